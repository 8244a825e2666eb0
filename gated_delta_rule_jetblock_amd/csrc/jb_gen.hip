// jb_gen.hip -- kernel generator (x -> conv taps), the standalone dynamic
// causal conv, the conv-cache tail copy and the matrix-core placement probe.
//
// Kernel generator (Jet-Nemotron csdn translation, section 2.4: it shares the
// Q/K/V projections' input, reduces with a Linear layer, applies SiLU, and a
// final Linear layer emits the conv-kernel weights; hidden width 32 and kernel
// size 4 per the xugj520 blog, section 2.2):
//     hidden = SiLU(W1 x + b1)   (32 units)     taps = W2 hidden + b2 (4 per head)
// The first layer is a [tokens x d_model] x [d_model x 32] product on the
// matrix cores (bf16 operands taken exactly from the inputs, fp32 accumulate;
// fp32 operands in the all-fp32 mode); SiLU and the small second layer run in
// fp32 on the vector ALUs.
#include "jb_device.h"
#include "jb_internal.h"

namespace jb {

constexpr int G = 32;        // generator hidden width

// Fragment of 8 contiguous K values (order 8g + j) straight from memory.
__device__ __forceinline__ void load8(const bf16_t* p, bool valid, bf16x8_t& out) {
  uint4 u = valid ? *reinterpret_cast<const uint4*>(p) : make_uint4(0u, 0u, 0u, 0u);
  out = *reinterpret_cast<bf16x8_t*>(&u);
}
__device__ __forceinline__ void load8(const float* p, bool valid, float (&out)[8]) {
  float4 a = valid ? *reinterpret_cast<const float4*>(p) : make_float4(0.f, 0.f, 0.f, 0.f);
  float4 b = valid ? *reinterpret_cast<const float4*>(p + 4) : make_float4(0.f, 0.f, 0.f, 0.f);
  out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
  out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
}

template <typename IO> struct GenFrag;
template <> struct GenFrag<bf16_t> {
  bf16x8_t v;
  __device__ __forceinline__ void load(const bf16_t* p, bool valid) { load8(p, valid, v); }
  __device__ __forceinline__ void mma(f4_t& acc, const GenFrag& b) const {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v, b.v, acc, 0, 0, 0);
  }
  __device__ __forceinline__ float get(int j) const { return (float)v[j]; }
};
template <> struct GenFrag<float> {
  float v[8];
  __device__ __forceinline__ void load(const float* p, bool valid) { load8(p, valid, v); }
  __device__ __forceinline__ float get(int j) const { return v[j]; }
  __device__ __forceinline__ void mma(f4_t& acc, const GenFrag& b) const {
#pragma unroll
    for (int j = 0; j < 8; ++j) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(v[j], b.v[j], acc, 0, 0, 0);
  }
};

// One workgroup: 16*NT tokens, NW wavefronts.  hidden^T (32 x tokens) =
// W1 (32 x D) x^T; wave w accumulates the K range [w D/NW, (w+1) D/NW) and
// the partials meet in LDS.  Few tokens per workgroup (decode) use many waves
// so that each wave's chain of dependent loads stays short.  The second
// layer, taps (tokens x 4H) = SiLU(hidden) W2^T, runs on the fp32 matrix
// cores, 16 x 16 tiles with the 32 hidden units as K.
template <typename IO, int NT, int NW>
__global__ __launch_bounds__(NW * 64, NT == 4 && sizeof(IO) == 2 ? 4 : 1) void gen_kernel(int64_t n, int D, int HK, const IO* x,
                                                                      const IO* W1, const IO* b1, const IO* W2,
                                                                      const IO* b2, float* taps, float* pre_out) {
  constexpr int NTOK = 16 * NT;
  constexpr int NTHREADS = NW * 64;
  constexpr int HALF = NW / 2;
  static_assert(NW % 2 == 0, "the cross-wave sum pairs the waves");
  __shared__ float red[HALF][G][NTOK];
  __shared__ float hid[NTOK][G + 1];
  __shared__ float b1s[G];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int m16 = lane & 15, g4 = lane >> 4;
  const int64_t n0 = (int64_t)blockIdx.x * NTOK;
  const float b1r = (tid < G && b1) ? to_f32<IO>(b1[tid]) : 0.f;

  f4_t acc[2][NT];
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[u][t] = zero4();

  // the wave's K range in blocks of KU 32-deep steps whose loads are all in
  // flight before the first product (one memory latency per block, not per step)
  constexpr int KU = NT == 1 ? 4 : 2;
  const int kq = D / NW, kend = (wave + 1) * kq;
  for (int k0 = wave * kq; k0 < kend; k0 += 32 * KU) {
    GenFrag<IO> A[KU][2], Bt[KU][NT];
#pragma unroll
    for (int s = 0; s < KU; ++s) {
      const int k = k0 + 32 * s;
      const bool kv = k < kend;
#pragma unroll
      for (int u = 0; u < 2; ++u) A[s][u].load(W1 + (int64_t)(u * 16 + m16) * D + k + 8 * g4, kv);
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const int64_t tok = n0 + t * 16 + m16;
        Bt[s][t].load(x + tok * D + k + 8 * g4, kv && tok < n);
      }
    }
#pragma unroll
    for (int s = 0; s < KU; ++s)
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int t = 0; t < NT; ++t) A[s][u].mma(acc[u][t], Bt[s][t]);  // zero fragments past kend add nothing
  }
  // lane holds hidden^T[u*16 + 4g + i][t*16 + m16].  Cross-wave sum in a
  // fixed order: waves HALF.. store, waves 0..HALF-1 add theirs, then the
  // HALF slots are summed.
  if (wave >= HALF) {
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) red[wave - HALF][u * 16 + 4 * g4 + i][t * 16 + m16] = acc[u][t][i];
  }
  if (tid < G) b1s[tid] = b1r;
  __syncthreads();
  if (wave < HALF) {
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) red[wave][u * 16 + 4 * g4 + i][t * 16 + m16] += acc[u][t][i];
  }
  __syncthreads();
  for (int e = tid; e < G * NTOK; e += NTHREADS) {
    const int u = e / NTOK, t = e % NTOK;
    float hsum = b1s[u];
#pragma unroll
    for (int w = 0; w < HALF; ++w) hsum += red[w][u][t];
    hid[t][u] = hsum / (1.0f + expf(-hsum));  // SiLU
    if (pre_out && n0 + t < n) pre_out[(n0 + t) * G + u] = hsum;  // for the backward pass
  }
  __syncthreads();
  // taps tile (rt, ct): rows n0 + 16 rt.., taps 16 ct..; lane supplies
  // hidden row 16 rt + m16 and W2 row 16 ct + m16 at K = 8g .. 8g + 7
  const int nct = (HK + 15) / 16;
  for (int tile = wave; tile < NT * nct; tile += NW) {
    const int rt = tile / nct, ct = tile % nct;
    const int r = ct * 16 + m16;
    const bool rv = r < HK;
    GenFrag<IO> w2f;
    w2f.load(W2 + (int64_t)min(r, HK - 1) * G + 8 * g4, rv);
    GenFrag<float> hf;
#pragma unroll
    for (int j = 0; j < 8; ++j) hf.v[j] = hid[rt * 16 + m16][8 * g4 + j];
    float wv[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) wv[j] = w2f.get(j);
    f4_t tp = zero4();
#pragma unroll
    for (int j = 0; j < 8; ++j) tp = __builtin_amdgcn_mfma_f32_16x16x4f32(hf.v[j], wv[j], tp, 0, 0, 0);
    // lane holds taps[n0 + 16 rt + 4g + i][16 ct + m16]
    const float bias = (rv && b2) ? to_f32<IO>(b2[r]) : 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t tok = n0 + rt * 16 + 4 * g4 + i;
      if (tok < n && rv) taps[tok * HK + r] = tp[i] + bias;
    }
  }
}

template <typename IO, int NT, int NW>
static void gen_launch(int64_t n, int D, int HK, const void* x, const void* W1, const void* b1, const void* W2,
                       const void* b2, float* taps, float* pre_out, hipStream_t stream) {
  const dim3 grid((unsigned)((n + 16 * NT - 1) / (16 * NT)));
  gen_kernel<IO, NT, NW><<<grid, NW * 64, 0, stream>>>(n, D, HK, (const IO*)x, (const IO*)W1, (const IO*)b1,
                                                      (const IO*)W2, (const IO*)b2, taps, pre_out);
}

template <typename IO>
static void gen_dispatch(int64_t n, int D, int HK, const void* x, const void* W1, const void* b1, const void* W2,
                         const void* b2, float* taps, float* pre_out, hipStream_t stream) {
  // few rows (decode): 16 tokens per workgroup over as many waves as d_model
  // allows, to spread the rows; many rows: 64 tokens per workgroup, 4 waves
  if (n <= 4096) {
    if ((D / 32) % 16 == 0) gen_launch<IO, 1, 16>(n, D, HK, x, W1, b1, W2, b2, taps, pre_out, stream);
    else if ((D / 32) % 8 == 0) gen_launch<IO, 1, 8>(n, D, HK, x, W1, b1, W2, b2, taps, pre_out, stream);
    else gen_launch<IO, 1, 4>(n, D, HK, x, W1, b1, W2, b2, taps, pre_out, stream);
  } else {
    gen_launch<IO, 4, 4>(n, D, HK, x, W1, b1, W2, b2, taps, pre_out, stream);
  }
}

hipError_t launch_gen_taps(int io, int64_t n, int D, int H, const void* x, const void* W1, const void* b1,
                           const void* W2, const void* b2, float* taps, hipStream_t stream, float* pre_out) {
  if (n == 0) return hipSuccess;
  if (io == IO_BF16) gen_dispatch<bf16_t>(n, D, 4 * H, x, W1, b1, W2, b2, taps, pre_out, stream);
  else gen_dispatch<float>(n, D, 4 * H, x, W1, b1, W2, b2, taps, pre_out, stream);
  return hipGetLastError();
}

// ------------------------------------------------------- standalone conv

// one thread per (b, t, h, column): v'_t = sum_j taps_t[j] v_{t-3+j}
template <typename IO>
__global__ void conv_kernel(int B, int T, int H, int dv, const float* taps, const IO* v, const IO* conv_in,
                            float* vconv) {
  const int64_t total = (int64_t)B * T * H * dv;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += (int64_t)gridDim.x * blockDim.x) {
    const int c = (int)(e % dv);
    const int64_t bth = e / dv;
    const int h = (int)(bth % H);
    const int64_t bt = bth / H;
    const int t = (int)(bt % T);
    const int b = (int)(bt / T);
    const float* tp = taps + bth * 4;
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int tt = t - 3 + j;
      float val = 0.f;
      if (tt >= 0) val = to_f32<IO>(v[(((int64_t)b * T + tt) * H + h) * dv + c]);
      else if (conv_in) val = to_f32<IO>(conv_in[(((int64_t)b * 3 + (3 + tt)) * H + h) * dv + c]);
      s += tp[j] * val;
    }
    vconv[e] = s;
  }
}

hipError_t launch_conv(int io, int B, int T, int H, int dv, const float* taps, const void* v, const void* conv_in,
                       float* vconv, hipStream_t stream) {
  const int64_t total = (int64_t)B * T * H * dv;
  if (total == 0) return hipSuccess;
  const int blocks = (int)((total + 255) / 256 < 65536 ? (total + 255) / 256 : 65536);
  if (io == IO_BF16)
    conv_kernel<bf16_t><<<blocks, 256, 0, stream>>>(B, T, H, dv, taps, (const bf16_t*)v, (const bf16_t*)conv_in, vconv);
  else
    conv_kernel<float><<<blocks, 256, 0, stream>>>(B, T, H, dv, taps, (const float*)v, (const float*)conv_in, vconv);
  return hipGetLastError();
}

// ------------------------------------------------------- conv cache tail

// conv_out[b][s] = row T_b-3+s of [conv_in; v] for sequence b; one thread
// per (b, h, c) reads all three sources before writing, so conv_out may alias
// conv_in.
template <typename IO>
__global__ void conv_tail_kernel(int B, int Tmax, int H, int dv, const IO* v, const IO* conv_in, IO* conv_out,
                                 const int* cu_seqlens, int64_t rows) {
  const int64_t total = (int64_t)B * H * dv;
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= total) return;
  const int c = (int)(e % dv);
  const int h = (int)((e / dv) % H);
  const int b = (int)(e / ((int64_t)dv * H));
  int64_t tok0;
  int T;
  seq_span(cu_seqlens, Tmax, rows, b, tok0, T);
  IO vals[3];
#pragma unroll
  for (int s = 0; s < 3; ++s) {
    const int t = T - 3 + s;
    if (t >= 0) vals[s] = v[((tok0 + t) * H + h) * dv + c];
    else if (conv_in) vals[s] = conv_in[(((int64_t)b * 3 + (3 + t)) * H + h) * dv + c];
    else vals[s] = from_f32<IO>(0.f);
  }
#pragma unroll
  for (int s = 0; s < 3; ++s) conv_out[(((int64_t)b * 3 + s) * H + h) * dv + c] = vals[s];
}

hipError_t launch_conv_tail(int io, int B, int T, int H, int dv, const void* v, const void* conv_in, void* conv_out,
                            hipStream_t stream, const int* cu_seqlens, int64_t rows) {
  const int64_t total = (int64_t)B * H * dv;
  if (rows < 0) rows = (int64_t)B * T;
  if (total == 0) return hipSuccess;
  const int blocks = (int)((total + 255) / 256);
  if (io == IO_BF16)
    conv_tail_kernel<bf16_t><<<blocks, 256, 0, stream>>>(B, T, H, dv, (const bf16_t*)v, (const bf16_t*)conv_in,
                                                         (bf16_t*)conv_out, cu_seqlens, rows);
  else
    conv_tail_kernel<float><<<blocks, 256, 0, stream>>>(B, T, H, dv, (const float*)v, (const float*)conv_in,
                                                        (float*)conv_out, cu_seqlens, rows);
  return hipGetLastError();
}

// ------------------------------------------------------- zero fill

__global__ void fill_zero_kernel(float* p, size_t n) {
  for (size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x; e < n; e += (size_t)gridDim.x * blockDim.x)
    p[e] = 0.f;
}

hipError_t launch_fill_zero(float* p, size_t n, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const size_t blocks = (n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096;
  fill_zero_kernel<<<(unsigned)blocks, 256, 0, stream>>>(p, n);
  return hipGetLastError();
}

// ------------------------------------------------------- placement probe

__global__ __launch_bounds__(64) void probe_kernel(int kind, const float* A, const float* B, float* D) {
  const int l = threadIdx.x, m = l & 15, g = l >> 4;
  f4_t acc = zero4();
  if (kind == 0) {
    Frag<_Float16> a, b;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      a.v[j] = (_Float16)A[m * 32 + kperm(g, j)];
      b.v[j] = (_Float16)B[kperm(g, j) * 16 + m];
    }
    mma(acc, a, b);
  } else if (kind == 1) {
    bf16_t ab[8], bb[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      ab[j] = f32_to_bf16(A[m * 32 + 8 * g + j]);
      bb[j] = f32_to_bf16(B[(8 * g + j) * 16 + m]);
    }
    bf16x8_t av = *reinterpret_cast<bf16x8_t*>(ab), bv = *reinterpret_cast<bf16x8_t*>(bb);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc, 0, 0, 0);
  } else {
    Frag<float> a, b;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      a.v[j] = A[m * 32 + kperm(g, j)];
      b.v[j] = B[kperm(g, j) * 16 + m];
    }
    mma(acc, a, b);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) D[(4 * g + i) * 16 + m] = acc[i];
}

hipError_t launch_probe_mfma(int kind, const float* A, const float* B, float* D, hipStream_t stream) {
  probe_kernel<<<1, 64, 0, stream>>>(kind, A, B, D);
  return hipGetLastError();
}

}  // namespace jb
