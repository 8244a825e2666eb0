// jb_backward.hip -- the gradient of the block (training; the pages train
// JetBlock inside the model: Jet-Nemotron csdn translation, sections 2.2 and
// 3.1), chunked like the forward pass.
//
// Per chunk of C = 64 tokens entering with state M0 and leaving with M_C
// (notation of jb_prefill.hip: A, T = (I + A)^{-1}, W = T diag(b gamma) K,
// U0 = T diag(b) V', U = U0 - W M0, P, gamma, D = e^{g_C - g}), given dO and
// the gradient dM of M_C:
//   chain (sequential, backwards over chunks):
//     dU = P^T dO + D K dM,   dM <- gamma_C dM + Q^T Gamma dO - W^T dU
//   per chunk (parallel):
//     dP = lower(dO U^T),  dQ = (dP.E) K + Gamma dO M0^T
//     dW = -dU M0^T,  dB_w = T^T dW,  dB_u = T^T dU,  dV' = diag(b) dB_u
//     dA = strictLower(-(dB_w W^T + dB_u U0^T)),  dS = dA . b_i E_ij
//     dK = (dP.E)^T Q + D (U dM^T) + diag(b gamma) dB_w + (dS + dS^T) K
//     db_i = gamma_i dB_w,i.k_i + dB_u,i.v'_i + sum_j dA_ij E_ij k_i.k_j
//     dg from P, from Gamma in O, from A, from gamma in W, from gamma_C and D
//     d ln a = reverse cumulative sum of dg within the chunk
// then through the L2 norms, the conv and the generator.  The gradients of o
// and S_final are scaled by a power of two (their largest magnitude brought
// to [0.5, 1)) before they meet fp16 matrix-core operands, and every result
// is scaled back, so the fp16 range never clips a gradient.  Likewise the
// forward values the pass re-forms (V', U0, U and the checkpointed states)
// carry one power of two sigma chosen from the largest |v|, |conv_in|, |taps|
// and |S0| (the block is linear in v' and S0): the gradients of q, k, alpha
// and beta, bilinear in forward and backward values, are scaled back by
// 1/sigma; those of v, conv_in, S0 and the taps do not depend on it.
#include "jb_chunk.h"
#include "jb_device.h"
#include "jb_internal.h"

namespace jb {

struct BwdArgs {
  int T, H, nchunks;
  const bf16_t* q;
  const bf16_t* k;
  const bf16_t* v;
  const bf16_t* conv_in;
  const float* alpha;
  const float* beta;
  const float* taps;      // [B][T][H][4]
  const float* dout;      // [B][T][H][DV]
  const float* dS_final;  // [B][H][DK][DV] or NULL
  const float* scale;     // [0] = s, [1] = 1/s, [2] = sigma, [3] = 1/(s sigma)
  const _Float16* Mck;    // [B][H][nchunks][DV/16][DK/16][64][4] fp16: the state entering each chunk, in
                          // accumulator tiles (lane l: rows 4 (l / 16) .. + 3 of column l % 16)
  _Float16* dMck;         // [B][H][nchunks][DK][DV]: s x the gradient of the state leaving each chunk (fp16: its
                          // products take it as an fp16 operand, and s keeps it in range)
  float* dU;              // [B][T][H][DV]: s x dU
  float* dS0;             // [B][H][DK][DV]
  float* dq;              // [B][T][H][DK]
  float* dk;
  float* dalpha;          // [B][T][H]
  float* dbeta;
  float* dvc;             // [B][T][H][DV]: dV'
  float* QO;              // [B][H][nchunks][C][DK]: s x dO M0^T per chunk
  float* WO;              // [B][H][nchunks][C][DK]: s x dU M0^T per chunk
  float* dgC;             // [B][H][nchunks]: s x sum(dM . M0) per chunk
  char* img;              // [B][H][nchunks] chain tiles (ChainImg)
};

// ------------------------------------------------------------ gradient scale

// The largest |dout| and |dS_final| as float bits (non-negative floats order
// like their bit patterns): a grid-stride pass, one atomic max per workgroup
// into word[0], which grad_scale_finish turns into scale[0] = 2^-e with
// max 2^-e in [0.5, 1) (1 when all are zero) and scale[1] = 2^e.
__global__ __launch_bounds__(256) void grad_absmax_kernel(const float* dout, int64_t n_out, const float* dS,
                                                          int64_t n_s, unsigned int* word) {
  __shared__ float sm[4];
  float m = 0.f;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  // dout in 16-byte pieces (its element count is a multiple of dv), dS_final by elements
  const float4* d4 = reinterpret_cast<const float4*>(dout);
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_out / 4; i += stride) {
    const float4 x = d4[i];
    m = fmaxf(m, fmaxf(fmaxf(fabsf(x.x), fabsf(x.y)), fmaxf(fabsf(x.z), fabsf(x.w))));
  }
  if (dS)
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_s; i += stride) m = fmaxf(m, fabsf(dS[i]));
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, WAVE));
  if ((threadIdx.x & 63) == 0) sm[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    const float mm = fmaxf(fmaxf(sm[0], sm[1]), fmaxf(sm[2], sm[3]));
    atomicMax(word, __float_as_uint(mm));
  }
}

// The largest |v| and |conv_in| (word[1]), |S0| (word[2]) and |taps| (word[3])
// as float bits, by the same grid-stride pattern (element counts are
// multiples of 8 for the bf16 tensors and of 4 for the float ones).
__global__ __launch_bounds__(256) void value_absmax_kernel(const bf16_t* v, int64_t n_v, const bf16_t* cin, int64_t n_c,
                                                           const float* S0, int64_t n_s, const float* taps,
                                                           int64_t n_t, unsigned int* word) {
  __shared__ unsigned int sm[3][4];
  unsigned int mv = 0u;
  float ms = 0.f, mt = 0.f;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x, i0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  // |bf16| orders like its low 15 bits
  for (int64_t i = i0; i < n_v / 8; i += stride) {
    const uint4 x = reinterpret_cast<const uint4*>(v)[i];
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) mv = max(mv, max(w[j] & 0x7fffu, (w[j] >> 16) & 0x7fffu));
  }
  if (cin)
    for (int64_t i = i0; i < n_c; i += stride) mv = max(mv, (uint32_t)cin[i] & 0x7fffu);
  if (S0)
    for (int64_t i = i0; i < n_s / 4; i += stride) {
      const float4 x = reinterpret_cast<const float4*>(S0)[i];
      ms = fmaxf(ms, fmaxf(fmaxf(fabsf(x.x), fabsf(x.y)), fmaxf(fabsf(x.z), fabsf(x.w))));
    }
  for (int64_t i = i0; i < n_t / 4; i += stride) {
    const float4 x = reinterpret_cast<const float4*>(taps)[i];
    mt = fmaxf(mt, fmaxf(fmaxf(fabsf(x.x), fabsf(x.y)), fmaxf(fabsf(x.z), fabsf(x.w))));
  }
  for (int o = 32; o > 0; o >>= 1) {
    mv = max(mv, (unsigned)__shfl_xor((int)mv, o, WAVE));
    ms = fmaxf(ms, __shfl_xor(ms, o, WAVE));
    mt = fmaxf(mt, __shfl_xor(mt, o, WAVE));
  }
  if ((threadIdx.x & 63) == 0) {
    sm[0][threadIdx.x >> 6] = mv << 16;  // the bf16 bits widened to a float's
    sm[1][threadIdx.x >> 6] = __float_as_uint(ms);
    sm[2][threadIdx.x >> 6] = __float_as_uint(mt);
  }
  __syncthreads();
  if (threadIdx.x < 3) {
    const unsigned int* r = sm[threadIdx.x];
    atomicMax(word + 1 + threadIdx.x, max(max(r[0], r[1]), max(r[2], r[3])));
  }
}

__global__ void grad_scale_start_kernel(unsigned int* word) {
#pragma unroll
  for (int i = 0; i < 4; ++i) word[i] = 0u;
}

// sigma = 2^-e with max(4 max|taps| max(|v|, |conv_in|), max|S0|) sigma in
// [2^8, 2^9) (1 when zero or not finite): the forward kernels' operand range.
__global__ void value_scale_finish_kernel(const unsigned int* word, float* scale) {
  const float mv = __uint_as_float(word[1]), ms = __uint_as_float(word[2]), mt = __uint_as_float(word[3]);
  const float mm = fmaxf(4.f * mt * mv, ms);
  int e = 9;
  if (mm > 0.f && isfinite(mm)) frexpf(mm, &e);  // mm = f 2^e, f in [0.5, 1)
  scale[2] = ldexpf(1.f, 9 - e);
  scale[3] = ldexpf(scale[1], e - 9);
}

__global__ void grad_scale_finish_kernel(const unsigned int* word, float* scale) {
  const float mm = __uint_as_float(word[0]);
  int e = 0;
  if (mm > 0.f && isfinite(mm)) frexpf(mm, &e);  // mm = f 2^e, f in [0.5, 1)
  scale[0] = ldexpf(1.f, -e);
  scale[1] = ldexpf(1.f, e);
}

// raw buffer loads: a wave-uniform resource and a per-lane byte offset; an
// offset at or beyond the resource's size reads as zero
__device__ __forceinline__ float buf_load_f32(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, 0, 0));
}
__device__ __forceinline__ float buf_load_bf16(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
  return bf16_to_f32(__builtin_amdgcn_raw_buffer_load_b16(r, (int)voff, 0, 0));
}

// ------------------------------------------------------------ chain kernel

// grid (nchunks, H, B), 8 waves: the Q^T and P^T chain tiles of one chunk
// (the checkpointing forward pass wrote its K, -W^T and gates): normalised q
// into LDS, the gated causal Q K^T blocks as P^T, both written out.  Every
// chunk is independent, so this runs at full occupancy ahead of the chain.
template <int DK>
__global__ __launch_bounds__(NTHR) void bwd_tiles_kernel(BwdArgs a) {
  using OP = _Float16;
  using I = ChainImg<DK>;
  constexpr int LDK = DK + 4, KB = DK / 32;
  constexpr int oKh = 0;                       // [C][LK] from the forward pass
  constexpr int oQh = oKh + C * I::LK * 2;     // [C][LDK]
  constexpr int oPt = oQh + C * LDK * 2;       // [C][LT]
  constexpr int oG = oPt + C * I::LT * 2;      // [C]
  constexpr int total = oG + C * 4;
  __shared__ __attribute__((aligned(16))) char smem[total];
  OP* sKh = reinterpret_cast<OP*>(smem + oKh);
  OP* sQh = reinterpret_cast<OP*>(smem + oQh);
  OP* sPt = reinterpret_cast<OP*>(smem + oPt);
  float* sG = reinterpret_cast<float*>(smem + oG);

  const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z, H = a.H, T = a.T;
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int m16 = lane & 15, g4 = lane >> 4;
  const int t0 = c * C, n = min(C, T - t0);
  const int64_t bh = (int64_t)b * H + h;
  char* im = a.img + (bh * a.nchunks + c) * I::bytes;

  // K and g from the forward pass
  for (int e = tid; e < C * I::LK * 2 / 16; e += NTHR)
    reinterpret_cast<uint4*>(sKh)[e] = reinterpret_cast<const uint4*>(im + I::oKh)[e];
  if (tid < C) sG[tid] = reinterpret_cast<const float*>(im + I::oG)[tid];
  // P^T below the block diagonal stays zero
  for (int e = tid; e < C * C; e += NTHR) {
    const int r = e / C, cc = e % C;
    if ((r >> 4) > (cc >> 4)) sPt[r * I::LT + cc] = (OP)0.f;
  }
  if (tid < PRO_THR) {
    Prologue<DK, bf16_t> pr;
    pr.load_global(a.q, a.k, ((int64_t)b * T + t0) * H + h, H, n);
    pr.finish(true);
#pragma unroll
    for (int e = 0; e < Prologue<DK, bf16_t>::E; ++e)
      sQh[pr.row * LDK + pr.part * Prologue<DK, bf16_t>::E + e] = (OP)pr.qv[e];
  }
  __syncthreads();
  // P^T block (tj, ti): keys of block tj against queries of block ti
  for (int t = wave; t < 10; t += NWAVE) {
    const int ti = (kLowI >> (2 * t)) & 3, tj = (kLowJ >> (2 * t)) & 3;
    f4_t acc = zero4();
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
      mma(acc, lds_frag<OP>(sKh, I::LK, tj * 16, kb * 32), lds_frag<OP>(sQh, LDK, ti * 16, kb * 32));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = tj * 16 + 4 * g4 + i, cc = ti * 16 + m16;
      sPt[r * I::LT + cc] = (OP)(cc >= r ? fast_exp2(sG[cc] - sG[r]) * acc[i] : 0.f);
    }
  }
  __syncthreads();
  for (int e = tid; e < C * I::LT * 2 / 16; e += NTHR)
    reinterpret_cast<uint4*>(im + I::oPt)[e] = reinterpret_cast<const uint4*>(sPt)[e];
  // Q^T from the row-major Q^ tile: 16-byte pieces of eight consecutive tokens
  // of one feature (the padding columns past C written as zeros)
  constexpr int PPT = I::LT / 8;  // pieces per Q^T row
  for (int e = tid; e < DK * PPT; e += NTHR) {
    const int d = e / PPT, r0 = (e % PPT) * 8;
    uint32_t w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = r0 + 2 * j;
      const OP lo = r < C ? sQh[r * LDK + d] : (OP)0.f, hi = r + 1 < C ? sQh[(r + 1) * LDK + d] : (OP)0.f;
      w[j] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
    }
    *reinterpret_cast<uint4*>(im + I::oQt + (d * I::LT + r0) * 2) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// grid (H, B), one wave per dv column tile (DV / 16 waves); wave w owns
// column tile w of dM, kept in accumulator registers while the chunks are
// walked backwards.  A chunk's tiles (bwd_tiles_kernel) stream into one of
// two LDS buffers while the previous chunk is worked, and its dO tile into
// registers, so a chunk costs one barrier and its products.
template <int DK, int DV>
__global__ __launch_bounds__(DV / 16 * 64, 1) void bwd_chain_kernel(BwdArgs a) {
  using OP = _Float16;
  using I = ChainImg<DK>;
  constexpr int NW = DV / 16, RT = DK / 16, KB = DK / 32;
  static_assert(NW <= 16, "one wave per column tile");
  __shared__ __attribute__((aligned(16))) char smem[2 * I::bytes];

  const int h = blockIdx.x, b = blockIdx.y, H = a.H, T = a.T;
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int m16 = lane & 15, g4 = lane >> 4;
  const int64_t bh = (int64_t)b * H + h;
  const float s = a.scale[0];
  const int col = wave * 16 + m16;

  f4_t dM[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      dM[rt][i] = a.dS_final ? s * a.dS_final[(bh * DK + rt * 16 + 4 * g4 + i) * DV + col] : 0.f;

  // dO, dU and dM rows through buffer resources: byte offsets are a 32-bit
  // lane part (row 4g, this column) plus a wave-uniform row part, and rows
  // past the chunk read zero / drop their stores
  const uint32_t rowb = (uint32_t)(H * DV * 4);
  const int ov = (int)(4 * g4 * rowb) + col * 4, om = (4 * g4 * DV + col) * 2;
  // chunk cc's tiles into LDS buffer cc & 1, its dO tile (accumulator layout, scaled) into dOn
  f4_t dOn[4];
  auto issue = [&](int cc) {
    const char* src = a.img + (bh * a.nchunks + cc) * I::bytes;
    char* dstl = smem + (cc & 1) * I::bytes;
    for (int j = wave; j * 64 < I::bytes / 16; j += NW) {
      const int p = j * 64 + lane;
      if (p < I::bytes / 16) dma16(src + p * 16, dstl + j * 64 * 16);
    }
    const int t0 = cc * C, n = min(C, T - t0);
    const __amdgpu_buffer_rsrc_t rO = make_rsrc(a.dout + (((int64_t)b * T + t0) * H + h) * DV, (uint32_t)n * rowb);
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        dOn[rt][i] = s * __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rO, ov, (int)((rt * 16 + i) * rowb), 0));
  };
  if (a.nchunks > 0) issue(a.nchunks - 1);

  for (int c = a.nchunks - 1; c >= 0; --c) {
    const int t0 = c * C, n = min(C, T - t0);
    __builtin_amdgcn_s_waitcnt(0);  // this wave's tile transfers and dO loads have landed
    __syncthreads();                // ... and every other wave's; the other buffer is free
    f4_t dOr[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) dOr[rt] = dOn[rt];
    if (c > 0) issue(c - 1);
    // an opaque buffer offset: the LDS addresses of both buffers would
    // otherwise be formed once, outside the loop, and held in registers
    int boff = (c & 1) * I::bytes;
    asm volatile("" : "+s"(boff));
    const char* img = smem + boff;
    const OP* sKh = reinterpret_cast<const OP*>(img + I::oKh);
    const OP* sQt = reinterpret_cast<const OP*>(img + I::oQt);
    const OP* sWt = reinterpret_cast<const OP*>(img + I::oWt);
    const OP* sPt = reinterpret_cast<const OP*>(img + I::oPt);
    const float* sGam = reinterpret_cast<const float*>(img + I::oGam);
    const float* sDec = reinterpret_cast<const float*>(img + I::oDec);
    const float gamC = sGam[C - 1];
    // dU = D (K dM) + P^T dO: K dM first, scaled by D row by row, then the
    // P^T dO products accumulate onto it (one accumulator set)
    f4_t dU[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) dU[rt] = zero4();
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const Frag<OP> fm = acc_frag<OP>(dM[2 * kb], dM[2 * kb + 1]);
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) mma(dU[rt], lds_frag<OP>(sKh, I::LK, rt * 16, kb * 32), fm);
    }
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i) dU[rt][i] *= sDec[rt * 16 + 4 * g4 + i];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const Frag<OP> fo = acc_frag<OP>(dOr[2 * kb], dOr[2 * kb + 1]);
#pragma unroll
      for (int rt = 0; rt < 4; ++rt)
        if (kb * 32 + 31 >= rt * 16) mma(dU[rt], lds_frag<OP>(sPt, I::LT, rt * 16, kb * 32), fo);
    }
    // the gradient of the chunk-end state and dU, for the per-chunk pass
    const __amdgpu_buffer_rsrc_t rM = make_rsrc(a.dMck + ((bh * a.nchunks + c) * DK) * DV, (uint32_t)(DK * DV * 2));
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        buf_store(rM, __builtin_bit_cast(bf16_t, (_Float16)dM[rt][i]), om, (rt * 16 + i) * DV * 2);  // fp16 bits
    const __amdgpu_buffer_rsrc_t rU = make_rsrc(a.dU + (((int64_t)b * T + t0) * H + h) * DV, (uint32_t)n * rowb);
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i) buf_store(rU, dU[rt][i], ov, (int)((rt * 16 + i) * rowb));  // rows past n dropped
    // dM <- gamma_C dM + Q^T Gamma dO - W^T dU
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i) dM[rt][i] *= gamC;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      Frag<OP> fo;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        fo.v[j] = (OP)(dOr[2 * kb][j] * sGam[kb * 32 + 4 * g4 + j]);
        fo.v[4 + j] = (OP)(dOr[2 * kb + 1][j] * sGam[kb * 32 + 16 + 4 * g4 + j]);
      }
      const Frag<OP> fu = acc_frag<OP>(dU[2 * kb], dU[2 * kb + 1]);
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        mma(dM[rt], lds_frag<OP>(sQt, I::LT, rt * 16, kb * 32), fo);
        mma(dM[rt], lds_frag<OP>(sWt, I::LT, rt * 16, kb * 32), fu);
      }
    }
  }

  const float inv = a.scale[1];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int i = 0; i < 4; ++i) a.dS0[(bh * DK + rt * 16 + 4 * g4 + i) * DV + col] = dM[rt][i] * inv;
}

// ------------------------------------------------------------ per-chunk gradients

// one DPP-moved copy of v: CTRL is a row rotation (0x12r) or a quad permutation
template <int CTRL> __device__ __forceinline__ float dpp_mov(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
// sum over the 16 lanes of a DPP row, in every lane of the row: rotations by 8
// and 4 within the row, then the two quad swaps
__device__ __forceinline__ float sum16(float v) {
  v += dpp_mov<0x128>(v);
  v += dpp_mov<0x124>(v);
  v += dpp_mov<0x4E>(v);
  v += dpp_mov<0xB1>(v);
  return v;
}

// sum of v over the 4 lane groups at the same lane position
__device__ __forceinline__ float sum_groups(float v) {
  v += __shfl_xor(v, 16, WAVE);
  v += __shfl_xor(v, 32, WAVE);
  return v;
}

// Y = (I + A)^{-T} R for a 64 x 16 right-hand side in accumulator layout:
// backward substitution over the transposed blocks; sAnT holds -A^T and sLiT
// the transposed diagonal-block inverses (columns 16..31 zero).
template <int LC, int LLI>
__device__ __forceinline__ void block_solve_t(f4_t (&Y)[4], const _Float16* sAnT, const _Float16* sLiT) {
  using OP = _Float16;
  const f4_t z = zero4();
  f4_t t = zero4();
  mma(t, lds_frag<OP>(sLiT, LLI, 48, 0), acc_frag<OP>(Y[3], z));
  Y[3] = t;
  mma(Y[2], lds_frag<OP>(sAnT, LC, 32, 32), acc_frag<OP>(z, Y[3]));
  t = zero4();
  mma(t, lds_frag<OP>(sLiT, LLI, 32, 0), acc_frag<OP>(Y[2], z));
  Y[2] = t;
  const Frag<OP> f23 = acc_frag<OP>(Y[2], Y[3]);
  mma(Y[1], lds_frag<OP>(sAnT, LC, 16, 32), f23);
  mma(Y[0], lds_frag<OP>(sAnT, LC, 0, 32), f23);
  t = zero4();
  mma(t, lds_frag<OP>(sLiT, LLI, 16, 0), acc_frag<OP>(Y[1], z));
  Y[1] = t;
  mma(Y[0], lds_frag<OP>(sAnT, LC, 0, 0), acc_frag<OP>(z, Y[1]));
  t = zero4();
  mma(t, lds_frag<OP>(sLiT, LLI, 0, 0), acc_frag<OP>(Y[0], z));
  Y[0] = t;
}

// dO M0^T and dU M0^T of every chunk (C x DK each, reduced over dv) and the
// chunk-end gate term sum(dM . M0).  grid (nchunks, H, B), 8 waves: M0 (kept
// in fp16) is read once into LDS (its rows are the B operand of both products),
// dM alongside it for the gate term; wave w then forms row tile w % 4 of
// dO M0^T (w < 4) or of dU M0^T, all DK columns, its A operand streamed from
// global memory.  No operand is read twice, and two workgroups share a
// compute unit.
template <int DK, int DV>
__global__ __launch_bounds__(NTHR, 2) void bwd_dvred_kernel(BwdArgs a) {
  using OP = _Float16;
  constexpr int LDM = DV + 8;              // fp16 row stride of the staged M0
  constexpr int CT = DK / 16;              // column tiles
  constexpr int KSTEP = DV / 32;           // 32-deep steps over dv
  constexpr int NV4 = DK * DV / 4 / NTHR;  // groups of four M0 (and dM) elements per thread
  constexpr int R = NV4 % 6 == 0 ? 6 : NV4 % 4 == 0 ? 4 : 1;  // groups per staging round
  static_assert(DK * DV % (4 * NTHR) == 0 && NV4 % R == 0, "whole float4s per thread");
  __shared__ __attribute__((aligned(16))) OP sM0[DK * LDM];
  __shared__ float sg[NWAVE];
  const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z, H = a.H, T = a.T;
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int m16 = lane & 15, g4 = lane >> 4;
  const int64_t bh = (int64_t)b * H + h;
  const int t0 = c * C, n = min(C, T - t0);
  const int64_t tokbase = ((int64_t)b * T + t0) * H + h;
  const uint2* M0 = reinterpret_cast<const uint2*>(a.Mck + ((bh * a.nchunks + c) * DK) * DV);  // a lane's 4 fp16
  const uint2* dMC = reinterpret_cast<const uint2*>(a.dMck + ((bh * a.nchunks + c) * DK) * DV);  // a lane's 4 fp16

  // this wave's A operand, 16 rows of dO (scaled) or of dU, issued first so
  // that its loads are in flight while M0 is staged
  const bool isU = wave >= 4;
  const int rt = wave & 3;
  const int row = rt * 16 + m16;
  const float* A = (isU ? a.dU : a.dout) + (tokbase + (int64_t)min(row, n - 1) * H) * DV + 4 * g4;
  const float sc = row < n ? (isU ? 1.f : a.scale[0]) : 0.f;  // clamped row, masked value
  float4 ra[KSTEP][2];
#pragma unroll
  for (int ks = 0; ks < KSTEP; ++ks) {
    ra[ks][0] = *reinterpret_cast<const float4*>(A + ks * 32);
    ra[ks][1] = *reinterpret_cast<const float4*>(A + ks * 32 + 16);
  }

  // M0 tiles (lane groups of 4 rows) into LDS rows
#pragma unroll
  for (int j0 = 0; j0 < NV4; j0 += R) {
    uint2 m[R];
#pragma unroll
    for (int j = 0; j < R; ++j) m[j] = M0[(j0 + j) * NTHR + tid];
#pragma unroll
    for (int j = 0; j < R; ++j) {
      const int e = (j0 + j) * NTHR + tid, tile = e >> 6, ln = e & 63;
      const int row = (tile % (DK / 16)) * 16 + 4 * (ln >> 4), col = (tile / (DK / 16)) * 16 + (ln & 15);
      const half4_t hv = __builtin_bit_cast(half4_t, m[j]);
#pragma unroll
      for (int i = 0; i < 4; ++i) sM0[(row + i) * LDM + col] = hv[i];
    }
  }
  lds_barrier();  // the A loads stay in flight
  // the gate term: dM rows (fp16, row-major) against the staged M0
  float part = 0.f;
#pragma unroll
  for (int j0 = 0; j0 < NV4; j0 += R) {
    uint2 d[R];
#pragma unroll
    for (int j = 0; j < R; ++j) d[j] = dMC[(j0 + j) * NTHR + tid];
#pragma unroll
    for (int j = 0; j < R; ++j) {
      const int e = (j0 + j) * NTHR + tid;
      const half4_t hv = *reinterpret_cast<const half4_t*>(sM0 + (e / (DV / 4)) * LDM + (e % (DV / 4)) * 4);
      const half4_t dv4 = __builtin_bit_cast(half4_t, d[j]);
      part += (float)hv[0] * (float)dv4[0] + (float)hv[1] * (float)dv4[1] + (float)hv[2] * (float)dv4[2] +
              (float)hv[3] * (float)dv4[3];
    }
  }
  part = wave_sum(part);
  if (lane == 0) sg[wave] = part;

  f4_t acc[CT];
#pragma unroll
  for (int j = 0; j < CT; ++j) acc[j] = zero4();
#pragma unroll
  for (int ks = 0; ks < KSTEP; ++ks) {
    Frag<OP> fa;
    const float4 lo = ra[ks][0], hi = ra[ks][1];
    fa.v[0] = (OP)(lo.x * sc); fa.v[1] = (OP)(lo.y * sc); fa.v[2] = (OP)(lo.z * sc); fa.v[3] = (OP)(lo.w * sc);
    fa.v[4] = (OP)(hi.x * sc); fa.v[5] = (OP)(hi.y * sc); fa.v[6] = (OP)(hi.z * sc); fa.v[7] = (OP)(hi.w * sc);
#pragma unroll
    for (int j = 0; j < CT; ++j) mma(acc[j], fa, lds_frag<OP>(sM0, LDM, j * 16, ks * 32));
  }
  float* out = (isU ? a.WO : a.QO) + ((bh * a.nchunks + c) * C + rt * 16 + 4 * g4) * DK + m16;
#pragma unroll
  for (int j = 0; j < CT; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) out[i * DK + j * 16] = acc[j][i];
  lds_barrier();  // sg
  if (tid == 0) {
    float tot = 0.f;
#pragma unroll
    for (int w = 0; w < NWAVE; ++w) tot += sg[w];
    a.dgC[bh * a.nchunks + c] = tot;
  }
}

// grid (nchunks, H, B), 8 waves.  The dv columns are taken 128 at a time:
// each wave forms one 16-column tile of that block's U0, U and dB_u
// (accumulator layout, staged in LDS as fp16), then every wave adds the
// block's share of the dv-reduced products it owns: C x C tiles of dP and
// dB_u U0^T (jobs spread over the waves), and for wave w < DK/16 column tile
// w of U dM^T.  dO M0^T and dU M0^T come from bwd_dvred_kernel.
template <int DK, int DV>
__global__ __launch_bounds__(NTHR, 1) void bwd_grad_kernel(BwdArgs a) {
  using OP = _Float16;
  constexpr int LDK = DK + 4, LC = C + 4, LAD = 20, LLI = 36, KW = DV >= 128 ? 128 : DV, LKW = KW + 8;
  constexpr int RT = DK / 16, KB = DK / 32, NKB = DV / KW, KS = KW / 32;
  // the per-row scalars first: below 64 KB every LDS address is one register
  // plus an immediate offset
  constexpr int oScal = 0;                            // g, gamma, beta, D, taps [C][4], norms, sums
  constexpr int nScal = 4 * C + 4 * C + 2 * C + 6 * C + 4;
  constexpr int oKh = oScal + nScal * 4;
  constexpr int oQh = oKh + C * LDK * 2;
  constexpr int oW = oQh + C * LDK * 2;
  constexpr int oAn = oW + C * LDK * 2;
  constexpr int oAnT = oAn + C * LC * 2;
  constexpr int oAd = oAnT + C * LC * 2;
  constexpr int oLi = oAd + C * LAD * 4;
  constexpr int oLiT = oLi + C * LLI * 2;
  constexpr int oU = oLiT + C * LLI * 2;              // union: staging during the dv loop, then dP.E, dS, dB_w
  constexpr int szStage = 4 * C * LKW * 2;
  constexpr int szPost = 2 * C * LC * 2 + C * LDK * 2;
  constexpr int total = oU + (szStage > szPost ? szStage : szPost);
  static_assert(total <= 160 * 1024, "LDS budget");
  static_assert(RT <= NWAVE, "one wave per dk column tile");
  __shared__ __attribute__((aligned(16))) char smem[total];
  OP* sKh = reinterpret_cast<OP*>(smem + oKh);
  OP* sQh = reinterpret_cast<OP*>(smem + oQh);
  OP* sW = reinterpret_cast<OP*>(smem + oW);      // [C][LDK] W
  OP* sAn = reinterpret_cast<OP*>(smem + oAn);    // [C][LC] -A
  OP* sAnT = reinterpret_cast<OP*>(smem + oAnT);  // [C][LC] -A^T
  float* sAd = reinterpret_cast<float*>(smem + oAd);
  OP* sLi = reinterpret_cast<OP*>(smem + oLi);
  OP* sLiT = reinterpret_cast<OP*>(smem + oLiT);
  float* sG = reinterpret_cast<float*>(smem + oScal);
  float* sGam = sG + C;
  float* sBeta = sG + 2 * C;
  float* sDec = sG + 3 * C;
  float* sTap = sG + 4 * C;        // [C][4]
  float* sNq = sTap + 4 * C;       // norms of the raw q, k rows
  float* sNk = sNq + C;
  float* sDg = sNk + C;            // d g (before the reverse cumsum)
  float* sDb = sDg + C;            // d beta
  float* sDD = sDb + C;            // k_i . (U dM^T)_i (the D term)
  float* sQd = sDD + C;            // q_i . dq^_i and k_i . dk^_i (norm backward)
  float* sKd = sQd + C;
  OP* sUb = reinterpret_cast<OP*>(smem + oU);        // [C][LKW] U of the current dv block
  OP* sU0b = sUb + C * LKW;                          // U0
  OP* sBub = sU0b + C * LKW;                         // dB_u
  OP* sdOb = sBub + C * LKW;                         // s dO
  OP* sdPE = reinterpret_cast<OP*>(smem + oU);       // after the loop: [C][LC] dP . E
  OP* sdS = sdPE + C * LC;                           // [C][LC] dS
  OP* sdBw = sdS + C * LC;                           // [C][LDK] dB_w

  const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z, H = a.H, T = a.T;
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int m16 = lane & 15, g4 = lane >> 4;
  const int64_t bh = (int64_t)b * H + h;
  const int t0 = c * C, n = min(C, T - t0);
  // s, 1/s: the gradient scale; vs: sigma, the forward values' scale; invq = 1/(s sigma)
  const float s = a.scale[0], inv = a.scale[1], vs = a.scale[2], invq = a.scale[3];
  const int64_t tokbase = ((int64_t)b * T + t0) * H + h;
  const _Float16* M0 = a.Mck + ((bh * a.nchunks + c) * DK) * DV;
  const _Float16* dMC = a.dMck + ((bh * a.nchunks + c) * DK) * DV;
  const float* dO = a.dout + tokbase * DV;
  const float* dUg = a.dU + tokbase * DV;

  // ---- prologue: normalised q, k, gates, taps, norms
  if (tid < PRO_THR) {
    Prologue<DK, bf16_t> pr;
    pr.load_global(a.q, a.k, tokbase, H, n);
    // raw norms for the backward of the normalisation
    float sk = 0.f, sq = 0.f;
#pragma unroll
    for (int e = 0; e < Prologue<DK, bf16_t>::E; ++e) { sk += pr.kv[e] * pr.kv[e]; sq += pr.qv[e] * pr.qv[e]; }
    sk = group_sum<8>(sk);
    sq = group_sum<8>(sq);
    if (pr.part == 0) {
      sNk[pr.row] = sqrtf(sk + 1e-6f);
      sNq[pr.row] = sqrtf(sq + 1e-6f);
    }
    pr.finish(true);
#pragma unroll
    for (int e = 0; e < Prologue<DK, bf16_t>::E; ++e) {
      const int d = pr.part * Prologue<DK, bf16_t>::E + e;
      sKh[pr.row * LDK + d] = (OP)pr.kv[e];
      sQh[pr.row * LDK + d] = (OP)pr.qv[e];
    }
  }
  if (wave == GATE_WAVE) {
    const bool valid = lane < n;
    const int64_t gi = tokbase + (int64_t)min(lane, n - 1) * H;  // clamped, then masked
    const float al0 = a.alpha[gi], be0 = a.beta[gi];
    const float4 tp0 = *reinterpret_cast<const float4*>(a.taps + gi * 4);
    const float al = valid ? al0 : 1.f;
    const float be = valid ? be0 : 0.f;
    const float4 tp = valid ? tp0 : make_float4(0.f, 0.f, 0.f, 0.f);
    const float g = chunk_gate_scan(al);
    const float gC = __shfl(g, C - 1, WAVE);
    sG[lane] = g;
    sGam[lane] = fast_exp2(g);
    sBeta[lane] = be;
    sDec[lane] = fast_exp2(gC - g);
    *reinterpret_cast<float4*>(sTap + lane * 4) = tp;
    sDg[lane] = 0.f;
    sDb[lane] = 0.f;
    sDD[lane] = 0.f;
    sQd[lane] = 0.f;
    sKd[lane] = 0.f;
  }
  __syncthreads();

  // ---- -A, its transpose and diagonal blocks
  for (int t = wave; t < 10; t += NWAVE) {
    const int ti = (kLowI >> (2 * t)) & 3, tj = (kLowJ >> (2 * t)) & 3;
    f4_t acc = zero4();
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
      mma(acc, lds_frag<OP>(sKh, LDK, ti * 16, kb * 32), lds_frag<OP>(sKh, LDK, tj * 16, kb * 32));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = ti * 16 + 4 * g4 + i, cc = tj * 16 + m16;
      const float av = cc < r ? sBeta[r] * fast_exp2(sG[r] - sG[cc]) * acc[i] : 0.f;
      sAn[r * LC + cc] = (OP)(-av);
      sAnT[cc * LC + r] = (OP)(-av);
      if (ti != tj) sAnT[r * LC + cc] = (OP)0.f;  // the mirror tile of -A^T is zero
      if (ti == tj) sAd[r * LAD + m16] = av;
    }
  }
  __syncthreads();
  if (wave == 0) {
    const int base = (lane >> 4) * 16, jc = lane & 15;
    float x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float acc = (i == jc) ? 1.f : 0.f;
      const float* arow = sAd + (base + i) * LAD;
#pragma unroll
      for (int k4 = 0; k4 < i; k4 += 4) {
        const float4 av = *reinterpret_cast<const float4*>(arow + k4);
        acc -= av.x * x[k4];
        if (k4 + 1 < i) acc -= av.y * x[k4 + 1];
        if (k4 + 2 < i) acc -= av.z * x[k4 + 2];
        if (k4 + 3 < i) acc -= av.w * x[k4 + 3];
      }
      x[i] = acc;
      if ((i & 3) == 3) __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      sLi[(base + i) * LLI + jc] = (OP)x[i];
      sLi[(base + i) * LLI + 16 + jc] = (OP)0.f;
      sLiT[(base + jc) * LLI + i] = (OP)x[i];
      sLiT[(base + i) * LLI + 16 + jc] = (OP)0.f;
    }
  }
  __syncthreads();
  if (wave < RT) {
    f4_t Y[4];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = rb * 16 + 4 * g4 + i;
        Y[rb][i] = sBeta[r] * sGam[r] * (float)sKh[r * LDK + wave * 16 + m16];
      }
    block_solve<OP, LC, LLI>(Y, sAn, sLi);
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
      for (int i = 0; i < 4; ++i) sW[(rb * 16 + 4 * g4 + i) * LDK + wave * 16 + m16] = (OP)Y[rb][i];
  }
  __syncthreads();

  // ---- the dv-reduced products, KW columns at a time
  f4_t accCC[3];                       // C x C jobs: wave, wave + 8, wave + 16 of {dP tiles, dB_u U0^T tiles}
  f4_t aQO[4], aKM[4], aW[4];          // column tile `wave` of dO M0^T, U dM^T, dU M0^T
#pragma unroll
  for (int i = 0; i < 3; ++i) accCC[i] = zero4();
#pragma unroll
  for (int i = 0; i < 4; ++i) { aQO[i] = zero4(); aKM[i] = zero4(); aW[i] = zero4(); }
  // Byte-addressed resources over the chunk's rows (row r at r * row stride):
  // rows at or beyond n fall outside them, so loads read zero and stores are
  // dropped without a branch.  The three value rows before the chunk come
  // from the previous chunk, or for the first chunk from the conv cache
  // (laid out [B][3][H][DV]: the same row stride), else read as zero.
  const uint32_t rowv = (uint32_t)(H * DV * 2), rowf = (uint32_t)(H * DV * 4);
  const __amdgpu_buffer_rsrc_t rV = make_rsrc(a.v + tokbase * DV, (uint32_t)(n - 1) * rowv + DV * 2);
  const bf16_t* halo = c > 0 ? a.v + (tokbase - 3 * (int64_t)H) * DV
                     : a.conv_in ? a.conv_in + ((int64_t)b * 3 * H + h) * DV : a.v;
  const __amdgpu_buffer_rsrc_t rVh = make_rsrc(halo, (c > 0 || a.conv_in) ? 2 * rowv + DV * 2 : 0u);
  const __amdgpu_buffer_rsrc_t rdU = make_rsrc(dUg, (uint32_t)(n - 1) * rowf + DV * 4);
  const __amdgpu_buffer_rsrc_t rdO = make_rsrc(dO, (uint32_t)(n - 1) * rowf + DV * 4);
  const __amdgpu_buffer_rsrc_t rdvc = make_rsrc(a.dvc + tokbase * DV, (uint32_t)(n - 1) * rowf + DV * 4);
#pragma unroll 1
  for (int kb = 0; kb < NKB; ++kb) {
    if (wave < KW / 16) {
      const int col = kb * KW + wave * 16 + m16;
      // the lane's row 4g of the chunk as byte offsets; an opaque copy, so that
      // the offsets derived from it are formed here and not kept in registers
      // across the loop
      uint32_t ov = 4 * g4 * rowv + col * 2, of = 4 * g4 * rowf + col * 4;
      asm volatile("" : "+v"(ov), "+v"(of));
      // V' (the conv of the raw value rows with the chunk's taps): a lane's
      // four rows 4g..4g+3 of a row tile read the seven value rows 4g-3..4g+3;
      // a row before the chunk has a negative offset in rV (out of range, so
      // zero) and its own in the halo resource
      f4_t Vp[4], Y[4];
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        float xr[7];
#pragma unroll
        for (int m = 0; m < 7; ++m) {
          const int dr = rt * 16 + m - 3;  // row offset from 4g
          xr[m] = buf_load_bf16(rV, ov + (uint32_t)dr * rowv);
          if (rt == 0 && m < 3) xr[m] += buf_load_bf16(rVh, ov + (uint32_t)(m * rowv));
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = rt * 16 + 4 * g4 + i;
          const float4 tp = *reinterpret_cast<const float4*>(sTap + r * 4);
          const float acc = (tp.x * xr[i] + tp.y * xr[i + 1] + tp.z * xr[i + 2] + tp.w * xr[i + 3]) * vs;
          Vp[rt][i] = acc;
          Y[rt][i] = sBeta[r] * acc;
        }
      }
      // the value loads and the conv stay ahead of the solve: interleaved with
      // it by the scheduler, the whole column pass takes half again as long
      __builtin_amdgcn_sched_barrier(0);
      block_solve<OP, LC, LLI>(Y, sAn, sLi);  // U0
      // U = U0 - W M0 (M0 tile in accumulator layout)
      f4_t m0[RT], tw[4];
      // M0 tiles of this column tile: one 8-byte load per row tile
      const half4_t* m0t = reinterpret_cast<const half4_t*>(M0) + (kb * (KW / 16) + wave) * RT * 64 + lane;
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const half4_t hv = m0t[rt * 64];
#pragma unroll
        for (int i = 0; i < 4; ++i) m0[rt][i] = (float)hv[i];
      }
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) tw[rt] = zero4();
#pragma unroll
      for (int k2 = 0; k2 < KB; ++k2) {
        const Frag<OP> fm = acc_frag<OP>(m0[2 * k2], m0[2 * k2 + 1]);
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) mma(tw[rt], lds_frag<OP>(sW, LDK, rt * 16, k2 * 32), fm);
      }
      // dB_u = T^T dU
      f4_t dB[4];
#pragma unroll
      for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i) dB[rt][i] = buf_load_f32(rdU, of + (uint32_t)(rt * 16 + i) * rowf);
      block_solve_t<LC, LLI>(dB, sAnT, sLiT);
      // this column of dO, staged in LDS for the dP jobs
      float xo[4][4];
#pragma unroll
      for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i) xo[rt][i] = buf_load_f32(rdO, of + (uint32_t)(rt * 16 + i) * rowf);
#pragma unroll
      for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = rt * 16 + 4 * g4 + i;
          const float u = Y[rt][i] - tw[rt][i];
          sUb[r * LKW + wave * 16 + m16] = (OP)u;
          sU0b[r * LKW + wave * 16 + m16] = (OP)Y[rt][i];
          sBub[r * LKW + wave * 16 + m16] = (OP)dB[rt][i];
          sdOb[r * LKW + wave * 16 + m16] = (OP)(s * xo[rt][i]);
          // dV' = b dB_u (unscaled), and b's share dB_u . V'
          buf_store(rdvc, sBeta[r] * dB[rt][i] * inv, (int)(of + (uint32_t)(rt * 16 + i) * rowf), 0);
          const float db = sum16(dB[rt][i] * Vp[rt][i]);
          if (m16 == 0) atomicAdd(&sDb[r], db);
        }
    }
    __syncthreads();
    // C x C jobs: 0..9 dP tiles, 10..19 dB_u U0^T tiles
#pragma unroll 1
    for (int ks = 0; ks < KS; ++ks) {
      const int k0 = kb * KW + ks * 32;
#pragma unroll
      for (int jj = 0; jj < 3; ++jj) {
        const int job = wave + jj * NWAVE;
        if (job < 20) {
          const int which = job >= 10, t = job - 10 * which;
          const int ti = (kLowI >> (2 * t)) & 3, tj = (kLowJ >> (2 * t)) & 3;
          if (which == 0)
            mma(accCC[jj], lds_frag<OP>(sdOb, LKW, ti * 16, ks * 32), lds_frag<OP>(sUb, LKW, tj * 16, ks * 32));
          else
            mma(accCC[jj], lds_frag<OP>(sBub, LKW, ti * 16, ks * 32), lds_frag<OP>(sU0b, LKW, tj * 16, ks * 32));
        }
      }
      if (wave < RT) {
        // dM rows 16 wave + m16 at K = k0 + 4 g4 .. + 3 and k0 + 16 + 4 g4 .. + 3 (fp16 as stored)
        Frag<OP> fdm;
        {
          const _Float16* pr = dMC + (wave * 16 + m16) * DV + k0 + 4 * g4;
          const half4_t lo = *reinterpret_cast<const half4_t*>(pr), hi = *reinterpret_cast<const half4_t*>(pr + 16);
#pragma unroll
          for (int j = 0; j < 4; ++j) { fdm.v[j] = lo[j]; fdm.v[4 + j] = hi[j]; }
        }
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) mma(aKM[rt], lds_frag<OP>(sUb, LKW, rt * 16, ks * 32), fdm);
      }
    }
    __syncthreads();
  }
  // dO M0^T and dU M0^T (bwd_dvred_kernel): column tile `wave` into registers
  if (wave < RT) {
    const float* qo = a.QO + ((bh * a.nchunks + c) * C) * DK + wave * 16 + m16;
    const float* wo = a.WO + ((bh * a.nchunks + c) * C) * DK + wave * 16 + m16;
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        aQO[rt][i] = qo[(rt * 16 + 4 * g4 + i) * DK];
        aW[rt][i] = wo[(rt * 16 + 4 * g4 + i) * DK];
      }
  }

  // ---- dP: the P and gate terms, dP . E to LDS; zero the upper tiles of dP.E and dS
  for (int e = tid; e < C * C; e += NTHR) {
    const int r = e / C, cc = e % C;
    if ((r >> 4) < (cc >> 4)) { sdPE[r * LC + cc] = (OP)0.f; sdS[r * LC + cc] = (OP)0.f; }
  }
#pragma unroll
  for (int jj = 0; jj < 3; ++jj) {
    const int job = wave + jj * NWAVE;
    if (job < 10) {
      const int ti = (kLowI >> (2 * job)) & 3, tj = (kLowJ >> (2 * job)) & 3;
      f4_t qk = zero4();
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
        mma(qk, lds_frag<OP>(sQh, LDK, ti * 16, kb * 32), lds_frag<OP>(sKh, LDK, tj * 16, kb * 32));
      float csum = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = ti * 16 + 4 * g4 + i, cc = tj * 16 + m16;
        const bool on = cc <= r;
        const float E = fast_exp2(sG[r] - sG[cc]);
        const float dp = on ? accCC[jj][i] : 0.f;
        const float x = dp * E * qk[i];  // dP_ij P_ij
        sdPE[r * LC + cc] = (OP)(dp * E);
        const float rs = sum16(x);
        if (m16 == 0) atomicAdd(&sDg[r], rs);
        csum += x;
      }
      csum = sum_groups(csum);
      if (g4 == 0) atomicAdd(&sDg[tj * 16 + m16], -csum);
    }
  }
  // ---- dk column owners: dB_w = T^T dW, the W-gate, O-gate and D terms
  f4_t dBw[4];
  if (wave < RT) {
    const int col = wave * 16 + m16;
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i) dBw[rt][i] = -aW[rt][i];
    block_solve_t<LC, LLI>(dBw, sAnT, sLiT);
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = rt * 16 + 4 * g4 + i;
        sdBw[r * LDK + col] = (OP)dBw[rt][i];
        const float kh = (float)sKh[r * LDK + col], qh = (float)sQh[r * LDK + col];
        const float xw = sum16(dBw[rt][i] * kh);    // dB_w,i . k_i (this tile's share)
        const float xo = sum16(aQO[rt][i] * qh);    // q_i . (dO M0^T)_i
        const float xd = sum16(aKM[rt][i] * kh);    // k_i . (U dM^T)_i
        if (m16 == 0) {
          atomicAdd(&sDb[r], sGam[r] * xw);
          atomicAdd(&sDg[r], sBeta[r] * sGam[r] * xw + sGam[r] * xo);
          atomicAdd(&sDD[r], xd);
        }
      }
  }
  __syncthreads();
  // ---- dA = strictLower(-(dB_w W^T + dB_u U0^T)): dS, the A gate and beta terms
#pragma unroll
  for (int jj = 0; jj < 3; ++jj) {
    const int job = wave + jj * NWAVE;
    if (job >= 10 && job < 20) {
      const int t = job - 10;
      const int ti = (kLowI >> (2 * t)) & 3, tj = (kLowJ >> (2 * t)) & 3;
      f4_t bw = zero4(), kk = zero4();
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        mma(bw, lds_frag<OP>(sdBw, LDK, ti * 16, kb * 32), lds_frag<OP>(sW, LDK, tj * 16, kb * 32));
        mma(kk, lds_frag<OP>(sKh, LDK, ti * 16, kb * 32), lds_frag<OP>(sKh, LDK, tj * 16, kb * 32));
      }
      float csum = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = ti * 16 + 4 * g4 + i, cc = tj * 16 + m16;
        const bool on = cc < r;
        const float E = fast_exp2(sG[r] - sG[cc]);
        const float dA = on ? -(bw[i] + accCC[jj][i]) : 0.f;
        sdS[r * LC + cc] = (OP)(dA * sBeta[r] * E);
        const float xb = sum16(dA * E * kk[i]);              // sum_j dA_ij E_ij S_ij
        const float xa = dA * sBeta[r] * E * kk[i];          // dA_ij A_ij
        const float rs = sum16(xa);
        if (m16 == 0) {
          atomicAdd(&sDb[r], xb);
          atomicAdd(&sDg[r], rs);
        }
        csum += xa;
      }
      csum = sum_groups(csum);
      if (g4 == 0) atomicAdd(&sDg[tj * 16 + m16], -csum);
    }
  }
  __syncthreads();
  // ---- dq^, dk^ column tiles, and the row dots for the normalisation
  f4_t dQh[4], dKh[4];
  if (wave < RT) {
    const int col = wave * 16 + m16;
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      dQh[rt] = zero4();
      dKh[rt] = zero4();
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const Frag<OP> fk = lds_fragT<OP>(sKh, LDK, wave * 16, kb * 32);
        mma(dQh[rt], lds_frag<OP>(sdPE, LC, rt * 16, kb * 32), fk);
        mma(dKh[rt], lds_fragT<OP>(sdPE, LC, rt * 16, kb * 32), lds_fragT<OP>(sQh, LDK, wave * 16, kb * 32));
        mma(dKh[rt], lds_frag<OP>(sdS, LC, rt * 16, kb * 32), fk);
        mma(dKh[rt], lds_fragT<OP>(sdS, LC, rt * 16, kb * 32), fk);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = rt * 16 + 4 * g4 + i;
        dQh[rt][i] += sGam[r] * aQO[rt][i];
        dKh[rt][i] += sDec[r] * aKM[rt][i] + sBeta[r] * sGam[r] * dBw[rt][i];
        // the normalisation's backward, dq = (dq^ - q^ (q^ . dq^)) / n, with q^ from LDS
        const float qv = (float)sQh[r * LDK + col], kv = (float)sKh[r * LDK + col];
        const float xq = sum16(qv * dQh[rt][i]), xk = sum16(kv * dKh[rt][i]);
        if (m16 == 0) {
          atomicAdd(&sQd[r], xq);
          atomicAdd(&sKd[r], xk);
        }
      }
    }
  }
  __syncthreads();
  if (wave < RT) {
    const int col = wave * 16 + m16;
    // rows past the chunk fall outside the resources and are dropped
    const uint32_t rowq = (uint32_t)(H * DK * 4);
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(a.dq + tokbase * DK, (uint32_t)(n - 1) * rowq + DK * 4);
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(a.dk + tokbase * DK, (uint32_t)(n - 1) * rowq + DK * 4);
    const int oq = (int)(4 * g4 * rowq) + col * 4;
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = rt * 16 + 4 * g4 + i;
        const float qv = (float)sQh[r * LDK + col], kv = (float)sKh[r * LDK + col];
        const float gq = (dQh[rt][i] - qv * sQd[r]) / sNq[r] * invq;
        const float gk = (dKh[rt][i] - kv * sKd[r]) / sNk[r] * invq;
        buf_store(rq, gq, oq, (int)((rt * 16 + i) * rowq));
        buf_store(rk, gk, oq, (int)((rt * 16 + i) * rowq));
      }
  }
  // ---- the gates: D and gamma_C terms, reverse cumulative sum, d alpha and d beta
  if (wave == GATE_WAVE) {
    const float D = sDec[lane], dd = sDD[lane];
    float dg = sDg[lane] - D * dd;
    const float tot = wave_sum(D * dd) + sGam[C - 1] * a.dgC[bh * a.nchunks + c];
    if (lane == C - 1) dg += tot;
    // reverse inclusive cumulative sum over the chunk
    float r = dg;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const float y = __shfl_down(r, o, WAVE);
      if (lane + o < 64) r += y;
    }
    if (lane < n) {
      const int64_t gi = tokbase + (int64_t)lane * H;
      a.dalpha[gi] = r / a.alpha[gi] * invq;
      a.dbeta[gi] = sDb[lane] * invq;
    }
  }
}

// ------------------------------------------------------------ conv backward

// grid (ceil((T + 3) / 32), H, B), 4 waves: wave w takes the 8 consecutive
// rows t = 8 (4 x + w) - 3 + k (t < 0: a conv-cache row).  The dV' rows
// t .. t + 3 and value rows t - 3 .. t the strip reads (11 of each) are
// loaded together up front, each lane taking DV / 64 adjacent columns.
// dv_raw[t] = sum_j taps_{t+3-j}[j] dV'_{t+3-j} over the tokens that read
// row t, plus the gradient of conv_out; dtaps_t[j] = dV'_t . raw_{t-3+j}.
template <int N> struct FVec;
template <> struct FVec<1> { typedef float F; typedef uint16_t B; };
template <> struct FVec<2> { typedef float2 F; typedef uint32_t B; };
template <> struct FVec<4> { typedef float4 F; typedef uint2 B; };

template <int DV>
__global__ __launch_bounds__(256) void conv_bwd_kernel(int T, int H, const bf16_t* v, const bf16_t* conv_in,
                                                       const float* taps, const float* dvc, const float* dconv_out,
                                                       float* dv, float* dconv_in, float* dtaps) {
  constexpr int CPL = DV / 64, STRIP = 8, NR = STRIP + 3;
  using FV = typename FVec<CPL>::F;
  using BV = typename FVec<CPL>::B;
  const int h = blockIdx.y, b = blockIdx.z, lane = threadIdx.x & 63;
  const int tw0 = (blockIdx.x * 4 + (threadIdx.x >> 6)) * STRIP - 3;
  if (tw0 >= T) return;
  float dw[NR][CPL], rw[NR][CPL], tp[NR][4];
#pragma unroll
  for (int k = 0; k < NR; ++k) {
    // dV' row u = tw0 + k and its taps (zero outside [0, T))
    const int u = tw0 + k;
    const bool ok = u >= 0 && u < T;
    const int64_t bu = ((int64_t)b * T + (ok ? u : 0)) * H + h;
    const float4 t4 = *reinterpret_cast<const float4*>(taps + bu * 4);
    tp[k][0] = ok ? t4.x : 0.f; tp[k][1] = ok ? t4.y : 0.f; tp[k][2] = ok ? t4.z : 0.f; tp[k][3] = ok ? t4.w : 0.f;
    const FV x = *reinterpret_cast<const FV*>(dvc + bu * DV + lane * CPL);
    const float* xf = reinterpret_cast<const float*>(&x);
#pragma unroll
    for (int i = 0; i < CPL; ++i) dw[k][i] = ok ? xf[i] : 0.f;
    // value row r = tw0 - 3 + k (r < 0: the conv cache; zero without one)
    const int r = tw0 - 3 + k;
    const bool inv = r >= 0 && r < T, inc = r < 0 && r >= -3 && conv_in != nullptr;
    const bf16_t* src = inv ? v + (((int64_t)b * T + r) * H + h) * DV
                      : inc ? conv_in + (((int64_t)b * 3 + 3 + r) * H + h) * DV : v;
    const BV rb = *reinterpret_cast<const BV*>(src + lane * CPL);
    const bf16_t* rbh = reinterpret_cast<const bf16_t*>(&rb);
#pragma unroll
    for (int i = 0; i < CPL; ++i) rw[k][i] = (inv || inc) ? bf16_to_f32(rbh[i]) : 0.f;
  }
#pragma unroll
  for (int k = 0; k < STRIP; ++k) {
    const int t = tw0 + k;
    if (t >= T) break;
    // token u = t + 3 - j (slot k + 3 - j) read row t with its tap j
    float acc[CPL];
#pragma unroll
    for (int i = 0; i < CPL; ++i) acc[i] = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < CPL; ++i) acc[i] += tp[k + 3 - j][j] * dw[k + 3 - j][i];
    if (dconv_out && t >= T - 3) {
      const int sl = t - (T - 3);
#pragma unroll
      for (int i = 0; i < CPL; ++i) acc[i] += dconv_out[(((int64_t)b * 3 + sl) * H + h) * DV + lane * CPL + i];
    }
    float* dst = t >= 0 ? dv + (((int64_t)b * T + t) * H + h) * DV : dconv_in + (((int64_t)b * 3 + 3 + t) * H + h) * DV;
    *reinterpret_cast<FV*>(dst + lane * CPL) = *reinterpret_cast<const FV*>(acc);
    if (t >= 0) {
      // dtaps_t[j] = dV'_t . raw_{t-3+j}: dV'_t in slot k, raw row t-3+j in slot k + j
      float d[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        d[j] = 0.f;
#pragma unroll
        for (int i = 0; i < CPL; ++i) d[j] += dw[k][i] * rw[k + j][i];
        d[j] = sum_groups(sum16(d[j]));
      }
      if (lane == 0)
        *reinterpret_cast<float4*>(dtaps + (((int64_t)b * T + t) * H + h) * 4) = make_float4(d[0], d[1], d[2], d[3]);
    }
  }
}

// ------------------------------------------------------------ generator backward

// dx = dp W1 and the partial dW1 = dp^T x of one token range, on the bf16
// matrix cores (dp in three bf16 parts, x and W1 exact; split3 below): grid
// (ceil(D / 128), NSPLIT), 4 waves; wave w owns the two 16-column tiles
// from d0 = 128 blockIdx.x + 32 w.  The range goes 64 tokens at a time: its
// dp rows and its x rows (128 columns) are staged in LDS by whole-row 16-byte
// loads and read there in the operand orientations, and the dx tile leaves
// through LDS as whole-row 16-byte stores, so every HBM access is a full
// row piece.
// x = hi + mid + lo with each part bf16 (round to nearest even at each step):
// the three parts keep x's 24 significant bits, so three bf16 matrix-core
// products against an operand exact in bf16 give the fp32 product.
__device__ __forceinline__ void split3(const float (&v)[8], bf16x8_t& h, bf16x8_t& m, bf16x8_t& l) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const __bf16 hj = (__bf16)v[j];
    const float r1 = v[j] - (float)hj;
    const __bf16 mj = (__bf16)r1;
    const float r2 = r1 - (float)mj;
    h[j] = hj;
    m[j] = mj;
    l[j] = (__bf16)r2;
  }
}

__global__ __launch_bounds__(256) void gen_bwd_x_kernel(int64_t n_tok, int D, const bf16_t* x, const bf16_t* W1,
                                                        const float* dp, float* dx, float* part_w1) {
  constexpr int LX = 128 + 8, LO = 128 + 4;  // row strides of the x (bf16) and dx (f32) tiles
  __shared__ float sdp[64][33];
  __shared__ __attribute__((aligned(16))) bf16_t sx[64 * LX];
  __shared__ __attribute__((aligned(16))) float sdx[64 * LO];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, m16 = lane & 15, g4 = lane >> 4;
  const int sp = blockIdx.y, nsp = gridDim.y;
  const int64_t t0 = n_tok * sp / nsp, t1 = n_tok * (sp + 1) / nsp;
  const int c0 = blockIdx.x * 128;                 // first column of the block
  const int cw = wave * 32;                        // the wave's columns within the block
  int dcol[2];
  bool dok[2];
  // W1 as the B operand of dx (K index = hidden unit 8g + j), held for the whole range
  bf16x8_t wb16[2];
#pragma unroll
  for (int dt = 0; dt < 2; ++dt) {
    dcol[dt] = c0 + cw + dt * 16 + m16;
    dok[dt] = dcol[dt] < D;
    const int dc = dok[dt] ? dcol[dt] : 0;  // clamped, then masked
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const bf16_t w = W1[(int64_t)(8 * g4 + j) * D + dc];
      wb16[dt][j] = __builtin_bit_cast(__bf16, dok[dt] ? w : (bf16_t)0);
    }
  }
  f4_t aw[2][2];  // dW1 tiles [unit tile][column tile]
#pragma unroll
  for (int ut = 0; ut < 2; ++ut)
#pragma unroll
    for (int dt = 0; dt < 2; ++dt) aw[ut][dt] = zero4();
  // a block's dp rows (64 x 32 floats, one 16-byte piece per thread and pass)
  // and x rows (64 x 128 bf16, 16 pieces per row) into registers: the next
  // block's move while the current one is multiplied
  float4 pdp[2];
  uint4 px[4];
  auto load_block = [&](int64_t tb) {
    const int nt = (int)(t1 - tb < 64 ? t1 - tb : 64);
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int e = it * 256 + tid, r = e >> 3, q = e & 7;
      pdp[it] = r < nt ? *reinterpret_cast<const float4*>(dp + (tb + r) * 32 + 4 * q) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int e = it * 256 + tid, r = e >> 4, q = e & 15, col = c0 + 8 * q;
      px[it] = (r < nt && col < D) ? *reinterpret_cast<const uint4*>(x + (tb + r) * D + col) : make_uint4(0u, 0u, 0u, 0u);
    }
  };
  if (t0 < t1) load_block(t0);
  for (int64_t tb = t0; tb < t1; tb += 64) {
    const int nt = (int)(t1 - tb < 64 ? t1 - tb : 64);
    __syncthreads();  // the previous block's tiles are read and its dx rows are out
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int e = it * 256 + tid, r = e >> 3, q = e & 7;
      sdp[r][4 * q] = pdp[it].x;
      sdp[r][4 * q + 1] = pdp[it].y;
      sdp[r][4 * q + 2] = pdp[it].z;
      sdp[r][4 * q + 3] = pdp[it].w;
    }
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int e = it * 256 + tid, r = e >> 4, q = e & 15;
      *reinterpret_cast<uint4*>(sx + r * LX + 8 * q) = px[it];
    }
    __syncthreads();
    if (tb + 64 < t1) load_block(tb + 64);
    for (int b32 = 0; b32 < nt; b32 += 32) {
      // dx tiles: A = dp rows b16 + m16 at K = hidden unit 8g + j, split into
      // three bf16 parts (hi + mid + lo keeps dp's 24 bits); B = W1, exact in bf16
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        const int b16 = b32 + 16 * hb;
        float da[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) da[j] = sdp[b16 + m16][8 * g4 + j];
        bf16x8_t ah, am, al;
        split3(da, ah, am, al);
#pragma unroll
        for (int dt = 0; dt < 2; ++dt) {
          f4_t o = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, wb16[dt], zero4(), 0, 0, 0);
          o = __builtin_amdgcn_mfma_f32_16x16x32_bf16(am, wb16[dt], o, 0, 0, 0);
          o = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, wb16[dt], o, 0, 0, 0);
          // lane holds dx[b16 + 4g + i][cw + 16 dt + m16]
#pragma unroll
          for (int i = 0; i < 4; ++i) sdx[(b16 + 4 * g4 + i) * LO + cw + dt * 16 + m16] = o[i];
        }
      }
      // dW1 tiles: A = dp^T rows 16 ut + m16 at K = token b32 + 8g + j (split
      // likewise); B = x rows b32 + 8g + j, exact in bf16
      bf16x8_t xb[2];
#pragma unroll
      for (int dt = 0; dt < 2; ++dt)
#pragma unroll
        for (int j = 0; j < 8; ++j)
          xb[dt][j] = __builtin_bit_cast(__bf16, sx[(b32 + 8 * g4 + j) * LX + cw + dt * 16 + m16]);
#pragma unroll
      for (int ut = 0; ut < 2; ++ut) {
        float pa[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) pa[j] = sdp[b32 + 8 * g4 + j][ut * 16 + m16];
        bf16x8_t ph, pm, pl;
        split3(pa, ph, pm, pl);
#pragma unroll
        for (int dt = 0; dt < 2; ++dt) {
          aw[ut][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ph, xb[dt], aw[ut][dt], 0, 0, 0);
          aw[ut][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pm, xb[dt], aw[ut][dt], 0, 0, 0);
          aw[ut][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pl, xb[dt], aw[ut][dt], 0, 0, 0);
        }
      }
    }
    __syncthreads();
    // the dx tile out: 32 pieces of 16 bytes per row, 8 rows per pass
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int r = it * 8 + (tid >> 5), q = tid & 31, col = c0 + 4 * q;
      if (r < nt && col < D)
        *reinterpret_cast<float4*>(dx + (tb + r) * D + col) = *reinterpret_cast<const float4*>(sdx + r * LO + 4 * q);
    }
  }
  // lane holds dW1[16 ut + 4g + i][dcol]
#pragma unroll
  for (int ut = 0; ut < 2; ++ut)
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
      if (dok[dt])
#pragma unroll
        for (int i = 0; i < 4; ++i) part_w1[((int64_t)sp * 32 + ut * 16 + 4 * g4 + i) * D + dcol[dt]] = aw[ut][dt][i];
}

// The generator's first backward step and its small partials, per token range
// (grid GEN_NSPLIT_SMALL ranges, 256 threads), in passes of 32 tokens whose
// taps gradients sit in LDS beside W2:
//   hid = SiLU(pre), dhid = W2^T dtaps, dp = dhid SiLU'(pre) with
//   SiLU'(p) = s (1 + p (1 - s)), s = sigmoid(p)   (dp written: dx and dW1 take it);
// then the range's partial dW2 = dtaps^T hid [4H][32], db2 = sum dtaps and
// db1 = sum dp, each summed over the range's tokens in order.
constexpr int GEN_SMALL_MAXH = 32;  // heads (4H taps) the LDS holds
__global__ __launch_bounds__(256) void gen_bwd_head_kernel(int64_t n_tok, int H, const bf16_t* W2, const float* pre,
                                                           const float* dtaps, float* dp, float* part_small) {
  constexpr int TB = 32, MAXHK = 4 * GEN_SMALL_MAXH;
  constexpr int NJ = (MAXHK * 32 + MAXHK + 32 + 255) / 256;  // outputs per thread, at most
  __shared__ float sW2[MAXHK * 32];
  __shared__ float sdt[TB][MAXHK + 1];
  __shared__ float shid[TB][33];
  __shared__ float sdp[TB][33];
  const int tid = threadIdx.x, sp = blockIdx.x, nsp = gridDim.x;
  const int64_t t0 = n_tok * sp / nsp, t1 = n_tok * (sp + 1) / nsp;
  const int HK = 4 * H, nsmall = HK * 32 + HK + 32;
  for (int e = tid; e < HK * 32; e += 256) sW2[e] = bf16_to_f32(W2[e]);
  float acc[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) acc[j] = 0.f;
  for (int64_t tb = t0; tb < t1; tb += TB) {
    const int nt = (int)(t1 - tb < TB ? t1 - tb : TB);
    __syncthreads();  // W2 is in; the previous pass's rows are read
    for (int e = tid; e < nt * HK; e += 256) sdt[e / HK][e % HK] = dtaps[tb * HK + e];
    __syncthreads();
    for (int e = tid; e < nt * 32; e += 256) {
      const int t = e >> 5, u = e & 31;
      const float p = pre[(tb + t) * 32 + u], sg = 1.f / (1.f + expf(-p));
      float dh = 0.f;
      for (int r = 0; r < HK; ++r) dh += sW2[r * 32 + u] * sdt[t][r];
      const float d = dh * sg * (1.f + p * (1.f - sg));
      dp[(tb + t) * 32 + u] = d;
      sdp[t][u] = d;
      shid[t][u] = p * sg;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int e = tid + 256 * j;
      if (e >= nsmall) continue;
      float a = acc[j];
      if (e < HK * 32) {
        const int r = e / 32, u = e % 32;
        for (int t = 0; t < nt; ++t) a += sdt[t][r] * shid[t][u];
      } else if (e < HK * 32 + HK) {
        const int r = e - HK * 32;
        for (int t = 0; t < nt; ++t) a += sdt[t][r];
      } else {
        const int u = e - HK * 32 - HK;
        for (int t = 0; t < nt; ++t) a += sdp[t][u];
      }
      acc[j] = a;
    }
  }
  float* ps = part_small + (int64_t)sp * nsmall;
#pragma unroll
  for (int j = 0; j < NJ; ++j)
    if (tid + 256 * j < nsmall) ps[tid + 256 * j] = acc[j];
}

// Sums of partials in a fixed order, `per` partials (a multiple of 4) per
// range: out[y][e] = sum over s in [y per, (y + 1) per) of part[s][e], with
// grid.y ranges.  Four running sums keep four loads in flight.
__global__ void sum_parts_kernel(int64_t n, int per, const float* part, float* out) {
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= n) return;
  const float* p = part + (int64_t)blockIdx.y * per * n + e;
  float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
#pragma unroll 4
  for (int s = 0; s < per; s += 4) {
    a0 += p[(int64_t)s * n];
    a1 += p[(int64_t)(s + 1) * n];
    a2 += p[(int64_t)(s + 2) * n];
    a3 += p[(int64_t)(s + 3) * n];
  }
  out[(int64_t)blockIdx.y * n + e] = (a0 + a1) + (a2 + a3);
}

// ------------------------------------------------------------ host side

// the (dk, dv) pairs built (backward_supported, in jb_prefill.hip, lists the same)
#define JB_BACKWARD_KERNEL_CASES(X) X(32, 64) X(64, 128) X(96, 256) X(128, 256)

static size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }
constexpr int GEN_NSPLIT = 128;       // token ranges of the dx / dW1 kernel
constexpr int GEN_NSPLIT_SMALL = 2048; // token ranges of the dW2, db1, db2 partials
constexpr int GEN_SMALL_PER = 64;      // partials per range in the first of their two sums
static_assert(GEN_NSPLIT % 4 == 0 && GEN_SMALL_PER % 4 == 0 && (GEN_NSPLIT_SMALL / GEN_SMALL_PER) % 4 == 0,
              "sum_parts_kernel takes partials four at a time");

size_t backward_workspace_bytes(int B, int T, int H, int dk, int dv, int D) {
  const PrefillPlan p = plan_prefill(B, T, H, dk, dv, IO_BF16, IO_F32, 0);
  const size_t n = (size_t)B * T;
  const size_t nch = (size_t)p.nchunks;
  size_t bytes = al256(prefill_base_bytes(p));                // taps, segment buffers (the forward pass)
  bytes += al256((size_t)B * H * nch * dk * dv * 2);           // Mck (fp16)
  bytes += al256((size_t)B * H * nch * dk * dv * 2);           // dMck (fp16)
  bytes += 2 * al256(n * H * dv * 4);                          // dU, dV'
  bytes += 2 * al256((size_t)B * H * nch * C * dk * 4);        // dO M0^T, dU M0^T per chunk
  bytes += al256((size_t)B * H * nch * chain_img_bytes(dk));   // the chain's tiles per chunk
  bytes += al256((size_t)B * H * nch * 4);                     // the chunk-end gate term
  bytes += al256(n * H * 4 * 4);                               // dtaps
  bytes += 2 * al256(n * 32 * 4);                              // pre, dp
  bytes += al256((size_t)GEN_NSPLIT * 32 * D * 4);             // dW1 partials
  bytes += al256((size_t)GEN_NSPLIT_SMALL * (4 * H * 32 + 4 * H + 32) * 4);
  bytes += al256((size_t)(GEN_NSPLIT_SMALL / GEN_SMALL_PER) * (4 * H * 32 + 4 * H + 32) * 4);
  bytes += al256(64);                                          // scales and their max words
  return bytes;
}

hipError_t launch_backward(int B, int T, int H, int dk, int dv, int D, const void* x, const void* q, const void* k,
                           const void* v, const float* alpha, const float* beta, const void* W1, const void* b1,
                           const void* W2, const void* b2, const float* S0, const void* conv_in, const float* dout,
                           const float* dS_final, const float* dconv_out, float* dx, float* dq, float* dk_,
                           float* dv_, float* dalpha, float* dbeta, float* dW1, float* db1, float* dW2, float* db2,
                           float* dS0, float* dconv_in, void* workspace, hipStream_t stream) {
  if (H > GEN_SMALL_MAXH) return hipErrorInvalidValue;
  const PrefillPlan p = plan_prefill(B, T, H, dk, dv, IO_BF16, IO_F32, 0);
  const int64_t n = (int64_t)B * T;
  const int nch = p.nchunks;
  char* ws = static_cast<char*>(workspace);
  char* fws = ws;                                   // taps first, then the segment buffers
  float* taps = reinterpret_cast<float*>(ws);
  ws += al256(prefill_base_bytes(p));
  _Float16* Mck = reinterpret_cast<_Float16*>(ws);
  ws += al256((size_t)B * H * nch * dk * dv * 2);
  _Float16* dMck = reinterpret_cast<_Float16*>(ws);
  ws += al256((size_t)B * H * nch * dk * dv * 2);
  float* dU = reinterpret_cast<float*>(ws);
  ws += al256((size_t)n * H * dv * 4);
  float* dvc = reinterpret_cast<float*>(ws);
  ws += al256((size_t)n * H * dv * 4);
  float* QO = reinterpret_cast<float*>(ws);
  ws += al256((size_t)B * H * nch * C * dk * 4);
  float* WO = reinterpret_cast<float*>(ws);
  ws += al256((size_t)B * H * nch * C * dk * 4);
  float* dgC = reinterpret_cast<float*>(ws);
  ws += al256((size_t)B * H * nch * 4);
  char* img = ws;
  ws += al256((size_t)B * H * nch * chain_img_bytes(dk));
  float* dtaps = reinterpret_cast<float*>(ws);
  ws += al256((size_t)n * H * 4 * 4);
  float* pre = reinterpret_cast<float*>(ws);
  ws += al256((size_t)n * 32 * 4);
  float* dp = reinterpret_cast<float*>(ws);
  ws += al256((size_t)n * 32 * 4);
  float* pw1 = reinterpret_cast<float*>(ws);
  ws += al256((size_t)GEN_NSPLIT * 32 * D * 4);
  float* psm = reinterpret_cast<float*>(ws);
  ws += al256((size_t)GEN_NSPLIT_SMALL * (4 * H * 32 + 4 * H + 32) * 4);
  float* psm2 = reinterpret_cast<float*>(ws);   // range sums of the small partials
  ws += al256((size_t)(GEN_NSPLIT_SMALL / GEN_SMALL_PER) * (4 * H * 32 + 4 * H + 32) * 4);
  float* scale = reinterpret_cast<float*>(ws);

  hipError_t e = hipSuccess;
  unsigned int* word = reinterpret_cast<unsigned int*>(scale + 8);
  grad_scale_start_kernel<<<1, 1, 0, stream>>>(word);
  grad_absmax_kernel<<<4096, 256, 0, stream>>>(dout, n * H * dv, dS_final, (int64_t)B * H * dk * dv, word);
  grad_scale_finish_kernel<<<1, 1, 0, stream>>>(word, scale);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // forward: taps, the forward values' scale and the state entering every chunk
  e = launch_gen_taps(IO_BF16, n, D, H, x, W1, b1, W2, b2, taps, stream, pre);
  if (e != hipSuccess) return e;
  value_absmax_kernel<<<4096, 256, 0, stream>>>((const bf16_t*)v, n * H * dv, (const bf16_t*)conv_in,
                                                conv_in ? (int64_t)B * 3 * H * dv : 0, S0, (int64_t)B * H * dk * dv,
                                                taps, n * H * 4, word);
  value_scale_finish_kernel<<<1, 1, 0, stream>>>(word, scale);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  e = launch_prefill_ckpt(p, q, k, v, alpha, beta, taps, conv_in, S0, Mck, img, fws, stream, scale + 2);
  if (e != hipSuccess) return e;
  BwdArgs a{};
  a.T = T; a.H = H; a.nchunks = nch;
  a.q = (const bf16_t*)q; a.k = (const bf16_t*)k; a.v = (const bf16_t*)v; a.conv_in = (const bf16_t*)conv_in;
  a.alpha = alpha; a.beta = beta; a.taps = taps; a.dout = dout; a.dS_final = dS_final; a.scale = scale;
  a.Mck = Mck; a.dMck = dMck; a.dU = dU; a.dS0 = dS0; a.dq = dq; a.dk = dk_; a.dalpha = dalpha; a.dbeta = dbeta;
  a.dvc = dvc; a.QO = QO; a.WO = WO; a.dgC = dgC; a.img = img;
  bool launched = false;
#define CASE(DK_, DV_)                                                                              \
  if (dk == DK_ && dv == DV_) {                                                                     \
    static_assert(ChainImg<DK_>::bytes == chain_img_bytes(DK_), "chain tile layout");               \
    bwd_tiles_kernel<DK_><<<dim3(nch, H, B), NTHR, 0, stream>>>(a);                                 \
    bwd_chain_kernel<DK_, DV_><<<dim3(H, B), DV_ / 16 * 64, 0, stream>>>(a);                        \
    bwd_dvred_kernel<DK_, DV_><<<dim3(nch, H, B), NTHR, 0, stream>>>(a);                            \
    bwd_grad_kernel<DK_, DV_><<<dim3(nch, H, B), NTHR, 0, stream>>>(a);                             \
    conv_bwd_kernel<DV_><<<dim3((T + 3 + 31) / 32, H, B), 256, 0, stream>>>(T, H, (const bf16_t*)v, \
        (const bf16_t*)conv_in, taps, dvc, dconv_out, dv_, dconv_in, dtaps);                        \
    launched = true;                                                                                \
  }
  JB_BACKWARD_KERNEL_CASES(CASE)
#undef CASE
  if (!launched) return hipErrorInvalidValue;
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // the generator
  gen_bwd_head_kernel<<<dim3(GEN_NSPLIT_SMALL), 256, 0, stream>>>(n, H, (const bf16_t*)W2, pre, dtaps, dp, psm);
  gen_bwd_x_kernel<<<dim3((D + 127) / 128, GEN_NSPLIT), 256, 0, stream>>>(n, D, (const bf16_t*)x,
                                                                         (const bf16_t*)W1, dp, dx, pw1);
  const int64_t nw1 = (int64_t)32 * D, nsm = (int64_t)4 * H * 32 + 4 * H + 32;
  sum_parts_kernel<<<dim3((unsigned)((nw1 + 255) / 256)), 256, 0, stream>>>(nw1, GEN_NSPLIT, pw1, dW1);
  // the small parts land in dW2 [4H][32], db2 [4H], db1 [32] (three sums over the same partial layout),
  // summed in two steps: ranges of GEN_SMALL_PER partials, then the ranges
  sum_parts_kernel<<<dim3((unsigned)((nsm + 255) / 256), GEN_NSPLIT_SMALL / GEN_SMALL_PER), 256, 0, stream>>>(
      nsm, GEN_SMALL_PER, psm, psm2);
  sum_parts_kernel<<<dim3((unsigned)((nsm + 255) / 256)), 256, 0, stream>>>(nsm, GEN_NSPLIT_SMALL / GEN_SMALL_PER,
                                                                             psm2, psm);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  e = hipMemcpyAsync(dW2, psm, (size_t)4 * H * 32 * 4, hipMemcpyDeviceToDevice, stream);
  if (e == hipSuccess) e = hipMemcpyAsync(db2, psm + 4 * H * 32, (size_t)4 * H * 4, hipMemcpyDeviceToDevice, stream);
  if (e == hipSuccess)
    e = hipMemcpyAsync(db1, psm + 4 * H * 32 + 4 * H, (size_t)32 * 4, hipMemcpyDeviceToDevice, stream);
  return e;
}

}  // namespace jb
