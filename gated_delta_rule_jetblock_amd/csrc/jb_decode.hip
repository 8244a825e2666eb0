// jb_decode.hip -- one decode step of the gated delta rule, HBM-streaming.
//
// Decoding is bound by memory bandwidth, and its cost is set by the size of
// the cached state (Jet-Nemotron csdn translation, section 2.5, finding 4).
// One step per (sequence, head), with M = S^T (dk x dv, fp32):
//     a = M^T khat,  c = M^T qhat               (both from one read of M)
//     u = b (v' - alpha a),  o = alpha c + (khat.qhat) u,  M' = alpha M + khat u^T
// which equals M' = alpha (M - b khat khat^T M) + b khat v'^T and o = M'^T qhat.
// v' is the dynamic causal conv (csdn section 2.4) of the cached raw rows and
// v_t with this token's taps.
//
// Workgroup per (head, sequence): 4 wavefronts; wave w owns dk/4 rows of M,
// lane l owns dv/64 adjacent columns, so every row is read and written as
// one contiguous dv-wide vector access per wave and M is read and written
// exactly once.  The two column reductions meet through LDS.  Plain (cached)
// vector accesses: on MI355X they stream the state faster than the
// non-temporal forms (measured 102 us vs 112 us per step at B=256, H=12,
// dk=96, dv=256).  The generator taps come from a separate small kernel:
// computing them inside every (sequence, head) workgroup repeats the
// 32 x d_model product per head and measured slower (146 us vs 115 us).
#include "jb_device.h"
#include "jb_internal.h"

namespace jb {

typedef float f2_t __attribute__((ext_vector_type(2)));
template <int CPL> struct VecF;
template <> struct VecF<1> { typedef float type; };
template <> struct VecF<2> { typedef f2_t type; };
template <> struct VecF<4> { typedef f4_t type; };

template <int CPL>
__device__ __forceinline__ void ld(const float* p, float (&o)[CPL]) {
  typedef typename VecF<CPL>::type V;
  V t = *reinterpret_cast<const V*>(p);
  const float* f = reinterpret_cast<const float*>(&t);
#pragma unroll
  for (int i = 0; i < CPL; ++i) o[i] = f[i];
}
template <int CPL>
__device__ __forceinline__ void st(float* p, const float (&o)[CPL]) {
  typedef typename VecF<CPL>::type V;
  V t;
  float* f = reinterpret_cast<float*>(&t);
#pragma unroll
  for (int i = 0; i < CPL; ++i) f[i] = o[i];
  *reinterpret_cast<V*>(p) = t;
}

template <int DK, int DV, typename IO, typename OUT>
__global__ __launch_bounds__(256) void decode_kernel(int H, const float* S_in, float* S_out, const IO* cache_in,
                                                     IO* cache_out, const IO* q_t, const IO* k_t, const IO* v_t,
                                                     const float* alpha_t, const float* beta_t, const float* taps,
                                                     OUT* o_t) {
  constexpr int RPW = DK / 4;   // rows per wave
  constexpr int CPL = DV / 64;  // columns per lane
  __shared__ float sk[DK], sq[DK], sv[DV];
  __shared__ float sred[2][4][DV];

  const int h = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int64_t bh = (int64_t)b * H + h;
  const float* Min = S_in + bh * DK * DV + (int64_t)(wave * RPW) * DV + lane * CPL;
  float* Mout = S_out + bh * DK * DV + (int64_t)(wave * RPW) * DV + lane * CPL;

  // issue the state loads first: they dominate the step
  float m[RPW][CPL];
#pragma unroll
  for (int r = 0; r < RPW; ++r) ld<CPL>(Min + (int64_t)r * DV, m[r]);

  const float al = alpha_t[bh], be = beta_t[bh];
  if (wave == 0) {
    // normalise q and k (each lane holds up to two elements)
    float kx[2], qx[2];
    float sk2 = 0.f, sq2 = 0.f;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int d = lane + 64 * e;
      kx[e] = d < DK ? to_f32<IO>(k_t[bh * DK + d]) : 0.f;
      qx[e] = d < DK ? to_f32<IO>(q_t[bh * DK + d]) : 0.f;
      sk2 += kx[e] * kx[e];
      sq2 += qx[e] * qx[e];
    }
    const float rk = l2_scale(wave_sum(sk2)), rq = l2_scale(wave_sum(sq2));
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int d = lane + 64 * e;
      if (d < DK) { sk[d] = kx[e] * rk; sq[d] = qx[e] * rq; }
    }
  } else if (wave == 1) {
    // conv of the cached raw rows and v_t with this token's taps; shift the cache
    const float4 tp = *reinterpret_cast<const float4*>(taps + bh * 4);
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      const int c = lane * CPL + i;
      const IO c0 = cache_in[((int64_t)b * 3 + 0) * H * DV + (int64_t)h * DV + c];
      const IO c1 = cache_in[((int64_t)b * 3 + 1) * H * DV + (int64_t)h * DV + c];
      const IO c2 = cache_in[((int64_t)b * 3 + 2) * H * DV + (int64_t)h * DV + c];
      const IO vt = v_t[bh * DV + c];
      sv[c] = tp.x * to_f32<IO>(c0) + tp.y * to_f32<IO>(c1) + tp.z * to_f32<IO>(c2) + tp.w * to_f32<IO>(vt);
      cache_out[((int64_t)b * 3 + 0) * H * DV + (int64_t)h * DV + c] = c1;
      cache_out[((int64_t)b * 3 + 1) * H * DV + (int64_t)h * DV + c] = c2;
      cache_out[((int64_t)b * 3 + 2) * H * DV + (int64_t)h * DV + c] = vt;
    }
  }
  __syncthreads();

  // partial column sums over this wave's rows
  float pa[CPL], pc[CPL];
#pragma unroll
  for (int i = 0; i < CPL; ++i) { pa[i] = 0.f; pc[i] = 0.f; }
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    const float kr = sk[wave * RPW + r], qr = sq[wave * RPW + r];
#pragma unroll
    for (int i = 0; i < CPL; ++i) { pa[i] += m[r][i] * kr; pc[i] += m[r][i] * qr; }
  }
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    sred[0][wave][lane * CPL + i] = pa[i];
    sred[1][wave][lane * CPL + i] = pc[i];
  }
  // k.q for the output term (every wave computes it from LDS)
  float kq = 0.f;
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int d = lane + 64 * e;
    if (d < DK) kq += sk[d] * sq[d];
  }
  kq = wave_sum(kq);
  __syncthreads();

  float u[CPL];
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    const int c = lane * CPL + i;
    const float av = sred[0][0][c] + sred[0][1][c] + sred[0][2][c] + sred[0][3][c];
    const float cv = sred[1][0][c] + sred[1][1][c] + sred[1][2][c] + sred[1][3][c];
    u[i] = be * (sv[c] - al * av);
    if (wave == 0) o_t[bh * DV + c] = from_f32<OUT>(al * cv + kq * u[i]);
  }
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    const float kr = sk[wave * RPW + r];
    float nm[CPL];
#pragma unroll
    for (int i = 0; i < CPL; ++i) nm[i] = al * m[r][i] + kr * u[i];
    st<CPL>(Mout + (int64_t)r * DV, nm);
  }
}

#define JB_DECODE_CASES(X) \
  X(32, 64) X(32, 128) X(32, 256) X(64, 64) X(64, 128) X(64, 256) \
  X(96, 64) X(96, 128) X(96, 256) X(128, 64) X(128, 128) X(128, 256)

bool decode_supported(int dk, int dv) {
#define CASE(DK_, DV_) if (dk == DK_ && dv == DV_) return true;
  JB_DECODE_CASES(CASE)
#undef CASE
  return false;
}

template <int DK, int DV, typename IO>
static hipError_t run_decode(int out, int B, int H, const float* S_in, float* S_out, const void* cache_in,
                             void* cache_out, const void* q_t, const void* k_t, const void* v_t, const float* alpha_t,
                             const float* beta_t, const float* taps, void* o_t, hipStream_t stream) {
  const dim3 grid(H, B);
  if (out == IO_F32)
    decode_kernel<DK, DV, IO, float><<<grid, 256, 0, stream>>>(
        H, S_in, S_out, (const IO*)cache_in, (IO*)cache_out, (const IO*)q_t, (const IO*)k_t, (const IO*)v_t,
        alpha_t, beta_t, taps, (float*)o_t);
  else
    decode_kernel<DK, DV, IO, bf16_t><<<grid, 256, 0, stream>>>(
        H, S_in, S_out, (const IO*)cache_in, (IO*)cache_out, (const IO*)q_t, (const IO*)k_t, (const IO*)v_t,
        alpha_t, beta_t, taps, (bf16_t*)o_t);
  return hipGetLastError();
}

hipError_t launch_decode(int io, int out, int B, int H, int dk, int dv, const float* S_in, float* S_out,
                         const void* cache_in, void* cache_out, const void* q_t, const void* k_t, const void* v_t,
                         const float* alpha_t, const float* beta_t, const float* taps, void* o_t,
                         hipStream_t stream) {
  if (B == 0) return hipSuccess;
#define CASE(DK_, DV_)                                                                                        \
  if (dk == DK_ && dv == DV_) {                                                                               \
    if (io == IO_BF16)                                                                                        \
      return run_decode<DK_, DV_, bf16_t>(out, B, H, S_in, S_out, cache_in, cache_out, q_t, k_t, v_t, alpha_t, \
                                          beta_t, taps, o_t, stream);                                         \
    return run_decode<DK_, DV_, float>(out, B, H, S_in, S_out, cache_in, cache_out, q_t, k_t, v_t, alpha_t,    \
                                       beta_t, taps, o_t, stream);                                            \
  }
  JB_DECODE_CASES(CASE)
#undef CASE
  return hipErrorInvalidValue;
}

}  // namespace jb
