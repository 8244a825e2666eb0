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

// The part of a decode step after staging, for the 4 waves of a (head,
// sequence) workgroup: wave `wave` holds rows wave*DK/4 .. of M in m, and
// sk, sq (normalised k, q) and sv (v') are in LDS behind a barrier.
template <int DK, int DV, typename OUT>
__device__ __forceinline__ void decode_update(float (&m)[DK / 4][DV / 64], const float* sk, const float* sq,
                                              const float* sv, float (&sred)[2][4][DV], float al, float be,
                                              int64_t bh, OUT* o_t, float* Mout, int wave, int lane) {
  constexpr int RPW = DK / 4;   // rows per wave
  constexpr int CPL = DV / 64;  // columns per lane
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

  decode_update<DK, DV, OUT>(m, sk, sq, sv, sred, al, be, bh, o_t, Mout, wave, lane);
}

// ------------------------------------------------------- fused decode step
//
// jb_decode_step in one launch, with no communication between workgroups.
// A workgroup of 16 waves owns one sequence b and a group of HPG of its
// heads (HPG = H when the sequences alone fill the GPU).  It computes the
// token's generator hidden layer once, then the taps, v' and the normalised
// q and k of its heads into LDS, and then streams the heads' states.  Even
// heads use one register tile and odd heads the other: head j+1's tile is in
// flight while head j is processed, and the barriers between phases order
// LDS only, so state loads and stores keep streaming across them.  Issue
// order matters because the hardware counts outstanding memory operations
// in order: the generator's loads go out before the state tiles, and each
// head's tile before the previous head's stores, so that no wait for a
// needed value also waits for a later, larger transfer.
constexpr int SEQ_NW = 8;       // waves per workgroup (two workgroups per CU)
constexpr int SEQ_MAXHPG = 16;  // heads per workgroup at most

template <int DK, int DV, int NW>
struct SeqSmem {
  float sk[SEQ_MAXHPG][DK], sq[SEQ_MAXHPG][DK];  // normalised k and q
  float sv[SEQ_MAXHPG][DV];                       // v'
  float sred[2][NW][DV];                          // per-wave column sums of M^T k and M^T q
  float su[DV];                                   // u of the current head
  float shraw[32], shid[32];                      // generator hidden layer before / after SiLU
  float sw2[SEQ_MAXHPG * 4][33];                  // second-layer rows of the group's taps
  float staps[SEQ_MAXHPG][4];
  float sal[SEQ_MAXHPG], sbe[SEQ_MAXHPG], skq[SEQ_MAXHPG];
};

// 16 bytes of IO elements from global memory (zeros when !valid)
template <typename IO>
__device__ __forceinline__ uint4 ld16(const IO* p, bool valid) {
  return valid ? *reinterpret_cast<const uint4*>(p) : make_uint4(0u, 0u, 0u, 0u);
}
// dot product of two 16-byte pieces of IO elements, accumulated in fp32
__device__ __forceinline__ float dot16(uint4 a, uint4 b, float acc, bf16_t) {
  const uint32_t av[4] = {a.x, a.y, a.z, a.w}, bv[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    acc += __uint_as_float(av[i] << 16) * __uint_as_float(bv[i] << 16);
    acc += __uint_as_float(av[i] & 0xffff0000u) * __uint_as_float(bv[i] & 0xffff0000u);
  }
  return acc;
}
__device__ __forceinline__ float dot16(uint4 a, uint4 b, float acc, float) {
  acc += __uint_as_float(a.x) * __uint_as_float(b.x);
  acc += __uint_as_float(a.y) * __uint_as_float(b.y);
  acc += __uint_as_float(a.z) * __uint_as_float(b.z);
  acc += __uint_as_float(a.w) * __uint_as_float(b.w);
  return acc;
}

// two adjacent IO elements as one register-sized load
template <typename IO> struct Two;
template <> struct Two<bf16_t> {
  uint32_t v;
  __device__ __forceinline__ float lo() const { return __uint_as_float(v << 16); }
  __device__ __forceinline__ float hi() const { return __uint_as_float(v & 0xffff0000u); }
};
template <> struct Two<float> {
  float2 v;
  __device__ __forceinline__ float lo() const { return v.x; }
  __device__ __forceinline__ float hi() const { return v.y; }
};

// The state updates of a workgroup's HPG heads (decode_seq_kernel and its
// static-conv twin): sk, sq, skq, sv, sal, sbe of every head are in LDS
// behind a barrier, head 0's tile is in ma and head 1's in (or on its way to)
// mb.  Head j+2's tile is loaded into the registers head j has just
// finished with, so one tile is always in flight.
template <int DK, int DV, typename OUT, int NW, typename LoadTile>
__device__ __forceinline__ void seq_update_heads(SeqSmem<DK, DV, NW>& sm, float (&ma)[DK / NW][DV / 64],
                                                 float (&mb)[DK / NW][DV / 64], int HPG, int64_t bh0, float* S_out,
                                                 OUT* o_t, int tid, int wave, int lane, LoadTile load_tile) {
  constexpr int RPW = DK / NW;
  constexpr int CPL = DV / 64;
  auto process = [&](float (&m)[RPW][CPL], int j) {
    const int64_t bh = bh0 + j;
    float pa[CPL], pc[CPL];
#pragma unroll
    for (int i = 0; i < CPL; ++i) { pa[i] = 0.f; pc[i] = 0.f; }
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      const float kr = sm.sk[j][wave * RPW + r], qr = sm.sq[j][wave * RPW + r];
#pragma unroll
      for (int i = 0; i < CPL; ++i) { pa[i] += m[r][i] * kr; pc[i] += m[r][i] * qr; }
    }
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      sm.sred[0][wave][lane * CPL + i] = pa[i];
      sm.sred[1][wave][lane * CPL + i] = pc[i];
    }
    lds_barrier();
    const float al = sm.sal[j];
    if (tid < DV) {
      float av = 0.f, cv = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) { av += sm.sred[0][w][tid]; cv += sm.sred[1][w][tid]; }
      const float u = sm.sbe[j] * (sm.sv[j][tid] - al * av);
      sm.su[tid] = u;
      o_t[bh * DV + tid] = from_f32<OUT>(al * cv + sm.skq[j] * u);
    }
    lds_barrier();
    float* Mo = S_out + bh * DK * DV + (int64_t)(wave * RPW) * DV + lane * CPL;
    float uu[CPL];
#pragma unroll
    for (int i = 0; i < CPL; ++i) uu[i] = sm.su[lane * CPL + i];
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      const float kr = sm.sk[j][wave * RPW + r];
      float nm[CPL];
#pragma unroll
      for (int i = 0; i < CPL; ++i) nm[i] = al * m[r][i] + kr * uu[i];
      st<CPL>(Mo + (int64_t)r * DV, nm);
    }
  };
  for (int j = 0; j < HPG; j += 2) {
    process(ma, j);
    if (j + 2 < HPG) load_tile(ma, j + 2);
    if (j + 1 < HPG) {
      process(mb, j + 1);
      if (j + 3 < HPG) load_tile(mb, j + 3);
    }
  }
}

template <int DK, int DV, typename IO, typename OUT, int NW>
__global__ __launch_bounds__(NW * 64) void decode_seq_kernel(int H, int HPG, int D, const float* S_in,
                                                                 float* S_out, const IO* cache_in, IO* cache_out,
                                                                 const IO* x_t, const IO* q_t, const IO* k_t,
                                                                 const IO* v_t, const float* alpha_t,
                                                                 const float* beta_t, const IO* W1, const IO* b1,
                                                                 const IO* W2, const IO* b2, OUT* o_t) {
  constexpr int NT = NW * 64;
  constexpr int RPW = DK / NW;                   // state rows per wave
  constexpr int UPW = 32 / NW;                   // generator hidden units per wave
  constexpr int CPL = DV / 64;                   // state columns per lane
  constexpr int EPC = 16 / (int)sizeof(IO);      // elements per 16-byte piece
  constexpr int GU = (sizeof(IO) == 2 ? 8 : 4) / UPW;  // generator pieces per lane in flight
  constexpr int NPAIR = (SEQ_MAXHPG * DV / 2 + NT - 1) / NT;  // (head, column pair) conv items per thread, at most
  constexpr bool EARLY_B = 2 * RPW * CPL <= 48;  // second state tile in flight during the generator
  __shared__ SeqSmem<DK, DV, NW> sm;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int b = blockIdx.y, h0 = blockIdx.x * HPG;
  const int64_t bh0 = (int64_t)b * H + h0;

  auto load_tile = [&](float (&m)[RPW][CPL], int j) {
    const float* p = S_in + (bh0 + j) * DK * DV + (int64_t)(wave * RPW) * DV + lane * CPL;
#pragma unroll
    for (int r = 0; r < RPW; ++r) ld<CPL>(p + (int64_t)r * DV, m[r]);
  };

  // ---- issue: generator pieces (wave w owns hidden units UPW w .. UPW w +
  // UPW-1, its lanes split d_model), the conv rows, then the state tiles
  const int npc = (D + 64 * EPC - 1) / (64 * EPC);  // pieces per lane over d_model
  uint4 gx[GU], gw[UPW][GU];
#pragma unroll
  for (int g = 0; g < GU; ++g) {
    const int e = (g * 64 + lane) * EPC;
    const bool ok = g < npc && e < D;
    gx[g] = ld16(x_t + (int64_t)b * D + e, ok);
#pragma unroll
    for (int u = 0; u < UPW; ++u) gw[u][g] = ld16(W1 + (int64_t)(UPW * wave + u) * D + e, ok);
  }
  // q and k of the wave's first head (each lane holds up to two elements)
  float kx[2] = {0.f, 0.f}, qx[2] = {0.f, 0.f};
  auto load_qk = [&](int jw) {
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int d = lane + 64 * e;
      if (d < DK) {
        kx[e] = to_f32<IO>(k_t[(bh0 + jw) * DK + d]);
        qx[e] = to_f32<IO>(q_t[(bh0 + jw) * DK + d]);
      }
    }
  };
  if (wave < HPG) load_qk(wave);
  Two<IO> raw[NPAIR][4];  // columns c, c+1 of the three cached rows and v_t
#pragma unroll
  for (int i = 0; i < NPAIR; ++i) {
    const int pr = tid + i * NT, j = pr / (DV / 2), c = 2 * (pr % (DV / 2));
    if (j < HPG) {
#pragma unroll
      for (int t = 0; t < 3; ++t)
        raw[i][t] = *reinterpret_cast<const Two<IO>*>(cache_in + ((int64_t)b * 3 + t) * H * DV + (int64_t)(h0 + j) * DV + c);
      raw[i][3] = *reinterpret_cast<const Two<IO>*>(v_t + (bh0 + j) * DV + c);
    }
  }
  float ma[RPW][CPL], mb[RPW][CPL];
  load_tile(ma, 0);
  if (EARLY_B && HPG > 1) load_tile(mb, 1);
  __builtin_amdgcn_sched_barrier(0);

  // ---- generator hidden layer (pre-activation), q / k normalisation, cache shift
  float hacc[UPW];
#pragma unroll
  for (int u = 0; u < UPW; ++u) hacc[u] = 0.f;
#pragma unroll
  for (int g = 0; g < GU; ++g) {
#pragma unroll
    for (int u = 0; u < UPW; ++u) hacc[u] = dot16(gw[u][g], gx[g], hacc[u], IO());
  }
  for (int p0 = GU; p0 < npc; p0 += GU) {  // d_model beyond one round of pieces
#pragma unroll
    for (int g = 0; g < GU; ++g) {
      const int e = ((p0 + g) * 64 + lane) * EPC;
      const bool ok = p0 + g < npc && e < D;
      gx[g] = ld16(x_t + (int64_t)b * D + e, ok);
#pragma unroll
      for (int u = 0; u < UPW; ++u) gw[u][g] = ld16(W1 + (int64_t)(UPW * wave + u) * D + e, ok);
    }
#pragma unroll
    for (int g = 0; g < GU; ++g) {
#pragma unroll
      for (int u = 0; u < UPW; ++u) hacc[u] = dot16(gw[u][g], gx[g], hacc[u], IO());
    }
  }
#pragma unroll
  for (int u = 0; u < UPW; ++u) {
    const float hs = wave_sum(hacc[u]);
    if (lane == 0) sm.shraw[UPW * wave + u] = hs;
  }
  for (int jw = wave; jw < HPG; jw += NW) {
    // normalise q and k of head jw (loaded above for the first)
    if (jw != wave) load_qk(jw);
    float sk2 = kx[0] * kx[0] + kx[1] * kx[1], sq2 = qx[0] * qx[0] + qx[1] * qx[1];
    const float rk = l2_scale(wave_sum(sk2)), rq = l2_scale(wave_sum(sq2));
    float kq = 0.f;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int d = lane + 64 * e;
      if (d < DK) {
        sm.sk[jw][d] = kx[e] * rk;
        sm.sq[jw][d] = qx[e] * rq;
        kq += kx[e] * rk * qx[e] * rq;
      }
    }
    kq = wave_sum(kq);
    if (lane == 0) {
      sm.skq[jw] = kq;
      sm.sal[jw] = alpha_t[bh0 + jw];
      sm.sbe[jw] = beta_t[bh0 + jw];
    }
  }
  for (int e = tid; e < HPG * 4 * 32; e += NT) sm.sw2[e / 32][e % 32] = to_f32<IO>(W2[(int64_t)h0 * 4 * 32 + e]);
  // shift the conv cache; the thread that read a (head, column) writes it,
  // so cache_out may alias cache_in
#pragma unroll
  for (int i = 0; i < NPAIR; ++i) {
    const int pr = tid + i * NT, j = pr / (DV / 2), c = 2 * (pr % (DV / 2));
    if (j < HPG) {
#pragma unroll
      for (int t = 0; t < 3; ++t)
        *reinterpret_cast<Two<IO>*>(cache_out + ((int64_t)b * 3 + t) * H * DV + (int64_t)(h0 + j) * DV + c) = raw[i][t + 1];
    }
  }
  if (!EARLY_B && HPG > 1) load_tile(mb, 1);
  lds_barrier();

  // ---- SiLU, second layer (the group's taps), conv
  if (tid < 32) {
    const float hv = sm.shraw[tid] + (b1 ? to_f32<IO>(b1[tid]) : 0.f);
    sm.shid[tid] = hv / (1.0f + expf(-hv));
  }
  lds_barrier();
  if (tid < 4 * HPG) {
    float t = b2 ? to_f32<IO>(b2[h0 * 4 + tid]) : 0.f;
#pragma unroll
    for (int u = 0; u < 32; ++u) t += sm.sw2[tid][u] * sm.shid[u];
    sm.staps[tid / 4][tid % 4] = t;
  }
  lds_barrier();
#pragma unroll
  for (int i = 0; i < NPAIR; ++i) {
    const int pr = tid + i * NT, j = pr / (DV / 2), c = 2 * (pr % (DV / 2));
    if (j < HPG) {
      const float t0 = sm.staps[j][0], t1 = sm.staps[j][1], t2 = sm.staps[j][2], t3 = sm.staps[j][3];
      sm.sv[j][c] = t0 * raw[i][0].lo() + t1 * raw[i][1].lo() + t2 * raw[i][2].lo() + t3 * raw[i][3].lo();
      sm.sv[j][c + 1] = t0 * raw[i][0].hi() + t1 * raw[i][1].hi() + t2 * raw[i][2].hi() + t3 * raw[i][3].hi();
    }
  }
  lds_barrier();

  // ---- the heads' state updates
  seq_update_heads<DK, DV, OUT, NW>(sm, ma, mb, HPG, bh0, S_out, o_t, tid, wave, lane, load_tile);
}

// heads per workgroup: the fewest groups per sequence that give every CU
// 16 waves (256 CUs) with at most SEQ_MAXHPG heads each (a divisor of H)
// One decode step of the static-conv block, the one JetBlock replaces
// (Jet-Nemotron csdn translation, section 2.4: earlier linear-attention
// blocks convolve with fixed kernels).  Read here as a causal depthwise conv
// of size 4 with fixed weights on each of q, k and v, no activation, q and k
// normalised after it.  Same workgroup layout as decode_seq_kernel, with the
// generator replaced by the three convs: wave w convolves q and k of heads
// w, w + NW, .. from their caches, every thread the v columns it owns; each
// cache element is written by the thread that read it, so the caches may be
// updated in place.  Issue order: the first heads' q / k rows and weights,
// the v rows and weights, then the state tiles.
template <int DK, int DV, typename IO, typename OUT, int NW>
__global__ __launch_bounds__(NW * 64) void decode_seq_static_kernel(
    int H, int HPG, const float* S_in, float* S_out, const IO* cq_in, const IO* ck_in, const IO* cv_in, IO* cq_out,
    IO* ck_out, IO* cv_out, const IO* q_t, const IO* k_t, const IO* v_t, const float* alpha_t, const float* beta_t,
    const float* wq, const float* wk, const float* wv, OUT* o_t) {
  constexpr int NT = NW * 64;
  constexpr int RPW = DK / NW;
  constexpr int CPL = DV / 64;
  constexpr int NPAIR = (SEQ_MAXHPG * DV / 2 + NT - 1) / NT;
  constexpr bool EARLY_B = 2 * RPW * CPL <= 48;
  __shared__ SeqSmem<DK, DV, NW> sm;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int b = blockIdx.y, h0 = blockIdx.x * HPG;
  const int64_t bh0 = (int64_t)b * H + h0;

  auto load_tile = [&](float (&m)[RPW][CPL], int j) {
    const float* p = S_in + (bh0 + j) * DK * DV + (int64_t)(wave * RPW) * DV + lane * CPL;
#pragma unroll
    for (int r = 0; r < RPW; ++r) ld<CPL>(p + (int64_t)r * DV, m[r]);
  };

  // raw q / k rows (three cached, the current one) and weights of head jw, up
  // to two elements per lane
  IO qr[2][4], kr[2][4];
  float4 wqd[2], wkd[2];
  auto load_qk = [&](int jw) {
    const int h = h0 + jw;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int d = lane + 64 * e;
      if (d < DK) {
        const int64_t r0 = (int64_t)b * 3 * H * DK + (int64_t)h * DK + d, rs = (int64_t)H * DK;
#pragma unroll
        for (int t = 0; t < 3; ++t) {
          qr[e][t] = cq_in[r0 + t * rs];
          kr[e][t] = ck_in[r0 + t * rs];
        }
        qr[e][3] = q_t[(bh0 + jw) * DK + d];
        kr[e][3] = k_t[(bh0 + jw) * DK + d];
        wqd[e] = *reinterpret_cast<const float4*>(wq + ((int64_t)h * DK + d) * 4);
        wkd[e] = *reinterpret_cast<const float4*>(wk + ((int64_t)h * DK + d) * 4);
      }
    }
  };
  if (wave < HPG) load_qk(wave);
  Two<IO> raw[NPAIR][4];  // columns c, c+1 of the three cached v rows and v_t
  float4 wvc[NPAIR][2];   // their weights
#pragma unroll
  for (int i = 0; i < NPAIR; ++i) {
    const int pr = tid + i * NT, j = pr / (DV / 2), c = 2 * (pr % (DV / 2));
    if (j < HPG) {
#pragma unroll
      for (int t = 0; t < 3; ++t)
        raw[i][t] = *reinterpret_cast<const Two<IO>*>(cv_in + ((int64_t)b * 3 + t) * H * DV + (int64_t)(h0 + j) * DV + c);
      raw[i][3] = *reinterpret_cast<const Two<IO>*>(v_t + (bh0 + j) * DV + c);
      wvc[i][0] = *reinterpret_cast<const float4*>(wv + ((int64_t)(h0 + j) * DV + c) * 4);
      wvc[i][1] = *reinterpret_cast<const float4*>(wv + ((int64_t)(h0 + j) * DV + c + 1) * 4);
    }
  }
  float ma[RPW][CPL], mb[RPW][CPL];
  load_tile(ma, 0);
  if (EARLY_B && HPG > 1) load_tile(mb, 1);
  __builtin_amdgcn_sched_barrier(0);

  // ---- q / k convs, normalisation and cache shift, per head of this wave
  for (int jw = wave; jw < HPG; jw += NW) {
    if (jw != wave) load_qk(jw);
    float kx[2] = {0.f, 0.f}, qx[2] = {0.f, 0.f};
#pragma unroll
    for (int e = 0; e < 2; ++e)
      if (lane + 64 * e < DK) {
        kx[e] = wkd[e].x * to_f32<IO>(kr[e][0]) + wkd[e].y * to_f32<IO>(kr[e][1]) + wkd[e].z * to_f32<IO>(kr[e][2]) +
                wkd[e].w * to_f32<IO>(kr[e][3]);
        qx[e] = wqd[e].x * to_f32<IO>(qr[e][0]) + wqd[e].y * to_f32<IO>(qr[e][1]) + wqd[e].z * to_f32<IO>(qr[e][2]) +
                wqd[e].w * to_f32<IO>(qr[e][3]);
      }
    float sk2 = kx[0] * kx[0] + kx[1] * kx[1], sq2 = qx[0] * qx[0] + qx[1] * qx[1];
    const float rk = l2_scale(wave_sum(sk2)), rq = l2_scale(wave_sum(sq2));
    float kq = 0.f;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int d = lane + 64 * e;
      if (d < DK) {
        sm.sk[jw][d] = kx[e] * rk;
        sm.sq[jw][d] = qx[e] * rq;
        kq += kx[e] * rk * qx[e] * rq;
        const int64_t r0 = (int64_t)b * 3 * H * DK + (int64_t)(h0 + jw) * DK + d, rs = (int64_t)H * DK;
#pragma unroll
        for (int t = 0; t < 3; ++t) {
          cq_out[r0 + t * rs] = qr[e][t + 1];
          ck_out[r0 + t * rs] = kr[e][t + 1];
        }
      }
    }
    kq = wave_sum(kq);
    if (lane == 0) {
      sm.skq[jw] = kq;
      sm.sal[jw] = alpha_t[bh0 + jw];
      sm.sbe[jw] = beta_t[bh0 + jw];
    }
  }
  // ---- v conv and cache shift
#pragma unroll
  for (int i = 0; i < NPAIR; ++i) {
    const int pr = tid + i * NT, j = pr / (DV / 2), c = 2 * (pr % (DV / 2));
    if (j < HPG) {
      const float4 w0 = wvc[i][0], w1 = wvc[i][1];
      sm.sv[j][c] = w0.x * raw[i][0].lo() + w0.y * raw[i][1].lo() + w0.z * raw[i][2].lo() + w0.w * raw[i][3].lo();
      sm.sv[j][c + 1] = w1.x * raw[i][0].hi() + w1.y * raw[i][1].hi() + w1.z * raw[i][2].hi() + w1.w * raw[i][3].hi();
#pragma unroll
      for (int t = 0; t < 3; ++t)
        *reinterpret_cast<Two<IO>*>(cv_out + ((int64_t)b * 3 + t) * H * DV + (int64_t)(h0 + j) * DV + c) = raw[i][t + 1];
    }
  }
  if (!EARLY_B && HPG > 1) load_tile(mb, 1);
  lds_barrier();

  // ---- the heads' state updates
  seq_update_heads<DK, DV, OUT, NW>(sm, ma, mb, HPG, bh0, S_out, o_t, tid, wave, lane, load_tile);
}

// Heads per workgroup: the fewest groups (each a divisor of H, at most
// SEQ_MAXHPG heads) that give at least 512 workgroups of nw = 8 waves, or 1024
// when a head's state is 128 rows or more.  Measured at B = 256, H = 12,
// dk = 96: 6 heads per workgroup 104 us per step, 4 or 3 heads 106-108 us; at
// B = 128, H = 16, dk = 128: 4 heads 96.7 us, 2 heads 93.0 us.
int decode_seq_heads_per_group(int B, int H, int dk, int nw) {
  const int64_t want = (int64_t)(dk >= 128 ? 1024 : 512) * 8 / nw;
  for (int ng = 1; ng <= H; ++ng)
    if (H % ng == 0 && H / ng <= SEQ_MAXHPG && (int64_t)B * ng >= want) return H / ng;
  return 1;
}

template <int DK, int DV, typename IO>
static hipError_t run_decode_seq(int out, int B, int H, int D, const float* S_in, float* S_out, const void* cache_in,
                                 void* cache_out, const void* x_t, const void* q_t, const void* k_t, const void* v_t,
                                 const float* alpha_t, const float* beta_t, const void* W1, const void* b1,
                                 const void* W2, const void* b2, void* o_t, hipStream_t stream) {
  constexpr int NW = SEQ_NW;
  const int hpg = decode_seq_heads_per_group(B, H, DK, NW);
  const dim3 grid(H / hpg, B);
#define JB_SEQ_ARGS(OUT_)                                                                                       \
  H, hpg, D, S_in, S_out, (const IO*)cache_in, (IO*)cache_out, (const IO*)x_t, (const IO*)q_t, (const IO*)k_t, \
      (const IO*)v_t, alpha_t, beta_t, (const IO*)W1, (const IO*)b1, (const IO*)W2, (const IO*)b2, (OUT_*)o_t
  if (out == IO_F32)
    decode_seq_kernel<DK, DV, IO, float, NW><<<grid, NW * 64, 0, stream>>>(JB_SEQ_ARGS(float));
  else
    decode_seq_kernel<DK, DV, IO, bf16_t, NW><<<grid, NW * 64, 0, stream>>>(JB_SEQ_ARGS(bf16_t));
#undef JB_SEQ_ARGS
  return hipGetLastError();
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

template <int DK, int DV, typename IO>
static hipError_t run_decode_static(int out, int B, int H, const float* S_in, float* S_out, const void* cq_in,
                                    const void* ck_in, const void* cv_in, void* cq_out, void* ck_out, void* cv_out,
                                    const void* q_t, const void* k_t, const void* v_t, const float* alpha_t,
                                    const float* beta_t, const float* wq, const float* wk, const float* wv, void* o_t,
                                    hipStream_t stream) {
  constexpr int NW = SEQ_NW;
  const int hpg = decode_seq_heads_per_group(B, H, DK, NW);
  const dim3 grid(H / hpg, B);
#define JB_STATIC_ARGS(OUT_)                                                                                    \
  H, hpg, S_in, S_out, (const IO*)cq_in, (const IO*)ck_in, (const IO*)cv_in, (IO*)cq_out, (IO*)ck_out,         \
      (IO*)cv_out, (const IO*)q_t, (const IO*)k_t, (const IO*)v_t, alpha_t, beta_t, wq, wk, wv, (OUT_*)o_t
  if (out == IO_F32)
    decode_seq_static_kernel<DK, DV, IO, float, NW><<<grid, NW * 64, 0, stream>>>(JB_STATIC_ARGS(float));
  else
    decode_seq_static_kernel<DK, DV, IO, bf16_t, NW><<<grid, NW * 64, 0, stream>>>(JB_STATIC_ARGS(bf16_t));
#undef JB_STATIC_ARGS
  return hipGetLastError();
}

hipError_t launch_decode_static(int io, int out, int B, int H, int dk, int dv, const float* S_in, float* S_out,
                                const void* cq_in, const void* ck_in, const void* cv_in, void* cq_out, void* ck_out,
                                void* cv_out, const void* q_t, const void* k_t, const void* v_t,
                                const float* alpha_t, const float* beta_t, const float* wq, const float* wk,
                                const float* wv, void* o_t, hipStream_t stream) {
  if (B == 0) return hipSuccess;
#define CASE(DK_, DV_)                                                                                          \
  if (dk == DK_ && dv == DV_) {                                                                                 \
    if (io == IO_BF16)                                                                                          \
      return run_decode_static<DK_, DV_, bf16_t>(out, B, H, S_in, S_out, cq_in, ck_in, cv_in, cq_out, ck_out,   \
                                                 cv_out, q_t, k_t, v_t, alpha_t, beta_t, wq, wk, wv, o_t, stream); \
    return run_decode_static<DK_, DV_, float>(out, B, H, S_in, S_out, cq_in, ck_in, cv_in, cq_out, ck_out,      \
                                              cv_out, q_t, k_t, v_t, alpha_t, beta_t, wq, wk, wv, o_t, stream);    \
  }
  JB_DECODE_CASES(CASE)
#undef CASE
  return hipErrorInvalidValue;
}

hipError_t launch_decode_step(int io, int out, int B, int H, int dk, int dv, int D, const float* S_in, float* S_out,
                              const void* cache_in, void* cache_out, const void* x_t, const void* q_t,
                              const void* k_t, const void* v_t, const float* alpha_t, const float* beta_t,
                              const void* W1, const void* b1, const void* W2, const void* b2, void* o_t,
                              hipStream_t stream) {
  if (B == 0) return hipSuccess;
#define CASE(DK_, DV_)                                                                                         \
  if (dk == DK_ && dv == DV_) {                                                                                \
    if (io == IO_BF16)                                                                                         \
      return run_decode_seq<DK_, DV_, bf16_t>(out, B, H, D, S_in, S_out, cache_in, cache_out, x_t, q_t, k_t, v_t, \
                                              alpha_t, beta_t, W1, b1, W2, b2, o_t, stream);                   \
    return run_decode_seq<DK_, DV_, float>(out, B, H, D, S_in, S_out, cache_in, cache_out, x_t, q_t, k_t, v_t,    \
                                           alpha_t, beta_t, W1, b1, W2, b2, o_t, stream);                      \
  }
  JB_DECODE_CASES(CASE)
#undef CASE
  return hipErrorInvalidValue;
}

}  // namespace jb
