// jb_chunk.h -- pieces of the chunked gated delta rule shared by the
// prefill kernels (jb_prefill.hip) and the backward kernels (jb_backward.hip):
// the chunk geometry, the normalisation prologue, the gate scan, the blocked
// triangular solve on the matrix cores and the LDS DMA wrappers.
#pragma once

#include "jb_device.h"

namespace jb {

// A fragment (kperm order) of the transpose of a row-major LDS tile: lane
// reads column c0 + l%16 at rows k0 + kperm(g, j).  As an A operand it is
// tile^T (rows c0..); as a B operand it is the tile itself (K = its rows).
template <typename OP>
__device__ __forceinline__ Frag<OP> lds_fragT(const OP* base, int ld, int c0, int k0) {
  const int l = lane_id(), m = l & 15, g = l >> 4;
  const OP* p = base + (k0 + 4 * g) * ld + c0 + m;
  Frag<OP> f;
#pragma unroll
  for (int j = 0; j < 4; ++j) { f.v[j] = p[j * ld]; f.v[4 + j] = p[(16 + j) * ld]; }
  return f;
}

// A fragment (kperm order) from a row-major fp32 matrix in global memory,
// scaled: rows r0 + l%16, K offset k0 (two 16-byte loads per lane); rows at
// or beyond nrows (at least 1) read as zero.
template <typename OP>
__device__ __forceinline__ Frag<OP> glb_frag(const float* base, int64_t ld, int r0, int k0, float scale,
                                             int nrows) {
  const int l = lane_id(), m = l & 15, g = l >> 4;
  // the row is clamped and the values masked, so the loads issue without a branch
  const bool ok = r0 + m < nrows;
  const float* p = base + (int64_t)min(r0 + m, nrows - 1) * ld + k0 + 4 * g;
  const float sc = ok ? scale : 0.f;
  const float4 lo = *reinterpret_cast<const float4*>(p), hi = *reinterpret_cast<const float4*>(p + 16);
  Frag<OP> f;
  f.v[0] = from_f32<OP>(lo.x * sc); f.v[1] = from_f32<OP>(lo.y * sc);
  f.v[2] = from_f32<OP>(lo.z * sc); f.v[3] = from_f32<OP>(lo.w * sc);
  f.v[4] = from_f32<OP>(hi.x * sc); f.v[5] = from_f32<OP>(hi.y * sc);
  f.v[6] = from_f32<OP>(hi.z * sc); f.v[7] = from_f32<OP>(hi.w * sc);
  return f;
}

constexpr int C = 64;        // chunk length
constexpr int NWAVE = 8;     // wavefronts per chunk workgroup
constexpr int NTHR = NWAVE * WAVE;
constexpr int PRO_THR = 512; // threads of the prologue mapping: 64 rows x 8 parts
constexpr int GATE_WAVE = 7; // the wave that loads and scans the gates
constexpr int NCU = 256;     // compute units of one MI355X


// Segments sequence b is cut into (at least one, which carries the state
// through an empty sequence).
__device__ __forceinline__ int seq_segments(int T, int seg_len) {
  const int nch = (T + C - 1) / C;
  return max(1, (nch + seg_len - 1) / seg_len);
}

// the lower-triangular tiles (i, j), j <= i, of a chunk's 4 x 4 tile grid in
// row order, two bits per coordinate: tile t is ((kLowI >> 2t) & 3, (kLowJ >> 2t) & 3)
constexpr uint32_t kLowI = 0xffa94u;  // rows    0 1 1 2 2 2 3 3 3 3
constexpr uint32_t kLowJ = 0xe4910u;  // columns 0 0 1 0 1 2 0 1 2 3

template <typename IO>
__device__ __forceinline__ void load_row_part(const IO* src, float* dst, int n, bool valid);

template <>
__device__ __forceinline__ void load_row_part<bf16_t>(const bf16_t* src, float* dst, int n, bool valid) {
  // n is a multiple of 4: 8-byte loads
  for (int e = 0; e < n; e += 4) {
    uint2 u = valid ? *reinterpret_cast<const uint2*>(src + e) : make_uint2(0u, 0u);
    dst[e + 0] = __uint_as_float(u.x << 16);
    dst[e + 1] = __uint_as_float(u.x & 0xffff0000u);
    dst[e + 2] = __uint_as_float(u.y << 16);
    dst[e + 3] = __uint_as_float(u.y & 0xffff0000u);
  }
}

template <>
__device__ __forceinline__ void load_row_part<float>(const float* src, float* dst, int n, bool valid) {
  for (int e = 0; e < n; e += 4) {
    float4 u = valid ? *reinterpret_cast<const float4*>(src + e) : make_float4(0.f, 0.f, 0.f, 0.f);
    dst[e + 0] = u.x;
    dst[e + 1] = u.y;
    dst[e + 2] = u.z;
    dst[e + 3] = u.w;
  }
}

// The normalisation part of the prologue for one chunk, as the first 512
// threads of a workgroup execute it: thread (row = tid/8, part = tid%8)
// handles DK/8 elements of q and k for token t0 + row.  Rows at or beyond
// `n` (ragged tail) are neutral tokens: q = k = 0 (and a = 1, b = 0).
// load() only issues the global loads; finish() reduces and scales.
template <int DK, typename IO>
struct Prologue {
  static constexpr int E = DK / 8;
  float kv[E], qv[E];
  int row, part;

  __device__ __forceinline__ void load(const IO* q, const IO* k, int64_t row_base, int H, int n, bool want_q) {
    row = threadIdx.x >> 3;
    part = threadIdx.x & 7;
    const bool valid = row < n;
    const int64_t off = (row_base + (int64_t)row * H) * DK + part * E;
    load_row_part<IO>(k + off, kv, E, valid);
    if (want_q) load_row_part<IO>(q + off, qv, E, valid);
  }
  // load() from global memory without branches: rows at or beyond n read
  // row n - 1 (n >= 1) and are zeroed, so every load issues at once
  __device__ __forceinline__ void load_global(const IO* q, const IO* k, int64_t row_base, int H, int n) {
    row = threadIdx.x >> 3;
    part = threadIdx.x & 7;
    const bool valid = row < n;
    const int64_t off = (row_base + (int64_t)min(row, n - 1) * H) * DK + part * E;
    load_row_part<IO>(k + off, kv, E, true);
    load_row_part<IO>(q + off, qv, E, true);
#pragma unroll
    for (int e = 0; e < E; ++e) {
      kv[e] = valid ? kv[e] : 0.f;
      qv[e] = valid ? qv[e] : 0.f;
    }
  }
  __device__ __forceinline__ void finish(bool want_q) {
    float sk = 0.f, sq = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) sk += kv[e] * kv[e];
    const float rk = l2_scale(group_sum<8>(sk));
#pragma unroll
    for (int e = 0; e < E; ++e) kv[e] *= rk;
    if (want_q) {
#pragma unroll
      for (int e = 0; e < E; ++e) sq += qv[e] * qv[e];
      const float rq = l2_scale(group_sum<8>(sq));
#pragma unroll
      for (int e = 0; e < E; ++e) qv[e] *= rq;
    }
  }
};

// Static-conv prologue: four channels d0 .. d0+3 of row `row` of the
// convolved q or k, from raw staged rows [C+3][DK] where row r + j holds
// token t0 + r - 3 + j, and tap-major weights w [4][DK]:
// x[i] = sum_j w[j][d0 + i] raw[row + j][d0 + i].
template <int DK, typename IO>
__device__ __forceinline__ void conv4(const IO* raw, const float* w, int row, int d0, bool valid, float (&x)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) x[i] = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float4 wj = *reinterpret_cast<const float4*>(w + j * DK + d0);
    float r[4];
    load_row_part<IO>(raw + (row + j) * DK + d0, r, 4, valid);
    x[0] += wj.x * r[0];
    x[1] += wj.y * r[1];
    x[2] += wj.z * r[2];
    x[3] += wj.w * r[3];
  }
}

// ------------------------------------------------------------ operand range
//
// The fp16 operands of the chunk products have 5 exponent bits: about 6e-5 to
// 6.5e4 at full precision.  The recurrence is linear in (v', S0), so a column
// tile of the state, its right-hand sides and its new values may be carried
// at any power-of-two scale and the outputs scaled back exactly.  Each tile
// keeps its own exponent E (held values = true values * 2^-E), chosen from
// the magnitudes the tile meets: after a change, the largest of |M| and the
// right-hand side sits in [2^8, 2^9), and it is changed again only when it
// leaves [2^4, 2^12) (a factor 128 of headroom under the fp16 maximum for the
// sums the products form).  Scaling every input by 2^k shifts every E by k
// and leaves the held values bit for bit unchanged.

// maximum over the wave: within quads, half rows, rows, then across rows by
// the row broadcasts (lane 63 ends with the total), read back from lane 63
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp<0xb1>(v, v));        // quad_perm [1,0,3,2]
  v = fmaxf(v, dpp<0x4e>(v, v));        // quad_perm [2,3,0,1]
  v = fmaxf(v, dpp<0x141>(v, v));       // row_half_mirror
  v = fmaxf(v, dpp<0x140>(v, v));       // row_mirror
  v = fmaxf(v, dpp<0x142, 0xa>(v, v));  // row_bcast:15 into rows 1, 3
  v = fmaxf(v, dpp<0x143, 0xc>(v, v));  // row_bcast:31 into rows 2, 3
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

// A tile starts "fresh" (E_FRESH: held in true units, no exponent chosen yet)
// so that its first choice does not depend on where the magnitudes happen to
// sit relative to 2^0; held_exp gives the exponent its held values carry.
constexpr int E_FRESH = -0x40000000;
__host__ __device__ constexpr int held_exp(int E) { return E == E_FRESH ? 0 : E; }

// The exponent for a tile currently at exponent E whose largest true
// magnitude is mx (wave-uniform).  Zero, infinite and NaN magnitudes keep E.
__device__ __forceinline__ int pick_exp(float mx, int E) {
  if (!(mx > 0.f) || !(mx <= 3.402823466e38f)) return E;
  const int ex = __builtin_amdgcn_frexp_expf(mx);  // mx in [2^(ex-1), 2^ex)
  const int t = ex - E;                            // held maximum in [2^(t-1), 2^t)
  return (E != E_FRESH && t >= 5 && t <= 12) ? E : ex - 9;
}

// One column tile before a chunk's solve: M (held at 2^-E, accumulator
// layout) and the chunk's right-hand side R (true units).  Picks the tile's
// exponent from both, re-expresses M if it changes, and brings R to it.
template <int RT>
__device__ __forceinline__ void rescale_tile(f4_t (&M)[RT], f4_t (&R)[4], int& E) {
  float mm = 0.f, mr = 0.f;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int i = 0; i < 4; ++i) mm = fmaxf(mm, fabsf(M[rt][i]));
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
#pragma unroll
    for (int i = 0; i < 4; ++i) mr = fmaxf(mr, fabsf(R[rb][i]));
  const int E0 = held_exp(E);
  const float mx = wave_max(fmaxf(ldexpf(mm, E0), mr));
  const int En = __builtin_amdgcn_readfirstlane(pick_exp(mx, E));
  if (En != E) {
    const int En0 = held_exp(En);
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i) M[rt][i] = ldexpf(M[rt][i], E0 - En0);
    E = En;
  }
  const int E1 = held_exp(E);
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
#pragma unroll
    for (int i = 0; i < 4; ++i) R[rb][i] = ldexpf(R[rb][i], -E1);
}

// g2 = inclusive cumsum of log2(alpha) over the chunk, lane = row (one wave).
// The chunk kernels keep the gates in base 2: e^{g_i - g_j} = 2^{g2_i - g2_j}.
__device__ __forceinline__ float chunk_gate_scan(float alpha_or_one) {
  return wave_inclusive_scan(fast_log2(alpha_or_one));
}

// Y = (I + A)^{-1} R for a 64 x 16 right-hand side in accumulator layout
// (Y[b] holds rows 16b..16b+15 of R on entry and of the solution on exit).
// Blocked forward substitution: Y_b = Linv_b (R_b - sum_{k<b} A_bk Y_k), on
// the matrix cores; sAn holds -A (row stride LC) and sLi the four diagonal
// block inverses (row stride LLI, columns 16..31 zero).
template <typename OP, int LC, int LLI>
__device__ __forceinline__ void block_solve(f4_t (&Y)[4], const OP* sAn, const OP* sLi) {
  const f4_t z = zero4();
  f4_t t = zero4();
  mma(t, lds_frag<OP>(sLi, LLI, 0, 0), acc_frag<OP>(Y[0], z));
  Y[0] = t;
  mma(Y[1], lds_frag<OP>(sAn, LC, 16, 0), acc_frag<OP>(Y[0], z));
  t = zero4();
  mma(t, lds_frag<OP>(sLi, LLI, 16, 0), acc_frag<OP>(Y[1], z));
  Y[1] = t;
  const Frag<OP> f01 = acc_frag<OP>(Y[0], Y[1]);
  mma(Y[2], lds_frag<OP>(sAn, LC, 32, 0), f01);
  mma(Y[3], lds_frag<OP>(sAn, LC, 48, 0), f01);
  t = zero4();
  mma(t, lds_frag<OP>(sLi, LLI, 32, 0), acc_frag<OP>(Y[2], z));
  Y[2] = t;
  mma(Y[3], lds_frag<OP>(sAn, LC, 48, 32), acc_frag<OP>(Y[2], z));
  t = zero4();
  mma(t, lds_frag<OP>(sLi, LLI, 48, 0), acc_frag<OP>(Y[3], z));
  Y[3] = t;
}

// ------------------------------------------------------------ chain tiles

// The state-independent tiles the backward chain needs of every chunk, in the
// padded LDS layout it reads them in (so that they move as one contiguous
// block): normalised K [C][DK], Q^T [DK][C], -W^T [DK][C], P^T [C][C] (fp16)
// and gamma, e^{g_C - g}, g [C] (fp32).  Row strides are padded by 8
// elements: 16-byte multiples whose 16 rows of a fragment read fall in
// distinct banks.  The checkpointing forward pass writes K, -W^T and the
// gates; the backward's tile kernel adds Q^T and P^T.
template <int DK>
struct ChainImg {
  static constexpr int LK = DK + 8, LT = C + 8;
  static constexpr int oKh = 0;
  static constexpr int oQt = oKh + C * LK * 2;
  static constexpr int oWt = oQt + DK * LT * 2;
  static constexpr int oPt = oWt + DK * LT * 2;
  static constexpr int oGam = oPt + C * LT * 2;
  static constexpr int oDec = oGam + C * 4;
  static constexpr int oG = oDec + C * 4;
  static constexpr int bytes = oG + C * 4;
  static_assert(bytes % 16 == 0 && (LK * 2) % 16 == 0 && (LT * 2) % 16 == 0, "16-byte pieces");
};
// bytes of one chunk's chain tiles (ChainImg<dk>::bytes)
constexpr size_t chain_img_bytes(int dk) {
  return (size_t)C * (dk + 8) * 2 + 2 * (size_t)dk * (C + 8) * 2 + (size_t)C * (C + 8) * 2 + 3 * (size_t)C * 4;
}

// ------------------------------------------------------------ LDS DMA

// Direct global -> LDS loads (gfx950): one wave instruction moves a 16-byte
// (or 4-byte) piece per active lane into consecutive LDS slots starting at the
// wave-uniform address `lds`; lanes that skip the call write nothing.
__device__ __forceinline__ void dma16(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)g,
                                   (__attribute__((address_space(3))) void*)lds, 16, 0, 0);
}
__device__ __forceinline__ void dma4(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)g,
                                   (__attribute__((address_space(3))) void*)lds, 4, 0, 0);
}

}  // namespace jb
