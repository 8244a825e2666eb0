// jb_device.h -- device-side building blocks shared by the libjetblock kernels
// (gfx950 / CDNA4, wave64).
//
// Matrix-core operand placement used everywhere (16x16 output tiles):
//   A (16 x K): lane l supplies row (l % 16); its lane group g = l / 16
//               supplies a quarter of the K values.
//   B (K x 16): lane l supplies column (l % 16), lane group g likewise.
//   D (16x16):  lane l holds D[4g + i][l % 16] for i = 0..3.
// A "fragment" is the 8 K-values one lane supplies for a 32-deep K block.
// Because the contraction sums over K, any bijection between (g, j) and the
// 32 K positions works as long as A and B use the same one.  Two orders are
// used:
//   kperm(g, j) = j < 4 ? 4g + j : 16 + 4g + (j - 4)
//       -- the rows a lane already holds in the accumulators of a 32-row
//          output block, so an accumulator block is a ready B fragment;
//   8g + j
//       -- contiguous, for operands streamed straight from memory.
// For fp16 a fragment feeds one v_mfma_f32_16x16x32_f16; for fp32 it feeds
// eight v_mfma_f32_16x16x4_f32, instruction j taking element j.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "jb_span.h"

namespace jb {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f4_t __attribute__((ext_vector_type(4)));
typedef uint16_t bf16_t;  // bfloat16 bits in memory

constexpr int WAVE = 64;

// ------------------------------------------------------------ conversions

__device__ __forceinline__ float bf16_to_f32(bf16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

// round-to-nearest-even float -> bfloat16 (one v_cvt_pk_bf16_f32 on gfx950)
__device__ __forceinline__ bf16_t f32_to_bf16(float f) { return __builtin_bit_cast(bf16_t, (__bf16)f); }

template <typename T> __device__ __forceinline__ float to_f32(T v);
template <> __device__ __forceinline__ float to_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ float to_f32<bf16_t>(bf16_t v) { return bf16_to_f32(v); }
template <> __device__ __forceinline__ float to_f32<_Float16>(_Float16 v) { return (float)v; }

template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float v) { return f32_to_bf16(v); }
template <> __device__ __forceinline__ _Float16 from_f32<_Float16>(float v) { return (_Float16)v; }

// ------------------------------------------------------------- fragments

__device__ __forceinline__ int lane_id() { return threadIdx.x & (WAVE - 1); }

__host__ __device__ constexpr int kperm(int g, int j) { return j < 4 ? 4 * g + j : 16 + 4 * g + (j - 4); }

template <typename OP> struct Frag { OP v[8]; };

__device__ __forceinline__ void mma(f4_t& acc, const Frag<_Float16>& a, const Frag<_Float16>& b) {
  half8_t av, bv;
#pragma unroll
  for (int j = 0; j < 8; ++j) { av[j] = a.v[j]; bv[j] = b.v[j]; }
  acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bv, acc, 0, 0, 0);
}

__device__ __forceinline__ void mma(f4_t& acc, const Frag<float>& a, const Frag<float>& b) {
#pragma unroll
  for (int j = 0; j < 8; ++j) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[j], b.v[j], acc, 0, 0, 0);
}

// A fragment (kperm order) from a row-major LDS tile: rows r0.., K offset k0.
// Lane reads row r0 + l%16 at columns k0 + 4g..4g+3 and k0 + 16 + 4g..+3.
template <typename OP>
__device__ __forceinline__ Frag<OP> lds_frag(const OP* base, int ld, int r0, int k0) {
  const int l = lane_id(), m = l & 15, g = l >> 4;
  const OP* p = base + (r0 + m) * ld + k0 + 4 * g;
  Frag<OP> f;
#pragma unroll
  for (int j = 0; j < 4; ++j) { f.v[j] = p[j]; f.v[4 + j] = p[16 + j]; }
  return f;
}

// B fragment (kperm order) from two accumulator tiles holding rows 0..15 and
// 16..31 of a 32-row block, each row optionally scaled.
template <typename OP>
__device__ __forceinline__ Frag<OP> acc_frag(const f4_t& lo, const f4_t& hi) {
  Frag<OP> f;
#pragma unroll
  for (int j = 0; j < 4; ++j) { f.v[j] = from_f32<OP>(lo[j]); f.v[4 + j] = from_f32<OP>(hi[j]); }
  return f;
}

__device__ __forceinline__ f4_t zero4() { return f4_t{0.f, 0.f, 0.f, 0.f}; }

// ----------------------------------------------------------- buffer stores
// A raw buffer resource over [base, base + bytes): stores beyond the range
// are dropped by the hardware.  Offsets are a per-lane 32-bit VGPR plus a
// wave-uniform SGPR, so a run of stores shares one address register.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ void buf_store(__amdgpu_buffer_rsrc_t r, float v, int voff, int soff) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, voff, soff, 0);  // bits, not a conversion
}
__device__ __forceinline__ void buf_store(__amdgpu_buffer_rsrc_t r, bf16_t v, int voff, int soff) {
  __builtin_amdgcn_raw_buffer_store_b16(v, r, voff, soff, 0);
}

// ----------------------------------------------------------- wave helpers

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, WAVE);
  return v;
}

// DPP lane exchange (data moves between lanes inside the VALU, no LDS round
// trip): dpp_ctrl as in the GFX9 ISA; rows outside row_mask keep `old`, and
// with bound_ctrl a lane whose source is outside its row reads zero
template <int CTRL, int ROWMASK = 0xf, bool BOUND = false>
__device__ __forceinline__ float dpp(float old, float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, old), __builtin_bit_cast(int, v),
                                                               CTRL, ROWMASK, 0xf, BOUND));
}

// sum over aligned groups of `n` consecutive lanes (n power of two <= 64);
// every lane of a group receives the same value
template <int N>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (N == 8) {
    v += dpp<0xb1>(v, v);   // quad_perm [1,0,3,2]
    v += dpp<0x4e>(v, v);   // quad_perm [2,3,0,1]
    v += dpp<0x141>(v, v);  // row_half_mirror: quad i of a half row meets quad 1 - i
    return v;
  } else {
#pragma unroll
    for (int off = N / 2; off >= 1; off >>= 1) v += __shfl_xor(v, off, WAVE);
    return v;
  }
}

// inclusive prefix sum across the 64 lanes of a wave: within rows of 16 by
// shifts of 1, 2, 4, 8, then across rows by the row broadcasts
__device__ __forceinline__ float wave_inclusive_scan(float v) {
  v += dpp<0x111, 0xf, true>(0.f, v);   // row_shr:1
  v += dpp<0x112, 0xf, true>(0.f, v);   // row_shr:2
  v += dpp<0x114, 0xf, true>(0.f, v);   // row_shr:4
  v += dpp<0x118, 0xf, true>(0.f, v);   // row_shr:8
  v += dpp<0x142, 0xa, false>(0.f, v);  // row_bcast:15 into rows 1, 3
  v += dpp<0x143, 0xc, false>(0.f, v);  // row_bcast:31 into rows 2, 3
  return v;
}

// Workgroup barrier ordering LDS only.  __syncthreads() also waits for the
// calling wave's outstanding global loads and stores; this one leaves them
// in flight, so prefetches and stores overlap the next phase.  Global data
// exchanged between waves still needs __syncthreads().
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// 2^x and log2(x) as single hardware instructions (1 ulp)
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// L2 normalisation factor (sum x^2 + 1e-6)^(-1/2)
__device__ __forceinline__ float l2_scale(float sumsq) { return 1.0f / sqrtf(sumsq + 1e-6f); }

// First row and length of sequence b of a batch: rows b T .. b T + T - 1 of
// the token-major tensors, or (packed sequences of different lengths) the
// span cu_seqlens gives (jb_span.h: clamped to the packed rows and to Tmax).
__device__ __forceinline__ void seq_span(const int* cu_seqlens, int Tmax, int64_t total, int b, int64_t& tok0,
                                         int& T) {
  if (!cu_seqlens) {
    tok0 = (int64_t)b * Tmax;
    T = Tmax;
    return;
  }
  clamp_span(cu_seqlens[b], cu_seqlens[b + 1], Tmax, total, tok0, T);
}

}  // namespace jb
