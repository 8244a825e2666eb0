// jb_frag.h -- matrix-core fragment helpers of the fused chunk kernels
// (jb_fwd.hip): LDS fragment reads along rows and down columns
// (ds_read_b64_tr_b16), accumulator-to-operand conversion, the LDS DMA wrapper
// and the LDS-only barrier.  Fragment orders as in jb_device.h.
//
// ds_read_b64_tr_b16: within each group of 16 lanes, lane 4a + b receives
// element b of the 8-byte pieces addressed by lanes 4j + a (j = 0..3), so one
// instruction yields four K values of a fragment read down a column.
#pragma once

#include "jb_device.h"

namespace jb {
typedef short s4_t __attribute__((ext_vector_type(4)));
typedef _Float16 h4_t __attribute__((ext_vector_type(4)));
typedef float f2_t __attribute__((ext_vector_type(2)));
typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u2_t __attribute__((ext_vector_type(2)));

typedef __attribute__((address_space(3))) s4_t lds_s4;
typedef __attribute__((address_space(3))) char lds_char;

// ------------------------------------------------------------ fragments

// A copy of x the compiler cannot see through.  Used for lane offsets, so that
// an LDS address stays one short chain of additions from its array (the
// compiler then still knows which array every access touches, and reads of the
// working tiles never wait for the DMA into the staging areas), and for values
// derived from the lane inside the chunk loop, which are then formed there
// instead of being hoisted out of the loop and held (or spilled) across it.
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

__device__ __forceinline__ half8_t cat8(h4_t lo, h4_t hi) {
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ __forceinline__ f4_t mfma(const half8_t& a, const half8_t& b, const f4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Fragment reads take this lane's base address in a tile, formed once, plus a
// byte offset that is a compile-time constant after unrolling, so that the
// constant lands in the LDS instruction's offset field instead of a register.

// four 16-bit values down a column of a row-major 16-bit tile: this lane
// supplies the address of its 8-byte piece (see the file header)
__device__ __forceinline__ s4_t tr4(const lds_char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)p);
}

// Lane bases for reads down the columns of a row-major 16-bit tile (row stride
// ld elements): the supplying lane 16g + 4j + a points at row r(g) + j,
// column 4a, with r(g) = 4g (kperm halves at rows k0 and k0 + 16) or 8g
// (contiguous halves at rows k0 and k0 + 4).
__device__ __forceinline__ const lds_char* tr_base_kp(const lds_char* tile, int ld) {
  const int l = lane_id();
  return tile + opaque(((4 * (l >> 4) + ((l >> 2) & 3)) * ld + 4 * (l & 3)) * 2);
}
__device__ __forceinline__ const lds_char* tr_base_ct(const lds_char* tile, int ld) {
  const int l = lane_id();
  return tile + opaque(((8 * (l >> 4) + ((l >> 2) & 3)) * ld + 4 * (l & 3)) * 2);
}
// Fragment down the columns from a kperm base: lane 16g + n receives
// tile[k0 + 4g + j][c0 + n], then tile[k0 + 16 + 4g + j][c0 + n]
template <int LD>
__device__ __forceinline__ half8_t tr_frag_kp(const lds_char* base, int k0, int c0) {
  const s4_t lo = tr4(base + (k0 * LD + c0) * 2);
  const s4_t hi = tr4(base + ((k0 + 16) * LD + c0) * 2);
  return __builtin_bit_cast(half8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}
// ... from a contiguous base: rows k0 + 8g + j, then k0 + 8g + 4 + j
template <int LD>
__device__ __forceinline__ half8_t tr_frag_ct(const lds_char* base, int k0, int c0) {
  const s4_t lo = tr4(base + (k0 * LD + c0) * 2);
  const s4_t hi = tr4(base + ((k0 + 4) * LD + c0) * 2);
  return __builtin_bit_cast(half8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Lane bases for reads along the rows (lane 16g + m: row m, column 4g (kperm)
// or 8g (contiguous)) of a row-major fp16 tile
__device__ __forceinline__ const _Float16* row_base_kp(const _Float16* tile, int ld) {
  const int l = lane_id();
  return tile + opaque((l & 15) * ld + 4 * (l >> 4));
}
__device__ __forceinline__ const _Float16* row_base_ct(const _Float16* tile, int ld) {
  const int l = lane_id();
  return tile + opaque((l & 15) * ld + 8 * (l >> 4));
}
// Fragment along rows r0.. with K in the accumulator-chaining order (kperm:
// columns k0 + 4g .. + 3 and k0 + 16 + 4g .. + 3)
template <int LD>
__device__ __forceinline__ half8_t row_frag_kp(const _Float16* base, int r0, int k0) {
  const int o = r0 * LD + k0;
  return cat8(*reinterpret_cast<const h4_t*>(base + o), *reinterpret_cast<const h4_t*>(base + (o + 16)));
}
// ... K contiguous (columns k0 + 8g .. + 7): one 16-byte read
template <int LD>
__device__ __forceinline__ half8_t row_frag_ct(const _Float16* base, int r0, int k0) {
  return *reinterpret_cast<const half8_t*>(base + (r0 * LD + k0));
}

// B fragment (kperm order) from two accumulator tiles: rows 0..15 and 16..31
__device__ __forceinline__ half8_t acc_frag2(const f4_t& lo, const f4_t& hi) {
  const h2_t a = __builtin_convertvector(f2_t{lo[0], lo[1]}, h2_t);
  const h2_t b = __builtin_convertvector(f2_t{lo[2], lo[3]}, h2_t);
  const h2_t c = __builtin_convertvector(f2_t{hi[0], hi[1]}, h2_t);
  const h2_t d = __builtin_convertvector(f2_t{hi[2], hi[3]}, h2_t);
  return half8_t{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// the same with every row scaled first (rows of lo by s0, of hi by s1)
__device__ __forceinline__ half8_t acc_frag2_scaled(const f4_t& lo, const f4_t& hi, const float4& s0,
                                                    const float4& s1) {
  return acc_frag2(f4_t{lo[0] * s0.x, lo[1] * s0.y, lo[2] * s0.z, lo[3] * s0.w},
                   f4_t{hi[0] * s1.x, hi[1] * s1.y, hi[2] * s1.z, hi[3] * s1.w});
}

// Direct buffer -> LDS loads: a piece of `size` bytes at byte offset voff of
// the resource for every active lane, landing at lds + size * lane (lds is
// wave-uniform); offsets past the resource read as zero
template <int SIZE>
__device__ __forceinline__ void dma_buf(__amdgpu_buffer_rsrc_t r, uint32_t voff, lds_char* lds) {
  if constexpr (SIZE == 16)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, (int)voff, 0, 0, 0);
  else
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 4, (int)voff, 0, 0, 0);
}

// Barrier for data exchanged through LDS: this wave's LDS accesses complete,
// then s_barrier.  Outstanding global loads (the next chunk's LDS DMA) and
// stores stay in flight.
__device__ __forceinline__ void bar() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

}  // namespace jb
