// jb_span.h -- the row span of one packed sequence, shared by the device
// kernels and a host-side check (no HIP dependency).
//
// A packed batch holds B sequences back to back in `total` rows; sequence b is
// rows c0 = cu_seqlens[b] .. c1 - 1 with c1 = cu_seqlens[b + 1].  The offsets
// live in device memory, so the host cannot validate them: every kernel clamps
// them instead.  The first row is clamped to [0, total], the length to
// [0, Tmax] (the grid is planned for Tmax) and to the rows left after the
// first one, so a malformed offset gives wrong rows but never an access
// outside the packed tensors.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define JB_SPAN_FN __host__ __device__ __forceinline__
#else
#define JB_SPAN_FN static inline
#endif

namespace jb {

JB_SPAN_FN void clamp_span(int c0, int c1, int Tmax, int64_t total, int64_t& tok0, int& T) {
  const int64_t t0 = c0 < 0 ? 0 : ((int64_t)c0 > total ? total : (int64_t)c0);
  int64_t n = (int64_t)c1 - (int64_t)c0;
  if (n < 0) n = 0;
  if (n > Tmax) n = Tmax;
  if (n > total - t0) n = total - t0;
  tok0 = t0;
  T = (int)n;
}

}  // namespace jb
