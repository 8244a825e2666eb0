// jb_api.hip -- the C ABI of libjetblock (declared in include/jetblock.h):
// host-side validation, workspace layout and kernel dispatch.  Validation is
// complete before the first HIP call, so a rejected call touches no device
// state; every entry point returns a jb_status and never throws.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <atomic>

#include "../../include/jetblock.h"
#include "jb_internal.h"

namespace {

thread_local char g_err[512];

jb_status fail(jb_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

jb_status ok() {
  g_err[0] = 0;
  return JB_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

#define JB_REQUIRE_PTR(p)                                                        \
  do {                                                                           \
    if (!(p)) return fail(JB_ERR_INVALID_ARG, "%s: %s is NULL", fn, #p);         \
    if (!aligned16(p)) return fail(JB_ERR_INVALID_ARG, "%s: %s is not 16-byte aligned", fn, #p); \
  } while (0)
#define JB_REQUIRE_SCALARS(p)                                                    \
  do {                                                                           \
    if (!(p)) return fail(JB_ERR_INVALID_ARG, "%s: %s is NULL", fn, #p);         \
    if ((uintptr_t)(p) & 3u) return fail(JB_ERR_INVALID_ARG, "%s: %s is not 4-byte aligned", fn, #p); \
  } while (0)
#define JB_OPTIONAL_PTR(p)                                                       \
  do {                                                                           \
    if ((p) && !aligned16(p)) return fail(JB_ERR_INVALID_ARG, "%s: %s is not 16-byte aligned", fn, #p); \
  } while (0)

// Shape checks common to every entry point; `decode` selects the T == 1 rules.
jb_status check_shape(const char* fn, const jb_shape* s, bool decode) {
  if (!s) return fail(JB_ERR_INVALID_ARG, "%s: shape is NULL", fn);
  if (s->B < 1) return fail(JB_ERR_INVALID_ARG, "%s: B = %d must be >= 1", fn, s->B);
  if (s->B > 65535) return fail(JB_ERR_UNSUPPORTED, "%s: B = %d exceeds 65535 (one grid dimension)", fn, s->B);
  if (decode ? s->T != 1 : s->T < 0)
    return fail(JB_ERR_INVALID_ARG, "%s: T = %d (%s)", fn, s->T, decode ? "decode needs T == 1" : "must be >= 0");
  if (s->T > (1 << 30)) return fail(JB_ERR_UNSUPPORTED, "%s: T = %d exceeds 2^30", fn, s->T);
  if (s->H < 1 || s->H > 32) return fail(JB_ERR_UNSUPPORTED, "%s: H = %d not in [1, 32]", fn, s->H);
  if (s->dk != 32 && s->dk != 64 && s->dk != 96 && s->dk != 128)
    return fail(JB_ERR_UNSUPPORTED, "%s: dk = %d not in {32, 64, 96, 128}", fn, s->dk);
  if (s->dv != 64 && s->dv != 128 && s->dv != 256)
    return fail(JB_ERR_UNSUPPORTED, "%s: dv = %d not in {64, 128, 256}", fn, s->dv);
  if (s->d_model < 128 || s->d_model % 128)
    return fail(JB_ERR_UNSUPPORTED, "%s: d_model = %d is not a positive multiple of 128", fn, s->d_model);
  if (s->gen_hidden != 32) return fail(JB_ERR_UNSUPPORTED, "%s: gen_hidden = %d (must be 32)", fn, s->gen_hidden);
  if (s->taps != 4) return fail(JB_ERR_UNSUPPORTED, "%s: taps = %d (must be 4)", fn, s->taps);
  if (s->chunk != 0 && s->chunk != 64) return fail(JB_ERR_UNSUPPORTED, "%s: chunk = %d (must be 0 or 64)", fn, s->chunk);
  if (s->io_dtype != JB_BF16 && s->io_dtype != JB_F32)
    return fail(JB_ERR_INVALID_ARG, "%s: io_dtype = %d is not a jb_dtype", fn, s->io_dtype);
  if (s->out_dtype != JB_BF16 && s->out_dtype != JB_F32)
    return fail(JB_ERR_INVALID_ARG, "%s: out_dtype = %d is not a jb_dtype", fn, s->out_dtype);
  const uint32_t extra = (uint32_t)s->flags & ~(0xffffu << 8);
  if (extra) return fail(JB_ERR_INVALID_ARG, "%s: unknown flags 0x%x", fn, extra);
  if (decode && s->flags) return fail(JB_ERR_INVALID_ARG, "%s: flags must be 0 for decode", fn);
  const int64_t tokens = (int64_t)s->B * s->T;
  if (tokens * s->H * (int64_t)(s->dv > s->d_model ? s->dv : s->d_model) >= ((int64_t)1 << 40))
    return fail(JB_ERR_UNSUPPORTED, "%s: tensor sizes exceed the supported range", fn);
  return JB_OK;
}

int seg_flag(const jb_shape* s) { return (int)(((uint32_t)s->flags >> 8) & 0xffffu); }

jb::PrefillPlan plan_of(const jb_shape* s) {
  return jb::plan_prefill(s->B, s->T, s->H, s->dk, s->dv, s->io_dtype == JB_F32 ? jb::IO_F32 : jb::IO_BF16,
                          s->out_dtype == JB_F32 ? jb::IO_F32 : jb::IO_BF16, seg_flag(s));
}

jb_status hip_status(const char* fn, hipError_t e) {
  if (e != hipSuccess) return fail(JB_ERR_HIP, "%s: %s", fn, hipGetErrorString(e));
  return ok();
}


}  // namespace

extern "C" {

const char* jb_status_string(jb_status st) {
  // a C caller may pass any int: read the bits as an int, not as the enum
  int v;
  memcpy(&v, &st, sizeof v);
  switch (v) {
    case JB_OK: return "JB_OK";
    case JB_ERR_INVALID_ARG: return "JB_ERR_INVALID_ARG";
    case JB_ERR_UNSUPPORTED: return "JB_ERR_UNSUPPORTED";
    case JB_ERR_WORKSPACE: return "JB_ERR_WORKSPACE";
    case JB_ERR_HIP: return "JB_ERR_HIP";
  }
  return "JB_ERR_UNKNOWN";
}

const char* jb_last_error(void) { return g_err; }

int32_t jb_version(void) { return 1 * 10000 + 0 * 100 + 0; }

jb_status jb_prefill_workspace_size(const jb_shape* s, size_t* bytes) {
  const char* fn = "jb_prefill_workspace_size";
  jb_status st = check_shape(fn, s, false);
  if (st) return st;
  if (!bytes) return fail(JB_ERR_INVALID_ARG, "%s: bytes is NULL", fn);
  *bytes = jb::prefill_workspace_bytes(plan_of(s));
  return ok();
}

// Shape and pointer checks of jb_prefill and jb_prefill_noalloc (everything but the workspace).
static jb_status check_prefill(const char* fn, const jb_shape* s, const void* x, const void* q, const void* k,
                               const void* v, const float* alpha, const float* beta, const void* W1, const void* b1,
                               const void* W2, const void* b2, const float* S0, const void* conv_in, const void* o,
                               const float* S_final, const void* conv_out) {
  jb_status st = check_shape(fn, s, false);
  if (st) return st;
  if (!jb::prefill_supported(plan_of(s)))
    return fail(JB_ERR_UNSUPPORTED, "%s: dk=%d dv=%d not built for io_dtype %d (the all-fp32 mode needs dk*dv <= 4096)",
                fn, s->dk, s->dv, s->io_dtype);
  if (seg_flag(s) < 0) return fail(JB_ERR_INVALID_ARG, "%s: bad segment flag", fn);
  if (s->T > 0) {
    JB_REQUIRE_PTR(x); JB_REQUIRE_PTR(q); JB_REQUIRE_PTR(k); JB_REQUIRE_PTR(v);
    JB_REQUIRE_SCALARS(alpha); JB_REQUIRE_SCALARS(beta); JB_REQUIRE_PTR(o);
  }
  JB_REQUIRE_PTR(W1); JB_REQUIRE_PTR(W2); JB_REQUIRE_PTR(S_final);
  JB_OPTIONAL_PTR(b1); JB_OPTIONAL_PTR(b2); JB_OPTIONAL_PTR(S0); JB_OPTIONAL_PTR(conv_in);
  JB_OPTIONAL_PTR(conv_out);
  return JB_OK;
}

static jb_status prefill_impl(const char* fn, const jb_shape* s, const void* x, const void* q, const void* k,
                              const void* v, const float* alpha, const float* beta, const void* W1, const void* b1,
                              const void* W2, const void* b2, const float* S0, const void* conv_in, void* o,
                              float* S_final, void* conv_out, void* workspace, size_t workspace_bytes,
                              void* stream) {
  jb_status st = check_prefill(fn, s, x, q, k, v, alpha, beta, W1, b1, W2, b2, S0, conv_in, o, S_final, conv_out);
  if (st) return st;
  const jb::PrefillPlan p = plan_of(s);
  const size_t need = jb::prefill_workspace_bytes(p);
  if (need && !workspace) return fail(JB_ERR_WORKSPACE, "%s: workspace is NULL (%zu bytes needed)", fn, need);
  if (workspace_bytes < need)
    return fail(JB_ERR_WORKSPACE, "%s: workspace has %zu bytes, %zu needed", fn, workspace_bytes, need);
  if (workspace && ((uintptr_t)workspace & 255u))
    return fail(JB_ERR_INVALID_ARG, "%s: workspace is not 256-byte aligned", fn);

  hipStream_t hs = static_cast<hipStream_t>(stream);
  const int io = s->io_dtype == JB_F32 ? jb::IO_F32 : jb::IO_BF16;
  hipError_t e = hipSuccess;
  if (s->T == 0) {
    // empty sequence: the state and cache pass through
    if (S0 && S0 != S_final)
      e = hipMemcpyAsync(S_final, S0, (size_t)s->B * s->H * s->dk * s->dv * sizeof(float), hipMemcpyDeviceToDevice, hs);
    else if (!S0)
      e = jb::launch_fill_zero(S_final, (size_t)s->B * s->H * s->dk * s->dv, hs);
    if (e == hipSuccess && conv_out) e = jb::launch_conv_tail(io, s->B, 0, s->H, s->dv, v, conv_in, conv_out, hs);
    return hip_status(fn, e);
  }
  float* taps = static_cast<float*>(workspace);
  e = jb::launch_gen_taps(io, (int64_t)s->B * s->T, s->d_model, s->H, x, W1, b1, W2, b2, taps, hs);
  if (e == hipSuccess) e = jb::launch_prefill(p, q, k, v, alpha, beta, taps, conv_in, S0, o, S_final, workspace, hs);
  if (e == hipSuccess && conv_out) e = jb::launch_conv_tail(io, s->B, s->T, s->H, s->dv, v, conv_in, conv_out, hs);
  return hip_status(fn, e);
}

jb_status jb_prefill(const jb_shape* s, const void* x, const void* q, const void* k, const void* v,
                     const float* alpha, const float* beta, const void* W1, const void* b1, const void* W2,
                     const void* b2, const float* S0, const void* conv_in, void* o, float* S_final,
                     void* conv_out, void* workspace, size_t workspace_bytes, void* stream) {
  return prefill_impl("jb_prefill", s, x, q, k, v, alpha, beta, W1, b1, W2, b2, S0, conv_in, o, S_final, conv_out,
                      workspace, workspace_bytes, stream);
}

}  // extern "C"

// ---- the allocation-free prefill: jb_prefill's kernels on a workspace that
// is a file-scope device array.  In host code `scratch` names a host-side
// stand-in, never the device memory: the kernels get the address that
// hipGetSymbolAddress returns for the current device, kept per device.
static __device__ __align__(256) unsigned char scratch[JB_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 256;
std::atomic<void*> g_scratch[kMaxDevices];

hipError_t scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* ptr = g_scratch[dev].load(std::memory_order_acquire);
  if (!ptr) {
    // first call on this device: look the array up with the device current
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!ptr) return hipErrorInvalidSymbol;
    g_scratch[dev].store(ptr, std::memory_order_release);
  }
  *out = ptr;
  return hipSuccess;
}

}  // namespace

extern "C" {

jb_status jb_prefill_noalloc(const jb_shape* s, const void* x, const void* q, const void* k, const void* v,
                             const float* alpha, const float* beta, const void* W1, const void* b1, const void* W2,
                             const void* b2, const float* S0, const void* conv_in, void* o, float* S_final,
                             void* conv_out, void* stream) {
  const char* fn = "jb_prefill_noalloc";
  jb_status st = check_prefill(fn, s, x, q, k, v, alpha, beta, W1, b1, W2, b2, S0, conv_in, o, S_final, conv_out);
  if (st) return st;
  const size_t need = jb::prefill_workspace_bytes(plan_of(s));
  if (need > JB_NOALLOC_SCRATCH_BYTES)
    return fail(JB_ERR_WORKSPACE, "%s: the shape needs %zu bytes of workspace, above the %zu this call holds; "
                "use jb_prefill with a workspace (or fewer tokens per call)", fn, need,
                (size_t)JB_NOALLOC_SCRATCH_BYTES);
  void* ptr = nullptr;
  const hipError_t e = scratch_address(&ptr);
  if (e != hipSuccess) return hip_status(fn, e);
  return prefill_impl(fn, s, x, q, k, v, alpha, beta, W1, b1, W2, b2, S0, conv_in, o, S_final, conv_out, ptr,
                      JB_NOALLOC_SCRATCH_BYTES, stream);
}

namespace {

jb_status check_varlen(const char* fn, const jb_shape* s, int64_t total_tokens, jb::PrefillPlan* p) {
  jb_status st = check_shape(fn, s, false);
  if (st) return st;
  if (total_tokens < 0 || total_tokens > (int64_t)s->B * s->T)
    return fail(JB_ERR_INVALID_ARG, "%s: total_tokens = %lld not in [0, B*T] (B = %d, T = %d the longest sequence)", fn,
                (long long)total_tokens, s->B, s->T);
  if (total_tokens > 0x7fffffffLL) return fail(JB_ERR_UNSUPPORTED, "%s: total_tokens exceeds 2^31 - 1", fn);
  *p = plan_of(s);
  if (!jb::prefill_supported(*p))
    return fail(JB_ERR_UNSUPPORTED, "%s: dk=%d dv=%d not built for io_dtype %d", fn, s->dk, s->dv, s->io_dtype);
  if (seg_flag(s) < 0) return fail(JB_ERR_INVALID_ARG, "%s: bad segment flag", fn);
  p->tokens = total_tokens;
  return JB_OK;
}

}  // namespace

jb_status jb_prefill_varlen_workspace_size(const jb_shape* s, int64_t total_tokens, size_t* bytes) {
  const char* fn = "jb_prefill_varlen_workspace_size";
  jb::PrefillPlan p;
  jb_status st = check_varlen(fn, s, total_tokens, &p);
  if (st) return st;
  if (!bytes) return fail(JB_ERR_INVALID_ARG, "%s: bytes is NULL", fn);
  *bytes = jb::prefill_workspace_bytes(p);
  return ok();
}

jb_status jb_prefill_varlen(const jb_shape* s, int64_t total_tokens, const int32_t* cu_seqlens, const void* x,
                            const void* q, const void* k, const void* v, const float* alpha, const float* beta,
                            const void* W1, const void* b1, const void* W2, const void* b2, const float* S0,
                            const void* conv_in, void* o, float* S_final, void* conv_out, void* workspace,
                            size_t workspace_bytes, void* stream) {
  const char* fn = "jb_prefill_varlen";
  jb::PrefillPlan p;
  jb_status st = check_varlen(fn, s, total_tokens, &p);
  if (st) return st;
  JB_REQUIRE_SCALARS(cu_seqlens);
  if (total_tokens > 0) {
    JB_REQUIRE_PTR(x); JB_REQUIRE_PTR(q); JB_REQUIRE_PTR(k); JB_REQUIRE_PTR(v);
    JB_REQUIRE_SCALARS(alpha); JB_REQUIRE_SCALARS(beta); JB_REQUIRE_PTR(o);
  }
  JB_REQUIRE_PTR(W1); JB_REQUIRE_PTR(W2); JB_REQUIRE_PTR(S_final);
  JB_OPTIONAL_PTR(b1); JB_OPTIONAL_PTR(b2); JB_OPTIONAL_PTR(S0); JB_OPTIONAL_PTR(conv_in);
  JB_OPTIONAL_PTR(conv_out);
  const size_t need = jb::prefill_workspace_bytes(p);
  if (need && !workspace) return fail(JB_ERR_WORKSPACE, "%s: workspace is NULL (%zu bytes needed)", fn, need);
  if (workspace_bytes < need)
    return fail(JB_ERR_WORKSPACE, "%s: workspace has %zu bytes, %zu needed", fn, workspace_bytes, need);
  if (workspace && ((uintptr_t)workspace & 255u))
    return fail(JB_ERR_INVALID_ARG, "%s: workspace is not 256-byte aligned", fn);

  hipStream_t hs = static_cast<hipStream_t>(stream);
  const int io = s->io_dtype == JB_F32 ? jb::IO_F32 : jb::IO_BF16;
  p.cu_seqlens = cu_seqlens;
  hipError_t e = hipSuccess;
  if (s->T == 0 || total_tokens == 0) {
    // every sequence is empty: the state and cache pass through
    if (S0 && S0 != S_final)
      e = hipMemcpyAsync(S_final, S0, (size_t)s->B * s->H * s->dk * s->dv * sizeof(float), hipMemcpyDeviceToDevice, hs);
    else if (!S0)
      e = jb::launch_fill_zero(S_final, (size_t)s->B * s->H * s->dk * s->dv, hs);
    if (e == hipSuccess && conv_out) e = jb::launch_conv_tail(io, s->B, 0, s->H, s->dv, v, conv_in, conv_out, hs);
    return hip_status(fn, e);
  }
  float* taps = static_cast<float*>(workspace);
  e = jb::launch_gen_taps(io, total_tokens, s->d_model, s->H, x, W1, b1, W2, b2, taps, hs);
  if (e == hipSuccess) e = jb::launch_prefill(p, q, k, v, alpha, beta, taps, conv_in, S0, o, S_final, workspace, hs);
  if (e == hipSuccess && conv_out)
    e = jb::launch_conv_tail(io, s->B, s->T, s->H, s->dv, v, conv_in, conv_out, hs, cu_seqlens, total_tokens);
  return hip_status(fn, e);
}

jb_status jb_decode_workspace_size(const jb_shape* s, size_t* bytes) {
  const char* fn = "jb_decode_workspace_size";
  jb_status st = check_shape(fn, s, true);
  if (st) return st;
  if (!bytes) return fail(JB_ERR_INVALID_ARG, "%s: bytes is NULL", fn);
  *bytes = 0;  // the fused step keeps its intermediates on chip
  return ok();
}

jb_status jb_decode_step(const jb_shape* s, const float* S_in, float* S_out, const void* cache_in, void* cache_out,
                         const void* x_t, const void* q_t, const void* k_t, const void* v_t, const float* alpha_t,
                         const float* beta_t, const void* W1, const void* b1, const void* W2, const void* b2,
                         void* o_t, void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "jb_decode_step";
  jb_status st = check_shape(fn, s, true);
  if (st) return st;
  if (!jb::decode_supported(s->dk, s->dv)) return fail(JB_ERR_UNSUPPORTED, "%s: dk=%d dv=%d not built", fn, s->dk, s->dv);
  JB_REQUIRE_PTR(S_in); JB_REQUIRE_PTR(S_out); JB_REQUIRE_PTR(cache_in); JB_REQUIRE_PTR(cache_out);
  JB_REQUIRE_PTR(x_t); JB_REQUIRE_PTR(q_t); JB_REQUIRE_PTR(k_t); JB_REQUIRE_PTR(v_t);
  JB_REQUIRE_SCALARS(alpha_t); JB_REQUIRE_SCALARS(beta_t); JB_REQUIRE_PTR(W1); JB_REQUIRE_PTR(W2);
  JB_REQUIRE_PTR(o_t);
  JB_OPTIONAL_PTR(b1); JB_OPTIONAL_PTR(b2);
  (void)workspace;
  (void)workspace_bytes;
  const int io = s->io_dtype == JB_F32 ? jb::IO_F32 : jb::IO_BF16;
  const int out = s->out_dtype == JB_F32 ? jb::IO_F32 : jb::IO_BF16;
  return hip_status(fn, jb::launch_decode_step(io, out, s->B, s->H, s->dk, s->dv, s->d_model, S_in, S_out, cache_in,
                                               cache_out, x_t, q_t, k_t, v_t, alpha_t, beta_t, W1, b1, W2, b2, o_t,
                                               static_cast<hipStream_t>(stream)));
}

jb_status jb_decode_update(const jb_shape* s, const float* S_in, float* S_out, const void* cache_in, void* cache_out,
                           const void* q_t, const void* k_t, const void* v_t, const float* alpha_t, const float* beta_t,
                           const float* taps, void* o_t, void* stream) {
  const char* fn = "jb_decode_update";
  jb_status st = check_shape(fn, s, true);
  if (st) return st;
  if (!jb::decode_supported(s->dk, s->dv)) return fail(JB_ERR_UNSUPPORTED, "%s: dk=%d dv=%d not built", fn, s->dk, s->dv);
  JB_REQUIRE_PTR(S_in); JB_REQUIRE_PTR(S_out); JB_REQUIRE_PTR(cache_in); JB_REQUIRE_PTR(cache_out);
  JB_REQUIRE_PTR(q_t); JB_REQUIRE_PTR(k_t); JB_REQUIRE_PTR(v_t); JB_REQUIRE_SCALARS(alpha_t);
  JB_REQUIRE_SCALARS(beta_t); JB_REQUIRE_PTR(taps); JB_REQUIRE_PTR(o_t);
  const int io = s->io_dtype == JB_F32 ? jb::IO_F32 : jb::IO_BF16;
  const int out = s->out_dtype == JB_F32 ? jb::IO_F32 : jb::IO_BF16;
  return hip_status(fn, jb::launch_decode(io, out, s->B, s->H, s->dk, s->dv, S_in, S_out, cache_in, cache_out, q_t,
                                          k_t, v_t, alpha_t, beta_t, taps, o_t, static_cast<hipStream_t>(stream)));
}

namespace {

size_t a256(size_t v) { return (v + 255) & ~(size_t)255; }

// bytes of q, k, v (bf16) and alpha, beta (fp32) for the tokens of `s`
size_t qkvab_bytes(const jb_shape* s) {
  const size_t n = (size_t)s->B * s->T;
  return 2 * a256(n * s->H * s->dk * 2) + a256(n * s->H * s->dv * 2) + 2 * a256(n * s->H * sizeof(float));
}

jb_status check_projection_args(const char* fn, const jb_shape* s) {
  jb_status st = check_shape(fn, s, false);
  if (st) return st;
  if (s->io_dtype != JB_BF16) return fail(JB_ERR_UNSUPPORTED, "%s: the projections take bf16 inputs only", fn);
  return JB_OK;
}

}  // namespace

jb_status jb_project_workspace_size(const jb_shape* s, size_t* bytes) {
  const char* fn = "jb_project_workspace_size";
  jb_status st = check_projection_args(fn, s);
  if (st) return st;
  if (!bytes) return fail(JB_ERR_INVALID_ARG, "%s: bytes is NULL", fn);
  *bytes = jb::project_workspace_bytes((int64_t)s->B * s->T, s->H, s->d_model);
  return ok();
}

#define JB_PROJECTION_PTRS()                                                                                \
  JB_REQUIRE_PTR(x); JB_REQUIRE_PTR(Wq); JB_REQUIRE_PTR(Wk); JB_REQUIRE_PTR(Wv); JB_REQUIRE_PTR(Wa);       \
  JB_REQUIRE_PTR(Wb); JB_REQUIRE_PTR(W1); JB_REQUIRE_PTR(W2); JB_OPTIONAL_PTR(ba); JB_OPTIONAL_PTR(bb);    \
  JB_OPTIONAL_PTR(b1); JB_OPTIONAL_PTR(b2)

jb_status jb_project(const jb_shape* s, const void* x, const void* Wq, const void* Wk, const void* Wv,
                     const void* Wa, const void* ba, const void* Wb, const void* bb,
                     const void* W1, const void* b1, const void* W2, const void* b2, void* q, void* k, void* v,
                     float* alpha, float* beta, float* taps, void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "jb_project";
  jb_status st = check_projection_args(fn, s);
  if (st) return st;
  if (s->T == 0) return ok();
  JB_PROJECTION_PTRS();
  JB_REQUIRE_PTR(q); JB_REQUIRE_PTR(k); JB_REQUIRE_PTR(v); JB_REQUIRE_SCALARS(alpha); JB_REQUIRE_SCALARS(beta);
  JB_REQUIRE_PTR(taps);
  (void)workspace;
  (void)workspace_bytes;
  return hip_status(fn, jb::launch_project((int64_t)s->B * s->T, s->H, s->dk, s->dv, s->d_model, x, Wq, Wk, Wv, Wa,
                                           ba, Wb, bb, W1, b1, W2, b2, q, k, v, alpha, beta, taps,
                                           workspace, static_cast<hipStream_t>(stream)));
}

jb_status jb_prefill_from_x_workspace_size(const jb_shape* s, size_t* bytes) {
  const char* fn = "jb_prefill_from_x_workspace_size";
  jb_status st = check_projection_args(fn, s);
  if (st) return st;
  if (!bytes) return fail(JB_ERR_INVALID_ARG, "%s: bytes is NULL", fn);
  *bytes = a256(jb::prefill_workspace_bytes(plan_of(s))) + qkvab_bytes(s);
  return ok();
}

jb_status jb_prefill_from_x(const jb_shape* s, const void* x, const void* Wq, const void* Wk, const void* Wv,
                            const void* Wa, const void* ba, const void* Wb, const void* bb, const void* W1,
                            const void* b1, const void* W2,
                            const void* b2, const float* S0, const void* conv_in, void* o, float* S_final,
                            void* conv_out, void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "jb_prefill_from_x";
  jb_status st = check_projection_args(fn, s);
  if (st) return st;
  const jb::PrefillPlan p = plan_of(s);
  if (!jb::prefill_supported(p)) return fail(JB_ERR_UNSUPPORTED, "%s: dk=%d dv=%d not built", fn, s->dk, s->dv);
  if (seg_flag(s) < 0) return fail(JB_ERR_INVALID_ARG, "%s: bad segment flag", fn);
  if (s->T > 0) {
    JB_PROJECTION_PTRS();
    JB_REQUIRE_PTR(o);
  }
  JB_REQUIRE_PTR(S_final); JB_OPTIONAL_PTR(S0); JB_OPTIONAL_PTR(conv_in); JB_OPTIONAL_PTR(conv_out);
  size_t need = 0;
  jb_prefill_from_x_workspace_size(s, &need);
  if (!workspace) return fail(JB_ERR_WORKSPACE, "%s: workspace is NULL (%zu bytes needed)", fn, need);
  if (workspace_bytes < need)
    return fail(JB_ERR_WORKSPACE, "%s: workspace has %zu bytes, %zu needed", fn, workspace_bytes, need);
  if ((uintptr_t)workspace & 255u) return fail(JB_ERR_INVALID_ARG, "%s: workspace is not 256-byte aligned", fn);

  hipStream_t hs = static_cast<hipStream_t>(stream);
  hipError_t e = hipSuccess;
  if (s->T == 0) {
    // empty sequence: the state and cache pass through
    if (S0 && S0 != S_final)
      e = hipMemcpyAsync(S_final, S0, (size_t)s->B * s->H * s->dk * s->dv * sizeof(float), hipMemcpyDeviceToDevice, hs);
    else if (!S0)
      e = jb::launch_fill_zero(S_final, (size_t)s->B * s->H * s->dk * s->dv, hs);
    if (e == hipSuccess && conv_out)
      e = jb::launch_conv_tail(jb::IO_BF16, s->B, 0, s->H, s->dv, nullptr, conv_in, conv_out, hs);
    return hip_status(fn, e);
  }
  // workspace: the prefill's own (taps first), then q, k, v, alpha, beta, then the projections'
  const size_t n = (size_t)s->B * s->T;
  char* ws = static_cast<char*>(workspace);
  float* taps = reinterpret_cast<float*>(ws);
  char* pre_ws = ws;
  ws += a256(jb::prefill_workspace_bytes(p));
  void* q = ws;
  ws += a256(n * s->H * s->dk * 2);
  void* k = ws;
  ws += a256(n * s->H * s->dk * 2);
  void* v = ws;
  ws += a256(n * s->H * s->dv * 2);
  float* alpha = reinterpret_cast<float*>(ws);
  ws += a256(n * s->H * sizeof(float));
  float* beta = reinterpret_cast<float*>(ws);
  e = jb::launch_project((int64_t)n, s->H, s->dk, s->dv, s->d_model, x, Wq, Wk, Wv, Wa, ba, Wb, bb, W1, b1, W2, b2, q,
                         k, v, alpha, beta, taps, nullptr, hs);
  if (e == hipSuccess) e = jb::launch_prefill(p, q, k, v, alpha, beta, taps, conv_in, S0, o, S_final, pre_ws, hs);
  if (e == hipSuccess && conv_out) e = jb::launch_conv_tail(jb::IO_BF16, s->B, s->T, s->H, s->dv, v, conv_in, conv_out, hs);
  return hip_status(fn, e);
}

jb_status jb_decode_step_from_x_workspace_size(const jb_shape* s, size_t* bytes) {
  const char* fn = "jb_decode_step_from_x_workspace_size";
  jb_status st = check_shape(fn, s, true);
  if (st) return st;
  if (s->io_dtype != JB_BF16) return fail(JB_ERR_UNSUPPORTED, "%s: the projections take bf16 inputs only", fn);
  if (!bytes) return fail(JB_ERR_INVALID_ARG, "%s: bytes is NULL", fn);
  // q, k, v and the gates of the B tokens
  *bytes = qkvab_bytes(s);
  return ok();
}

jb_status jb_decode_step_from_x(const jb_shape* s, const float* S_in, float* S_out, const void* cache_in,
                                void* cache_out, const void* x, const void* Wq, const void* Wk, const void* Wv,
                                const void* Wa, const void* ba, const void* Wb, const void* bb, const void* W1,
                                const void* b1, const void* W2, const void* b2, void* o_t, void* workspace,
                                size_t workspace_bytes, void* stream) {
  const char* fn = "jb_decode_step_from_x";
  jb_status st = check_shape(fn, s, true);
  if (st) return st;
  if (s->io_dtype != JB_BF16) return fail(JB_ERR_UNSUPPORTED, "%s: the projections take bf16 inputs only", fn);
  if (!jb::decode_supported(s->dk, s->dv)) return fail(JB_ERR_UNSUPPORTED, "%s: dk=%d dv=%d not built", fn, s->dk, s->dv);
  JB_PROJECTION_PTRS();
  JB_REQUIRE_PTR(S_in); JB_REQUIRE_PTR(S_out); JB_REQUIRE_PTR(cache_in); JB_REQUIRE_PTR(cache_out);
  JB_REQUIRE_PTR(o_t);
  size_t need = 0;
  jb_decode_step_from_x_workspace_size(s, &need);
  if (!workspace) return fail(JB_ERR_WORKSPACE, "%s: workspace is NULL (%zu bytes needed)", fn, need);
  if (workspace_bytes < need)
    return fail(JB_ERR_WORKSPACE, "%s: workspace has %zu bytes, %zu needed", fn, workspace_bytes, need);
  if ((uintptr_t)workspace & 255u) return fail(JB_ERR_INVALID_ARG, "%s: workspace is not 256-byte aligned", fn);
  hipStream_t hs = static_cast<hipStream_t>(stream);
  const size_t n = (size_t)s->B;
  char* ws = static_cast<char*>(workspace);
  void* q = ws;
  ws += a256(n * s->H * s->dk * 2);
  void* k = ws;
  ws += a256(n * s->H * s->dk * 2);
  void* v = ws;
  ws += a256(n * s->H * s->dv * 2);
  float* alpha = reinterpret_cast<float*>(ws);
  ws += a256(n * s->H * sizeof(float));
  float* beta = reinterpret_cast<float*>(ws);
  const int out = s->out_dtype == JB_F32 ? jb::IO_F32 : jb::IO_BF16;
  // q, k, v and the gates of the batch from the projection kernel; the step
  // forms the taps itself (its workgroups hold x_t of their sequence)
  hipError_t e = jb::launch_project((int64_t)n, s->H, s->dk, s->dv, s->d_model, x, Wq, Wk, Wv, Wa, ba, Wb, bb, W1,
                                    nullptr, nullptr, nullptr, q, k, v, alpha, beta, nullptr, nullptr, hs);
  if (e == hipSuccess)
    e = jb::launch_decode_step(jb::IO_BF16, out, s->B, s->H, s->dk, s->dv, s->d_model, S_in, S_out, cache_in,
                               cache_out, x, q, k, v, alpha, beta, W1, b1, W2, b2, o_t, hs);
  return hip_status(fn, e);
}

namespace {

jb_status check_static_prefill(const char* fn, const jb_shape* s, jb::PrefillPlan* p) {
  jb_status st = check_shape(fn, s, false);
  if (st) return st;
  *p = plan_of(s);
  if (!jb::prefill_static_supported(*p))
    return fail(JB_ERR_UNSUPPORTED,
                "%s: the static-conv prefill is built for bf16 inputs and (dk, dv) in {(32,64), (64,128), (96,256), "
                "(128,256)}; got io_dtype %d, dk=%d dv=%d", fn, s->io_dtype, s->dk, s->dv);
  if (seg_flag(s) < 0) return fail(JB_ERR_INVALID_ARG, "%s: bad segment flag", fn);
  return JB_OK;
}

}  // namespace

jb_status jb_prefill_static_workspace_size(const jb_shape* s, size_t* bytes) {
  const char* fn = "jb_prefill_static_workspace_size";
  jb::PrefillPlan p;
  jb_status st = check_static_prefill(fn, s, &p);
  if (st) return st;
  if (!bytes) return fail(JB_ERR_INVALID_ARG, "%s: bytes is NULL", fn);
  *bytes = jb::prefill_static_workspace_bytes(p);
  return ok();
}

jb_status jb_prefill_static(const jb_shape* s, const void* q, const void* k, const void* v, const float* alpha,
                            const float* beta, const float* wq, const float* wk, const float* wv, const float* S0,
                            const void* cache_q_in, const void* cache_k_in, const void* cache_v_in, void* o,
                            float* S_final, void* cache_q_out, void* cache_k_out, void* cache_v_out, void* workspace,
                            size_t workspace_bytes, void* stream) {
  const char* fn = "jb_prefill_static";
  jb::PrefillPlan p;
  jb_status st = check_static_prefill(fn, s, &p);
  if (st) return st;
  if (s->T > 0) {
    JB_REQUIRE_PTR(q); JB_REQUIRE_PTR(k); JB_REQUIRE_PTR(v);
    JB_REQUIRE_SCALARS(alpha); JB_REQUIRE_SCALARS(beta); JB_REQUIRE_PTR(o);
  }
  JB_REQUIRE_PTR(wq); JB_REQUIRE_PTR(wk); JB_REQUIRE_PTR(wv); JB_REQUIRE_PTR(S_final);
  JB_OPTIONAL_PTR(S0); JB_OPTIONAL_PTR(cache_q_in); JB_OPTIONAL_PTR(cache_k_in); JB_OPTIONAL_PTR(cache_v_in);
  JB_OPTIONAL_PTR(cache_q_out); JB_OPTIONAL_PTR(cache_k_out); JB_OPTIONAL_PTR(cache_v_out);
  if (!cache_q_in != !cache_k_in || !cache_q_in != !cache_v_in)
    return fail(JB_ERR_INVALID_ARG, "%s: cache_q_in, cache_k_in and cache_v_in must be all set or all NULL", fn);
  const size_t need = jb::prefill_static_workspace_bytes(p);
  if (need && !workspace) return fail(JB_ERR_WORKSPACE, "%s: workspace is NULL (%zu bytes needed)", fn, need);
  if (workspace_bytes < need)
    return fail(JB_ERR_WORKSPACE, "%s: workspace has %zu bytes, %zu needed", fn, workspace_bytes, need);
  if (workspace && ((uintptr_t)workspace & 255u))
    return fail(JB_ERR_INVALID_ARG, "%s: workspace is not 256-byte aligned", fn);

  hipStream_t hs = static_cast<hipStream_t>(stream);
  hipError_t e = hipSuccess;
  if (s->T == 0) {
    if (S0 && S0 != S_final)
      e = hipMemcpyAsync(S_final, S0, (size_t)s->B * s->H * s->dk * s->dv * sizeof(float), hipMemcpyDeviceToDevice, hs);
    else if (!S0)
      e = jb::launch_fill_zero(S_final, (size_t)s->B * s->H * s->dk * s->dv, hs);
  } else {
    e = jb::launch_prefill_static(p, q, k, v, alpha, beta, wq, wk, wv, cache_q_in, cache_k_in, cache_v_in, S0, o,
                                  S_final, workspace, hs);
  }
  // the caches' tails after the chunk kernels, which read the incoming caches
  if (e == hipSuccess && cache_q_out)
    e = jb::launch_conv_tail(jb::IO_BF16, s->B, s->T, s->H, s->dk, q, cache_q_in, cache_q_out, hs);
  if (e == hipSuccess && cache_k_out)
    e = jb::launch_conv_tail(jb::IO_BF16, s->B, s->T, s->H, s->dk, k, cache_k_in, cache_k_out, hs);
  if (e == hipSuccess && cache_v_out)
    e = jb::launch_conv_tail(jb::IO_BF16, s->B, s->T, s->H, s->dv, v, cache_v_in, cache_v_out, hs);
  return hip_status(fn, e);
}

jb_status jb_decode_step_static(const jb_shape* s, const float* S_in, float* S_out, const void* cache_q_in,
                                const void* cache_k_in, const void* cache_v_in, void* cache_q_out, void* cache_k_out,
                                void* cache_v_out, const void* q_t, const void* k_t, const void* v_t,
                                const float* alpha_t, const float* beta_t, const float* wq, const float* wk,
                                const float* wv, void* o_t, void* stream) {
  const char* fn = "jb_decode_step_static";
  jb_status st = check_shape(fn, s, true);
  if (st) return st;
  if (!jb::decode_supported(s->dk, s->dv)) return fail(JB_ERR_UNSUPPORTED, "%s: dk=%d dv=%d not built", fn, s->dk, s->dv);
  JB_REQUIRE_PTR(S_in); JB_REQUIRE_PTR(S_out);
  JB_REQUIRE_PTR(cache_q_in); JB_REQUIRE_PTR(cache_k_in); JB_REQUIRE_PTR(cache_v_in);
  JB_REQUIRE_PTR(cache_q_out); JB_REQUIRE_PTR(cache_k_out); JB_REQUIRE_PTR(cache_v_out);
  JB_REQUIRE_PTR(q_t); JB_REQUIRE_PTR(k_t); JB_REQUIRE_PTR(v_t);
  JB_REQUIRE_SCALARS(alpha_t); JB_REQUIRE_SCALARS(beta_t);
  JB_REQUIRE_PTR(wq); JB_REQUIRE_PTR(wk); JB_REQUIRE_PTR(wv); JB_REQUIRE_PTR(o_t);
  const int io = s->io_dtype == JB_F32 ? jb::IO_F32 : jb::IO_BF16;
  const int out = s->out_dtype == JB_F32 ? jb::IO_F32 : jb::IO_BF16;
  return hip_status(fn, jb::launch_decode_static(io, out, s->B, s->H, s->dk, s->dv, S_in, S_out, cache_q_in,
                                                 cache_k_in, cache_v_in, cache_q_out, cache_k_out, cache_v_out, q_t,
                                                 k_t, v_t, alpha_t, beta_t, wq, wk, wv, o_t,
                                                 static_cast<hipStream_t>(stream)));
}

namespace {

jb_status check_backward(const char* fn, const jb_shape* s) {
  jb_status st = check_shape(fn, s, false);
  if (st) return st;
  if (s->io_dtype != JB_BF16) return fail(JB_ERR_UNSUPPORTED, "%s: the backward pass takes bf16 inputs only", fn);
  if (!jb::backward_supported(jb::IO_BF16, s->dk, s->dv))
    return fail(JB_ERR_UNSUPPORTED, "%s: (dk, dv) = (%d, %d) not built (built: (32,64), (64,128), (96,256), (128,256))",
                fn, s->dk, s->dv);
  if (s->flags) return fail(JB_ERR_INVALID_ARG, "%s: flags must be 0", fn);
  return JB_OK;
}

}  // namespace

jb_status jb_backward_workspace_size(const jb_shape* s, size_t* bytes) {
  const char* fn = "jb_backward_workspace_size";
  jb_status st = check_backward(fn, s);
  if (st) return st;
  if (!bytes) return fail(JB_ERR_INVALID_ARG, "%s: bytes is NULL", fn);
  *bytes = jb::backward_workspace_bytes(s->B, s->T, s->H, s->dk, s->dv, s->d_model);
  return ok();
}

jb_status jb_backward(const jb_shape* s, const void* x, const void* q, const void* k, const void* v,
                      const float* alpha, const float* beta, const void* W1, const void* b1, const void* W2,
                      const void* b2, const float* S0, const void* conv_in, const float* dout, const float* dS_final,
                      const float* dconv_out, float* dx, float* dq, float* dk, float* dv, float* dalpha,
                      float* dbeta, float* dW1, float* db1, float* dW2, float* db2, float* dS0, float* dconv_in,
                      void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "jb_backward";
  jb_status st = check_backward(fn, s);
  if (st) return st;
  if (s->T > 0) {
    JB_REQUIRE_PTR(x); JB_REQUIRE_PTR(q); JB_REQUIRE_PTR(k); JB_REQUIRE_PTR(v);
    JB_REQUIRE_SCALARS(alpha); JB_REQUIRE_SCALARS(beta); JB_REQUIRE_PTR(dout);
    JB_REQUIRE_PTR(dx); JB_REQUIRE_PTR(dq); JB_REQUIRE_PTR(dk); JB_REQUIRE_PTR(dv);
    JB_REQUIRE_SCALARS(dalpha); JB_REQUIRE_SCALARS(dbeta);
  }
  JB_REQUIRE_PTR(W1); JB_REQUIRE_PTR(W2); JB_OPTIONAL_PTR(b1); JB_OPTIONAL_PTR(b2);
  JB_OPTIONAL_PTR(S0); JB_OPTIONAL_PTR(conv_in); JB_OPTIONAL_PTR(dS_final); JB_OPTIONAL_PTR(dconv_out);
  JB_REQUIRE_PTR(dW1); JB_REQUIRE_SCALARS(db1); JB_REQUIRE_PTR(dW2); JB_REQUIRE_SCALARS(db2);
  JB_REQUIRE_PTR(dS0); JB_REQUIRE_PTR(dconv_in);
  const size_t need = jb::backward_workspace_bytes(s->B, s->T, s->H, s->dk, s->dv, s->d_model);
  if (!workspace) return fail(JB_ERR_WORKSPACE, "%s: workspace is NULL (%zu bytes needed)", fn, need);
  if (workspace_bytes < need)
    return fail(JB_ERR_WORKSPACE, "%s: workspace has %zu bytes, %zu needed", fn, workspace_bytes, need);
  if ((uintptr_t)workspace & 255u) return fail(JB_ERR_INVALID_ARG, "%s: workspace is not 256-byte aligned", fn);
  hipStream_t hs = static_cast<hipStream_t>(stream);
  hipError_t e = hipSuccess;
  if (s->T == 0) {
    // nothing was computed: the state and cache gradients pass through, the weights get none
    const size_t ns = (size_t)s->B * s->H * s->dk * s->dv, nc = (size_t)s->B * 3 * s->H * s->dv;
    e = dS_final ? hipMemcpyAsync(dS0, dS_final, ns * 4, hipMemcpyDeviceToDevice, hs) : jb::launch_fill_zero(dS0, ns, hs);
    if (e == hipSuccess)
      e = dconv_out ? hipMemcpyAsync(dconv_in, dconv_out, nc * 4, hipMemcpyDeviceToDevice, hs)
                    : jb::launch_fill_zero(dconv_in, nc, hs);
    if (e == hipSuccess) e = jb::launch_fill_zero(dW1, (size_t)32 * s->d_model, hs);
    if (e == hipSuccess) e = jb::launch_fill_zero(db1, 32, hs);
    if (e == hipSuccess) e = jb::launch_fill_zero(dW2, (size_t)4 * s->H * 32, hs);
    if (e == hipSuccess) e = jb::launch_fill_zero(db2, (size_t)4 * s->H, hs);
    return hip_status(fn, e);
  }
  return hip_status(fn, jb::launch_backward(s->B, s->T, s->H, s->dk, s->dv, s->d_model, x, q, k, v, alpha, beta, W1,
                                            b1, W2, b2, S0, conv_in, dout, dS_final, dconv_out, dx, dq, dk, dv,
                                            dalpha, dbeta, dW1, db1, dW2, db2, dS0, dconv_in, workspace, hs));
}

jb_status jb_gen_taps(const jb_shape* s, const void* x, const void* W1, const void* b1, const void* W2, const void* b2,
                      float* taps, void* stream) {
  const char* fn = "jb_gen_taps";
  jb_status st = check_shape(fn, s, false);
  if (st) return st;
  if (s->T > 0) { JB_REQUIRE_PTR(x); JB_REQUIRE_PTR(taps); }
  JB_REQUIRE_PTR(W1); JB_REQUIRE_PTR(W2); JB_OPTIONAL_PTR(b1); JB_OPTIONAL_PTR(b2);
  const int io = s->io_dtype == JB_F32 ? jb::IO_F32 : jb::IO_BF16;
  return hip_status(fn, jb::launch_gen_taps(io, (int64_t)s->B * s->T, s->d_model, s->H, x, W1, b1, W2, b2, taps,
                                            static_cast<hipStream_t>(stream)));
}

jb_status jb_gen_conv(const jb_shape* s, const void* x, const void* W1, const void* b1, const void* W2, const void* b2,
                      const void* v, const void* conv_in, float* taps, float* vconv, void* stream) {
  const char* fn = "jb_gen_conv";
  jb_status st = check_shape(fn, s, false);
  if (st) return st;
  if (s->T > 0) { JB_REQUIRE_PTR(x); JB_REQUIRE_PTR(v); JB_REQUIRE_PTR(taps); JB_REQUIRE_PTR(vconv); }
  JB_REQUIRE_PTR(W1); JB_REQUIRE_PTR(W2); JB_OPTIONAL_PTR(b1); JB_OPTIONAL_PTR(b2); JB_OPTIONAL_PTR(conv_in);
  const int io = s->io_dtype == JB_F32 ? jb::IO_F32 : jb::IO_BF16;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  hipError_t e = jb::launch_gen_taps(io, (int64_t)s->B * s->T, s->d_model, s->H, x, W1, b1, W2, b2, taps, hs);
  if (e == hipSuccess) e = jb::launch_conv(io, s->B, s->T, s->H, s->dv, taps, v, conv_in, vconv, hs);
  return hip_status(fn, e);
}

jb_status jb_prologue(const jb_shape* s, const void* q, const void* k, const float* alpha, float* qhat, float* khat,
                      float* g, void* stream) {
  const char* fn = "jb_prologue";
  jb_status st = check_shape(fn, s, false);
  if (st) return st;
  if (s->T > 0) {
    JB_REQUIRE_PTR(q); JB_REQUIRE_PTR(k); JB_REQUIRE_SCALARS(alpha);
    JB_REQUIRE_PTR(qhat); JB_REQUIRE_PTR(khat); JB_REQUIRE_PTR(g);
  }
  const int io = s->io_dtype == JB_F32 ? jb::IO_F32 : jb::IO_BF16;
  return hip_status(fn, jb::launch_prologue(io, s->B, s->T, s->H, s->dk, q, k, alpha, qhat, khat, g,
                                            static_cast<hipStream_t>(stream)));
}

jb_status jb_probe_mfma(int32_t kind, const float* A, const float* B, float* D, void* stream) {
  const char* fn = "jb_probe_mfma";
  if (kind < 0 || kind > 2) return fail(JB_ERR_INVALID_ARG, "%s: kind = %d not in {0, 1, 2}", fn, kind);
  JB_REQUIRE_PTR(A); JB_REQUIRE_PTR(B); JB_REQUIRE_PTR(D);
  return hip_status(fn, jb::launch_probe_mfma(kind, A, B, D, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
