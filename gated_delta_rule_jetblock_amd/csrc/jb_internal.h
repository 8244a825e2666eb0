// jb_internal.h -- host-side launchers shared between the libjetblock
// translation units.  Each launcher enqueues kernels on `stream` and returns
// the hipError_t of hipGetLastError() after the launch.  Arguments have been
// validated by the C-ABI layer (jb_api.hip) before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace jb {

enum IoType { IO_BF16 = 0, IO_F32 = 1 };

// Kernel generator over n rows of x [n][D] -> taps [n][H*4] f32 (and, when
// pre_out is given, the hidden layer before SiLU [n][32] f32).
hipError_t launch_gen_taps(int io, int64_t n, int D, int H, const void* x, const void* W1,
                           const void* b1, const void* W2, const void* b2, float* taps,
                           hipStream_t stream, float* pre_out = nullptr);

// Dynamic causal conv: vconv [B][T][H][dv] f32 from taps [B][T][H][4].
hipError_t launch_conv(int io, int B, int T, int H, int dv, const float* taps, const void* v,
                       const void* conv_in, float* vconv, hipStream_t stream);

// Normalised q, k (f32) and chunk-local cumulative log-gate g.
hipError_t launch_prologue(int io, int B, int T, int H, int dk, const void* q, const void* k,
                           const float* alpha, float* qhat, float* khat, float* g,
                           hipStream_t stream);

// Copy of the last 3 raw value rows of [conv_in; v] into conv_out, per
// sequence (cu_seqlens: packed sequences of at most T rows in `rows` packed
// rows, else dense: rows < 0 means B T).
hipError_t launch_conv_tail(int io, int B, int T, int H, int dv, const void* v,
                            const void* conv_in, void* conv_out, hipStream_t stream,
                            const int* cu_seqlens = nullptr, int64_t rows = -1);

// Chunked prefill (segment summaries, scan, outputs).
struct PrefillPlan {
  int B, T, H, dk, dv;
  int io, out;       // IoType of inputs and of o
  int nchunks;       // ceil(T / 64)
  int seg_len;       // chunks per segment
  int nseg;          // number of segments (per sequence, at most)
  int64_t tokens;    // rows of the token-major tensors (B T, or the packed total)
  const int* cu_seqlens;  // packed batch: B + 1 row offsets on the device, T the longest; NULL: dense
};
PrefillPlan plan_prefill(int B, int T, int H, int dk, int dv, int io, int out, int seg_len);
size_t prefill_workspace_bytes(const PrefillPlan& p);
// taps and segment buffers only (the checkpointing forward pass of the backward)
size_t prefill_base_bytes(const PrefillPlan& p);
bool prefill_supported(const PrefillPlan& p);
hipError_t launch_prefill(const PrefillPlan& p, const void* q, const void* k, const void* v,
                          const float* alpha, const float* beta, const float* taps,
                          const void* conv_in, const float* S0, void* o, float* S_final,
                          void* workspace, hipStream_t stream);

// The fused chunk passes for bf16 inputs (jb_fwd.hip): passes bit 0 runs the
// segment summaries (segments 0 .. nseg-2: Dsum, Phi), bit 1 the output pass
// (o, S_final) from S0 (one segment) or Mstart.  bf16 tensors are passed as
// their 16-bit patterns.
struct FwdArgs {
  int T, H, seg_len, nseg;
  const int* cu_seqlens;   // packed batch (NULL: dense, rows b T ..)
  int64_t total;           // rows of the token-major tensors
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* conv_in;
  const float* alpha;
  const float* beta;
  const float* taps;
  const float* S0;
  const float* Mstart;     // [B][H][nseg][dk][dv]
  float* Dsum;             // [B][H][nseg][dk][dv]
  float* Phi;              // [B][H][nseg][dk][dk]
  void* o;
  float* S_final;
};
bool fwd_supported(int dk, int dv);
hipError_t launch_fwd(const FwdArgs& a, int passes, int dk, int dv, bool out_bf16, int nseg, int H, int B,
                      hipStream_t stream);

// The static-conv variant: q, k, v each pass a causal conv with fixed
// per-channel weights wq, wk [H*dk][4], wv [H*dv][4] (f32) instead of the
// dynamic conv on v; caches cq/ck/cv [B][3][H][d] (NULL: zeros) hold the raw
// rows before the sequence.  bf16 inputs; workspace of
// prefill_static_workspace_bytes (segment buffers only).
size_t prefill_static_workspace_bytes(const PrefillPlan& p);
bool prefill_static_supported(const PrefillPlan& p);
hipError_t launch_prefill_static(const PrefillPlan& p, const void* q, const void* k, const void* v,
                                 const float* alpha, const float* beta, const float* wq, const float* wk,
                                 const float* wv, const void* cq_in, const void* ck_in, const void* cv_in,
                                 const float* S0, void* o, float* S_final, void* workspace, hipStream_t stream);

// The forward pass storing the state entering every chunk, Mck
// [B][H][nchunks][dk][dv] fp16, as the true state times *ck_scale (a power of
// two in device memory; bf16 inputs; workspace as launch_prefill's).
hipError_t launch_prefill_ckpt(const PrefillPlan& p, const void* q, const void* k, const void* v, const float* alpha,
                               const float* beta, const float* taps, const void* conv_in, const float* S0,
                               _Float16* Mck, char* img, void* workspace, hipStream_t stream,
                               const float* ck_scale);

// The gradient of jb_prefill (bf16 inputs, fp32 gradients; one segment per
// sequence).  Shapes built: (dk, dv) in {(32,64), (64,128), (96,256), (128,256)}.
bool backward_supported(int io, int dk, int dv);
size_t backward_workspace_bytes(int B, int T, int H, int dk, int dv, int D);
hipError_t launch_backward(int B, int T, int H, int dk, int dv, int D, const void* x, const void* q, const void* k,
                           const void* v, const float* alpha, const float* beta, const void* W1, const void* b1,
                           const void* W2, const void* b2, const float* S0, const void* conv_in, const float* dout,
                           const float* dS_final, const float* dconv_out, float* dx, float* dq, float* dk_,
                           float* dv_, float* dalpha, float* dbeta, float* dW1, float* db1, float* dW2, float* db2,
                           float* dS0, float* dconv_in, void* workspace, hipStream_t stream);

// One decode step's state update (taps precomputed).
bool decode_supported(int dk, int dv);
hipError_t launch_decode(int io, int out, int B, int H, int dk, int dv, const float* S_in,
                         float* S_out, const void* cache_in, void* cache_out, const void* q_t,
                         const void* k_t, const void* v_t, const float* alpha_t,
                         const float* beta_t, const float* taps, void* o_t, hipStream_t stream);

// One decode step of the static-conv block: caches cq/ck/cv [B][3][H][d]
// (updated in place when out == in), weights as for launch_prefill_static.
hipError_t launch_decode_static(int io, int out, int B, int H, int dk, int dv, const float* S_in, float* S_out,
                                const void* cq_in, const void* ck_in, const void* cv_in, void* cq_out, void* ck_out,
                                void* cv_out, const void* q_t, const void* k_t, const void* v_t,
                                const float* alpha_t, const float* beta_t, const float* wq, const float* wk,
                                const float* wv, void* o_t, hipStream_t stream);

// One whole decode step in one launch (generator taps, conv and state update
// for B tokens); no workspace.
int decode_seq_heads_per_group(int B, int H, int dk, int nw);
hipError_t launch_decode_step(int io, int out, int B, int H, int dk, int dv, int D, const float* S_in, float* S_out,
                              const void* cache_in, void* cache_out, const void* x_t, const void* q_t,
                              const void* k_t, const void* v_t, const float* alpha_t, const float* beta_t,
                              const void* W1, const void* b1, const void* W2, const void* b2, void* o_t,
                              hipStream_t stream);

// The input projections (q, k, v, gates) and the generator taps from x
// (bf16 inputs only) in one kernel; no workspace (project_workspace_bytes is
// 0).  With W1 == NULL only q, k, v are formed.
size_t project_workspace_bytes(int64_t n, int H, int D);
hipError_t launch_project(int64_t n, int H, int dk, int dv, int D, const void* x, const void* Wq, const void* Wk,
                          const void* Wv, const void* Wa, const void* ba, const void* Wb, const void* bb,
                          const void* W1, const void* b1,
                          const void* W2, const void* b2, void* q, void* k, void* v, float* alpha, float* beta,
                          float* taps, void* workspace, hipStream_t stream);

// Zero-fill n floats with a kernel (no memset node, safe under graph capture).
hipError_t launch_fill_zero(float* p, size_t n, hipStream_t stream);

hipError_t launch_probe_mfma(int kind, const float* A, const float* B, float* D, hipStream_t stream);

}  // namespace jb
