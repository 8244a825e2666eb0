/*
 * jetblock.h -- C ABI of libjetblock, the JetBlock token mixer on one AMD
 * MI355X (gfx950).
 *
 * The block (Jet-Nemotron paper, Chinese translation on csdn, section 2.4
 * "new attention block design"; parameters from the xugj520 blog, section
 * 2.2): a kernel generator that shares the Q/K/V projections' input x
 * (Linear -> SiLU -> Linear, hidden width 32) emits 4 causal conv taps per
 * head for every token; the taps convolve the value tokens only (no static
 * conv on Q or K); Gated DeltaNet mixes time.  With L2-normalised q, k and
 * the convolved value v':
 *
 *     S_t = a_t S_{t-1} (I - b_t k_t k_t^T) + b_t v'_t k_t^T,   o_t = S_t q_t
 *
 * The library stores the state transposed, M = S^T, as [dk][dv] with dv
 * contiguous ("dk x dv fp32 state per head").
 *
 * Conventions shared by every entry point
 *   - Every tensor argument is a DEVICE pointer owned by the caller,
 *     contiguous, row-major in the layout given, and 16-byte aligned (alpha
 *     and beta: 4-byte aligned).  The library never allocates, frees or keeps
 *     a pointer after a call returns.
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL means
 *     the default stream).  Inputs must stay valid until the work completes.
 *   - Arguments are validated on the host before anything is enqueued.  On
 *     an error nothing is written, a status is returned and jb_last_error()
 *     names the offending argument.  No exception crosses the ABI.
 *     JB_ERR_HIP reports a failed launch (hipGetLastError after enqueue).
 *   - I/O dtype (shape.io_dtype) applies to x, q, k, v, W1, b1, W2, b2 and
 *     the conv cache: JB_BF16 (bfloat16) or JB_F32.  alpha, beta, the state
 *     and the taps are always float32.  o is shape.out_dtype.
 *   - JB_F32 I/O selects the all-fp32 arithmetic mode (fp32 MFMA); JB_BF16
 *     I/O selects fp16-operand MFMA with fp32 accumulation and fp32 state.
 *
 * Layouts (B sequences, T tokens, H heads, K = taps = 4, G = gen_hidden = 32)
 *   x        [B][T][d_model]         q, k   [B][T][H][dk]
 *   v        [B][T][H][dv]           alpha, beta [B][T][H]  (float32)
 *   W1       [G][d_model]            b1     [G]          (nullable)
 *   W2       [H*K][G]  row h*K+j is tap j of head h;  b2 [H*K] (nullable)
 *   taps     [B][T][H][K] float32, tap j multiplies v_{t-(K-1)+j} (j = K-1
 *            is the current token)
 *   S0, S_final, decode state  [B][H][dk][dv] float32 (M = S^T)
 *   conv cache [B][K-1][H][dv], the last K-1 raw value rows, oldest first
 *   o        [B][T][H][dv]
 *
 * Supported shapes: dk in {32, 64, 96, 128}; dv in {64, 128, 256};
 * gen_hidden == 32; taps == 4; chunk == 64 (0 selects 64); d_model a
 * positive multiple of 128; 1 <= B <= 65535; H <= 32; 0 <= T <= 2^30 for
 * prefill, T == 1 for decode; fewer than 2^40 elements in any tensor.
 * The all-fp32 mode of jb_prefill additionally needs dk*dv <= 64*64 (its
 * tiles must fit in the 160 KB of LDS of one compute unit).
 */
#ifndef JETBLOCK_H
#define JETBLOCK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  JB_OK = 0,
  JB_ERR_INVALID_ARG = 1,  /* null pointer, bad size, misalignment */
  JB_ERR_UNSUPPORTED = 2,  /* valid but not built: shape or dtype combination */
  JB_ERR_WORKSPACE = 3,    /* workspace missing or smaller than required */
  JB_ERR_HIP = 4           /* the HIP runtime reported an error on launch */
} jb_status;

typedef enum { JB_BF16 = 0, JB_F32 = 1 } jb_dtype;

typedef struct {
  int32_t B, T, H, dk, dv, d_model;
  int32_t gen_hidden;   /* must be 32 */
  int32_t taps;         /* must be 4 */
  int32_t chunk;        /* 0 or 64 */
  int32_t io_dtype;     /* jb_dtype of x, q, k, v, W1, b1, W2, b2, conv cache */
  int32_t out_dtype;    /* jb_dtype of o */
  int32_t flags;        /* 0, or JB_FLAG_SEGMENT(n) (jb_prefill only) */
} jb_shape;

/* Tuning knob for jb_prefill: split each sequence into segments of exactly
 * n chunks (1 <= n <= 65535) instead of the automatic choice.  Results agree
 * with any other segmentation up to rounding. */
#define JB_FLAG_SEGMENT(n) ((int32_t)(((uint32_t)(n) & 0xffffu) << 8))

/* Human-readable name of a status code (static string). */
const char* jb_status_string(jb_status status);

/* Message describing the last error raised on the calling thread ("" if
 * none).  The string stays valid until the next call on that thread. */
const char* jb_last_error(void);

/* Library version as major*10000 + minor*100 + patch. */
int32_t jb_version(void);

/*
 * Workspace bytes jb_prefill needs for `shape` (device memory, 256-byte
 * aligned, contents ignored on entry).  Writes *bytes; returns JB_OK or a
 * validation error.  It holds the per-token conv taps (B*T*H*4 floats)
 * and, when a sequence is cut into segments, each segment's start state and
 * its two summaries (2*dk*dv + dk*dk floats per (sequence, head, segment)).
 */
jb_status jb_prefill_workspace_size(const jb_shape* shape, size_t* bytes);

/*
 * jb_prefill -- run the block over B sequences of T tokens.
 *
 * Computes, for every sequence and head, the generator taps from x
 * (csdn section 2.4: Linear, SiLU, Linear emitting conv-kernel weights), the
 * dynamic causal conv of v with those taps (rows before the start come from
 * conv_in, or are zero when conv_in is NULL), and the gated delta-rule
 * recurrence above from S0 (zero when NULL), writing every o_t and the final
 * state.  The sequential recurrence is evaluated in chunks of 64 tokens with
 * a WY/UT intra-chunk transform; long single sequences are split into
 * segments whose transitions are composed by a scan, so results agree with
 * the token-by-token definition up to rounding.
 *
 * Arguments: x, q, k, v, alpha, beta, W1, W2 required; b1, b2, S0, conv_in
 * nullable; o required when T > 0; S_final required; conv_out nullable (the
 * last K-1 raw value rows of [conv_in; v]).  S_final may alias S0 and
 * conv_out may alias conv_in.  alpha should lie in (0, 1] and beta in
 * [0, 1]; other values are not rejected but the result is then undefined
 * in precision.  workspace must hold jb_prefill_workspace_size() bytes.
 */
jb_status jb_prefill(const jb_shape* shape, const void* x, const void* q, const void* k,
                     const void* v, const float* alpha, const float* beta, const void* W1,
                     const void* b1, const void* W2, const void* b2, const float* S0,
                     const void* conv_in, void* o, float* S_final, void* conv_out,
                     void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of device memory jb_prefill_noalloc holds per GPU (its workspace). */
#define JB_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/*
 * jb_prefill_noalloc -- jb_prefill for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  Same arguments, layouts, results and errors as
 * jb_prefill, without the workspace: the call runs jb_prefill's kernels on a
 * file-scope device array of JB_NOALLOC_SCRATCH_BYTES bytes (each GPU the
 * library runs on holds its own copy until the process ends) and calls no
 * hipMalloc, hipFree or allocating library routine.
 *
 * The array of the calling thread's current device is used, so `stream`
 * must belong to that device; its address is looked up on the first call on
 * each device.  Returns JB_ERR_WORKSPACE, launching nothing, when the shape
 * needs more than JB_NOALLOC_SCRATCH_BYTES (jb_prefill_workspace_size tells).
 * At dk = 96, dv = 256, H = 12: one sequence of T = 16384 needs 56 MiB,
 * 64 sequences of 1024 tokens 12 MiB, one of T = 65536 68 MiB (rejected).
 * Nothing in the array has to start at zero.  Every call on one GPU shares
 * that GPU's array: calls that overlap in time on one GPU (different streams
 * or threads) race and must be serialised by the caller.
 */
jb_status jb_prefill_noalloc(const jb_shape* shape, const void* x, const void* q, const void* k,
                             const void* v, const float* alpha, const float* beta, const void* W1,
                             const void* b1, const void* W2, const void* b2, const float* S0,
                             const void* conv_in, void* o, float* S_final, void* conv_out,
                             void* stream);

/* Workspace bytes jb_decode_step needs for `shape` (shape.T must be 1).
 * Currently 0: the step keeps its intermediates on chip. */
jb_status jb_decode_workspace_size(const jb_shape* shape, size_t* bytes);

/*
 * jb_decode_step -- one token for each of B sequences (shape.T == 1).
 *
 * The same block as jb_prefill for a single token: generator taps from x_t,
 * v' from the conv cache and v_t, then with a = M^T k, c = M^T q (one read
 * of the state): u = b (v' - alpha a), o_t = alpha c + (k.q) u,
 * M' = alpha M + k u^T, written to S_out; the cache shifts in the raw v_t.
 * Decode is bound by the state's HBM traffic (csdn section 2.5, finding 4:
 * decoding is memory-bandwidth-bound), which this call reads and writes once.
 *
 * One launch: each workgroup takes one sequence (or a group of its heads),
 * computes that token's generator hidden layer once, and streams the heads'
 * states through registers.
 *
 * Layouts: S_in, S_out [B][H][dk][dv] f32 (S_out may alias S_in);
 * cache_in, cache_out [B][K-1][H][dv] (may alias); x_t [B][d_model];
 * q_t, k_t [B][H][dk]; v_t [B][H][dv]; alpha_t, beta_t [B][H] f32;
 * o_t [B][H][dv] (out_dtype).  workspace may be NULL when
 * jb_decode_workspace_size() reports 0; it is accepted for the signature's
 * stability and not touched.
 */
jb_status jb_decode_step(const jb_shape* shape, const float* S_in, float* S_out,
                         const void* cache_in, void* cache_out, const void* x_t,
                         const void* q_t, const void* k_t, const void* v_t,
                         const float* alpha_t, const float* beta_t, const void* W1,
                         const void* b1, const void* W2, const void* b2, void* o_t,
                         void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Packed batches of sequences of different lengths: the serving side of the
 * pages' throughput method (Jet-Nemotron csdn translation, section 3.1 on the
 * throughput test bed, and appendix A.3: chunked prefill, the decode batch
 * made as large as memory allows).
 * The token-major tensors hold the sequences back to back: sequence b is rows
 * cu_seqlens[b] .. cu_seqlens[b+1] - 1.  S0, S_final [B][H][dk][dv] and
 * conv_in, conv_out [B][3][H][dv] are per sequence, in the layouts
 * jb_decode_step takes, so a prefill's outputs are a decode batch's inputs.
 * ------------------------------------------------------------------------- */

/* Workspace bytes of jb_prefill_varlen for `shape` and `total_tokens` rows. */
jb_status jb_prefill_varlen_workspace_size(const jb_shape* shape, int64_t total_tokens,
                                           size_t* bytes);

/*
 * jb_prefill_varlen -- jb_prefill over B packed sequences.
 *   shape.B      number of sequences; shape.T the longest sequence's length
 *                (the grid is planned for it: a longer sequence is cut to its
 *                first shape.T tokens)
 *   total_tokens rows of the packed tensors, = cu_seqlens[B] (<= B * T)
 *   cu_seqlens   int32 [B+1] in device memory: 0, then non-decreasing row
 *                offsets up to total_tokens (the library cannot check device
 *                memory on the host: other values make it read and write
 *                outside the tensors); an empty sequence passes its state and
 *                cache through
 *   x [total][d_model], q, k [total][H][dk], v [total][H][dv],
 *   alpha, beta [total][H], o [total][H][dv]; the rest as in jb_prefill.
 */
jb_status jb_prefill_varlen(const jb_shape* shape, int64_t total_tokens,
                            const int32_t* cu_seqlens, const void* x, const void* q,
                            const void* k, const void* v, const float* alpha,
                            const float* beta, const void* W1, const void* b1,
                            const void* W2, const void* b2, const float* S0,
                            const void* conv_in, void* o, float* S_final, void* conv_out,
                            void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * The block from its layer input x.  The kernel generator takes the same
 * input as the Q/K/V projection layers (csdn translation, section 2.4), so the
 * projections and the generator's first layer share one pass over x:
 *   q = Wq x, k = Wk x, v = Wv x     (bf16, nearest-even from the fp32 sum)
 *   alpha = sigmoid(Wa x + ba), beta = sigmoid(Wb x + bb)   (fp32, per head)
 *   taps  = W2 SiLU(W1 x + b1) + b2                          (fp32, 4 per head)
 * The pages do not describe the gate projections; a sigmoid keeps both
 * gates in (0, 1).  bf16 inputs only (shape.io_dtype == JB_BF16); other
 * dtypes return JB_ERR_UNSUPPORTED.
 *
 * Weights (bf16, row-major, caller-owned): Wq, Wk [H*dk][d_model];
 * Wv [H*dv][d_model]; Wa, Wb [H][d_model]; W1 [32][d_model]; W2 [4H][32].
 * The Q/K/V layers take no bias; the biases ba, bb [H], b1 [32], b2 [4H] are
 * nullable (NULL means zero).  All pointers 16-byte aligned.
 * ------------------------------------------------------------------------- */

/* Workspace bytes of jb_project for `shape` (B*T tokens): always 0, kept so
 * that callers size every entry point the same way. */
jb_status jb_project_workspace_size(const jb_shape* shape, size_t* bytes);

/*
 * jb_project -- the projections above for the B*T rows of x [B][T][d_model]:
 * writes q, k [B][T][H][dk] and v [B][T][H][dv] (bf16), alpha, beta
 * [B][T][H] and taps [B][T][H][4] (fp32).  One kernel reads x once per
 * token tile and forms every output on bf16 matrix cores with fp32
 * accumulation (q, k, v rounded once; SiLU, the generator's second layer and
 * the sigmoids in fp32).  workspace and workspace_bytes are not used (may be
 * NULL and 0).
 */
jb_status jb_project(const jb_shape* shape, const void* x, const void* Wq, const void* Wk,
                     const void* Wv, const void* Wa, const void* ba, const void* Wb, const void* bb,
                     const void* W1, const void* b1, const void* W2, const void* b2,
                     void* q, void* k, void* v, float* alpha, float* beta, float* taps,
                     void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes of jb_prefill_from_x for `shape`. */
jb_status jb_prefill_from_x_workspace_size(const jb_shape* shape, size_t* bytes);

/*
 * jb_prefill_from_x -- jb_project followed by jb_prefill's recurrence: the
 * block over B sequences of T tokens from x.  q, k, v and the gates live in
 * the workspace.  S0, conv_in, o, S_final, conv_out as in jb_prefill.
 */
jb_status jb_prefill_from_x(const jb_shape* shape, const void* x, const void* Wq, const void* Wk,
                            const void* Wv, const void* Wa, const void* ba, const void* Wb, const void* bb,
                            const void* W1, const void* b1, const void* W2, const void* b2,
                            const float* S0, const void* conv_in, void* o, float* S_final,
                            void* conv_out, void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes of jb_decode_step_from_x for `shape` (shape.T must be 1). */
jb_status jb_decode_step_from_x_workspace_size(const jb_shape* shape, size_t* bytes);

/*
 * jb_decode_step_from_x -- one decode step for B sequences from the layer
 * input x_t [B][d_model]: the projection kernel forms q, k, v of the B tokens
 * in the workspace, then the decode step, which forms the taps and the gates
 * from x_t itself.  S_in, S_out, cache_in, cache_out, o_t as in
 * jb_decode_step.
 */
jb_status jb_decode_step_from_x(const jb_shape* shape, const float* S_in, float* S_out,
                                const void* cache_in, void* cache_out, const void* x_t,
                                const void* Wq, const void* Wk, const void* Wv, const void* Wa,
                                const void* ba, const void* Wb, const void* bb, const void* W1,
                                const void* b1, const void* W2, const void* b2, void* o_t,
                                void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * The static-conv Gated DeltaNet block, the block JetBlock replaces (csdn
 * translation, section 2.4: earlier linear-attention blocks convolve with
 * fixed kernels; JetBlock makes the V kernel dynamic and drops the Q and K
 * convs), kept for measuring the two side by side.  The pages give no
 * detail; read here as a causal depthwise conv of size 4 with fixed weights
 * on each of q, k and v (tap j multiplies token t-3+j, no activation), then
 * L2 normalisation of q and k and the same gated delta rule:
 *   q'_t[c] = sum_j wq[c][j] q_{t-3+j}[c]   (likewise k' with wk, v' with wv)
 *
 * Weights (fp32, row-major, 16-byte aligned): wq, wk [H*dk][4]; wv [H*dv][4],
 * row h*d + c for channel c of head h.  Caches of raw rows, oldest first:
 * cache_q, cache_k [B][3][H][dk]; cache_v [B][3][H][dv] (I/O dtype).
 * ------------------------------------------------------------------------- */

/* Workspace bytes of jb_prefill_static for `shape` (0 with one segment). */
jb_status jb_prefill_static_workspace_size(const jb_shape* shape, size_t* bytes);

/*
 * jb_prefill_static -- the static-conv block over B sequences of T tokens.
 * q, k, v, alpha, beta, S0, o, S_final and shape.flags as in jb_prefill.
 * cache_q_in, cache_k_in, cache_v_in: all three or none (NULL: zero rows
 * before the sequence).  cache_*_out: each nullable; written after the
 * recurrence has read the incoming caches, so an out cache may alias its in
 * cache.  Built for bf16 inputs and (dk, dv) in {(32, 64), (64, 128),
 * (96, 256), (128, 256)}; other shapes return JB_ERR_UNSUPPORTED.
 */
jb_status jb_prefill_static(const jb_shape* shape, const void* q, const void* k, const void* v,
                            const float* alpha, const float* beta, const float* wq, const float* wk,
                            const float* wv, const float* S0, const void* cache_q_in,
                            const void* cache_k_in, const void* cache_v_in, void* o, float* S_final,
                            void* cache_q_out, void* cache_k_out, void* cache_v_out, void* workspace,
                            size_t workspace_bytes, void* stream);

/*
 * jb_decode_step_static -- one decode step of the static-conv block for B
 * sequences (shape.T == 1): q_t, k_t [B][H][dk], v_t [B][H][dv], alpha_t,
 * beta_t [B][H]; S_in, S_out, o_t as in jb_decode_step.  All six caches are
 * required; each out cache may alias its in cache (updated in place).  Both
 * I/O dtypes, every (dk, dv) of jb_decode_step.  No workspace.
 */
jb_status jb_decode_step_static(const jb_shape* shape, const float* S_in, float* S_out,
                                const void* cache_q_in, const void* cache_k_in,
                                const void* cache_v_in, void* cache_q_out, void* cache_k_out,
                                void* cache_v_out, const void* q_t, const void* k_t,
                                const void* v_t, const float* alpha_t, const float* beta_t,
                                const float* wq, const float* wk, const float* wv, void* o_t,
                                void* stream);

/* ---------------------------------------------------------------------------
 * The gradient of jb_prefill, for training the block (the pages train
 * JetBlock inside the model: csdn translation, sections 2.2 and 3.1).
 * ------------------------------------------------------------------------- */

/* Workspace bytes of jb_backward for `shape`. */
jb_status jb_backward_workspace_size(const jb_shape* shape, size_t* bytes);

/*
 * jb_backward -- reverse-mode gradient of jb_prefill over B sequences of T
 * tokens.  Inputs as in jb_prefill (bf16 I/O only, shape.flags == 0); dout
 * [B][T][H][dv] is the gradient of o, dS_final [B][H][dk][dv] and dconv_out
 * [B][K-1][H][dv] those of S_final and conv_out (both nullable: zero), all
 * float32.  Outputs, all float32 and required:
 *   dx [B][T][d_model]; dq, dk [B][T][H][dk]; dv [B][T][H][dv];
 *   dalpha, dbeta [B][T][H]; dW1 [32][d_model], db1 [32]; dW2 [4H][32],
 *   db2 [4H]; dS0 [B][H][dk][dv]; dconv_in [B][K-1][H][dv]
 * (dS0 and dconv_in are returned also when S0 / conv_in are NULL: the
 * gradient with respect to the zeros used in their place).  The pass
 * recomputes the forward states chunk by chunk; the gradients of o and
 * S_final are scaled internally by a power of two so that the fp16
 * matrix-core operands cannot overflow.  Built for (dk, dv) in {(32, 64),
 * (64, 128), (96, 256), (128, 256)}.  workspace: jb_backward_workspace_size()
 * bytes, 256-byte aligned.
 */
jb_status jb_backward(const jb_shape* shape, const void* x, const void* q, const void* k,
                      const void* v, const float* alpha, const float* beta, const void* W1,
                      const void* b1, const void* W2, const void* b2, const float* S0,
                      const void* conv_in, const float* dout, const float* dS_final,
                      const float* dconv_out, float* dx, float* dq, float* dk, float* dv,
                      float* dalpha, float* dbeta, float* dW1, float* db1, float* dW2, float* db2,
                      float* dS0, float* dconv_in, void* workspace, size_t workspace_bytes,
                      void* stream);

/* ---------------------------------------------------------------------------
 * Single-stage entry points.  Each runs one stage of the path by itself so
 * that it can be checked on its own; the two calls above fuse these stages.
 * ------------------------------------------------------------------------- */

/*
 * jb_gen_taps -- kernel generator (csdn section 2.4; hidden width 32 from
 * the xugj520 blog, section 2.2) on the B*T rows of x:
 * taps = W2 SiLU(W1 x + b1) + b2, written as taps [B][T][H][K] float32.
 */
jb_status jb_gen_taps(const jb_shape* shape, const void* x, const void* W1, const void* b1,
                      const void* W2, const void* b2, float* taps, void* stream);

/*
 * jb_gen_conv -- kernel generator followed by the dynamic causal conv of v
 * (csdn section 2.4: dynamic kernels applied to the value tokens):
 * v'_t[h][c] = sum_j taps_t[h][j] v_{t-(K-1)+j}[h][c], rows before the start
 * from conv_in or zero.  Writes taps (nullable) and vconv [B][T][H][dv]
 * float32.
 */
jb_status jb_gen_conv(const jb_shape* shape, const void* x, const void* W1, const void* b1,
                      const void* W2, const void* b2, const void* v, const void* conv_in,
                      float* taps, float* vconv, void* stream);

/*
 * jb_prologue -- the gate and normalisation stage on its own:
 * qhat = q (sum q^2 + 1e-6)^(-1/2), khat likewise (float32, [B][T][H][dk]),
 * and g [B][T][H] float32, the inclusive cumulative sum of ln(alpha) within
 * each 64-token chunk (the log of the chunk-local decay products).
 */
jb_status jb_prologue(const jb_shape* shape, const void* q, const void* k,
                      const float* alpha, float* qhat, float* khat, float* g, void* stream);

/*
 * jb_decode_update -- the state-update stage of jb_decode_step on its own,
 * with the taps [B][H][K] float32 already computed (e.g. by jb_gen_taps on
 * x_t): conv of the cache and v_t, q/k normalisation, the one-pass update
 * of the state (csdn section 2.5, finding 4: decode is bound by memory
 * bandwidth) and the cache shift.  Arguments as in jb_decode_step.
 */
jb_status jb_decode_update(const jb_shape* shape, const float* S_in, float* S_out,
                           const void* cache_in, void* cache_out, const void* q_t,
                           const void* k_t, const void* v_t, const float* alpha_t,
                           const float* beta_t, const float* taps, void* o_t, void* stream);

/*
 * jb_probe_mfma -- runs one 16x16x32 matrix-core product D = A B on one
 * wavefront with the operand placement the library's kernels assume
 * (A [16][32], B [32][16], D [16][16], row-major float32 device buffers).
 * kind 0: fp16 operands in the accumulator-chaining K order; kind 1: bf16
 * operands in contiguous K order; kind 2: fp32 operands (eight 16x16x4
 * products).  Operands are rounded to the operand type on load.  Exposed so
 * that a test can check the placement against a host product.
 */
jb_status jb_probe_mfma(int32_t kind, const float* A, const float* B, float* D, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* JETBLOCK_H */
