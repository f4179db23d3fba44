/*
 * gdn.h -- C ABI of the GatedDeltaNet layer library for AMD MI355X (gfx950).
 *
 * The layer, over one packed row of N variable-length sequences:
 *
 *   conv:   y = SiLU(causal depthwise conv1d(x)), then each q and k head is
 *           L2-normalised:  y <- y / sqrt(|y|^2 + eps)
 *   chunk:  the gated delta rule per sequence and v-head,
 *           S_t = e^{g_t} S_{t-1} (I - b_t k_t k_t^T) + b_t v_t k_t^T,
 *           o_t = scale * S_t q_t,
 *           evaluated chunk by chunk in the WY form
 *   norm:   RMSNormGated:  y = o * rsqrt(mean(o^2) + eps) * w * SiLU(z)
 *
 * and the reverse mode of each step.  Where the pages name these pieces:
 *  - "[Qwen3.5 MoE] Add hybrid decoder model (GatedDeltaNet + full attention +
 *    MoE)", Summary: GatedDeltaNet linear attention, RMSNormGated, depthwise
 *    conv1d, softplus gate.
 *  - "Support Qwen35 SFT", XTuner changes: GatedDeltaNet with varlen support
 *    on causal_conv1d and flash-linear-attention; per-token sequence ids.
 *  - "feat(models): dense Qwen3.5 custom attention", Summary and review fix:
 *    cu_seqlens derived from position_ids; the path receives one packed row.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All tensor pointers are DEVICE pointers.  The caller allocates every
 *    buffer, including workspace (sized by the *_workspace queries).  The
 *    library allocates no device memory, never synchronises and never reads
 *    device memory from the host; its only mutable global state is the opt-in
 *    timing record of gdn_profile_enable (mutex-guarded) and the per-device
 *    scratch array of gdn_norm_gate_bwd_noalloc.  All work is enqueued on `stream`
 *    (a hipStream_t; NULL means the default stream).
 *  - The compute calls enqueue kernel launches only: no memset, copy, event
 *    or wait (while gdn_profile_enable is off).  A sequence of them can be
 *    recorded into a HIP graph by stream capture; each replay re-runs every
 *    kernel on the captured pointers and reads their current contents.
 *  - Arguments are validated on the host before anything is enqueued; on any
 *    error nothing is launched.  Device-side contents that break a documented
 *    precondition (for example a cu_seqlens that is not non-decreasing or
 *    does not end at total_tokens) give undefined results.
 *  - cu_seqlens: int32 [N+1] on the device, cu[0] = 0, cu[N] = T,
 *    non-decreasing; sequence n owns tokens [cu[n], cu[n+1]).  Zero-length
 *    sequences are allowed, and so is an empty row (T = 0): then the
 *    token-indexed pointers (x, y, q, k, v, g, beta, o, z and their
 *    gradients) may be NULL, states are still written (ht = h0 or 0,
 *    dh0 = dht or 0) and weight gradients are zero.
 *  - Element type of x, y, q, k, v, o, z, w_conv, w_norm and their gradients
 *    is shape->dtype (GDN_F32 = float, GDN_BF16 = bfloat16).  g, beta,
 *    states, dg, dbeta, dw_conv, dw_norm and state gradients are always
 *    float32.  All arithmetic is float32 (bf16 values are MFMA operands).
 *  - Layouts are token-major:  x, y [T][Cch] with Cch = 2*Hk*dk + Hv*dv and
 *    channel blocks [q (Hk*dk) | k (Hk*dk) | v (Hv*dv)];  o, z, norm output
 *    [T][Hv][dv];  g, beta [T][Hv];  states [N][Hv][dk][dv] holding H = S^T
 *    (row i = key dimension, column c = value dimension).
 *  - V-head h reads q/k head h / (Hv/Hk).
 *  - Pointers must be 16-byte aligned; token strides (in elements) must keep
 *    every row 16-byte aligned.
 *  - Outputs are overwritten, never accumulated into.  Every result is
 *    deterministic: the same inputs give the same bits on every run.
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum gdn_status {
  GDN_OK = 0,
  GDN_ERR_INVALID_ARG = -1,  /* null required pointer, bad size, misaligned pointer/stride */
  GDN_ERR_UNSUPPORTED = -2,  /* valid but unsupported shape (head dim, chunk, dtype, width) */
  GDN_ERR_WORKSPACE = -3,    /* workspace pointer null or smaller than the query returns */
  GDN_ERR_HIP = -4           /* a kernel launch failed (hipGetLastError) */
} gdn_status;

enum { GDN_F32 = 0, GDN_BF16 = 1 };

typedef struct gdn_shape {
  int32_t n_seqs;       /* N >= 1 */
  int32_t total_tokens; /* T >= 0, equals cu_seqlens[N] */
  int32_t h_qk;         /* Hk >= 1 */
  int32_t h_v;          /* Hv >= 1, Hv % Hk == 0 */
  int32_t d_k;          /* 16, 32, 64 or 128 */
  int32_t d_v;          /* must equal d_k */
  int32_t chunk;        /* 16, 32 or 64 (GDN_F32 needs chunk <= 32) */
  int32_t dtype;        /* GDN_F32 or GDN_BF16 */
  float scale;          /* query scale (o_t = scale * S_t q_t) */
} gdn_shape;

typedef void* gdn_stream; /* hipStream_t */

/* Human-readable name of a status code (static string). */
const char* gdn_status_string(gdn_status status);

/* --------------------------------------------------------------------------
 * Chunk index (varlen bookkeeping).  Chunks of `chunk` tokens restart at each
 * sequence start and never straddle two sequences; the last chunk of a
 * sequence may be shorter.  Pages: "feat(models): dense Qwen3.5 custom
 * attention" (cu_seqlens; seq_lens as the packed-sample boundary contract),
 * "Support Qwen35 SFT" (review: per-token seq_idx needed by GatedDeltaNet).
 *
 * gdn_max_chunks: upper bound ceil(T/chunk) + N used to size every grid and
 *   buffer without reading cu_seqlens on the host.
 * gdn_chunk_index writes
 *   table      int32 [max_chunks][4]: (sequence, first token, length, 0) for
 *              chunk c < n_chunks, and (-1, 0, 0, 0) after the last chunk;
 *   seq_chunk0 int32 [N+1]: index of the first chunk of each sequence,
 *              seq_chunk0[N] = n_chunks.
 * -------------------------------------------------------------------------- */
int64_t gdn_max_chunks(const gdn_shape* shape);
gdn_status gdn_chunk_index(const gdn_shape* shape, const int32_t* cu_seqlens,
                           int32_t* table, int32_t* seq_chunk0, gdn_stream stream);

/* --------------------------------------------------------------------------
 * Causal depthwise conv1d + SiLU + L2 normalisation of q and k heads.
 * Pages: "[Qwen3.5 MoE] Add hybrid decoder model", Summary (depthwise conv1d
 * in GatedDeltaNet); "Support Qwen35 SFT", Notes and XTuner changes
 * (causal_conv1d, varlen mode).
 *   c[t, ch] = sum_{i < width} w_conv[ch][i] * x[t - width + 1 + i][ch], terms
 *              before the first token of t's sequence are zero (no history is
 *              carried into a sequence);
 *   y = c * sigmoid(c);  q/k heads (channels < 2*Hk*dk, groups of dk):
 *   y <- y / sqrt(sum(y^2) + l2_eps).
 * x, y: [T][Cch] (y must not alias x); w_conv: [Cch][width]; width in 2..4.
 * -------------------------------------------------------------------------- */
gdn_status gdn_conv1d(const gdn_shape* shape, const void* x, const void* w_conv, int32_t width,
                      float l2_eps, const int32_t* cu_seqlens, void* y, gdn_stream stream);

/* gdn_conv1d for a prefill that continues earlier calls (chunked prefill): each
 * sequence starts from its carried window of previous inputs instead of zero
 * history.  Page: "feat(models): dense Qwen3.5 custom attention", KL mismatch
 * table and review overview (continuation outside the training path).
 *   window_in:  [N][width-1][Cch] (dtype), sequence n's previous width-1
 *               inputs, oldest first, or NULL (zero history, as gdn_conv1d);
 *   window_out: NULL, or [N][width-1][Cch]: the last width-1 inputs of
 *               [window_in[n] ; x rows of sequence n] (gdn_conv1d_window);
 *               must not alias window_in, x or y.  N <= 65535 when given.
 * Other arguments as gdn_conv1d. */
gdn_status gdn_conv1d_prefill(const gdn_shape* shape, const void* x, const void* w_conv, int32_t width,
                              float l2_eps, const int32_t* cu_seqlens, const void* window_in, void* y,
                              void* window_out, gdn_stream stream);

/* Reverse mode of gdn_conv1d.  dy: gradient w.r.t. y [T][Cch]; writes dx
 * [T][Cch] (dtype) and dw_conv [Cch][width] (float32, summed over all tokens
 * in a fixed order).  Workspace: gdn_conv1d_bwd_workspace bytes. */
size_t gdn_conv1d_bwd_workspace(const gdn_shape* shape, int32_t width);
gdn_status gdn_conv1d_bwd(const gdn_shape* shape, const void* dy, const void* x, const void* w_conv,
                          int32_t width, float l2_eps, const int32_t* cu_seqlens, void* dx,
                          float* dw_conv, void* ws, size_t ws_bytes, gdn_stream stream);

/* --------------------------------------------------------------------------
 * Gates of the recurrence.  Page: "[Qwen3.5 MoE] Add hybrid decoder model",
 * Summary (softplus registered as a pointwise op for the GatedDeltaNet gate).
 *   g[t,h]    = -exp(A_log[h]) * softplus(a[t,h] + dt_bias[h])   (log-decay, < 0)
 *   beta[t,h] = sigmoid(b[t,h])
 * a, b, g, beta: float32 [T][Hv] (g, beta as gdn_chunk_fwd takes them);
 * A_log, dt_bias: float32 [Hv].  Only shape->total_tokens and h_v are used
 * (the other fields must still be valid).  Pointers need 4-byte alignment;
 * g and beta must not alias a or b.  An empty row (T = 0) launches nothing.
 * -------------------------------------------------------------------------- */
gdn_status gdn_gates(const gdn_shape* shape, const float* a, const float* b, const float* A_log,
                     const float* dt_bias, float* g, float* beta, gdn_stream stream);

/* Reverse mode of gdn_gates.  dg, dbeta: float32 [T][Hv] gradients w.r.t. g
 * and beta (gdn_chunk_bwd writes them).  Writes da, db [T][Hv] and dA_log,
 * ddt_bias [Hv] (float32, sums over all tokens in a fixed order; zero for an
 * empty row).  Workspace: gdn_gates_bwd_workspace bytes, 16-byte aligned. */
size_t gdn_gates_bwd_workspace(const gdn_shape* shape);
gdn_status gdn_gates_bwd(const gdn_shape* shape, const float* a, const float* b, const float* A_log,
                         const float* dt_bias, const float* dg, const float* dbeta, float* da, float* db,
                         float* dA_log, float* ddt_bias, void* ws, size_t ws_bytes, gdn_stream stream);

/* --------------------------------------------------------------------------
 * Gated delta rule, chunked.  Pages: "[Qwen3.5 MoE] Add hybrid decoder
 * model", Summary (GatedDeltaNet linear attention, FLA kernels optional with a
 * naive fallback); "Support Qwen35 SFT", XTuner changes (varlen mode).
 *   q, k: element (t, j, i) at q[t*tok_stride_qk + j*dk + i] (k likewise);
 *   v:    element (t, h, c) at v[t*tok_stride_v + h*dv + c];
 *   q and k are used as given (the caller normalises them: gdn_conv1d does);
 *   g, beta: float32 [T][Hv]; g <= 0 is assumed for the stated accuracy;
 *   h0: float32 [N][Hv][dk][dv] initial states, or NULL for zero states;
 *   o:  [T][Hv][dv] output;  ht: float32 [N][Hv][dk][dv] final states or NULL.
 * A zero-length sequence leaves its state unchanged (ht = h0 or 0).
 * -------------------------------------------------------------------------- */
size_t gdn_chunk_fwd_workspace(const gdn_shape* shape);
gdn_status gdn_chunk_fwd(const gdn_shape* shape, const void* q, const void* k, const void* v,
                         int64_t tok_stride_qk, int64_t tok_stride_v, const float* g,
                         const float* beta, const int32_t* cu_seqlens, const float* h0, void* o,
                         float* ht, void* ws, size_t ws_bytes, gdn_stream stream);

/* Reverse mode of gdn_chunk_fwd (recomputes the forward internally).
 *   d_o: [T][Hv][dv] gradient w.r.t. o;  dht: float32 gradient w.r.t. ht, or NULL;
 *   dq, dk: written with tok_stride_qk like q and k (may point into a
 *           [T][Cch] buffer next to dv);  dv: written with tok_stride_v;
 *   dg, dbeta: float32 [T][Hv];  dh0: float32 [N][Hv][dk][dv] or NULL. */
size_t gdn_chunk_bwd_workspace(const gdn_shape* shape);
gdn_status gdn_chunk_bwd(const gdn_shape* shape, const void* q, const void* k, const void* v,
                         int64_t tok_stride_qk, int64_t tok_stride_v, const float* g,
                         const float* beta, const int32_t* cu_seqlens, const float* h0,
                         const void* d_o, const float* dht, void* dq, void* dk, void* dv,
                         float* dg, float* dbeta, float* dh0, void* ws, size_t ws_bytes,
                         gdn_stream stream);

/* Training pair: the forward keeps, in a backward-sized workspace, the
 * per-chunk products that gdn_chunk_bwd would otherwise recompute (the WY
 * factors and their transposes, the state entering every chunk, W), and the
 * backward reads them instead.  Same computation and same results, bit for
 * bit, as gdn_chunk_fwd followed by gdn_chunk_bwd.  Pages: "Support Qwen35
 * SFT", feature list (training the layer).
 *   gdn_chunk_fwd_save: arguments as gdn_chunk_fwd; ws_bytes >=
 *     gdn_chunk_bwd_workspace(shape).
 *   gdn_chunk_bwd_saved: arguments as gdn_chunk_bwd, with the same ws and the
 *     same shape, q, k, v, strides, g, beta, cu_seqlens and h0 (contents
 *     unchanged) as the gdn_chunk_fwd_save call it follows; the workspace must
 *     not be used by any other call in between.  The caller owns that pairing:
 *     a mismatch is not detected and gives undefined results. */
gdn_status gdn_chunk_fwd_save(const gdn_shape* shape, const void* q, const void* k, const void* v,
                              int64_t tok_stride_qk, int64_t tok_stride_v, const float* g,
                              const float* beta, const int32_t* cu_seqlens, const float* h0, void* o,
                              float* ht, void* ws, size_t ws_bytes, gdn_stream stream);
gdn_status gdn_chunk_bwd_saved(const gdn_shape* shape, const void* q, const void* k, const void* v,
                               int64_t tok_stride_qk, int64_t tok_stride_v, const float* g,
                               const float* beta, const int32_t* cu_seqlens, const float* h0,
                               const void* d_o, const float* dht, void* dq, void* dk, void* dv,
                               float* dg, float* dbeta, float* dh0, void* ws, size_t ws_bytes,
                               gdn_stream stream);

/* gdn_chunk_fwd on fp8 inputs: q, k and v arrive as OCP e4m3 bytes (1 sign,
 * 4 exponent bits with bias 7, 3 mantissa bits) with one scale per tensor,
 * value = e4m3 value * scale.  Pages: "Support Qwen35 SFT", feature list
 * (fp8 training).  The scales must be powers of two (2^-100 .. 2^100;
 * GDN_ERR_INVALID_ARG otherwise), so every dequantised input is a bf16 value:
 * the kernels decode the bytes exactly as they load them and run the bf16
 * path, and the results are bit-identical to gdn_chunk_fwd's on the
 * dequantised bf16 tensors.  Token strides are in elements (bytes) and must
 * be multiples of 16; shape->dtype is GDN_BF16 (the element type of o);
 * supported at d = 128, chunk 64 (GDN_ERR_UNSUPPORTED otherwise).  The e4m3
 * NaN code (0x7f, 0xff) is not a valid input.  Other arguments and the
 * workspace (gdn_chunk_fwd_workspace) as gdn_chunk_fwd. */
gdn_status gdn_chunk_fwd_fp8(const gdn_shape* shape, const void* q, const void* k, const void* v,
                             int64_t tok_stride_qk, int64_t tok_stride_v, float scale_q, float scale_k, float scale_v,
                             const float* g, const float* beta, const int32_t* cu_seqlens, const float* h0, void* o,
                             float* ht, void* ws, size_t ws_bytes, gdn_stream stream);

/* --------------------------------------------------------------------------
 * Fused gates: the chunked recurrence with g and beta computed inside its
 * kernels from the gates' raw inputs, as gdn_gates would (same functions,
 * same bits), so g and beta are never written or read as arrays; the
 * backward returns the gradients w.r.t. those raw inputs, as gdn_gates_bwd
 * would from dg and dbeta.  Page: "[Qwen3.5 MoE] Add hybrid decoder model",
 * Summary (the softplus gate of GatedDeltaNet).
 *   gates:  a, b float32 [T][Hv]; A_log, dt_bias float32 [Hv];
 *           g = -exp(A_log[h]) softplus(a[t,h] + dt_bias[h]), beta = sigmoid(b[t,h]).
 *   dgates: da, db float32 [T][Hv]; dA_log, ddt_bias float32 [Hv] (sums over
 *           every token in a fixed order: deterministic; zero for an empty row).
 * Every other argument, the workspace sizes and the pairing rules of the
 * saved forms are those of gdn_chunk_fwd, gdn_chunk_fwd_save, gdn_chunk_bwd and
 * gdn_chunk_bwd_saved.  Pointers need 4-byte alignment. */
typedef struct gdn_gate_inputs {
  const float* a;
  const float* b;
  const float* A_log;
  const float* dt_bias;
} gdn_gate_inputs;

typedef struct gdn_gate_grads {
  float* da;
  float* db;
  float* dA_log;
  float* ddt_bias;
} gdn_gate_grads;

gdn_status gdn_chunk_fwd_gated(const gdn_shape* shape, const void* q, const void* k, const void* v,
                               int64_t tok_stride_qk, int64_t tok_stride_v, const gdn_gate_inputs* gates,
                               const int32_t* cu_seqlens, const float* h0, void* o, float* ht, void* ws,
                               size_t ws_bytes, gdn_stream stream);
gdn_status gdn_chunk_fwd_save_gated(const gdn_shape* shape, const void* q, const void* k, const void* v,
                                    int64_t tok_stride_qk, int64_t tok_stride_v, const gdn_gate_inputs* gates,
                                    const int32_t* cu_seqlens, const float* h0, void* o, float* ht, void* ws,
                                    size_t ws_bytes, gdn_stream stream);
gdn_status gdn_chunk_bwd_gated(const gdn_shape* shape, const void* q, const void* k, const void* v,
                               int64_t tok_stride_qk, int64_t tok_stride_v, const gdn_gate_inputs* gates,
                               const int32_t* cu_seqlens, const float* h0, const void* d_o, const float* dht,
                               void* dq, void* dk, void* dv, const gdn_gate_grads* dgates, float* dh0, void* ws,
                               size_t ws_bytes, gdn_stream stream);
gdn_status gdn_chunk_bwd_saved_gated(const gdn_shape* shape, const void* q, const void* k, const void* v,
                                     int64_t tok_stride_qk, int64_t tok_stride_v, const gdn_gate_inputs* gates,
                                     const int32_t* cu_seqlens, const float* h0, const void* d_o,
                                     const float* dht, void* dq, void* dk, void* dv, const gdn_gate_grads* dgates,
                                     float* dh0, void* ws, size_t ws_bytes, gdn_stream stream);

/* --------------------------------------------------------------------------
 * RMSNormGated epilogue.  Page: "[Qwen3.5 MoE] Add hybrid decoder model",
 * Summary (RMSNormGated).
 *   per row (token, v-head) of dv values:
 *   y = o * rsqrt(mean(o^2) + eps) * w_norm * z * sigmoid(z)
 * o, z, y: [T][Hv][dv]; w_norm: [dv] (dtype).  y may alias o.
 * -------------------------------------------------------------------------- */
gdn_status gdn_norm_gate(const gdn_shape* shape, const void* o, const void* z, const void* w_norm,
                         float eps, void* y, gdn_stream stream);

/* Reverse mode of gdn_norm_gate.  Writes d_o, dz [T][Hv][dv] (dtype) and
 * dw_norm [dv] (float32, fixed-order sum over rows). */
size_t gdn_norm_gate_bwd_workspace(const gdn_shape* shape);
gdn_status gdn_norm_gate_bwd(const gdn_shape* shape, const void* dy, const void* o, const void* z,
                             const void* w_norm, float eps, void* d_o, void* dz, float* dw_norm,
                             void* ws, size_t ws_bytes, gdn_stream stream);

/* gdn_norm_gate_bwd without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  It allocates nothing: the backward's dw
 * partials live in a scratch array inside the library, 512 KiB per device
 * (1024 blocks x d_v floats, d_v <= 128), created with the library's code
 * object on each device it runs on and held until the process ends.  Every
 * call on one device shares that device's scratch: calls that overlap in time
 * on one device (for example on two concurrently running streams) race and
 * give undefined results; calls ordered on one stream, or on different
 * devices, are independent.  `stream` must belong to the current device
 * (GDN_ERR_INVALID_ARG otherwise).  Shapes whose partials exceed the scratch
 * return GDN_ERR_UNSUPPORTED (none among the supported d_v).  Results are
 * bit-identical to gdn_norm_gate_bwd's; other arguments as there. */
gdn_status gdn_norm_gate_bwd_noalloc(const gdn_shape* shape, const void* dy, const void* o, const void* z,
                                     const void* w_norm, float eps, void* d_o, void* dz, float* dw_norm,
                                     gdn_stream stream);

/* --------------------------------------------------------------------------
 * Token-by-token continuation (decode).  Page: "feat(models): dense Qwen3.5
 * custom attention", KL mismatch table (RL rollouts come from an inference
 * engine and are scored by the trainer, so the layer also runs one token at a
 * time) and review overview (the training path keeps no cache: a continuation
 * carries the recurrent state and the conv window instead).  Each call takes
 * ONE new token for each of N sequences: shape->total_tokens must equal
 * shape->n_seqs, and token n belongs to sequence n (no cu_seqlens).
 *
 * gdn_recurrent_step: the gated delta rule on that token,
 *   S' = e^{g} S (I - b k k^T) + b v k^T,  o = scale * S' q   (per v-head),
 *   q, k, v, g, beta laid out and strided as for gdn_chunk_fwd with T = N;
 *   state_in:  float32 [N][Hv][dk][dv] (H = S^T), or NULL for zero states;
 *   state_out: float32 [N][Hv][dk][dv], may equal state_in (updated in place)
 *              but must not overlap it otherwise;  o: [N][Hv][dv].
 * gdn_conv1d_step: conv1d + SiLU + L2 (as gdn_conv1d) of that token, with
 *   conv_window [N][width-1][Cch] (dtype) holding each sequence's previous
 *   width-1 inputs, oldest first; it is read and then advanced by one token
 *   in place.  x, y: [N][Cch]; y must not alias x or conv_window.  N <= 65535.
 * gdn_conv1d_window: the conv window after a prefill call: for sequence n,
 *   the last width-1 rows of [window_in[n] ; x rows of sequence n] (window_in
 *   NULL means zeros, i.e. a fresh sequence), into window_out (must not alias
 *   window_in).  x: [T][Cch] with cu_seqlens as in gdn_conv1d.  N <= 65535.
 * A prefill with gdn_conv1d / gdn_chunk_fwd (ht) and gdn_conv1d_window,
 * followed by these steps, continues every sequence exactly as one longer
 * prefill would.
 * -------------------------------------------------------------------------- */
gdn_status gdn_recurrent_step(const gdn_shape* shape, const void* q, const void* k, const void* v,
                              int64_t tok_stride_qk, int64_t tok_stride_v, const float* g, const float* beta,
                              const float* state_in, float* state_out, void* o, gdn_stream stream);
gdn_status gdn_conv1d_step(const gdn_shape* shape, const void* x, const void* w_conv, int32_t width,
                           float l2_eps, void* conv_window, void* y, gdn_stream stream);
gdn_status gdn_conv1d_window(const gdn_shape* shape, const void* x, int32_t width,
                             const int32_t* cu_seqlens, const void* window_in, void* window_out,
                             gdn_stream stream);

/* --------------------------------------------------------------------------
 * Diagnostics: per-kernel timing with HIP events.  For benchmarks and
 * profiling only (not part of the layer's computation).
 * gdn_profile_enable(1) clears earlier records and brackets every later kernel
 * launch of the library with hipEventRecord on its stream; (0) stops.
 * gdn_profile_report writes "kernel_name launches total_ms" lines into buf
 * (at most cap bytes including the terminating zero), waiting for the
 * recorded events, and returns the full length.  State-pass records carry the
 * variant that ran after a colon (wide128 / wide64: the whole or half state
 * per workgroup; tiled16 / tiled32: column tiles of that width).  The records
 * are guarded by a mutex, so launches from several host threads each time
 * their own kernel; the event objects are created once and reused.
 * -------------------------------------------------------------------------- */
void gdn_profile_enable(int on);
size_t gdn_profile_report(char* buf, size_t cap);

/* Diagnostics: achievable-peak probes (not part of the layer).
 * gdn_probe_copy: copies `bytes` (a multiple of 16; both pointers 16-byte
 *   aligned, not overlapping) from src to dst with 16-byte loads and stores:
 *   the HBM bandwidth a streaming kernel reaches.
 * gdn_probe_mfma: `blocks` workgroups of 4 waves, each wave running
 *   independent chains of `iters` bf16 matrix-core products: shape 0, 8
 *   chains of 16x16x32 (blocks * 4 * 8 * iters * 16384 flops); shape 1, 4
 *   chains of 32x32x16 (blocks * 4 * 4 * iters * 32768 flops); writes one
 *   float per thread to out [blocks * 256]: the matrix-core rate a kernel
 *   can reach with that instruction. */
gdn_status gdn_probe_copy(const void* src, void* dst, size_t bytes, gdn_stream stream);
gdn_status gdn_probe_mfma(float* out, int32_t blocks, int32_t iters, int32_t shape, gdn_stream stream);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H */
