// C ABI of the library: host-side argument checks, workspace sizing, and
// launches on the caller's stream.  Every check runs before anything is
// enqueued.
#include <hip/hip_runtime.h>

#include <cmath>

#include "gdn_internal.h"

using namespace gdn;

namespace {

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned4(const void* p) { return ((uintptr_t)p & 3u) == 0; }

bool dim_ok(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }

// shape checks shared by every entry point
gdn_status check_shape(const gdn_shape* s) {
  if (!s) return GDN_ERR_INVALID_ARG;
  if (s->n_seqs < 1 || s->total_tokens < 0 || s->h_qk < 1 || s->h_v < 1) return GDN_ERR_INVALID_ARG;
  if (s->h_v % s->h_qk != 0) return GDN_ERR_INVALID_ARG;
  if (s->dtype != GDN_F32 && s->dtype != GDN_BF16) return GDN_ERR_UNSUPPORTED;
  if (!dim_ok(s->d_k) || s->d_v != s->d_k) return GDN_ERR_UNSUPPORTED;
  if ((int64_t)s->total_tokens * (2 * s->h_qk * s->d_k + s->h_v * s->d_v) > ((int64_t)1 << 40))
    return GDN_ERR_INVALID_ARG;
  return GDN_OK;
}

gdn_status check_chunk(const gdn_shape* s) {
  if (s->chunk != 16 && s->chunk != 32 && s->chunk != 64) return GDN_ERR_UNSUPPORTED;
  if (!chunk_supported(s)) return GDN_ERR_UNSUPPORTED;
  if (max_chunks(s) > (int64_t)1 << 30) return GDN_ERR_INVALID_ARG;
  return GDN_OK;
}

size_t esize(const gdn_shape* s) { return s->dtype == GDN_BF16 ? 2 : 4; }

bool stride_ok(const gdn_shape* s, int64_t stride, int64_t min_elems) {
  return stride >= min_elems && (stride * (int64_t)esize(s)) % 16 == 0;
}

gdn_status launched() { return hipGetLastError() == hipSuccess ? GDN_OK : GDN_ERR_HIP; }

bool gates_ok(const gdn_gate_inputs* gi, bool any) {
  if (!gi || !gi->A_log || !gi->dt_bias || (any && (!gi->a || !gi->b))) return false;
  return aligned4(gi->a) && aligned4(gi->b) && aligned4(gi->A_log) && aligned4(gi->dt_bias);
}

bool gate_grads_ok(const gdn_gate_grads* gg, bool any) {
  if (!gg || !gg->dA_log || !gg->ddt_bias || (any && (!gg->da || !gg->db))) return false;
  return aligned4(gg->da) && aligned4(gg->db) && aligned4(gg->dA_log) && aligned4(gg->ddt_bias);
}

// forward; with save, the workspace (backward-sized) keeps what the backward reads;
// with gi, g and beta come from the raw gate inputs
gdn_status chunk_fwd_call(const gdn_shape* shape, const void* q, const void* k, const void* v, int64_t tok_stride_qk,
                          int64_t tok_stride_v, const float* g, const float* beta, const gdn_gate_inputs* gi,
                          bool gated, const int32_t* cu_seqlens, const float* h0, void* o, float* ht, void* ws,
                          size_t ws_bytes, bool save, gdn_stream stream) {
  gdn_status st = check_shape(shape);
  if (st != GDN_OK) return st;
  if ((st = check_chunk(shape)) != GDN_OK) return st;
  const bool any = shape->total_tokens > 0;
  if (gated ? !gates_ok(gi, any) : (any && (!g || !beta))) return GDN_ERR_INVALID_ARG;
  if (!cu_seqlens || (any && (!q || !k || !v || !o))) return GDN_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return GDN_ERR_INVALID_ARG;
  if (!stride_ok(shape, tok_stride_qk, (int64_t)shape->h_qk * shape->d_k) ||
      !stride_ok(shape, tok_stride_v, (int64_t)shape->h_v * shape->d_v))
    return GDN_ERR_INVALID_ARG;
  const size_t need = save ? chunk_bwd_ws_bytes(shape) : chunk_fwd_ws_bytes(shape);
  if (!ws || !aligned16(ws) || ws_bytes < need) return GDN_ERR_WORKSPACE;
  if (!run_chunk_fwd(shape, q, k, v, tok_stride_qk, tok_stride_v, g, beta, gated ? gi : nullptr, cu_seqlens, h0,
                     o, ht, ws, save, (hipStream_t)stream))
    return GDN_ERR_UNSUPPORTED;
  return launched();
}

// backward; with saved, the workspace holds what gdn_chunk_fwd_save left there
gdn_status chunk_bwd_call(const gdn_shape* shape, const void* q, const void* k, const void* v, int64_t tok_stride_qk,
                          int64_t tok_stride_v, const float* g, const float* beta, const gdn_gate_inputs* gi,
                          bool gated, const int32_t* cu_seqlens, const float* h0, const void* d_o, const float* dht,
                          void* dq, void* dk, void* dv, float* dg, float* dbeta, const gdn_gate_grads* gg,
                          float* dh0, void* ws, size_t ws_bytes, bool saved, gdn_stream stream) {
  gdn_status st = check_shape(shape);
  if (st != GDN_OK) return st;
  if ((st = check_chunk(shape)) != GDN_OK) return st;
  const bool any = shape->total_tokens > 0;
  if (gated ? (!gates_ok(gi, any) || !gate_grads_ok(gg, any)) : (any && (!g || !beta || !dg || !dbeta)))
    return GDN_ERR_INVALID_ARG;
  if (!cu_seqlens || (any && (!q || !k || !v || !d_o || !dq || !dk || !dv))) return GDN_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(d_o) || !aligned16(dq) || !aligned16(dk) ||
      !aligned16(dv))
    return GDN_ERR_INVALID_ARG;
  if (!stride_ok(shape, tok_stride_qk, (int64_t)shape->h_qk * shape->d_k) ||
      !stride_ok(shape, tok_stride_v, (int64_t)shape->h_v * shape->d_v))
    return GDN_ERR_INVALID_ARG;
  if (!ws || !aligned16(ws) || ws_bytes < chunk_bwd_ws_bytes(shape)) return GDN_ERR_WORKSPACE;
  if (!run_chunk_bwd(shape, q, k, v, tok_stride_qk, tok_stride_v, g, beta, gated ? gi : nullptr, cu_seqlens, h0,
                     d_o, dht, dq, dk, dv, dg, dbeta, gated ? gg : nullptr, dh0, ws, saved, (hipStream_t)stream))
    return GDN_ERR_UNSUPPORTED;
  return launched();
}

}  // namespace

extern "C" {

const char* gdn_status_string(gdn_status status) {
  switch (status) {
    case GDN_OK: return "GDN_OK";
    case GDN_ERR_INVALID_ARG: return "GDN_ERR_INVALID_ARG: invalid argument";
    case GDN_ERR_UNSUPPORTED: return "GDN_ERR_UNSUPPORTED: unsupported shape or dtype";
    case GDN_ERR_WORKSPACE: return "GDN_ERR_WORKSPACE: workspace missing or too small";
    case GDN_ERR_HIP: return "GDN_ERR_HIP: kernel launch failed";
  }
  return "unknown gdn_status";
}

int64_t gdn_max_chunks(const gdn_shape* shape) {
  if (check_shape(shape) != GDN_OK || shape->chunk < 1) return -1;
  return max_chunks(shape);
}

gdn_status gdn_chunk_index(const gdn_shape* shape, const int32_t* cu_seqlens, int32_t* table, int32_t* seq_chunk0,
                           gdn_stream stream) {
  gdn_status st = check_shape(shape);
  if (st != GDN_OK) return st;
  if (shape->chunk != 16 && shape->chunk != 32 && shape->chunk != 64) return GDN_ERR_UNSUPPORTED;
  if (!cu_seqlens || !table || !seq_chunk0 || !aligned16(table)) return GDN_ERR_INVALID_ARG;
  run_chunk_index(shape, cu_seqlens, table, seq_chunk0, (hipStream_t)stream);
  return launched();
}

gdn_status gdn_conv1d(const gdn_shape* shape, const void* x, const void* w_conv, int32_t width, float l2_eps,
                      const int32_t* cu_seqlens, void* y, gdn_stream stream) {
  gdn_status st = check_shape(shape);
  if (st != GDN_OK) return st;
  if (width < 2 || width > 4) return GDN_ERR_UNSUPPORTED;
  const bool any = shape->total_tokens > 0;  // token-indexed pointers may be null for an empty row
  if (!w_conv || !cu_seqlens || (any && (!x || !y || x == y))) return GDN_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(y)) return GDN_ERR_INVALID_ARG;
  if (!(l2_eps >= 0.f)) return GDN_ERR_INVALID_ARG;
  if (!run_conv_fwd(shape, x, w_conv, width, cu_seqlens, nullptr, l2_eps, y, (hipStream_t)stream))
    return GDN_ERR_UNSUPPORTED;
  return launched();
}

gdn_status gdn_conv1d_prefill(const gdn_shape* shape, const void* x, const void* w_conv, int32_t width, float l2_eps,
                              const int32_t* cu_seqlens, const void* window_in, void* y, void* window_out,
                              gdn_stream stream) {
  gdn_status st = check_shape(shape);
  if (st != GDN_OK) return st;
  if (width < 2 || width > 4) return GDN_ERR_UNSUPPORTED;
  if (window_out && shape->n_seqs > 65535) return GDN_ERR_UNSUPPORTED;
  const bool any = shape->total_tokens > 0;
  if (!w_conv || !cu_seqlens || (any && (!x || !y || x == y))) return GDN_ERR_INVALID_ARG;
  if (window_in && (window_in == window_out || window_in == y)) return GDN_ERR_INVALID_ARG;
  if (window_out && (window_out == x || window_out == y)) return GDN_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(y) || !aligned16(window_in) || !aligned16(window_out)) return GDN_ERR_INVALID_ARG;
  if (!(l2_eps >= 0.f)) return GDN_ERR_INVALID_ARG;
  if (!run_conv_fwd(shape, x, w_conv, width, cu_seqlens, window_in, l2_eps, y, (hipStream_t)stream))
    return GDN_ERR_UNSUPPORTED;
  if (window_out && !run_conv_window(shape, x, width, cu_seqlens, window_in, window_out, (hipStream_t)stream))
    return GDN_ERR_UNSUPPORTED;
  return launched();
}

size_t gdn_conv1d_bwd_workspace(const gdn_shape* shape, int32_t width) {
  if (check_shape(shape) != GDN_OK || width < 2 || width > 4) return 0;
  return conv_bwd_ws_bytes(shape, width);
}

gdn_status gdn_conv1d_bwd(const gdn_shape* shape, const void* dy, const void* x, const void* w_conv, int32_t width,
                          float l2_eps, const int32_t* cu_seqlens, void* dx, float* dw_conv, void* ws,
                          size_t ws_bytes, gdn_stream stream) {
  gdn_status st = check_shape(shape);
  if (st != GDN_OK) return st;
  if (width < 2 || width > 4) return GDN_ERR_UNSUPPORTED;
  const bool any = shape->total_tokens > 0;
  if (!w_conv || !cu_seqlens || !dw_conv || (any && (!dy || !x || !dx))) return GDN_ERR_INVALID_ARG;
  if (!aligned16(dy) || !aligned16(x) || !aligned16(dx) || (any && (dx == x || dx == dy))) return GDN_ERR_INVALID_ARG;
  if (!(l2_eps >= 0.f)) return GDN_ERR_INVALID_ARG;
  if (!ws || !aligned16(ws) || ws_bytes < conv_bwd_ws_bytes(shape, width)) return GDN_ERR_WORKSPACE;
  if (!run_conv_bwd(shape, dy, x, w_conv, width, cu_seqlens, l2_eps, dx, dw_conv, ws, (hipStream_t)stream))
    return GDN_ERR_UNSUPPORTED;
  return launched();
}

size_t gdn_chunk_fwd_workspace(const gdn_shape* shape) {
  if (check_shape(shape) != GDN_OK || check_chunk(shape) != GDN_OK) return 0;
  return chunk_fwd_ws_bytes(shape);
}

gdn_status gdn_chunk_fwd(const gdn_shape* shape, const void* q, const void* k, const void* v, int64_t tok_stride_qk,
                         int64_t tok_stride_v, const float* g, const float* beta, const int32_t* cu_seqlens,
                         const float* h0, void* o, float* ht, void* ws, size_t ws_bytes, gdn_stream stream) {
  return chunk_fwd_call(shape, q, k, v, tok_stride_qk, tok_stride_v, g, beta, nullptr, false, cu_seqlens, h0, o, ht,
                        ws, ws_bytes, false, stream);
}

gdn_status gdn_chunk_fwd_save(const gdn_shape* shape, const void* q, const void* k, const void* v,
                              int64_t tok_stride_qk, int64_t tok_stride_v, const float* g, const float* beta,
                              const int32_t* cu_seqlens, const float* h0, void* o, float* ht, void* ws,
                              size_t ws_bytes, gdn_stream stream) {
  return chunk_fwd_call(shape, q, k, v, tok_stride_qk, tok_stride_v, g, beta, nullptr, false, cu_seqlens, h0, o, ht,
                        ws, ws_bytes, true, stream);
}

size_t gdn_chunk_bwd_workspace(const gdn_shape* shape) {
  if (check_shape(shape) != GDN_OK || check_chunk(shape) != GDN_OK) return 0;
  return chunk_bwd_ws_bytes(shape);
}

gdn_status gdn_chunk_bwd(const gdn_shape* shape, const void* q, const void* k, const void* v, int64_t tok_stride_qk,
                         int64_t tok_stride_v, const float* g, const float* beta, const int32_t* cu_seqlens,
                         const float* h0, const void* d_o, const float* dht, void* dq, void* dk, void* dv, float* dg,
                         float* dbeta, float* dh0, void* ws, size_t ws_bytes, gdn_stream stream) {
  return chunk_bwd_call(shape, q, k, v, tok_stride_qk, tok_stride_v, g, beta, nullptr, false, cu_seqlens, h0, d_o,
                        dht, dq, dk, dv, dg, dbeta, nullptr, dh0, ws, ws_bytes, false, stream);
}

gdn_status gdn_chunk_bwd_saved(const gdn_shape* shape, const void* q, const void* k, const void* v,
                               int64_t tok_stride_qk, int64_t tok_stride_v, const float* g, const float* beta,
                               const int32_t* cu_seqlens, const float* h0, const void* d_o, const float* dht,
                               void* dq, void* dk, void* dv, float* dg, float* dbeta, float* dh0, void* ws,
                               size_t ws_bytes, gdn_stream stream) {
  return chunk_bwd_call(shape, q, k, v, tok_stride_qk, tok_stride_v, g, beta, nullptr, false, cu_seqlens, h0, d_o,
                        dht, dq, dk, dv, dg, dbeta, nullptr, dh0, ws, ws_bytes, true, stream);
}

gdn_status gdn_chunk_fwd_fp8(const gdn_shape* shape, const void* q, const void* k, const void* v,
                             int64_t tok_stride_qk, int64_t tok_stride_v, float scale_q, float scale_k, float scale_v,
                             const float* g, const float* beta, const int32_t* cu_seqlens, const float* h0, void* o,
                             float* ht, void* ws, size_t ws_bytes, gdn_stream stream) {
  gdn_status st = check_shape(shape);
  if (st != GDN_OK) return st;
  if ((st = check_chunk(shape)) != GDN_OK) return st;
  if (shape->dtype != GDN_BF16 || shape->d_k != 128 || shape->chunk != 64) return GDN_ERR_UNSUPPORTED;
  const float scales[3] = {scale_q, scale_k, scale_v};
  for (float x : scales) {  // powers of two: the decoded inputs are then exact bf16 values
    int e = 0;
    if (!(x > 0.f) || !std::isfinite(x) || std::frexp(x, &e) != 0.5f || e < -100 || e > 100)
      return GDN_ERR_INVALID_ARG;
  }
  const bool any = shape->total_tokens > 0;
  if (!cu_seqlens || (any && (!q || !k || !v || !g || !beta || !o))) return GDN_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return GDN_ERR_INVALID_ARG;
  const int64_t nqk = (int64_t)shape->h_qk * shape->d_k, nv = (int64_t)shape->h_v * shape->d_v;
  if (tok_stride_qk < nqk || tok_stride_qk % 16 || tok_stride_v < nv || tok_stride_v % 16) return GDN_ERR_INVALID_ARG;
  if (!ws || !aligned16(ws) || ws_bytes < chunk_fwd_ws_bytes(shape)) return GDN_ERR_WORKSPACE;
  if (!run_chunk_fwd_f8(shape, q, k, v, tok_stride_qk, tok_stride_v, scales, g, beta, cu_seqlens, h0, o, ht, ws,
                        (hipStream_t)stream))
    return GDN_ERR_UNSUPPORTED;
  return launched();
}

gdn_status gdn_chunk_fwd_gated(const gdn_shape* shape, const void* q, const void* k, const void* v,
                               int64_t tok_stride_qk, int64_t tok_stride_v, const gdn_gate_inputs* gates,
                               const int32_t* cu_seqlens, const float* h0, void* o, float* ht, void* ws,
                               size_t ws_bytes, gdn_stream stream) {
  return chunk_fwd_call(shape, q, k, v, tok_stride_qk, tok_stride_v, nullptr, nullptr, gates, true, cu_seqlens, h0, o,
                        ht, ws, ws_bytes, false, stream);
}

gdn_status gdn_chunk_fwd_save_gated(const gdn_shape* shape, const void* q, const void* k, const void* v,
                                    int64_t tok_stride_qk, int64_t tok_stride_v, const gdn_gate_inputs* gates,
                                    const int32_t* cu_seqlens, const float* h0, void* o, float* ht, void* ws,
                                    size_t ws_bytes, gdn_stream stream) {
  return chunk_fwd_call(shape, q, k, v, tok_stride_qk, tok_stride_v, nullptr, nullptr, gates, true, cu_seqlens, h0, o,
                        ht, ws, ws_bytes, true, stream);
}

gdn_status gdn_chunk_bwd_gated(const gdn_shape* shape, const void* q, const void* k, const void* v,
                               int64_t tok_stride_qk, int64_t tok_stride_v, const gdn_gate_inputs* gates,
                               const int32_t* cu_seqlens, const float* h0, const void* d_o, const float* dht,
                               void* dq, void* dk, void* dv, const gdn_gate_grads* dgates, float* dh0, void* ws,
                               size_t ws_bytes, gdn_stream stream) {
  return chunk_bwd_call(shape, q, k, v, tok_stride_qk, tok_stride_v, nullptr, nullptr, gates, true, cu_seqlens, h0,
                        d_o, dht, dq, dk, dv, nullptr, nullptr, dgates, dh0, ws, ws_bytes, false, stream);
}

gdn_status gdn_chunk_bwd_saved_gated(const gdn_shape* shape, const void* q, const void* k, const void* v,
                                     int64_t tok_stride_qk, int64_t tok_stride_v, const gdn_gate_inputs* gates,
                                     const int32_t* cu_seqlens, const float* h0, const void* d_o,
                                     const float* dht, void* dq, void* dk, void* dv, const gdn_gate_grads* dgates,
                                     float* dh0, void* ws, size_t ws_bytes, gdn_stream stream) {
  return chunk_bwd_call(shape, q, k, v, tok_stride_qk, tok_stride_v, nullptr, nullptr, gates, true, cu_seqlens, h0,
                        d_o, dht, dq, dk, dv, nullptr, nullptr, dgates, dh0, ws, ws_bytes, true, stream);
}

gdn_status gdn_norm_gate(const gdn_shape* shape, const void* o, const void* z, const void* w_norm, float eps, void* y,
                         gdn_stream stream) {
  gdn_status st = check_shape(shape);
  if (st != GDN_OK) return st;
  const bool any = shape->total_tokens > 0;
  if (!w_norm || (any && (!o || !z || !y))) return GDN_ERR_INVALID_ARG;
  if (!aligned16(o) || !aligned16(z) || !aligned16(w_norm) || !aligned16(y)) return GDN_ERR_INVALID_ARG;
  if (!(eps >= 0.f)) return GDN_ERR_INVALID_ARG;
  if (!run_norm_fwd(shape, o, z, w_norm, eps, y, (hipStream_t)stream)) return GDN_ERR_UNSUPPORTED;
  return launched();
}

gdn_status gdn_gates(const gdn_shape* shape, const float* a, const float* b, const float* A_log, const float* dt_bias,
                     float* g, float* beta, gdn_stream stream) {
  gdn_status st = check_shape(shape);
  if (st != GDN_OK) return st;
  const bool any = shape->total_tokens > 0;
  if (!A_log || !dt_bias || (any && (!a || !b || !g || !beta))) return GDN_ERR_INVALID_ARG;
  if (!aligned4(a) || !aligned4(b) || !aligned4(A_log) || !aligned4(dt_bias) || !aligned4(g) || !aligned4(beta))
    return GDN_ERR_INVALID_ARG;
  if (any && (g == a || g == b || beta == a || beta == b || g == beta)) return GDN_ERR_INVALID_ARG;
  run_gates_fwd(shape, a, b, A_log, dt_bias, g, beta, (hipStream_t)stream);
  return launched();
}

size_t gdn_gates_bwd_workspace(const gdn_shape* shape) {
  if (check_shape(shape) != GDN_OK) return 0;
  return gates_bwd_ws_bytes(shape);
}

gdn_status gdn_gates_bwd(const gdn_shape* shape, const float* a, const float* b, const float* A_log,
                         const float* dt_bias, const float* dg, const float* dbeta, float* da, float* db,
                         float* dA_log, float* ddt_bias, void* ws, size_t ws_bytes, gdn_stream stream) {
  gdn_status st = check_shape(shape);
  if (st != GDN_OK) return st;
  const bool any = shape->total_tokens > 0;
  if (!A_log || !dt_bias || !dA_log || !ddt_bias || (any && (!a || !b || !dg || !dbeta || !da || !db)))
    return GDN_ERR_INVALID_ARG;
  if (!aligned4(a) || !aligned4(b) || !aligned4(A_log) || !aligned4(dt_bias) || !aligned4(dg) || !aligned4(dbeta) ||
      !aligned4(da) || !aligned4(db) || !aligned4(dA_log) || !aligned4(ddt_bias))
    return GDN_ERR_INVALID_ARG;
  if (!ws || !aligned16(ws) || ws_bytes < gates_bwd_ws_bytes(shape)) return GDN_ERR_WORKSPACE;
  run_gates_bwd(shape, a, b, A_log, dt_bias, dg, dbeta, da, db, dA_log, ddt_bias, ws, (hipStream_t)stream);
  return launched();
}

gdn_status gdn_recurrent_step(const gdn_shape* shape, const void* q, const void* k, const void* v,
                              int64_t tok_stride_qk, int64_t tok_stride_v, const float* g, const float* beta,
                              const float* state_in, float* state_out, void* o, gdn_stream stream) {
  gdn_status st = check_shape(shape);
  if (st != GDN_OK) return st;
  if (shape->total_tokens != shape->n_seqs) return GDN_ERR_INVALID_ARG;  // one token per sequence
  if (!q || !k || !v || !g || !beta || !state_out || !o) return GDN_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(state_in) ||
      !aligned16(state_out) || !aligned4(g) || !aligned4(beta))
    return GDN_ERR_INVALID_ARG;
  if (!stride_ok(shape, tok_stride_qk, (int64_t)shape->h_qk * shape->d_k) ||
      !stride_ok(shape, tok_stride_v, (int64_t)shape->h_v * shape->d_v))
    return GDN_ERR_INVALID_ARG;
  if (!run_recurrent_step(shape, q, k, v, tok_stride_qk, tok_stride_v, g, beta, state_in, state_out, o,
                          (hipStream_t)stream))
    return GDN_ERR_UNSUPPORTED;
  return launched();
}

gdn_status gdn_conv1d_step(const gdn_shape* shape, const void* x, const void* w_conv, int32_t width, float l2_eps,
                           void* conv_window, void* y, gdn_stream stream) {
  gdn_status st = check_shape(shape);
  if (st != GDN_OK) return st;
  if (width < 2 || width > 4) return GDN_ERR_UNSUPPORTED;
  if (shape->total_tokens != shape->n_seqs) return GDN_ERR_INVALID_ARG;
  if (shape->n_seqs > 65535) return GDN_ERR_UNSUPPORTED;  // one grid row per sequence
  if (!x || !w_conv || !conv_window || !y || y == x || y == conv_window || x == conv_window)
    return GDN_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(y) || !aligned16(conv_window)) return GDN_ERR_INVALID_ARG;
  if (!(l2_eps >= 0.f)) return GDN_ERR_INVALID_ARG;
  if (!run_conv_step(shape, x, w_conv, width, l2_eps, conv_window, y, (hipStream_t)stream))
    return GDN_ERR_UNSUPPORTED;
  return launched();
}

gdn_status gdn_conv1d_window(const gdn_shape* shape, const void* x, int32_t width, const int32_t* cu_seqlens,
                             const void* window_in, void* window_out, gdn_stream stream) {
  gdn_status st = check_shape(shape);
  if (st != GDN_OK) return st;
  if (width < 2 || width > 4) return GDN_ERR_UNSUPPORTED;
  if (shape->n_seqs > 65535) return GDN_ERR_UNSUPPORTED;
  const bool any = shape->total_tokens > 0;
  if (!cu_seqlens || !window_out || (any && !x) || window_in == window_out) return GDN_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(window_in) || !aligned16(window_out)) return GDN_ERR_INVALID_ARG;
  if (!run_conv_window(shape, x, width, cu_seqlens, window_in, window_out, (hipStream_t)stream))
    return GDN_ERR_UNSUPPORTED;
  return launched();
}

size_t gdn_norm_gate_bwd_workspace(const gdn_shape* shape) {
  if (check_shape(shape) != GDN_OK) return 0;
  return norm_bwd_ws_bytes(shape);
}

gdn_status gdn_norm_gate_bwd(const gdn_shape* shape, const void* dy, const void* o, const void* z, const void* w_norm,
                             float eps, void* d_o, void* dz, float* dw_norm, void* ws, size_t ws_bytes,
                             gdn_stream stream) {
  gdn_status st = check_shape(shape);
  if (st != GDN_OK) return st;
  const bool any = shape->total_tokens > 0;
  if (!w_norm || !dw_norm || (any && (!dy || !o || !z || !d_o || !dz))) return GDN_ERR_INVALID_ARG;
  if (!aligned16(dy) || !aligned16(o) || !aligned16(z) || !aligned16(w_norm) || !aligned16(d_o) || !aligned16(dz))
    return GDN_ERR_INVALID_ARG;
  if (!(eps >= 0.f)) return GDN_ERR_INVALID_ARG;
  if (!ws || !aligned16(ws) || ws_bytes < norm_bwd_ws_bytes(shape)) return GDN_ERR_WORKSPACE;
  if (!run_norm_bwd(shape, dy, o, z, w_norm, eps, d_o, dz, dw_norm, ws, (hipStream_t)stream))
    return GDN_ERR_UNSUPPORTED;
  return launched();
}

gdn_status gdn_norm_gate_bwd_noalloc(const gdn_shape* shape, const void* dy, const void* o, const void* z,
                                     const void* w_norm, float eps, void* d_o, void* dz, float* dw_norm,
                                     gdn_stream stream) {
  gdn_status st = check_shape(shape);
  if (st != GDN_OK) return st;
  const bool any = shape->total_tokens > 0;
  if (!w_norm || !dw_norm || (any && (!dy || !o || !z || !d_o || !dz))) return GDN_ERR_INVALID_ARG;
  if (!aligned16(dy) || !aligned16(o) || !aligned16(z) || !aligned16(w_norm) || !aligned16(d_o) || !aligned16(dz))
    return GDN_ERR_INVALID_ARG;
  if (!(eps >= 0.f)) return GDN_ERR_INVALID_ARG;
  if (norm_bwd_ws_bytes(shape) > norm_scratch_bytes()) return GDN_ERR_UNSUPPORTED;
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess) return GDN_ERR_HIP;
  if (stream) {  // the scratch used is the current device's: the stream must belong to it
    hipDevice_t sdev = -1;
    if (hipStreamGetDevice((hipStream_t)stream, &sdev) != hipSuccess) return GDN_ERR_HIP;
    if ((int)sdev != cur) return GDN_ERR_INVALID_ARG;
  }
  void* ws = norm_scratch_ptr();
  if (!ws) return GDN_ERR_HIP;
  if (!run_norm_bwd(shape, dy, o, z, w_norm, eps, d_o, dz, dw_norm, ws, (hipStream_t)stream))
    return GDN_ERR_UNSUPPORTED;
  return launched();
}

}  // extern "C"
