// Host-side declarations shared by the kernel translation units and the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/gdn.h"

namespace gdn {

// conv1d.hip
size_t conv_bwd_ws_bytes(const gdn_shape* s, int width);
// win: NULL, or the carried window [N][width-1][Cch] of each sequence's previous inputs
bool run_conv_fwd(const gdn_shape* s, const void* x, const void* w, int width, const int32_t* cu, const void* win,
                  float eps, void* y, hipStream_t st);
bool run_conv_bwd(const gdn_shape* s, const void* dy, const void* x, const void* w, int width, const int32_t* cu,
                  float eps, void* dx, float* dw, void* ws, hipStream_t st);

// norm_gate.hip
size_t norm_bwd_ws_bytes(const gdn_shape* s);
size_t norm_scratch_bytes();  // capacity of the allocation-free backward's device scratch
void* norm_scratch_ptr();     // its device address on the current device, or NULL on a HIP error
bool run_norm_fwd(const gdn_shape* s, const void* o, const void* z, const void* w, float eps, void* y,
                  hipStream_t st);
bool run_norm_bwd(const gdn_shape* s, const void* dy, const void* o, const void* z, const void* w, float eps,
                  void* d_o, void* dz, float* dw, void* ws, hipStream_t st);

// gates.hip
size_t gates_bwd_ws_bytes(const gdn_shape* s);
void run_gates_fwd(const gdn_shape* s, const float* a, const float* b, const float* A_log, const float* dt_bias,
                   float* g, float* beta, hipStream_t st);
void run_gates_bwd(const gdn_shape* s, const float* a, const float* b, const float* A_log, const float* dt_bias,
                   const float* dg, const float* dbeta, float* da, float* db, float* dA_log, float* ddt_bias,
                   void* ws, hipStream_t st);

// recurrent.hip
bool run_recurrent_step(const gdn_shape* s, const void* q, const void* k, const void* v, int64_t sqk, int64_t sv,
                        const float* g, const float* beta, const float* state_in, float* state_out, void* o,
                        hipStream_t st);
bool run_conv_step(const gdn_shape* s, const void* x, const void* w, int width, float eps, void* window, void* y,
                   hipStream_t st);
bool run_conv_window(const gdn_shape* s, const void* x, int width, const int32_t* cu, const void* win_in,
                     void* win_out, hipStream_t st);

// chunk_fwd.hip / chunk_bwd.hip
int64_t max_chunks(const gdn_shape* s);
bool chunk_supported(const gdn_shape* s);
void run_chunk_index(const gdn_shape* s, const int32_t* cu, int32_t* table, int32_t* seq_chunk0, hipStream_t st);
size_t chunk_fwd_ws_bytes(const gdn_shape* s);
size_t chunk_bwd_ws_bytes(const gdn_shape* s);
// fp8 (e4m3) q, k, v with power-of-two scales (q, k, v scale): bf16, d = 128, chunk 64 only
bool run_chunk_fwd_f8(const gdn_shape* s, const void* q, const void* k, const void* v, int64_t sqk, int64_t sv,
                      const float scales[3], const float* g, const float* beta, const int32_t* cu, const float* h0,
                      void* o, float* ht, void* ws, hipStream_t st);
// gi / gg non-NULL: the fused-gate forms (g, beta and dg, dbeta unused)
bool run_chunk_fwd(const gdn_shape* s, const void* q, const void* k, const void* v, int64_t sqk, int64_t sv,
                   const float* g, const float* beta, const gdn_gate_inputs* gi, const int32_t* cu,
                   const float* h0, void* o, float* ht, void* ws, bool save, hipStream_t st);
bool run_chunk_bwd(const gdn_shape* s, const void* q, const void* k, const void* v, int64_t sqk, int64_t sv,
                   const float* g, const float* beta, const gdn_gate_inputs* gi, const int32_t* cu,
                   const float* h0, const void* d_o, const float* dht, void* dq, void* dk, void* dv, float* dg,
                   float* dbeta, const gdn_gate_grads* gg, float* dh0, void* ws, bool saved, hipStream_t st);

}  // namespace gdn
