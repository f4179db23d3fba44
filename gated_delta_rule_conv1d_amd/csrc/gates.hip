// Gates of the recurrence and their reverse mode.
//
// Page: "[Qwen3.5 MoE] Add hybrid decoder model", Summary (softplus registered
// as a pointwise op for the GatedDeltaNet gate).  Per token t and v-head h:
//   g    = -exp(A_log[h]) * softplus(a[t,h] + dt_bias[h])     (log-decay, < 0)
//   beta = sigmoid(b[t,h])                                   (write strength)
// softplus(x) = max(x, 0) + log1p(exp(-|x|)): no overflow for large x, no loss
// of the small values for very negative x.  Reverse mode:
//   da = -exp(A_log) sigmoid(a + dt_bias) dg,   db = beta (1 - beta) dbeta,
//   dA_log[h] = sum_t dg g,   ddt_bias[h] = sum_t da   (per-block partials
//   summed in a fixed order: deterministic).
// Elementwise over [T][Hv] float32: HBM streaming, no LDS staging needed.
#include "gdn_common.cuh"
#include "gdn_internal.h"
#include "profile.h"

namespace gdn {

constexpr int kGateThreads = 256;
constexpr int kGateBwdTokens = 256;  // tokens per backward block (one partial row each)

__device__ __forceinline__ float softplus_f(float x) { return gate_softplus(x); }
__device__ __forceinline__ float sigmoid_f(float x) { return gate_sigmoid(x); }

__global__ __launch_bounds__(kGateThreads) void gates_fwd_kernel(const float* __restrict__ a,
                                                                 const float* __restrict__ b,
                                                                 const float* __restrict__ A_log,
                                                                 const float* __restrict__ dt_bias, long n, int Hv,
                                                                 float* __restrict__ g, float* __restrict__ beta) {
  const long e = (long)blockIdx.x * kGateThreads + threadIdx.x;
  if (e >= n) return;
  const int h = (int)(e % Hv);
  g[e] = -__expf(A_log[h]) * softplus_f(a[e] + dt_bias[h]);
  beta[e] = sigmoid_f(b[e]);
}

// Block (bx, by) covers tokens [bx*256, bx*256 + 256) and heads
// [by*HB, by*HB + HB); thread (tl, hl) = (tid / HB, tid % HB) walks the block's
// tokens tl, tl + TL, ...  so a row of HB threads reads HB consecutive floats.
// The per-head sums over the block's tokens go to part[bx][h] (dA_log) and
// part[nbx + bx][h] (ddt_bias), added in token order per thread, then over tl.
__global__ __launch_bounds__(kGateThreads) void gates_bwd_kernel(
    const float* __restrict__ a, const float* __restrict__ b, const float* __restrict__ A_log,
    const float* __restrict__ dt_bias, const float* __restrict__ dg, const float* __restrict__ dbeta, int T, int Hv,
    int HB, float* __restrict__ da, float* __restrict__ db, float* __restrict__ part) {
  __shared__ float red[2][kGateThreads];
  const int tid = threadIdx.x;
  const int hl = tid % HB, tl = tid / HB, TL = kGateThreads / HB;
  const int h = blockIdx.y * HB + hl;
  const int t0 = blockIdx.x * kGateBwdTokens, t1 = min(t0 + kGateBwdTokens, T);
  float sA = 0.f, sdt = 0.f;
  if (h < Hv) {
    const float ea = __expf(A_log[h]), bias = dt_bias[h];
    for (int t = t0 + tl; t < t1; t += TL) {
      const long e = (long)t * Hv + h;
      const float x = a[e] + bias;
      const float gv = -ea * softplus_f(x);
      const float dgv = dg[e];
      const float dav = -ea * sigmoid_f(x) * dgv;
      const float bb = b[e];
      da[e] = dav;
      // beta (1 - beta) as sigmoid(b) sigmoid(-b): no cancellation in 1 - beta
      db[e] = sigmoid_f(bb) * sigmoid_f(-bb) * dbeta[e];
      sA += dgv * gv;
      sdt += dav;
    }
  }
  red[0][tid] = sA;
  red[1][tid] = sdt;
  __syncthreads();
  if (tl == 0 && h < Hv) {
    float s0 = 0.f, s1 = 0.f;
    for (int i = 0; i < TL; ++i) {
      s0 += red[0][i * HB + hl];
      s1 += red[1][i * HB + hl];
    }
    part[(size_t)blockIdx.x * Hv + h] = s0;
    part[((size_t)gridDim.x + blockIdx.x) * Hv + h] = s1;
  }
}

static int gate_bwd_blocks(int T) { return (T + kGateBwdTokens - 1) / kGateBwdTokens; }

size_t gates_bwd_ws_bytes(const gdn_shape* s) {
  const int nb = gate_bwd_blocks(s->total_tokens);
  return (size_t)2 * (nb > 0 ? nb : 1) * s->h_v * sizeof(float);
}

void run_gates_fwd(const gdn_shape* s, const float* a, const float* b, const float* A_log, const float* dt_bias,
                   float* g, float* beta, hipStream_t st) {
  const long n = (long)s->total_tokens * s->h_v;
  if (n == 0) return;
  GDN_PROF("gates_fwd", st);
  gates_fwd_kernel<<<(unsigned)((n + kGateThreads - 1) / kGateThreads), kGateThreads, 0, st>>>(
      a, b, A_log, dt_bias, n, s->h_v, g, beta);
}

void run_gates_bwd(const gdn_shape* s, const float* a, const float* b, const float* A_log, const float* dt_bias,
                   const float* dg, const float* dbeta, float* da, float* db, float* dA_log, float* ddt_bias,
                   void* ws, hipStream_t st) {
  const int T = s->total_tokens, Hv = s->h_v;
  const int nb = gate_bwd_blocks(T);
  float* part = (float*)ws;
  if (nb > 0) {
    int HB = 1;
    while (HB < Hv && HB < 64) HB <<= 1;
    GDN_PROF("gates_bwd", st);
    gates_bwd_kernel<<<dim3(nb, (Hv + HB - 1) / HB), kGateThreads, 0, st>>>(a, b, A_log, dt_bias, dg, dbeta, T, Hv,
                                                                          HB, da, db, part);
  }
  GDN_PROF("gates_dw_sum", st);
  launch_colsum(part, nb, Hv, dA_log, st);
  launch_colsum(part + (size_t)nb * Hv, nb, Hv, ddt_bias, st);
}

}  // namespace gdn
