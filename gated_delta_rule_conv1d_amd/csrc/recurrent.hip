// One-token continuation (decode) of the layer: the gated delta rule applied to
// one new token of each of N sequences, and the causal conv1d + SiLU + L2 step
// with its rolling window of the last width-1 inputs.
//
// Pages: "feat(models): dense Qwen3.5 custom attention", KL mismatch table (RL
// rollouts come from an inference engine and are scored by the trainer: the
// same layer also runs token by token) and the review overview (the training
// path itself carries no cache; a continuation carries the recurrent state and
// the conv window instead).
//
// Recurrent step, per sequence n and v-head h (H = S^T, [dk][dv] fp32):
//   H' = e^g H + k u^T,   u = beta (v - e^g H^T k)
//   o  = scale H'^T q = scale (e^g H^T q + (k . q) u)
// so one read of H gives both column sums H^T k and H^T q, and one write
// stores H'.  A workgroup owns one (sequence, v-head): thread (rg, cq) holds
// columns 4cq..4cq+3 of rows rg, rg + RG, ... (each load instruction covers RG
// whole rows: coalesced), sums its rows, and the RG partial sums of every
// column are added in a fixed order through LDS.  Pure HBM streaming of the
// state (2 * dk * dv * 4 bytes per sequence and v-head).
#include "gdn_common.cuh"
#include "gdn_internal.h"
#include "profile.h"

namespace gdn {

template <int D>
constexpr int rec_threads() { return D * D / 4 < 256 ? D * D / 4 : 256; }

template <typename E, int D>
__global__ __launch_bounds__(rec_threads<D>()) void recurrent_step_kernel(
    const E* __restrict__ q, const E* __restrict__ k, const E* __restrict__ v, int64_t sqk, int64_t sv,
    const float* __restrict__ g, const float* __restrict__ beta, const float* state_in, float* state_out,
    E* __restrict__ o, int Hv, int G, float scale) {
  constexpr int NTH = rec_threads<D>();
  constexpr int CQ = D / 4;     // column quads
  constexpr int RG = NTH / CQ;  // row groups
  constexpr int R = D / RG;     // rows per thread
  __shared__ float ks[D], qs[D];
  __shared__ float pk[RG][D], pq[RG][D];
  const int n = blockIdx.x / Hv, h = blockIdx.x % Hv, j = h / G;
  const int tid = threadIdx.x, cq = tid % CQ, rg = tid / CQ;
  const int64_t sidx = ((int64_t)n * Hv + h) * D * D;

  float4 Hr[R];
#pragma unroll
  for (int i = 0; i < R; ++i) {
    Hr[i] = state_in ? *reinterpret_cast<const float4*>(state_in + sidx + (int64_t)(rg + i * RG) * D + cq * 4)
                     : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  for (int i = tid; i < D; i += NTH) {
    ks[i] = to_f<E>(k[(int64_t)n * sqk + (int64_t)j * D + i]);
    qs[i] = to_f<E>(q[(int64_t)n * sqk + (int64_t)j * D + i]);
  }
  const float eg = __expf(g[(int64_t)n * Hv + h]);
  const float bt = beta[(int64_t)n * Hv + h];
  float vv[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) vv[c] = to_f<E>(v[(int64_t)n * sv + (int64_t)h * D + cq * 4 + c]);
  __syncthreads();

  float sk[4] = {0.f, 0.f, 0.f, 0.f}, sq[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const int r = rg + i * RG;
    const float kr = ks[r], qr = qs[r];
    const float hv[4] = {Hr[i].x, Hr[i].y, Hr[i].z, Hr[i].w};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      sk[c] += hv[c] * kr;
      sq[c] += hv[c] * qr;
    }
  }
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    pk[rg][cq * 4 + c] = sk[c];
    pq[rg][cq * 4 + c] = sq[c];
  }
  __syncthreads();
  float kq = 0.f;
  for (int i = 0; i < D; ++i) kq += ks[i] * qs[i];
  float u[4], ov[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    float tk = 0.f, tq = 0.f;
    for (int r = 0; r < RG; ++r) {
      tk += pk[r][cq * 4 + c];
      tq += pq[r][cq * 4 + c];
    }
    u[c] = bt * (vv[c] - eg * tk);
    ov[c] = scale * (eg * tq + kq * u[c]);
  }
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const float kr = ks[rg + i * RG];
    float4 y;
    y.x = eg * Hr[i].x + kr * u[0];
    y.y = eg * Hr[i].y + kr * u[1];
    y.z = eg * Hr[i].z + kr * u[2];
    y.w = eg * Hr[i].w + kr * u[3];
    *reinterpret_cast<float4*>(state_out + sidx + (int64_t)(rg + i * RG) * D + cq * 4) = y;
  }
  if (rg == 0) {
    E* op = o + ((int64_t)n * Hv + h) * D + cq * 4;
#pragma unroll
    for (int c = 0; c < 4; ++c) op[c] = from_f<E>(ov[c]);
  }
}

// Conv step: token n of x is the next input of sequence n.  window [N][W-1][Cch]
// holds that sequence's previous W-1 inputs, oldest first; it is read, then
// shifted by one with x appended (in place: each thread owns its channels).
// y = SiLU(sum_i w[ch][i] * [window ; x][i]), then L2 over each q/k head.  A
// lane owns 16 bytes of consecutive channels; an L2 group of dk channels is an
// aligned lane group reduced with xor shuffles (as in the prefill kernel).
template <typename E, int D, int W>
__global__ __launch_bounds__(256) void conv_step_kernel(const E* __restrict__ x, const E* __restrict__ w,
                                                        E* window, int N, int Cch, int n_qk, float eps,
                                                        E* __restrict__ y) {
  constexpr int V = Vec<E>::N;
  constexpr int LPH = D / V;
  const int n = blockIdx.y;
  const int ch = (blockIdx.x * blockDim.x + threadIdx.x) * V;
  const bool active = ch < Cch;
  float xin[W][V];
  float acc[V];
  if (active) {
#pragma unroll
    for (int i = 0; i < W - 1; ++i) Vec<E>::load(window + ((int64_t)n * (W - 1) + i) * Cch + ch, xin[i]);
    Vec<E>::load(x + (int64_t)n * Cch + ch, xin[W - 1]);
#pragma unroll
    for (int c = 0; c < V; ++c) {
      float s = 0.f;
#pragma unroll
      for (int i = 0; i < W; ++i) s += to_f<E>(w[(int64_t)(ch + c) * W + i]) * xin[i][c];
      acc[c] = s * sigmoidf_(s);
    }
  } else {
#pragma unroll
    for (int c = 0; c < V; ++c) acc[c] = 0.f;
  }
  float ss = 0.f;
#pragma unroll
  for (int c = 0; c < V; ++c) ss += acc[c] * acc[c];
  ss = group_sum<LPH>(ss);
  if (ch < n_qk) {
    const float inv = rsqrtf(ss + eps);
#pragma unroll
    for (int c = 0; c < V; ++c) acc[c] *= inv;
  }
  if (active) {
    Vec<E>::store(y + (int64_t)n * Cch + ch, acc);
#pragma unroll
    for (int i = 0; i < W - 1; ++i) Vec<E>::store(window + ((int64_t)n * (W - 1) + i) * Cch + ch, xin[i + 1]);
  }
}

// Window after a prefill: for each sequence, the last W-1 inputs of
// [window_in ; x of the sequence] (window_in NULL: zeros before the sequence).
// Thread per (sequence, slot, 16-byte channel group).
template <typename E, int W>
__global__ __launch_bounds__(256) void conv_window_kernel(const E* __restrict__ x, const int32_t* __restrict__ cu,
                                                          const E* window_in, int Cch, E* window_out) {
  constexpr int V = Vec<E>::N;
  const int n = blockIdx.z, slot = blockIdx.y;
  const int ch = (blockIdx.x * blockDim.x + threadIdx.x) * V;
  if (ch >= Cch) return;
  const int L = cu[n + 1] - cu[n];
  const int back = (W - 1) - slot;  // this slot holds the input `back` steps before the end
  float val[V];
  if (back <= L) {
    Vec<E>::load(x + (int64_t)(cu[n] + L - back) * Cch + ch, val);
  } else if (window_in) {
    // back - L steps before the sequence's first token: old window slot
    Vec<E>::load(window_in + ((int64_t)n * (W - 1) + (W - 1) - (back - L)) * Cch + ch, val);
  } else {
#pragma unroll
    for (int c = 0; c < V; ++c) val[c] = 0.f;
  }
  Vec<E>::store(window_out + ((int64_t)n * (W - 1) + slot) * Cch + ch, val);
}

// --------------------------------------------------------------------------
// host side
// --------------------------------------------------------------------------
bool run_recurrent_step(const gdn_shape* s, const void* q, const void* k, const void* v, int64_t sqk, int64_t sv,
                        const float* g, const float* beta, const float* state_in, float* state_out, void* o,
                        hipStream_t st) {
  const int N = s->n_seqs, Hv = s->h_v, G = s->h_v / s->h_qk;
#define GDN_REC(E, D)                                                                                    \
  if (s->d_k == D) {                                                                                     \
    GDN_PROF("recurrent_step", st);                                                                      \
    recurrent_step_kernel<E, D><<<N * Hv, rec_threads<D>(), 0, st>>>(                                    \
        (const E*)q, (const E*)k, (const E*)v, sqk, sv, g, beta, state_in, state_out, (E*)o, Hv, G,     \
        s->scale);                                                                                       \
    return true;                                                                                         \
  }
  if (s->dtype == GDN_BF16) {
    GDN_REC(bf16, 16) GDN_REC(bf16, 32) GDN_REC(bf16, 64) GDN_REC(bf16, 128)
  } else {
    GDN_REC(float, 16) GDN_REC(float, 32) GDN_REC(float, 64) GDN_REC(float, 128)
  }
#undef GDN_REC
  return false;
}

template <typename E, int D>
static bool conv_step_w(const gdn_shape* s, const void* x, const void* w, int width, float eps, void* window,
                        void* y, hipStream_t st) {
  constexpr int V = Vec<E>::N;
  const int Cch = 2 * s->h_qk * s->d_k + s->h_v * s->d_v;
  const dim3 grid((Cch / V + 255) / 256, s->n_seqs);
  const int nqk = 2 * s->h_qk * s->d_k;
  GDN_PROF("conv_step", st);
  switch (width) {
    case 2: conv_step_kernel<E, D, 2><<<grid, 256, 0, st>>>((const E*)x, (const E*)w, (E*)window, s->n_seqs, Cch,
                                                           nqk, eps, (E*)y); return true;
    case 3: conv_step_kernel<E, D, 3><<<grid, 256, 0, st>>>((const E*)x, (const E*)w, (E*)window, s->n_seqs, Cch,
                                                           nqk, eps, (E*)y); return true;
    case 4: conv_step_kernel<E, D, 4><<<grid, 256, 0, st>>>((const E*)x, (const E*)w, (E*)window, s->n_seqs, Cch,
                                                           nqk, eps, (E*)y); return true;
  }
  return false;
}

bool run_conv_step(const gdn_shape* s, const void* x, const void* w, int width, float eps, void* window, void* y,
                   hipStream_t st) {
#define GDN_CS(E, D) \
  if (s->d_k == D) return conv_step_w<E, D>(s, x, w, width, eps, window, y, st);
  if (s->dtype == GDN_BF16) {
    GDN_CS(bf16, 16) GDN_CS(bf16, 32) GDN_CS(bf16, 64) GDN_CS(bf16, 128)
  } else {
    GDN_CS(float, 16) GDN_CS(float, 32) GDN_CS(float, 64) GDN_CS(float, 128)
  }
#undef GDN_CS
  return false;
}

template <typename E>
static bool conv_window_e(const gdn_shape* s, const void* x, int width, const int32_t* cu, const void* win_in,
                          void* win_out, hipStream_t st) {
  constexpr int V = Vec<E>::N;
  const int Cch = 2 * s->h_qk * s->d_k + s->h_v * s->d_v;
  const dim3 grid((Cch / V + 255) / 256, width - 1, s->n_seqs);
  GDN_PROF("conv_window", st);
  switch (width) {
    case 2: conv_window_kernel<E, 2><<<grid, 256, 0, st>>>((const E*)x, cu, (const E*)win_in, Cch, (E*)win_out);
      return true;
    case 3: conv_window_kernel<E, 3><<<grid, 256, 0, st>>>((const E*)x, cu, (const E*)win_in, Cch, (E*)win_out);
      return true;
    case 4: conv_window_kernel<E, 4><<<grid, 256, 0, st>>>((const E*)x, cu, (const E*)win_in, Cch, (E*)win_out);
      return true;
  }
  return false;
}

bool run_conv_window(const gdn_shape* s, const void* x, int width, const int32_t* cu, const void* win_in,
                     void* win_out, hipStream_t st) {
  return s->dtype == GDN_BF16 ? conv_window_e<bf16>(s, x, width, cu, win_in, win_out, st)
                              : conv_window_e<float>(s, x, width, cu, win_in, win_out, st);
}

}  // namespace gdn
