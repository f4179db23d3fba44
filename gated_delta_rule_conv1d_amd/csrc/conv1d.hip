// Causal depthwise conv1d + SiLU + per-head L2 normalisation, forward and
// backward, over one packed varlen row.
//
// Pages: "[Qwen3.5 MoE] Add hybrid decoder model", Summary (depthwise conv1d
// inside GatedDeltaNet); "Support Qwen35 SFT", Notes and XTuner changes
// (causal_conv1d dependency, varlen mode).
//
// Layout: x, y [T][Cch] channel-last.  A lane owns 16 bytes of consecutive
// channels (8 bf16 or 4 float), so a wave reads/writes 1 KiB (bf16) of one
// token per instruction, fully coalesced.  Each wave walks TB consecutive
// tokens of its channel block, keeping the width-1 previous inputs in
// registers; the sequence containing the wave's first token is found by
// binary search in cu_seqlens and the history is cleared at every sequence
// start.  L2 groups (one q/k head = d channels) are aligned lane groups and
// reduce with xor shuffles.
#include "gdn_common.cuh"
#include "gdn_internal.h"
#include "profile.h"

namespace gdn {

constexpr int kConvTB = 64;       // tokens per wave, forward (at most; fewer on short rows)
constexpr int kConvTBB = 128;     // tokens per wave, backward (its W-1 look-ahead
                                  // tokens and dw partials amortise over more)
constexpr int kConvWaves = 4;     // waves (token blocks) per workgroup
constexpr int kConvCUs = 256;     // MI355X compute units

__device__ __forceinline__ int find_seq(const int32_t* cu, int N, int t) {
  // largest n with cu[n] <= t (so cu[n] <= t < cu[n+1] when t < T)
  int lo = 0, hi = N;  // answer in [0, N-1]
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (cu[mid] <= t) lo = mid; else hi = mid - 1;
  }
  return lo < N ? lo : N - 1;
}

// Prologue loads through buffer resources: a lane whose value does not exist
// (channel past Cch, token outside its sequence) reads an out-of-range offset
// and gets zeros, so every load is issued at once and waited for once (loads
// under a per-lane branch were each waited for inside it).
constexpr int kOob = 0x7fffff00;

// this lane's V x W taps, w[(ch + c) * W + i]
template <typename E, int V, int W>
__device__ __forceinline__ void load_taps(const E* w, int Cch, int ch, float (&wr)[V][W]) {
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<E*>(w), 0, Cch * W * (int)sizeof(E), 0x00020000);
  const int base = ch < Cch ? ch * W * (int)sizeof(E) : kOob;
#pragma unroll
  for (int c = 0; c < V; ++c)
#pragma unroll
    for (int i = 0; i < W; ++i) {
      const int k = (c * W + i) * (int)sizeof(E);
      if constexpr (sizeof(E) == 2)
        wr[c][i] = to_f<E>(__builtin_bit_cast(E, (uint16_t)__builtin_amdgcn_raw_buffer_load_b16(rs, base + k, 0, 0)));
      else
        wr[c][i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, base + k, 0, 0));
    }
}

// 16 bytes (V channels) at byte offset off of rs, as floats (zeros out of range)
template <typename E>
__device__ __forceinline__ void load_vec_buf(__amdgpu_buffer_rsrc_t rs, int off, float* out) {
  const uint4 raw = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0));
  const E* e = reinterpret_cast<const E*>(&raw);
#pragma unroll
  for (int i = 0; i < Vec<E>::N; ++i) out[i] = to_f<E>(e[i]);
}

template <typename E, int D, int W>
__global__ __launch_bounds__(256) void conv_fwd_kernel(const E* __restrict__ x, const E* __restrict__ w,
                                                       const int32_t* __restrict__ cu, const E* __restrict__ win,
                                                       int N, int T, int Cch, int n_qk, float eps, int tpw,
                                                       E* __restrict__ y) {
  constexpr int V = Vec<E>::N;      // channels per lane
  constexpr int LPH = D / V;        // lanes per L2 group
  const int lane = lane_id();
  // the wave index read as a scalar: the token range, the sequence search and
  // its cu_seqlens reads are then scalar too
  const int tb = blockIdx.x * kConvWaves + __builtin_amdgcn_readfirstlane(wave_id());
  const int t0 = tb * tpw;          // tpw tokens per wave
  if (t0 >= T) return;
  const int t1 = min(t0 + tpw, T);
  const int ch = (blockIdx.y * kWave + lane) * V;
  const bool active = ch < Cch;
  const bool is_qk = ch < n_qk;

  float wr[V][W];
  load_taps<E, V, W>(w, Cch, ch, wr);

  // ring[k] holds x of the token t with (t - t0) % W == k; the token loop is
  // unrolled by W so every slot index is a constant (no register shifting)
  float ring[W][V];
  int n = find_seq(cu, N, t0);
  int seq_start = cu[n], seq_end = cu[n + 1];
#pragma unroll
  for (int c = 0; c < V; ++c) ring[0][c] = 0.f;
  {
    // history: token s = t0 - (W-1) + i from x inside the sequence, else its
    // carried window (slot s - seq_start + W - 1), else zeros
    const int b0 = max(t0 - (W - 1), 0);
    const int es = (int)sizeof(E);
    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<E*>(x) + (size_t)b0 * Cch, 0, (t0 - b0) * Cch * es, 0x00020000);
    const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<E*>(win) + (win ? (size_t)n * (W - 1) * Cch : 0), 0, win ? (W - 1) * Cch * es : 0, 0x00020000);
#pragma unroll
    for (int i = 0; i < W - 1; ++i) {
      const int s = t0 - (W - 1) + i;
      const bool in_seq = s >= seq_start;
      float fx[V], fw[V];
      load_vec_buf<E>(rx, active && in_seq ? ((s - b0) * Cch + ch) * es : kOob, fx);
      load_vec_buf<E>(rw, active && !in_seq ? ((s - seq_start + W - 1) * Cch + ch) * es : kOob, fw);
#pragma unroll
      for (int c = 0; c < V; ++c) ring[i + 1][c] = in_seq ? fx[c] : fw[c];
    }
  }

  // the next W tokens' x are loaded while the current W compute (W loads in
  // flight per wave)
  uint4 cx[W];
#pragma unroll
  for (int p = 0; p < W; ++p)
    cx[p] = (active && t0 + p < t1) ? *reinterpret_cast<const uint4*>(x + (size_t)(t0 + p) * Cch + ch)
                                    : make_uint4(0, 0, 0, 0);
  for (int tb = t0; tb < t1; tb += W) {
    uint4 nx[W];
#pragma unroll
    for (int p = 0; p < W; ++p)
      nx[p] = (active && tb + W + p < t1) ? *reinterpret_cast<const uint4*>(x + (size_t)(tb + W + p) * Cch + ch)
                                          : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int p = 0; p < W; ++p) {
      const int t = tb + p;
      if (t >= t1) break;
      const uint4 rx = cx[p];
      if (t >= seq_end) {  // entering a new sequence (skip empty ones): t is its first token
        while (cu[n + 1] <= t) ++n;
        seq_start = cu[n];
        seq_end = cu[n + 1];
        // history: the sequence's carried window (token t - (W-1) + i in window
        // slot i), or zeros
#pragma unroll
        for (int i = 0; i < W - 1; ++i) {
          if (active && win) Vec<E>::load(win + ((size_t)n * (W - 1) + i) * Cch + ch, ring[(p + 1 + i) % W]);
          else
#pragma unroll
            for (int c = 0; c < V; ++c) ring[(p + 1 + i) % W][c] = 0.f;
        }
      }
      {
        const E* ex = reinterpret_cast<const E*>(&rx);
#pragma unroll
        for (int c = 0; c < V; ++c) ring[p][c] = to_f<E>(ex[c]);
      }
      float a[V];
      float ss = 0.f;
#pragma unroll
      for (int c = 0; c < V; ++c) {
        float acc = wr[c][W - 1] * ring[p][c];
#pragma unroll
        for (int i = 0; i < W - 1; ++i) acc += wr[c][i] * ring[(p + 1 + i) % W][c];  // token t - (W-1) + i
        a[c] = acc * sigmoidf_(acc);
        ss += a[c] * a[c];
      }
      ss = group_sum<LPH>(ss);
      if (is_qk) {
        const float inv = rsqrtf(ss + eps);
#pragma unroll
        for (int c = 0; c < V; ++c) a[c] *= inv;
      }
      if (active) Vec<E>::store(y + (size_t)t * Cch + ch, a);
    }
#pragma unroll
    for (int p = 0; p < W; ++p) cx[p] = nx[p];
  }
}

// Backward.  For token t: recompute c, a = SiLU(c), the L2 norm; then
// da = dy/n - a (a.dy)/n^3 (q/k) or dy (v); dc = da * s (1 + c (1 - s)).
// dx[s] = sum_i w_i dc[s + W-1 - i] over terms in s's sequence; each wave
// computes dc for its TB tokens plus W-1 look-ahead tokens.  dw partial sums
// per (workgroup, channel, tap) go to workspace in a fixed order.
template <typename E, int D, int W>
__global__ __launch_bounds__(256, 2) void conv_bwd_kernel(const E* __restrict__ dy, const E* __restrict__ x,
                                                       const E* __restrict__ w, const int32_t* __restrict__ cu,
                                                       int N, int T, int Cch, int n_qk, float eps,
                                                       E* __restrict__ dx, float* __restrict__ dw_part) {
  constexpr int V = Vec<E>::N;
  constexpr int LPH = D / V;
  __shared__ float red[kConvWaves][kWave * V * W];
  const int lane = lane_id();
  const int wv = __builtin_amdgcn_readfirstlane(wave_id());  // scalar: so are the token range and the cu_seqlens reads
  const int tb = blockIdx.x * kConvWaves + wv;
  const int t0 = tb * kConvTBB;
  const int ch = (blockIdx.y * kWave + lane) * V;
  const bool active = ch < Cch;
  const bool is_qk = ch < n_qk;

  float dwacc[V][W];
#pragma unroll
  for (int c = 0; c < V; ++c)
#pragma unroll
    for (int i = 0; i < W; ++i) dwacc[c][i] = 0.f;

  if (t0 < T) {
    const int t1 = min(t0 + kConvTBB, T);
    const int tend = min(t1 + W - 1, T);
    float wr[V][W];
    load_taps<E, V, W>(w, Cch, ch, wr);

    int n = find_seq(cu, N, t0);
    int seq_start = cu[n], seq_end = cu[n + 1];
    // xr[k] holds x of the token t with (t - t0) % W == k, dcr[k] / dcs[k] its
    // dc and the start of its sequence; the token loop is unrolled by W so
    // every slot index is a constant (no register shifting)
    float xr[W][V], dcr[W][V];
    int dcs[W];
#pragma unroll
    for (int i = 0; i < W; ++i) {
      dcs[i] = 0x7fffffff;
#pragma unroll
      for (int c = 0; c < V; ++c) xr[i][c] = dcr[i][c] = 0.f;
    }
    {
      const int b0 = max(t0 - (W - 1), 0);
      const int es = (int)sizeof(E);
      const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<E*>(x) + (size_t)b0 * Cch, 0, (t0 - b0) * Cch * es, 0x00020000);
#pragma unroll
      for (int i = 0; i < W - 1; ++i) {
        const int s = t0 - (W - 1) + i;
        load_vec_buf<E>(rx, active && s >= seq_start ? ((s - b0) * Cch + ch) * es : kOob, xr[i + 1]);
      }
    }
    // the next W tokens' x and dy are loaded while the current W compute
    uint4 cx[W], cg[W];
#pragma unroll
    for (int p = 0; p < W; ++p) {
      const bool ok = active && t0 + p < tend;
      cx[p] = ok ? *reinterpret_cast<const uint4*>(x + (size_t)(t0 + p) * Cch + ch) : make_uint4(0, 0, 0, 0);
      cg[p] = ok ? *reinterpret_cast<const uint4*>(dy + (size_t)(t0 + p) * Cch + ch) : make_uint4(0, 0, 0, 0);
    }
    for (int tb = t0; tb < tend; tb += W) {
      uint4 nx[W], ng[W];
#pragma unroll
      for (int p = 0; p < W; ++p) {
        const int tn = tb + W + p;
        const bool ok = active && tn < tend;
        nx[p] = ok ? *reinterpret_cast<const uint4*>(x + (size_t)tn * Cch + ch) : make_uint4(0, 0, 0, 0);
        ng[p] = ok ? *reinterpret_cast<const uint4*>(dy + (size_t)tn * Cch + ch) : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int p = 0; p < W; ++p) {
        const int t = tb + p;
        if (t >= tend) break;
        const uint4 rx = cx[p], rg = cg[p];
        if (t >= seq_end) {  // entering a new sequence (skip empty ones): no history
          while (cu[n + 1] <= t) ++n;
          seq_start = cu[n];
          seq_end = cu[n + 1];
#pragma unroll
          for (int i = 0; i < W; ++i)
#pragma unroll
            for (int c = 0; c < V; ++c) xr[i][c] = 0.f;
        }
        float g[V];
        {
          const E* ex = reinterpret_cast<const E*>(&rx);
          const E* eg = reinterpret_cast<const E*>(&rg);
#pragma unroll
          for (int c = 0; c < V; ++c) {
            xr[p][c] = to_f<E>(ex[c]);
            g[c] = to_f<E>(eg[c]);
          }
        }
        float cc[V], sg[V], a[V];
        float ss = 0.f, dot = 0.f;
#pragma unroll
        for (int c = 0; c < V; ++c) {
          float acc = wr[c][W - 1] * xr[p][c];
#pragma unroll
          for (int i = 0; i < W - 1; ++i) acc += wr[c][i] * xr[(p + 1 + i) % W][c];  // token t - (W-1) + i
          cc[c] = acc;
          sg[c] = sigmoidf_(acc);
          a[c] = acc * sg[c];
          ss += a[c] * a[c];
          dot += a[c] * g[c];
        }
        ss = group_sum<LPH>(ss);
        dot = group_sum<LPH>(dot);
        const float inv = rsqrtf(ss + eps);
        const float inv3 = inv * inv * inv;
#pragma unroll
        for (int c = 0; c < V; ++c) {
          const float da = is_qk ? (g[c] * inv - a[c] * dot * inv3) : g[c];
          dcr[p][c] = da * sg[c] * (1.f + cc[c] * (1.f - sg[c]));
        }
        dcs[p] = seq_start;
        if (t < t1) {  // own token: weight gradient
#pragma unroll
          for (int c = 0; c < V; ++c) {
#pragma unroll
            for (int i = 0; i < W - 1; ++i) dwacc[c][i] += dcr[p][c] * xr[(p + 1 + i) % W][c];
            dwacc[c][W - 1] += dcr[p][c] * xr[p][c];
          }
        }
        // dx for token s = t - (W-1): dc[s + m] sits in slot (p + 1 + m) % W and
        // tap W-1-m multiplies it; only terms inside s's sequence count
        const int s = t - (W - 1);
        if (s >= t0 && active) {
          float o[V];
#pragma unroll
          for (int c = 0; c < V; ++c) o[c] = 0.f;
#pragma unroll
          for (int m = 0; m < W; ++m) {
            const int k = (p + 1 + m) % W;
            if (dcs[k] <= s) {
#pragma unroll
              for (int c = 0; c < V; ++c) o[c] += wr[c][W - 1 - m] * dcr[k][c];
            }
          }
          Vec<E>::store(dx + (size_t)s * Cch + ch, o);
        }
      }
#pragma unroll
      for (int p = 0; p < W; ++p) {
        cx[p] = nx[p];
        cg[p] = ng[p];
      }
    }
    // tokens whose W-1 successors run past the end of the row: dc of token u
    // (u < tend) is in slot (u - t0) % W
    if (active) {
      for (int s = max(t0, tend - (W - 1)); s < t1; ++s) {
        float o[V];
#pragma unroll
        for (int c = 0; c < V; ++c) o[c] = 0.f;
#pragma unroll
        for (int m = 0; m < W; ++m) {
          const int k = (s + m - t0) % W;
          if (s + m < tend && dcs[k] <= s) {
#pragma unroll
            for (int c = 0; c < V; ++c) o[c] += wr[c][W - 1 - m] * dcr[k][c];
          }
        }
        Vec<E>::store(dx + (size_t)s * Cch + ch, o);
      }
    }
  }
  // reduce dw over the workgroup's waves in a fixed order
#pragma unroll
  for (int c = 0; c < V; ++c)
#pragma unroll
    for (int i = 0; i < W; ++i) red[wv][(lane * V + c) * W + i] = dwacc[c][i];
  __syncthreads();
  for (int e = threadIdx.x; e < kWave * V * W; e += blockDim.x) {
    const int chl = e / W;  // channel within the block
    const int gch = blockIdx.y * kWave * V + chl;
    if (gch < Cch) {
      float s = 0.f;
#pragma unroll
      for (int k = 0; k < kConvWaves; ++k) s += red[k][e];
      dw_part[((size_t)blockIdx.x * Cch + gch) * W + (e % W)] = s;
    }
  }
}

// --------------------------------------------------------------------------
// host side
// --------------------------------------------------------------------------
static int conv_grid_x(int T, int tb) {
  const int ntb = (T + tb - 1) / tb;
  return (ntb + kConvWaves - 1) / kConvWaves;
}

size_t conv_bwd_ws_bytes(const gdn_shape* s, int width) {
  const int Cch = 2 * s->h_qk * s->d_k + s->h_v * s->d_v;
  const int gx = conv_grid_x(s->total_tokens, kConvTBB) > 0 ? conv_grid_x(s->total_tokens, kConvTBB) : 1;
  return (size_t)gx * Cch * width * sizeof(float);
}

template <typename E, int D, int W>
static void launch_conv_fwd(const gdn_shape* s, const void* x, const void* w, const int32_t* cu, const void* win,
                            float eps, void* y, hipStream_t st) {
  constexpr int V = Vec<E>::N;
  const int Cch = 2 * s->h_qk * s->d_k + s->h_v * s->d_v;
  // tokens per wave: 64, or fewer where that would leave under 16 waves per CU
  // (each wave keeps one width of tokens in flight, so short rows need more
  // waves to cover the memory latency; each extra wave re-reads W - 1 tokens of
  // history)
  const int cgroups = (Cch + kWave * V - 1) / (kWave * V);
  int tpw = kConvTB;
  while (tpw > 16 && (int64_t)((s->total_tokens + tpw - 1) / tpw) * cgroups < 16 * kConvCUs) tpw /= 2;
  dim3 grid(conv_grid_x(s->total_tokens, tpw), cgroups);
  GDN_PROF("conv_fwd", st);
  conv_fwd_kernel<E, D, W><<<grid, 256, 0, st>>>((const E*)x, (const E*)w, cu, (const E*)win, s->n_seqs,
                                                 s->total_tokens, Cch, 2 * s->h_qk * s->d_k, eps, tpw, (E*)y);
}

template <typename E, int D, int W>
static void launch_conv_bwd(const gdn_shape* s, const void* dy, const void* x, const void* w, const int32_t* cu,
                            float eps, void* dx, float* dw, void* ws, hipStream_t st) {
  constexpr int V = Vec<E>::N;
  const int Cch = 2 * s->h_qk * s->d_k + s->h_v * s->d_v;
  dim3 grid(conv_grid_x(s->total_tokens, kConvTBB), (Cch + kWave * V - 1) / (kWave * V));
  float* part = (float*)ws;
  {
    GDN_PROF("conv_bwd", st);
    conv_bwd_kernel<E, D, W><<<grid, 256, 0, st>>>((const E*)dy, (const E*)x, (const E*)w, cu, s->n_seqs,
                                                   s->total_tokens, Cch, 2 * s->h_qk * s->d_k, eps, (E*)dx, part);
  }
  const int n = Cch * W;
  GDN_PROF("conv_dw_sum", st);
  launch_colsum(part, (int)grid.x, n, dw, st);
}

template <typename E, int D>
static bool conv_fwd_w(const gdn_shape* s, const void* x, const void* w, int width, const int32_t* cu,
                       const void* win, float eps, void* y, hipStream_t st) {
  switch (width) {
    case 2: launch_conv_fwd<E, D, 2>(s, x, w, cu, win, eps, y, st); return true;
    case 3: launch_conv_fwd<E, D, 3>(s, x, w, cu, win, eps, y, st); return true;
    case 4: launch_conv_fwd<E, D, 4>(s, x, w, cu, win, eps, y, st); return true;
  }
  return false;
}

template <typename E, int D>
static bool conv_bwd_w(const gdn_shape* s, const void* dy, const void* x, const void* w, int width,
                       const int32_t* cu, float eps, void* dx, float* dw, void* ws, hipStream_t st) {
  switch (width) {
    case 2: launch_conv_bwd<E, D, 2>(s, dy, x, w, cu, eps, dx, dw, ws, st); return true;
    case 3: launch_conv_bwd<E, D, 3>(s, dy, x, w, cu, eps, dx, dw, ws, st); return true;
    case 4: launch_conv_bwd<E, D, 4>(s, dy, x, w, cu, eps, dx, dw, ws, st); return true;
  }
  return false;
}

bool run_conv_fwd(const gdn_shape* s, const void* x, const void* w, int width, const int32_t* cu, const void* win,
                  float eps, void* y, hipStream_t st) {
  if (s->total_tokens == 0) return true;
#define GDN_CONV_D(E, D) \
  if (s->d_k == D) return conv_fwd_w<E, D>(s, x, w, width, cu, win, eps, y, st);
  if (s->dtype == GDN_BF16) {
    GDN_CONV_D(bf16, 16) GDN_CONV_D(bf16, 32) GDN_CONV_D(bf16, 64) GDN_CONV_D(bf16, 128)
  } else {
    GDN_CONV_D(float, 16) GDN_CONV_D(float, 32) GDN_CONV_D(float, 64) GDN_CONV_D(float, 128)
  }
#undef GDN_CONV_D
  return false;
}

bool run_conv_bwd(const gdn_shape* s, const void* dy, const void* x, const void* w, int width, const int32_t* cu,
                  float eps, void* dx, float* dw, void* ws, hipStream_t st) {
  if (s->total_tokens == 0) {
    const int n = (2 * s->h_qk * s->d_k + s->h_v * s->d_v) * width;
    launch_colsum((const float*)ws, 0, n, dw, st);
    return true;
  }
#define GDN_CONV_D(E, D) \
  if (s->d_k == D) return conv_bwd_w<E, D>(s, dy, x, w, width, cu, eps, dx, dw, ws, st);
  if (s->dtype == GDN_BF16) {
    GDN_CONV_D(bf16, 16) GDN_CONV_D(bf16, 32) GDN_CONV_D(bf16, 64) GDN_CONV_D(bf16, 128)
  } else {
    GDN_CONV_D(float, 16) GDN_CONV_D(float, 32) GDN_CONV_D(float, 64) GDN_CONV_D(float, 128)
  }
#undef GDN_CONV_D
  return false;
}

}  // namespace gdn
