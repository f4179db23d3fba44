/*
 * Plain CPU oracle for the GatedDeltaNet layer over packed varlen rows.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may call this code; the library never does.
 * It shares no code with the GPU path.
 *
 * Built twice: with REAL=double (the oracle proper) and REAL=float (used only
 * to show that a correct single-precision implementation meets the fp32
 * tolerance).  Every step is the plain definition, token by token, with no
 * blocking, chunking or reordering.
 *
 * Where the layer comes from on the pages:
 *  - "[Qwen3.5 MoE] Add hybrid decoder model (GatedDeltaNet + full attention +
 *    MoE)", Summary: GatedDeltaNet linear attention, RMSNormGated, a depthwise
 *    conv1d, the softplus gate, and a naive torch fallback (the role this file
 *    plays).
 *  - "Support Qwen35 SFT", XTuner changes and Notes: GatedDeltaNet in varlen
 *    mode built on causal_conv1d and flash-linear-attention.
 *  - "feat(models): dense Qwen3.5 custom attention", Summary: cu_seqlens derived
 *    from position_ids, one packed row per call.
 * The pages print no formula; the definitions below are the layer's standard
 * ones (causal depthwise conv + SiLU, L2-normalised q/k, the gated delta rule
 * S_t = e^{g_t} S_{t-1} (I - b_t k_t k_t^T) + b_t v_t k_t^T with o_t = S_t q_t,
 * RMSNormGated), with the readings listed alongside the library's design notes.
 *
 * State convention: H = S^T is stored [d_k][d_v] row-major, so o_t = H^T q_t.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifndef REAL
#define REAL double
#endif
typedef REAL real;

#if defined(_OPENMP)
#include <omp.h>
#endif

#define EXPORT __attribute__((visibility("default")))

static real sigm(real x) { return (real)1 / ((real)1 + exp(-x)); }

/* ---------------------------------------------------------------------------
 * Causal depthwise conv1d + SiLU, then L2 normalisation of each q/k head.
 *   c[t,ch] = sum_{i<W} w[ch,i] * x[t-(W-1)+i, ch], terms before the start of
 *             t's sequence are zero (every sequence starts from zero history);
 *   y = c * sigmoid(c);
 *   for channels ch < n_qk_ch (the q and k blocks), per head of d_k channels:
 *             y <- y / sqrt(sum y^2 + eps).
 * x, y: [T][Cch]; w: [Cch][W]; cu: [N+1] token offsets.
 * ------------------------------------------------------------------------- */
EXPORT void oracle_conv1d(int N, const int32_t* cu, int Cch, int W, int n_qk_ch, int d_k,
                          real eps, const real* x, const real* w, real* y) {
  const long T = cu[N];
#pragma omp parallel for schedule(static)
  for (int ch = 0; ch < Cch; ++ch) {
    for (int n = 0; n < N; ++n) {
      for (long t = cu[n]; t < cu[n + 1]; ++t) {
        real c = 0;
        for (int i = 0; i < W; ++i) {
          long s = t - (W - 1) + i;
          if (s >= cu[n]) c += w[(long)ch * W + i] * x[s * Cch + ch];
        }
        y[t * Cch + ch] = c * sigm(c);
      }
    }
  }
  if (n_qk_ch <= 0) return;
#pragma omp parallel for schedule(static)
  for (long t = 0; t < T; ++t) {
    for (int h0 = 0; h0 < n_qk_ch; h0 += d_k) {
      real ss = 0;
      for (int i = 0; i < d_k; ++i) ss += y[t * Cch + h0 + i] * y[t * Cch + h0 + i];
      real inv = (real)1 / sqrt(ss + eps);
      for (int i = 0; i < d_k; ++i) y[t * Cch + h0 + i] *= inv;
    }
  }
}

/* Backward of oracle_conv1d.  dy: gradient w.r.t. y [T][Cch].
 * dx [T][Cch] and dw [Cch][W] are overwritten.  For each channel the weight
 * gradient sums over sequences, then tokens, in order. */
EXPORT void oracle_conv1d_bwd(int N, const int32_t* cu, int Cch, int W, int n_qk_ch, int d_k,
                              real eps, const real* x, const real* w, const real* dy,
                              real* dx, real* dw) {
  const long T = cu[N];
  real* c = (real*)malloc(sizeof(real) * T * Cch);
  real* dc = (real*)malloc(sizeof(real) * T * Cch);
  /* pre-activation */
#pragma omp parallel for schedule(static)
  for (int ch = 0; ch < Cch; ++ch)
    for (int n = 0; n < N; ++n)
      for (long t = cu[n]; t < cu[n + 1]; ++t) {
        real acc = 0;
        for (int i = 0; i < W; ++i) {
          long s = t - (W - 1) + i;
          if (s >= cu[n]) acc += w[(long)ch * W + i] * x[s * Cch + ch];
        }
        c[t * Cch + ch] = acc;
      }
  /* through the L2 normalisation (q/k heads) and the SiLU */
#pragma omp parallel for schedule(static)
  for (long t = 0; t < T; ++t) {
    for (int ch0 = 0; ch0 < Cch;) {
      const int width = ch0 < n_qk_ch ? d_k : 1;
      if (ch0 < n_qk_ch) {
        real ss = 0, dot = 0;
        for (int i = 0; i < width; ++i) {
          real cc = c[t * Cch + ch0 + i], a = cc * sigm(cc);
          ss += a * a;
          dot += a * dy[t * Cch + ch0 + i];
        }
        real nrm = sqrt(ss + eps);
        for (int i = 0; i < width; ++i) {
          real cc = c[t * Cch + ch0 + i], sg = sigm(cc), a = cc * sg;
          real da = dy[t * Cch + ch0 + i] / nrm - a * dot / (nrm * nrm * nrm);
          dc[t * Cch + ch0 + i] = da * sg * ((real)1 + cc * ((real)1 - sg));
        }
      } else {
        real cc = c[t * Cch + ch0], sg = sigm(cc);
        dc[t * Cch + ch0] = dy[t * Cch + ch0] * sg * ((real)1 + cc * ((real)1 - sg));
      }
      ch0 += width;
    }
  }
  /* through the causal conv: dx[s] = sum_i w_i dc[s+(W-1)-i] within the sequence */
#pragma omp parallel for schedule(static)
  for (int ch = 0; ch < Cch; ++ch) {
    for (int i = 0; i < W; ++i) dw[(long)ch * W + i] = 0;
    for (int n = 0; n < N; ++n)
      for (long s = cu[n]; s < cu[n + 1]; ++s) {
        real acc = 0;
        for (int i = 0; i < W; ++i) {
          long t = s + (W - 1) - i;
          if (t < cu[n + 1]) acc += w[(long)ch * W + i] * dc[t * Cch + ch];
        }
        dx[s * Cch + ch] = acc;
      }
    for (int n = 0; n < N; ++n)
      for (long t = cu[n]; t < cu[n + 1]; ++t)
        for (int i = 0; i < W; ++i) {
          long s = t - (W - 1) + i;
          if (s >= cu[n]) dw[(long)ch * W + i] += dc[t * Cch + ch] * x[s * Cch + ch];
        }
  }
  free(c);
  free(dc);
}

/* ---------------------------------------------------------------------------
 * Gated delta rule, token by token, per sequence and v-head h (k-head h*Hk/Hv).
 *   H <- e^{g_t} H                      (decay the whole previous state)
 *   p  = H^T k_t                        (prediction of the decayed state)
 *   u  = b_t (v_t - p)
 *   H <- H + k_t u^T                    (S_t = e^{g}S(I - b k k^T) + b v k^T)
 *   o_t = scale * H^T q_t
 * q, k: element (t, j, i) at [t*sqk + j*d_k + i]; v: (t, h, i) at [t*sv + h*d_v + i].
 * g, beta: [T][Hv]; h0, ht: [N][Hv][d_k][d_v] (either may be NULL); o: [T][Hv][d_v].
 * ------------------------------------------------------------------------- */
EXPORT void oracle_recurrence(int N, const int32_t* cu, int Hk, int Hv, int dk, int dv, real scale,
                              const real* q, const real* k, long sqk, const real* v, long sv,
                              const real* g, const real* beta, const real* h0,
                              real* o, real* ht) {
  const int G = Hv / Hk;
#pragma omp parallel for schedule(dynamic, 1)
  for (long task = 0; task < (long)N * Hv; ++task) {
    const int n = (int)(task / Hv), h = (int)(task % Hv), j = h / G;
    real* H = (real*)malloc(sizeof(real) * dk * dv);
    real* p = (real*)malloc(sizeof(real) * dv);
    if (h0) memcpy(H, h0 + ((long)n * Hv + h) * dk * dv, sizeof(real) * dk * dv);
    else memset(H, 0, sizeof(real) * dk * dv);
    for (long t = cu[n]; t < cu[n + 1]; ++t) {
      const real* kt = k + t * sqk + (long)j * dk;
      const real* qt = q + t * sqk + (long)j * dk;
      const real* vt = v + t * sv + (long)h * dv;
      const real decay = exp(g[t * Hv + h]), b = beta[t * Hv + h];
      for (int e = 0; e < dk * dv; ++e) H[e] *= decay;
      for (int c = 0; c < dv; ++c) p[c] = 0;
      for (int i = 0; i < dk; ++i)
        for (int c = 0; c < dv; ++c) p[c] += H[i * dv + c] * kt[i];
      for (int c = 0; c < dv; ++c) p[c] = b * (vt[c] - p[c]); /* p now holds u */
      for (int i = 0; i < dk; ++i)
        for (int c = 0; c < dv; ++c) H[i * dv + c] += kt[i] * p[c];
      real* ot = o + (t * Hv + h) * dv;
      for (int c = 0; c < dv; ++c) ot[c] = 0;
      for (int i = 0; i < dk; ++i)
        for (int c = 0; c < dv; ++c) ot[c] += H[i * dv + c] * qt[i];
      for (int c = 0; c < dv; ++c) ot[c] *= scale;
    }
    if (ht) memcpy(ht + ((long)n * Hv + h) * dk * dv, H, sizeof(real) * dk * dv);
    free(H);
    free(p);
  }
}

/* Reverse mode of oracle_recurrence.  d_o: [T][Hv][d_v]; dht may be NULL (zero).
 * Outputs (overwritten): dq, dk dense [T][Hk][d_k]; dv [T][Hv][d_v]; dg, dbeta
 * [T][Hv]; dh0 [N][Hv][d_k][d_v] (may be NULL).  The state is checkpointed every
 * CKPT tokens and recomputed inside each block.  One task per (sequence,
 * k-head) handles its v-heads in order, so dq and dk need no shared writes. */
#define CKPT 64
EXPORT void oracle_recurrence_bwd(int N, const int32_t* cu, int Hk, int Hv, int dk, int dv, real scale,
                                  const real* q, const real* k, long sqk, const real* v, long sv,
                                  const real* g, const real* beta, const real* h0,
                                  const real* d_o, const real* dht,
                                  real* dq, real* dk_out, real* dv_out, real* dg, real* dbeta,
                                  real* dh0) {
  const int G = Hv / Hk;
  const long S = (long)dk * dv;
#pragma omp parallel for schedule(dynamic, 1)
  for (long task = 0; task < (long)N * Hk; ++task) {
    const int n = (int)(task / Hk), j = (int)(task % Hk);
    const long t0 = cu[n], L = cu[n + 1] - cu[n];
    for (long t = t0; t < t0 + L; ++t)
      for (int i = 0; i < dk; ++i) {
        dq[(t * Hk + j) * dk + i] = 0;
        dk_out[(t * Hk + j) * dk + i] = 0;
      }
    const long nblk = (L + CKPT - 1) / CKPT;
    real* ck = (real*)malloc(sizeof(real) * S * (nblk > 0 ? nblk : 1));
    real* states = (real*)malloc(sizeof(real) * S * (CKPT + 1)); /* states[0] = before block */
    real* H = (real*)malloc(sizeof(real) * S);
    real* dH = (real*)malloc(sizeof(real) * S);
    real* Hd = (real*)malloc(sizeof(real) * S);
    real* u = (real*)malloc(sizeof(real) * dv);
    real* pv = (real*)malloc(sizeof(real) * dv);
    real* du = (real*)malloc(sizeof(real) * dv);
    real* dp = (real*)malloc(sizeof(real) * dv);
    for (int h = j * G; h < (j + 1) * G; ++h) {
      /* forward: checkpoint the state entering each block */
      if (h0) memcpy(H, h0 + ((long)n * Hv + h) * S, sizeof(real) * S);
      else memset(H, 0, sizeof(real) * S);
      for (long t = t0; t < t0 + L; ++t) {
        const long r = t - t0;
        if (r % CKPT == 0) memcpy(ck + (r / CKPT) * S, H, sizeof(real) * S);
        const real* kt = k + t * sqk + (long)j * dk;
        const real* vt = v + t * sv + (long)h * dv;
        const real decay = exp(g[t * Hv + h]), b = beta[t * Hv + h];
        for (long e = 0; e < S; ++e) H[e] *= decay;
        for (int c = 0; c < dv; ++c) u[c] = 0;
        for (int i = 0; i < dk; ++i)
          for (int c = 0; c < dv; ++c) u[c] += H[i * dv + c] * kt[i];
        for (int c = 0; c < dv; ++c) u[c] = b * (vt[c] - u[c]);
        for (int i = 0; i < dk; ++i)
          for (int c = 0; c < dv; ++c) H[i * dv + c] += kt[i] * u[c];
      }
      /* reverse */
      if (dht) memcpy(dH, dht + ((long)n * Hv + h) * S, sizeof(real) * S);
      else memset(dH, 0, sizeof(real) * S);
      for (long blk = nblk - 1; blk >= 0; --blk) {
        const long rb = blk * CKPT, re = (rb + CKPT < L) ? rb + CKPT : L;
        memcpy(states, ck + blk * S, sizeof(real) * S);
        for (long r = rb; r < re; ++r) { /* states[r-rb+1] = state after token r */
          const long t = t0 + r;
          const real* kt = k + t * sqk + (long)j * dk;
          const real* vt = v + t * sv + (long)h * dv;
          const real decay = exp(g[t * Hv + h]), b = beta[t * Hv + h];
          real* Hp = states + (r - rb) * S;
          real* Hn = states + (r - rb + 1) * S;
          for (long e = 0; e < S; ++e) Hn[e] = Hp[e] * decay;
          for (int c = 0; c < dv; ++c) u[c] = 0;
          for (int i = 0; i < dk; ++i)
            for (int c = 0; c < dv; ++c) u[c] += Hn[i * dv + c] * kt[i];
          for (int c = 0; c < dv; ++c) u[c] = b * (vt[c] - u[c]);
          for (int i = 0; i < dk; ++i)
            for (int c = 0; c < dv; ++c) Hn[i * dv + c] += kt[i] * u[c];
        }
        for (long r = re - 1; r >= rb; --r) {
          const long t = t0 + r;
          const real* kt = k + t * sqk + (long)j * dk;
          const real* qt = q + t * sqk + (long)j * dk;
          const real* vt = v + t * sv + (long)h * dv;
          const real* dot = d_o + (t * Hv + h) * dv;
          const real decay = exp(g[t * Hv + h]), b = beta[t * Hv + h];
          const real* Hprev = states + (r - rb) * S;
          const real* Hcur = states + (r - rb + 1) * S;
          real* dqt = dq + (t * Hk + j) * dk;
          real* dkt = dk_out + (t * Hk + j) * dk;
          real* dvt = dv_out + (t * Hv + h) * dv;
          /* decayed state and the write u */
          for (long e = 0; e < S; ++e) Hd[e] = Hprev[e] * decay;
          for (int c = 0; c < dv; ++c) pv[c] = 0;
          for (int i = 0; i < dk; ++i)
            for (int c = 0; c < dv; ++c) pv[c] += Hd[i * dv + c] * kt[i];
          for (int c = 0; c < dv; ++c) u[c] = b * (vt[c] - pv[c]);
          /* o = scale H^T q */
          for (int i = 0; i < dk; ++i) {
            real acc = 0;
            for (int c = 0; c < dv; ++c) acc += Hcur[i * dv + c] * dot[c];
            dqt[i] += scale * acc;
          }
          for (int i = 0; i < dk; ++i)
            for (int c = 0; c < dv; ++c) dH[i * dv + c] += scale * qt[i] * dot[c];
          /* H = Hd + k u^T */
          for (int c = 0; c < dv; ++c) du[c] = 0;
          for (int i = 0; i < dk; ++i)
            for (int c = 0; c < dv; ++c) du[c] += dH[i * dv + c] * kt[i];
          for (int i = 0; i < dk; ++i) {
            real acc = 0;
            for (int c = 0; c < dv; ++c) acc += dH[i * dv + c] * u[c];
            dkt[i] += acc;
          }
          /* u = b (v - p) */
          real db = 0;
          for (int c = 0; c < dv; ++c) db += du[c] * (vt[c] - pv[c]);
          dbeta[t * Hv + h] = db;
          for (int c = 0; c < dv; ++c) {
            dvt[c] = b * du[c];
            dp[c] = -b * du[c];
          }
          /* p = Hd^T k: dHd = dH + k dp^T; dk += Hd dp */
          for (int i = 0; i < dk; ++i)
            for (int c = 0; c < dv; ++c) dH[i * dv + c] += kt[i] * dp[c];
          for (int i = 0; i < dk; ++i) {
            real acc = 0;
            for (int c = 0; c < dv; ++c) acc += Hd[i * dv + c] * dp[c];
            dkt[i] += acc;
          }
          /* Hd = e^g Hprev */
          real dgt = 0;
          for (long e = 0; e < S; ++e) dgt += dH[e] * Hd[e];
          dg[t * Hv + h] = dgt;
          for (long e = 0; e < S; ++e) dH[e] *= decay;
        }
      }
      if (dh0) memcpy(dh0 + ((long)n * Hv + h) * S, dH, sizeof(real) * S);
    }
    free(ck); free(states); free(H); free(dH); free(Hd);
    free(u); free(pv); free(du); free(dp);
  }
}

/* ---------------------------------------------------------------------------
 * RMSNormGated over each row of d_v values (one row = one token and v-head):
 *   r = (mean(o^2) + eps)^(-1/2);  y = o * r * w * silu(z).
 * ------------------------------------------------------------------------- */
EXPORT void oracle_norm_gate(long rows, int dv, real eps, const real* o, const real* z,
                             const real* w, real* y) {
#pragma omp parallel for schedule(static)
  for (long r = 0; r < rows; ++r) {
    const real* orow = o + r * dv;
    const real* zrow = z + r * dv;
    real ss = 0;
    for (int c = 0; c < dv; ++c) ss += orow[c] * orow[c];
    const real rs = (real)1 / sqrt(ss / dv + eps);
    for (int c = 0; c < dv; ++c) y[r * dv + c] = orow[c] * rs * w[c] * (zrow[c] * sigm(zrow[c]));
  }
}

/* Backward of oracle_norm_gate.  d_o, dz: [rows][d_v]; dw: [d_v], each entry
 * summed over rows in row order. */
EXPORT void oracle_norm_gate_bwd(long rows, int dv, real eps, const real* dy, const real* o,
                                 const real* z, const real* w, real* d_o, real* dz, real* dw) {
  real* rsv = (real*)malloc(sizeof(real) * (rows > 0 ? rows : 1));
#pragma omp parallel for schedule(static)
  for (long r = 0; r < rows; ++r) {
    const real* orow = o + r * dv;
    const real* zrow = z + r * dv;
    const real* dyr = dy + r * dv;
    real ss = 0, ao = 0;
    for (int c = 0; c < dv; ++c) ss += orow[c] * orow[c];
    const real rs = (real)1 / sqrt(ss / dv + eps);
    rsv[r] = rs;
    for (int c = 0; c < dv; ++c) {
      const real sz = zrow[c] * sigm(zrow[c]);
      ao += dyr[c] * w[c] * sz * orow[c];
    }
    ao /= dv;
    for (int c = 0; c < dv; ++c) {
      const real sg = sigm(zrow[c]), sz = zrow[c] * sg;
      const real a = dyr[c] * w[c] * sz;
      d_o[r * dv + c] = rs * (a - orow[c] * rs * rs * ao);
      dz[r * dv + c] = dyr[c] * orow[c] * rs * w[c] * sg * ((real)1 + zrow[c] * ((real)1 - sg));
    }
  }
#pragma omp parallel for schedule(static)
  for (int c = 0; c < dv; ++c) {
    real acc = 0;
    for (long r = 0; r < rows; ++r) {
      const real zz = z[r * dv + c];
      acc += dy[r * dv + c] * o[r * dv + c] * rsv[r] * zz * sigm(zz);
    }
    dw[c] = acc;
  }
  free(rsv);
}

/* ---------------------------------------------------------------------------
 * Gates of the recurrence, per token t and v-head h (page: "[Qwen3.5 MoE] Add
 * hybrid decoder model", Summary: the softplus gate):
 *   g[t,h]    = -exp(A_log[h]) * softplus(a[t,h] + dt_bias[h])   (decay, < 0)
 *   beta[t,h] = sigmoid(b[t,h])                                 (write strength)
 * softplus(x) = log(1 + e^x), written as max(x, 0) + log1p(e^-|x|) so that it
 * neither overflows for large x nor loses the small values for negative x.
 * a, b, g, beta: [T][Hv]; A_log, dt_bias: [Hv].
 * ------------------------------------------------------------------------- */
static real softplus_(real x) { return (x > 0 ? x : (real)0) + log1p(exp(-fabs(x))); }

EXPORT void oracle_gates(long T, int Hv, const real* a, const real* b, const real* A_log,
                         const real* dt_bias, real* g, real* beta) {
  for (long t = 0; t < T; ++t)
    for (int h = 0; h < Hv; ++h) {
      const long e = t * Hv + h;
      g[e] = -exp(A_log[h]) * softplus_(a[e] + dt_bias[h]);
      beta[e] = sigm(b[e]);
    }
}

/* Reverse mode of oracle_gates.  dg, dbeta: [T][Hv] gradients w.r.t. g, beta.
 * d softplus(x)/dx = sigmoid(x);  dg/dA_log = g;  dbeta/db = beta (1 - beta).
 *   da[t,h] = -exp(A_log[h]) sigmoid(a + dt_bias) dg[t,h];   db = beta (1-beta) dbeta
 *   dA_log[h] = sum_t dg[t,h] g[t,h];   ddt_bias[h] = sum_t da[t,h]   (t in order) */
EXPORT void oracle_gates_bwd(long T, int Hv, const real* a, const real* b, const real* A_log,
                             const real* dt_bias, const real* dg, const real* dbeta, real* da,
                             real* db, real* dA_log, real* ddt_bias) {
  for (int h = 0; h < Hv; ++h) {
    dA_log[h] = 0;
    ddt_bias[h] = 0;
  }
  for (long t = 0; t < T; ++t)
    for (int h = 0; h < Hv; ++h) {
      const long e = t * Hv + h;
      const real x = a[e] + dt_bias[h];
      const real gv = -exp(A_log[h]) * softplus_(x);
      const real bv = sigm(b[e]);
      da[e] = -exp(A_log[h]) * sigm(x) * dg[e];
      db[e] = bv * ((real)1 - bv) * dbeta[e];
      dA_log[h] += dg[e] * gv;
      ddt_bias[h] += da[e];
    }
}

EXPORT int oracle_real_bytes(void) { return (int)sizeof(real); }

/* Thread count of the OpenMP loops (the CPU baseline also times one thread). */
EXPORT void oracle_set_threads(int n) {
#if defined(_OPENMP)
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

EXPORT int oracle_threads(void) {
#if defined(_OPENMP)
  return omp_get_max_threads();
#else
  return 1;
#endif
}
