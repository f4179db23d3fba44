/*
 * Host-memory and undefined-behaviour check of the CPU oracle -- TEST
 * INFRASTRUCTURE ONLY.  Built together with gdn_oracle.c under gcc's
 * AddressSanitizer and UndefinedBehaviorSanitizer (tests/test_sanitize.py)
 * and run as a plain program: every entry point of the oracle is called on a
 * small packed row that holds the edge cases of the varlen contract (empty
 * sequences, a single token, a sequence longer than the backward's
 * checkpoint block, a ragged tail) and on an empty row.  A sanitizer report
 * aborts the run; otherwise it prints a checksum of every output and exits 0.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

typedef double real;

void oracle_conv1d(int N, const int32_t* cu, int Cch, int W, int n_qk_ch, int d_k, real eps, const real* x,
                   const real* w, real* y);
void oracle_conv1d_bwd(int N, const int32_t* cu, int Cch, int W, int n_qk_ch, int d_k, real eps, const real* x,
                       const real* w, const real* dy, real* dx, real* dw);
void oracle_recurrence(int N, const int32_t* cu, int Hk, int Hv, int dk, int dv, real scale, const real* q,
                       const real* k, long sqk, const real* v, long sv, const real* g, const real* beta,
                       const real* h0, real* o, real* ht);
void oracle_recurrence_bwd(int N, const int32_t* cu, int Hk, int Hv, int dk, int dv, real scale, const real* q,
                           const real* k, long sqk, const real* v, long sv, const real* g, const real* beta,
                           const real* h0, const real* d_o, const real* dht, real* dq, real* dk_out,
                           real* dv_out, real* dg, real* dbeta, real* dh0);
void oracle_norm_gate(long rows, int dv, real eps, const real* o, const real* z, const real* w, real* y);
void oracle_norm_gate_bwd(long rows, int dv, real eps, const real* dy, const real* o, const real* z,
                          const real* w, real* d_o, real* dz, real* dw);
void oracle_gates(long T, int Hv, const real* a, const real* b, const real* A_log, const real* dt_bias, real* g,
                  real* beta);
void oracle_gates_bwd(long T, int Hv, const real* a, const real* b, const real* A_log, const real* dt_bias,
                      const real* dg, const real* dbeta, real* da, real* db, real* dA_log, real* ddt_bias);

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static real urand(void) { /* xorshift64*, uniform in (-1, 1) */
  rng_state ^= rng_state >> 12;
  rng_state ^= rng_state << 25;
  rng_state ^= rng_state >> 27;
  return (real)((rng_state * 0x2545F4914F6CDD1Dull) >> 11) / (real)(1ull << 53) * 2.0 - 1.0;
}

/* exactly-sized heap buffers, so any overrun is a sanitizer report */
static real* buf(long n, int fill) {
  real* p = (real*)malloc(sizeof(real) * (size_t)(n > 0 ? n : 1));
  for (long i = 0; i < n; ++i) p[i] = fill ? urand() : 0.0;
  return p;
}

static double sum(const real* p, long n) {
  double s = 0;
  for (long i = 0; i < n; ++i) s += fabs(p[i]);
  return s;
}

static int run(int N, const int32_t* cu, int Hk, int Hv, int d, int W) {
  const long T = cu[N], Cch = 2L * Hk * d + (long)Hv * d, S = (long)d * d;
  real *x = buf(T * Cch, 1), *w = buf(Cch * W, 1), *y = buf(T * Cch, 0), *dyc = buf(T * Cch, 1);
  real *dx = buf(T * Cch, 0), *dw = buf(Cch * W, 0);
  oracle_conv1d(N, cu, (int)Cch, W, 2 * Hk * d, d, 1e-6, x, w, y);
  oracle_conv1d_bwd(N, cu, (int)Cch, W, 2 * Hk * d, d, 1e-6, x, w, dyc, dx, dw);
  real *a = buf(T * Hv, 1), *b = buf(T * Hv, 1), *A_log = buf(Hv, 1), *dt = buf(Hv, 1);
  real *g = buf(T * Hv, 0), *beta = buf(T * Hv, 0);
  oracle_gates(T, Hv, a, b, A_log, dt, g, beta);
  real *h0 = buf(N * Hv * S, 1), *o = buf(T * Hv * d, 0), *ht = buf(N * Hv * S, 0);
  /* q, k, v as strided views of the conv output, as the layer passes them */
  oracle_recurrence(N, cu, Hk, Hv, d, d, 1.0, y, y + Hk * d, Cch, y + 2 * Hk * d, Cch, g, beta, h0, o, ht);
  real *d_o = buf(T * Hv * d, 1), *dht = buf(N * Hv * S, 1);
  real *dq = buf(T * Hk * d, 0), *dk = buf(T * Hk * d, 0), *dv = buf(T * Hv * d, 0);
  real *dg = buf(T * Hv, 0), *dbeta = buf(T * Hv, 0), *dh0 = buf(N * Hv * S, 0);
  oracle_recurrence_bwd(N, cu, Hk, Hv, d, d, 0.75, y, y + Hk * d, Cch, y + 2 * Hk * d, Cch, g, beta, h0, d_o, dht,
                        dq, dk, dv, dg, dbeta, dh0);
  oracle_recurrence_bwd(N, cu, Hk, Hv, d, d, 1.0, y, y + Hk * d, Cch, y + 2 * Hk * d, Cch, g, beta, NULL, d_o,
                        NULL, dq, dk, dv, dg, dbeta, NULL);
  real *z = buf(T * Hv * d, 1), *wn = buf(d, 1), *yn = buf(T * Hv * d, 0), *dyn = buf(T * Hv * d, 1);
  real *dz = buf(T * Hv * d, 0), *dwn = buf(d, 0), *do2 = buf(T * Hv * d, 0);
  oracle_norm_gate(T * Hv, d, 1e-6, o, z, wn, yn);
  oracle_norm_gate_bwd(T * Hv, d, 1e-6, dyn, o, z, wn, do2, dz, dwn);
  real *da = buf(T * Hv, 0), *db = buf(T * Hv, 0), *dA = buf(Hv, 0), *ddt = buf(Hv, 0);
  oracle_gates_bwd(T, Hv, a, b, A_log, dt, dg, dbeta, da, db, dA, ddt);
  const double cs = sum(y, T * Cch) + sum(dx, T * Cch) + sum(dw, Cch * W) + sum(o, T * Hv * d) +
                    sum(ht, N * Hv * S) + sum(dq, T * Hk * d) + sum(dk, T * Hk * d) + sum(dv, T * Hv * d) +
                    sum(dg, T * Hv) + sum(dbeta, T * Hv) + sum(yn, T * Hv * d) + sum(dz, T * Hv * d) +
                    sum(dwn, d) + sum(da, T * Hv) + sum(db, T * Hv) + sum(dA, Hv) + sum(ddt, Hv);
  printf("N=%d T=%ld Hk=%d Hv=%d d=%d W=%d checksum=%.6e\n", N, T, Hk, Hv, d, W, cs);
  real* all[] = {x, w, y, dyc, dx, dw, a, b, A_log, dt, g, beta, h0, o, ht, d_o, dht, dq, dk, dv, dg, dbeta, dh0,
                 z, wn, yn, dyn, dz, dwn, do2, da, db, dA, ddt};
  for (size_t i = 0; i < sizeof all / sizeof all[0]; ++i) free(all[i]);
  return isfinite(cs) ? 0 : 1;
}

int main(void) {
  const int32_t cu1[] = {0, 0, 1, 1, 151, 168, 168}; /* empty, one token, 150 (> checkpoint), 17, empty */
  const int32_t cu2[] = {0, 0};                      /* an empty row */
  const int32_t cu3[] = {0, 70};
  int bad = 0;
  bad |= run(6, cu1, 2, 4, 8, 4);
  bad |= run(1, cu2, 1, 2, 16, 4);
  bad |= run(1, cu3, 1, 1, 16, 3);
  return bad;
}
