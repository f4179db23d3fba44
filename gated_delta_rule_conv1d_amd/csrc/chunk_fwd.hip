// Chunked gated delta rule: chunk index, per-chunk WY preparation, and the
// serial inter-chunk state pass (forward).
//
// Pages: "[Qwen3.5 MoE] Add hybrid decoder model", Summary (GatedDeltaNet
// linear attention; FLA kernels optional); "Support Qwen35 SFT", XTuner changes
// (GatedDeltaNet varlen mode); "feat(models): dense Qwen3.5 custom attention",
// Summary (cu_seqlens from position_ids; one packed row).
//
// Per chunk (rows r, s; gamma = within-chunk cumulative gate, Gam = e^gamma,
// D_rs = e^{gamma_r - gamma_s} for r >= s, H = S^T entering the chunk):
//   A  = strict_lower(diag(beta) (D * K K^T)),   T = (I + A)^-1
//   U  = T diag(beta) V,   Wk = T diag(beta Gam) K,   W = U - Wk H
//   O  = scale (diag(Gam) Q H + lower_incl(D * Q K^T) W)
//   H' = Gam_last H + K^T diag(e^{gamma_last - gamma}) W
// which is the token recurrence re-associated exactly.  Only non-positive
// differences gamma_r - gamma_s (r >= s) are ever exponentiated; the mask is
// applied before the exponential.
#include <cstddef>

#include "chunk_common.cuh"
#include "profile.h"

namespace gdn {

// ---------------------------------------------------------------------------
// Chunk index: one workgroup scans the per-sequence chunk counts, then fills
// the table for every slot below the max_chunks bound.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void chunk_index_kernel(const int32_t* __restrict__ cu, int N, int C,
                                                           int max_chunks, int32_t* __restrict__ table,
                                                           int32_t* __restrict__ seq_chunk0) {
  __shared__ int scan[1024];
  __shared__ int base_s;
  const int tid = threadIdx.x;
  if (tid == 0) base_s = 0;
  __syncthreads();
  for (int n0 = 0; n0 < N; n0 += 1024) {
    const int n = n0 + tid;
    const int cnt = n < N ? (cu[n + 1] - cu[n] + C - 1) / C : 0;
    scan[tid] = cnt;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
      const int add = tid >= off ? scan[tid - off] : 0;
      __syncthreads();
      scan[tid] += add;
      __syncthreads();
    }
    const int base = base_s;
    if (n < N) seq_chunk0[n] = base + scan[tid] - cnt;
    __syncthreads();
    if (tid == 0) base_s = base + scan[1023];
    __syncthreads();
  }
  const int n_chunks = base_s;
  if (tid == 0) seq_chunk0[N] = n_chunks;
  __syncthreads();
  for (int c = tid; c < max_chunks; c += 1024) {
    int4 ent = make_int4(-1, 0, 0, 0);
    if (c < n_chunks) {
      int lo = 0, hi = N - 1;  // last n with seq_chunk0[n] <= c
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (seq_chunk0[mid] <= c) lo = mid; else hi = mid - 1;
      }
      const int tok0 = cu[lo] + (c - seq_chunk0[lo]) * C;
      ent = make_int4(lo, tok0, min(C, cu[lo + 1] - tok0), 0);
    }
    reinterpret_cast<int4*>(table)[c] = ent;
  }
}

// ---------------------------------------------------------------------------
// WY preparation, persistent workgroups walking (chunk, k-head) items, each
// looping over the k-head's v-heads.  K K^T and Q K^T on MFMA (operand type E),
// the unit-lower triangular inverse in fp32 (16x16 diagonal blocks by per-lane
// forward substitution, off-diagonal blocks by block substitution on fp32
// MFMA), U and Wk on MFMA.  At bf16, d = 128, chunk 64 the outputs only the
// state passes read leave in the order those passes load them.
// ---------------------------------------------------------------------------
template <typename E, int D, int C, bool LO_OUT, int NTH, bool F8 = false>
__global__ __launch_bounds__(NTH) void prep_kernel(ChunkArgs a) {
  constexpr int NW = NTH / kWave;
  using S = PrepSmem<E, D, C>;
  __shared__ S sm;
  constexpr int V = Vec<E>::N;
  constexpr int NT = C / 16, ND = D / 16;
  // Wk, K^T, U (and P of the inference forward) in the state passes' load
  // order at the shapes those passes serve
  constexpr bool FRAG = use_wide_state<E, D, C>();
  const int tid = threadIdx.x, w = wave_id(), lane = lane_id();
  // Persistent: the workgroup walks items (chunk, k-head) = (it / Hk, it % Hk)
  // from blockIdx.x in steps of gridDim.x, and requests the next item's q, k
  // rows, first v rows and gates while the current item finishes, so that no
  // item starts on a cold global round trip.  Padding chunks past the last
  // one end the table, so the first of them ends the walk.
  const int n_items = a.max_chunks * a.Hk;
  auto item_entry = [&](int it) { return it < n_items ? chunk_entry(a.table, it / a.Hk) : make_int4(-1, 0, 0, 0); };
  TileRegs<E, C, D, NTH, true> pV;  // a v-head's v rows; rows first: written transposed
  TileRegs<E, C, D, NTH> rQ;
  TileRegs<E, C, D, NTH, true> rK;  // rows first: also written transposed
  // wave 0: this lane's raw gate inputs (g or a; beta or b) and the head's
  // A_log and dt_bias (fused gates), finished where the v-head starts
  float gx = 0.f, bx = 0.f, gA = 0.f, gdt = 0.f;
  // The next v-head's v rows and gate inputs, and at an item's last v-head
  // the next item's q and k rows: every path issues the same loads, and what
  // it does not need (q and k within an item, gates outside wave 0, anything
  // past the last item) reads through a zero-size buffer (zeros, no memory
  // access).  Loads issued on some paths only make the compiler join register
  // copies that wait for them at once.  F8: q, k, v arrive as e4m3 bytes and
  // are decoded on load (exactly: the registers then hold the bf16 tile of the
  // dequantised inputs).
  auto load_next = [&](bool item_start, int tok, int n, int jj, int hh) {
    const int nqk = item_start ? n : 0;
    if constexpr (F8) {
      rQ.load_f8((const uint8_t*)a.q + (int64_t)tok * a.sqk + (int64_t)jj * D, a.sqk, nqk, a.f8_scale[0]);
      rK.load_f8((const uint8_t*)a.k + (int64_t)tok * a.sqk + (int64_t)jj * D, a.sqk, nqk, a.f8_scale[1]);
      pV.load_f8((const uint8_t*)a.v + (int64_t)tok * a.sv + (int64_t)hh * D, a.sv, n, a.f8_scale[2]);
    } else {
      rQ.load((const E*)a.q + (int64_t)tok * a.sqk + (int64_t)jj * D, a.sqk, nqk);
      rK.load((const E*)a.k + (int64_t)tok * a.sqk + (int64_t)jj * D, a.sqk, nqk);
      pV.load((const E*)a.v + (int64_t)tok * a.sv + (int64_t)hh * D, a.sv, n);
    }
    // token tok + lane's value at lane * Hv floats; the wave index made
    // visibly uniform, so the buffer's size stays a scalar
    const int ng = __builtin_amdgcn_readfirstlane(w) == 0 ? n : 0;
    const int gbytes = ng > 0 ? ((ng - 1) * a.Hv + 1) * 4 : 0;
    const int64_t o = (int64_t)tok * a.Hv + hh;
    gx = buf_load_f32((a.ga ? a.ga : a.g) + o, gbytes, lane * a.Hv * 4);
    bx = buf_load_f32((a.gb ? a.gb : a.beta) + o, gbytes, lane * a.Hv * 4);
    const int hbytes = a.ga && ng > 0 ? 4 : 0;
    gA = buf_load_f32(a.ga ? a.A_log + hh : nullptr, hbytes, 0);
    gdt = buf_load_f32(a.ga ? a.dt_bias + hh : nullptr, hbytes, 0);
  };
  int item = blockIdx.x;
  int4 ent = item_entry(item);
  load_next(true, ent.y, ent.x >= 0 ? ent.z : 0, item % a.Hk, (item % a.Hk) * a.G);
  while (ent.x >= 0) {
    const int ci = item / a.Hk, j = item % a.Hk;
    const int tok0 = ent.y, len = ent.z;
    const int next = item + (int)gridDim.x;
    const int4 nent = item_entry(next);
    rQ.store(&sm.Qs[0][0], S::LDQ);
    rK.store(&sm.Ks[0][0], S::LDQ);
    rK.template store_t<E>(&sm.Kt[0][0], S::LDCE);
    __syncthreads();
    if constexpr (FRAG) {
      // K^T (plain: the same for every v-head of the k-head) once per item,
      // in fragment order, for the state passes (zero past len)
      E* Kg = (E*)a.Kt + ((int64_t)ci * a.Hk + j) * D * C;
      for_strided<D * C / 8, NTH>(tid, [&](int e) {
        const int f = e >> 6, l = e & 63;
        *reinterpret_cast<uint4*>(Kg + e * 8) =
            *reinterpret_cast<const uint4*>(&sm.Kt[(f / (C / 32)) * 16 + (l & 15)][(f % (C / 32)) * 32 + (l >> 4) * 8]);
      });
    }
    if constexpr (FRAG && !LO_OUT && !F8) {
      if (a.q_frag) {  // q rows in fragment order for the state pass (zero past len)
        E* Qg = (E*)a.Qf + ((int64_t)ci * a.Hk + j) * C * D;
        for_strided<C * D / 8, NTH>(tid, [&](int e) {
          const int f = e >> 6, l = e & 63;
          *reinterpret_cast<uint4*>(Qg + e * 8) =
              *reinterpret_cast<const uint4*>(&sm.Qs[(f / (D / 32)) * 16 + (l & 15)][(f % (D / 32)) * 32 + (l >> 4) * 8]);
        });
      }
    }
    for (int t = w; t < NT * NT; t += NW) {
      const int rt = t / NT, ct = t % NT;
      const f32x4 acc = mm_tile<E, D>(zero4(), &sm.Ks[rt * 16][0], S::LDQ, &sm.Ks[ct * 16][0], S::LDQ);
#pragma unroll
      for (int e = 0; e < 4; ++e) sm.Sk[rt * 16 + acc_row(e)][ct * 16 + acc_col()] = acc[e];
    }
    __syncthreads();

    for (int gi = 0; gi < a.G; ++gi) {
      const int h = j * a.G + gi;
      const int64_t slot = (int64_t)ci * a.Hv + h;
      if (w == 0) {  // within-chunk cumulative gate
        float x = chunk_g_fin(a, GateRaw{gx, gA, gdt});
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) {
          const float y = __shfl_up(x, off, kWave);
          if (lane >= off) x += y;
        }
        if (lane < C) {
          sm.gam[lane] = x;
          sm.beta[lane] = chunk_beta_fin(a, bx);
          a.gam[slot * C + lane] = x;
        }
      }
      pV.template store_t<E>(&sm.Vt[0][0], S::LDCE);  // V^T
      {  // in flight during this v-head: its next v-head, or the next item
        const bool last = gi + 1 == a.G;
        const int nj = next % a.Hk;
        load_next(last, last ? nent.y : tok0, last ? (nent.x >= 0 ? nent.z : 0) : len, nj, last ? nj * a.G : h + 1);
      }
      __syncthreads();

      // P = lower_incl(D * Q K^T) (fp32 to workspace), A = strict_lower(beta_r D * K K^T)
      {
        float* Pg = a.P + slot * C * C;
        for_strided<NT * NT, NW>(w, [&](int t) {
          const int rt = t / NT, ct = t % NT;
          if constexpr (LO_OUT) {  // P tiles: P^T also leaves, as 4-element runs
            const f32x4 acc = mm_tile<E, D>(zero4(), &sm.Qs[rt * 16][0], S::LDQ, &sm.Ks[ct * 16][0], S::LDQ);
            f32x4 pv;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int r = rt * 16 + acc_row(e), s = ct * 16 + acc_col();
              const float dd = (s <= r) ? __expf(sm.gam[r] - sm.gam[s]) : 0.f;
              pv[e] = (r < len) ? dd * acc[e] : 0.f;
              sm.Am[r][s] = (s < r) ? sm.beta[r] * dd * sm.Sk[r][s] : 0.f;
            }
            store_tile<float>(Pg, C, rt * 16, ct * 16, pv, C);
            // (the whole-state reverse pass, kt_plain, gathers P^T from P itself)
            if (!a.kt_plain) store_tile_t(a.Ptr + slot * C * C, C, rt * 16, ct * 16, pv);
          } else {  // P^T = K Q^T tiles: a lane holds P[r][s..s+3] (one 16-byte store) and the same piece of A
            const f32x4 acc = mm_tile<E, D>(zero4(), &sm.Ks[ct * 16][0], S::LDQ, &sm.Qs[rt * 16][0], S::LDQ);
            const int r = rt * 16 + acc_col(), s0 = ct * 16 + acc_row(0);
            f32x4 pv, av;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int s = s0 + e;
              const float dd = (s <= r) ? __expf(sm.gam[r] - sm.gam[s]) : 0.f;
              pv[e] = (r < len) ? dd * acc[e] : 0.f;
              av[e] = (s < r) ? sm.beta[r] * dd * sm.Sk[r][s] : 0.f;
            }
            *reinterpret_cast<float4*>(&sm.Am[r][s0]) = make_float4(av[0], av[1], av[2], av[3]);
            st4<float>(Pg + (FRAG ? pf_off(r, s0, C) : r * C + s0), pv);
          }
        });
      }
      __syncthreads();
      // Outputs that need only gamma, K and Q (K~^T hi / lo; for the backward
      // also the K~ rows and (Gam q)^T): written by waves 1.. while wave 0 runs
      // the diagonal solve of the inverse
      auto gate_outputs = [&](int t0, int nt) {
        // Kt_e[d][s] = e^{gamma_last - gamma_s} k_s[d]  (s < len), 0 past len;
        // with kt_plain the unscaled k_s[d] (exact: no lo part)
        if (!FRAG) {  // (FRAG: written once per item above)
          E* Kg = (E*)a.Kt + slot * D * C;
          const float glast = sm.gam[len - 1];
          const bool plain = a.kt_plain;
          for (int e = t0; e < D * (C / V); e += nt) {
            const int d = e / (C / V), s0 = (e % (C / V)) * V;
            float val[V], lo[V];
#pragma unroll
            for (int i = 0; i < V; ++i) {
              const int s = s0 + i;
              const float es = plain ? 1.f : __expf(glast - sm.gam[s]);
              val[i] = (s < len) ? to_f<E>(sm.Kt[d][s]) * es : 0.f;
              lo[i] = val[i] - to_f<E>(from_f<E>(val[i]));
            }
            Vec<E>::store(Kg + d * C + s0, val);
            if constexpr (Split<E>::on)
              if (!plain) Vec<E>::store((E*)a.Ktl + slot * D * C + d * C + s0, lo);
          }
          // rows e_s k_s [C][D] and (Gam_r q_r)^T [D][C], hi / lo, for the
          // reverse state pass (the whole-state pass, kt_plain, reads k and q
          // and forms them itself)
          if (LO_OUT && !plain) {
            for (int e = t0; e < C * (D / V); e += nt) {
              const int s = e / (D / V), c0 = (e % (D / V)) * V;
              const float es = (s < len) ? __expf(glast - sm.gam[s]) : 0.f;
              float val[V], lo[V];
#pragma unroll
              for (int i = 0; i < V; ++i) {
                val[i] = es * to_f<E>(sm.Ks[s][c0 + i]);
                lo[i] = val[i] - to_f<E>(from_f<E>(val[i]));
              }
              const int64_t o = slot * C * D + (int64_t)s * D + c0;
              Vec<E>::store((E*)a.Krh + o, val);
              if constexpr (Split<E>::on) Vec<E>::store((E*)a.Krl + o, lo);
            }
            // Q^T through V x V register blocks: a thread reads V rows of V
            // consecutive d and writes V rows of Q^T; adjacent lanes take adjacent
            // d blocks (conflict-free LDS reads), and the C / V lanes sharing a d
            // block write whole rows of Q^T
            constexpr int DB = D / V, SB = C / V, DF = DB >= 8 ? 8 : DB;
            for (int e = t0; e < DB * SB; e += nt) {
              const int d0 = (e % DF + DF * (e / (DF * SB))) * V, s0 = ((e / DF) % SB) * V;
              float blk[V][V], gs[V];
#pragma unroll
              for (int i = 0; i < V; ++i) {
                Vec<E>::load(&sm.Qs[s0 + i][d0], blk[i]);
                gs[i] = __expf(sm.gam[s0 + i]);
              }
#pragma unroll
              for (int dd = 0; dd < V; ++dd) {
                float val[V], lo[V];
#pragma unroll
                for (int i = 0; i < V; ++i) {
                  val[i] = gs[i] * blk[i][dd];
                  lo[i] = val[i] - to_f<E>(from_f<E>(val[i]));
                }
                const int64_t o = slot * D * C + (int64_t)(d0 + dd) * C + s0;
                Vec<E>::store((E*)a.Qth + o, val);
                if constexpr (Split<E>::on) Vec<E>::store((E*)a.Qtl + o, lo);
              }
            }
          }
        }
      };
      unit_lower_inverse<C, S::LDCF, NTH>(sm.Am, sm.Tm, sm.Tt, sm.Xs, gate_outputs);  // ends with a barrier
      if constexpr (LO_OUT) {  // T for the WY gradients
        for_strided<C * (C / 4), NTH>(tid, [&](int e) {
          const int r = e / (C / 4), c = (e % (C / 4)) * 4;
          *reinterpret_cast<float4*>(a.Tw + slot * C * C + r * C + c) = *reinterpret_cast<const float4*>(&sm.Tm[r][c]);
        });
      }

      // U = (T diag(beta)) V and Wk = (T diag(beta Gam)) K, their left factors
      // split into hi + lo parts in one pass (the Wk factor in the LDS of A and
      // T^T, which the inverse no longer needs), then both products' tiles in
      // one phase; fp32 results
      E (*const TB2)[S::LDCE] = reinterpret_cast<E (*)[S::LDCE]>(&sm.Am[0][0]);
      E (*const TB2l)[S::LDCE] = reinterpret_cast<E (*)[S::LDCE]>(&sm.Tt[0][0]);
      static_assert(sizeof(E) * S::LDCE <= sizeof(float) * S::LDCF, "the Wk factor fits A's rows");
      static_assert(offsetof(S, gam) % 16 == 0 && offsetof(S, beta) % 16 == 0, "16-byte gate reads");
      for_strided<C * C / 4, NTH>(tid, [&](int e) {  // 4 consecutive s per step: 16-byte reads, 8-byte writes
        const int r = e / (C / 4), s = (e % (C / 4)) * 4;
        const float4 t4 = *reinterpret_cast<const float4*>(&sm.Tm[r][s]);
        const float4 b4 = *reinterpret_cast<const float4*>(&sm.beta[s]);
        const float4 g4 = *reinterpret_cast<const float4*>(&sm.gam[s]);
        const f32x4 tb = {t4.x * b4.x, t4.y * b4.y, t4.z * b4.z, t4.w * b4.w};
        const f32x4 tb2 = {tb[0] * __expf(g4.x), tb[1] * __expf(g4.y), tb[2] * __expf(g4.z), tb[3] * __expf(g4.w)};
        st4_split<E>(&sm.TB[r][s], &sm.TBl[0][0] + r * S::LDCE + s, tb);
        st4_split<E>(&TB2[r][s], &TB2l[r][s], tb2);
      });
      __syncthreads();
      auto u_tile = [&](int t) {
        float* Ug = a.U + slot * C * D;
        if constexpr (FRAG) {  // U tiles, each lane's 4 values one 16-byte write in accumulator order
          const int rt = t / ND, dt = t % ND;
          f32x4 acc = mm_tile<E, C>(zero4(), &sm.TB[rt * 16][0], S::LDCE, &sm.Vt[dt * 16][0], S::LDCE);
          if constexpr (Split<E>::on)
            acc = mm_tile<E, C>(acc, &sm.TBl[rt * 16][0], S::LDCE, &sm.Vt[dt * 16][0], S::LDCE);
          st4<float>(Ug + (t * 64 + lane) * 4, acc);
        } else {
          // formed as U^T = V^T (T diag(beta))^T tiles: a lane then holds 4
          // consecutive d of one row of U, stored as one 16-byte write
          const int dt = t / NT, rt = t % NT;
          f32x4 acc = mm_tile<E, C>(zero4(), &sm.Vt[dt * 16][0], S::LDCE, &sm.TB[rt * 16][0], S::LDCE);
          if constexpr (Split<E>::on)
            acc = mm_tile<E, C>(acc, &sm.Vt[dt * 16][0], S::LDCE, &sm.TBl[rt * 16][0], S::LDCE);
          st4<float>(Ug + (int64_t)(rt * 16 + acc_col()) * D + dt * 16 + acc_row(0), acc);
        }
      };
      auto wk_tile = [&](int t) {
        E* Wg = (E*)a.Wk + slot * C * D;
        if constexpr (LO_OUT) {  // Wk tiles: Wk^T [D][C] (hi / lo) leaves as 4-element runs
          const int rt = t / ND, ct = t % ND;
          f32x4 acc = mm_tile<E, C>(zero4(), &TB2[rt * 16][0], S::LDCE, &sm.Kt[ct * 16][0], S::LDCE);
          if constexpr (Split<E>::on)
            acc = mm_tile<E, C>(acc, &TB2l[rt * 16][0], S::LDCE, &sm.Kt[ct * 16][0], S::LDCE);
          if constexpr (FRAG) {
#pragma unroll
            for (int e = 0; e < 4; ++e) Wg[af_off(rt * 16 + acc_row(e), ct * 16 + acc_col(), D)] = from_f<E>(acc[e]);
          } else {
            store_tile<E>(Wg, D, rt * 16, ct * 16, acc, C);
          }
          const int64_t o = slot * D * C + (int64_t)(ct * 16 + acc_col()) * C + rt * 16 + acc_row(0);
          st4_split<E>((E*)a.Wth + o, (E*)a.Wtl + o, acc);
        } else {  // Wk^T = K^T (T diag(beta Gam))^T tiles: 4 consecutive d of a Wk row per lane
          const int dt = t / NT, rt = t % NT;
          f32x4 acc = mm_tile<E, C>(zero4(), &sm.Kt[dt * 16][0], S::LDCE, &TB2[rt * 16][0], S::LDCE);
          if constexpr (Split<E>::on)
            acc = mm_tile<E, C>(acc, &sm.Kt[dt * 16][0], S::LDCE, &TB2l[rt * 16][0], S::LDCE);
          const int r = rt * 16 + acc_col(), d0 = dt * 16 + acc_row(0);
          st4<E>(Wg + (FRAG ? af_off(r, d0, D) : r * D + d0), acc);
        }
      };
      for_strided<NT * ND, NW>(w, u_tile);
      for_strided<NT * ND, NW>(w, wk_tile);
      __syncthreads();
    }
    item = next;
    ent = nent;
  }
}

// ---------------------------------------------------------------------------
// Inter-chunk state pass, one workgroup per (sequence, v-head, dv tile of DVT
// columns).  The state tile H [D][DVT] stays in registers (fp32) for the whole
// sequence; each chunk stages Wk, Kt_e (and Q, P for the output) in LDS, and
// H^T / W^T as bf16 MFMA operands.  Dv tiles are independent: the update acts
// on the state by left multiplication only.
//   OUT   = true : writes o and the final state ht
//   OUT   = false: writes, per chunk, the entering state Hc and W (for the
//                  backward pass), and the final state if asked
// ---------------------------------------------------------------------------
template <typename E, int D, int C, int DVT, int MODE>
__global__ __launch_bounds__(kChunkThreads) void state_fwd_kernel(ChunkArgs a) {
  constexpr bool OUT = MODE & kFwdOut, STORE = MODE & kFwdStore;
  using S = StateSmem<E, D, C, DVT, OUT>;
  __shared__ S sm;
  constexpr bool LO = Split<E>::on;
  constexpr bool KL = LO;  // Kt has a lo part
  constexpr int NVT = D / DVT;
  constexpr int NCT = DVT / 16;                 // column tiles
  constexpr int NHT = (D / 16) * NCT;           // state tiles
  constexpr int NHW = (NHT + kChunkWaves - 1) / kChunkWaves;
  constexpr int NWT = (C / 16) * NCT;           // W / O tiles
  constexpr int NWW = (NWT + kChunkWaves - 1) / kChunkWaves;
  int n, h, vt;
  if (!state_block(blockIdx.x, a.N, a.Hk, a.G, NVT, n, h, vt)) return;
  const int j = h / a.G;
  const int w = wave_id();
  const int col0 = vt * DVT;

  f32x4 Hr[NHW];
#pragma unroll
  for (int i = 0; i < NHW; ++i) {
    const int t = w + kChunkWaves * i;
    Hr[i] = zero4();
    if (t < NHT && a.h0) {
      const int rt = t / NCT, ct = t % NCT;
      const float* src = a.h0 + ((int64_t)n * a.Hv + h) * D * D;
#pragma unroll
      for (int e = 0; e < 4; ++e) Hr[i][e] = src[(rt * 16 + acc_row(e)) * D + col0 + ct * 16 + acc_col()];
    }
  }
  // H^T as the B operand of the next chunk's products, hi + lo parts
  auto write_Ht = [&]() {
#pragma unroll
    for (int i = 0; i < NHW; ++i) {
      const int t = w + kChunkWaves * i;
      if (t < NHT) {
        const int rt = t / NCT, ct = t % NCT;
        const int c = ct * 16 + acc_col(), r = rt * 16 + acc_row(0);
        st4_split<E>(&sm.Ht[c][r], &sm.Htl[0][0] + c * S::LDQ + r, Hr[i]);
      }
    }
  };

  // next chunk's tiles, staged in registers (guarded loads: see TileRegs::load_each)
  constexpr int TN = kChunkThreads;
  TileRegs<E, C, D, TN, false, false> pWk;
  TileRegs<E, D, C, TN, false, false> pKt;
  TileRegs<E, KL ? D : 1, KL ? C : 16 / (int)sizeof(E), TN, false, false> pKtl;
  TileRegs<E, OUT ? C : 16, OUT ? D : 16 / (int)sizeof(E), TN, false, false> pQ;
  TileRegs<float, OUT ? C : 1, OUT ? C : 4, TN, false, false> pP;
  TileRegs<float, C, DVT, TN, false, false> pU;
  TileRegs<float, 1, C, TN, false, false> pG;
  // the sequence's chunks are consecutive table entries: (first token, length)
  // follow from cu_seqlens, so no table load sits in front of the Q load
  // the sequence's bounds as scalars (buffer sizes formed from them stay uniform)
  const int c0 = __builtin_amdgcn_readfirstlane(a.seq_chunk0[n]);
  const int c1 = __builtin_amdgcn_readfirstlane(a.seq_chunk0[n + 1]);
  const int s0 = __builtin_amdgcn_readfirstlane(a.cu[n]), s1 = __builtin_amdgcn_readfirstlane(a.cu[n + 1]);
  int ptok = 0, plen = 0;
  auto prefetch = [&](int ci) {
    ptok = s0 + (ci - c0) * C;
    plen = min(C, s1 - ptok);
    const int64_t slot = (int64_t)ci * a.Hv + h;
    pWk.load((const E*)a.Wk + slot * C * D, D, C);
    pKt.load((const E*)a.Kt + slot * D * C, C, D);
    if constexpr (KL) pKtl.load((const E*)a.Ktl + slot * D * C, C, D);
    if constexpr (OUT) {
      pQ.load((const E*)a.q + (int64_t)ptok * a.sqk + (int64_t)j * D, a.sqk, plen);
      pP.load(a.P + slot * C * C, C, C);
    }
    pU.load(a.U + slot * C * D + col0, D, C);
    pG.load(a.gam + slot * C, C, 1);
  };

  if (c0 < c1) prefetch(c0);
  write_Ht();
  for (int ci = c0; ci < c1; ++ci) {
    const int tok0 = ptok, len = plen;
    const int64_t slot = (int64_t)ci * a.Hv + h;
    __syncthreads();  // the previous chunk is done with the LDS tiles
    pWk.store(&sm.Wk[0][0], S::LDQ);
    pKt.store(&sm.Kt[0][0], S::LDCE);
    if constexpr (KL) pKtl.store(&sm.Ktl[0][0], S::LDCE);
    if constexpr (OUT) {
      pQ.store(&sm.Q[0][0], S::LDQ);
      pP.template store_split<E>(&sm.P[0][0], &sm.Pl[0][0], S::LDCE);
    }
    pU.store(&sm.U[0][0], S::LDU);
    pG.store(&sm.gam[0], C);
    if constexpr (STORE) {
      // state entering this chunk, for the backward pass
      float* Hg = a.Hc + slot * D * D;
#pragma unroll
      for (int i = 0; i < NHW; ++i) {
        const int t = w + kChunkWaves * i;
        if (t < NHT) store_tile<float>(Hg, D, (t / NCT) * 16, col0 + (t % NCT) * 16, Hr[i], D);
      }
    }
    __syncthreads();
    if (ci + 1 < c1) prefetch(ci + 1);  // in flight during this chunk's compute

    f32x4 Or[NWW];
#pragma unroll
    for (int i = 0; i < NWW; ++i) {
      const int t = w + kChunkWaves * i;
      Or[i] = zero4();
      if (t < NWT) {
        const int rt = t / NCT, ct = t % NCT;
        f32x4 x = mm_tile<E, D>(zero4(), &sm.Wk[rt * 16][0], S::LDQ, &sm.Ht[ct * 16][0], S::LDQ);
        if constexpr (LO) x = mm_tile<E, D>(x, &sm.Wk[rt * 16][0], S::LDQ, &sm.Htl[ct * 16][0], S::LDQ);
        f32x4 wv;
#pragma unroll
        for (int e = 0; e < 4; ++e) wv[e] = sm.U[rt * 16 + acc_row(e)][ct * 16 + acc_col()] - x[e];
        {
          const int c = ct * 16 + acc_col(), r = rt * 16 + acc_row(0);
          st4_split<E>(&sm.Wt[c][r], &sm.Wtl[0][0] + c * S::LDCE + r, wv);
        }
        if constexpr (STORE) store_tile<float>(a.W + slot * C * D, D, rt * 16, col0 + ct * 16, wv, C);
        if constexpr (OUT) {
          f32x4 xo = mm_tile<E, D>(zero4(), &sm.Q[rt * 16][0], S::LDQ, &sm.Ht[ct * 16][0], S::LDQ);
          if constexpr (LO) xo = mm_tile<E, D>(xo, &sm.Q[rt * 16][0], S::LDQ, &sm.Htl[ct * 16][0], S::LDQ);
#pragma unroll
          for (int e = 0; e < 4; ++e) Or[i][e] = __expf(sm.gam[rt * 16 + acc_row(e)]) * xo[e];
        }
      }
    }
    __syncthreads();

    const float gl = __expf(sm.gam[len - 1]);
#pragma unroll
    for (int i = 0; i < NHW; ++i) {
      const int t = w + kChunkWaves * i;
      if (t < NHT) {
        const int rt = t / NCT, ct = t % NCT;
        f32x4 y = mm_tile<E, C>(zero4(), &sm.Kt[rt * 16][0], S::LDCE, &sm.Wt[ct * 16][0], S::LDCE);
        if constexpr (LO) {
          y = mm_tile<E, C>(y, &sm.Kt[rt * 16][0], S::LDCE, &sm.Wtl[ct * 16][0], S::LDCE);
          y = mm_tile<E, C>(y, &sm.Ktl[rt * 16][0], S::LDCE, &sm.Wt[ct * 16][0], S::LDCE);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) Hr[i][e] = gl * Hr[i][e] + y[e];
      }
    }
    if constexpr (OUT) {
      E* og = (E*)a.o + (int64_t)tok0 * a.Hv * D + (int64_t)h * D + col0;
#pragma unroll
      for (int i = 0; i < NWW; ++i) {
        const int t = w + kChunkWaves * i;
        if (t < NWT) {
          const int rt = t / NCT, ct = t % NCT;
          f32x4 y = mm_tile<E, C>(zero4(), &sm.P[rt * 16][0], S::LDCE, &sm.Wt[ct * 16][0], S::LDCE);
          if constexpr (LO) {
            y = mm_tile<E, C>(y, &sm.P[rt * 16][0], S::LDCE, &sm.Wtl[ct * 16][0], S::LDCE);
            y = mm_tile<E, C>(y, &sm.Pl[rt * 16][0], S::LDCE, &sm.Wt[ct * 16][0], S::LDCE);
          }
          f32x4 ov;
#pragma unroll
          for (int e = 0; e < 4; ++e) ov[e] = a.scale * (Or[i][e] + y[e]);
          store_tile<E>(og, (int64_t)a.Hv * D, rt * 16, ct * 16, ov, len);
        }
      }
    }
    write_Ht();  // phase 1 (the only reader of Ht) is over for every wave
  }
  if (a.ht) {
    float* dst = a.ht + ((int64_t)n * a.Hv + h) * D * D;
#pragma unroll
    for (int i = 0; i < NHW; ++i) {
      const int t = w + kChunkWaves * i;
      if (t < NHT) {
        const int rt = t / NCT, ct = t % NCT;
#pragma unroll
        for (int e = 0; e < 4; ++e) dst[(rt * 16 + acc_row(e)) * D + col0 + ct * 16 + acc_col()] = Hr[i][e];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
int64_t max_chunks(const gdn_shape* s) {
  return ((int64_t)s->total_tokens + s->chunk - 1) / s->chunk + s->n_seqs;
}

void run_chunk_index(const gdn_shape* s, const int32_t* cu, int32_t* table, int32_t* seq_chunk0, hipStream_t st) {
  GDN_PROF("chunk_index", st);
  chunk_index_kernel<<<1, 1024, 0, st>>>(cu, s->n_seqs, s->chunk, (int)max_chunks(s), table, seq_chunk0);
}

template <typename E, int D>
constexpr int state_dvt() { return D >= 32 ? 32 : D; }

// The one-workgroup-per-(sequence, v-head) state pass runs one serial chain of
// chunk steps per workgroup; with fewer chains than compute units most of the
// chip idles (a single long sequence has only Hv of them).  The state's dv
// columns are independent (the update multiplies it from the left only), so
// it can be split:
//  - at most 64 chains: 16-column tiles, eight 256-thread workgroups per chain
//    that read their operand rows straight into matrix-core fragments
//    (state_wide.hip; one 65536-token sequence at d = 128: 8.0 ms with whole
//    states, 2.8 ms with LDS-staged 16-column tiles, 2.15 ms now);
//  - two workgroups per chain with 64 columns each (the whole-state pass
//    halved, with the same arithmetic per element, so the same bits): when
//    there are fewer chains than CUs, and for inference up to four chains per
//    CU, where the shorter serial steps outweigh the doubled staging (dense
//    4 x 2048: 0.28 -> 0.20 ms; varlen 32768: 0.94 -> 0.80 ms); the passes
//    that also store H_c and W are bandwidth-bound from one chain per CU on
//    (training 8 x 8192: 1.64 ms whole, 2.01 ms halved);
//  - otherwise one workgroup per chain, the whole state.
// The 16-column choice must not depend on the mode (it changes the order of
// the sums, and the saved training pair and the recomputing backward must see
// the same H_c and W bits); the halving may.  Returns the column count per
// workgroup.
inline int state_columns(const ChunkArgs& a, int D, int mode) {
  const int chains = a.N * a.Hv;
  if (chains * 4 <= kNumCUs) return 16;
  return chains < (mode == kFwdOut ? 4 * kNumCUs : kNumCUs) ? D / 2 : D;
}

template <typename E, int D, int C, int DVT>
static void launch_state_fwd_tiled(const ChunkArgs& a, hipStream_t st, int mode) {
  const dim3 grid(state_grid(a.N, a.Hk, a.G, D / DVT));
  if (mode == kFwdOut) state_fwd_kernel<E, D, C, DVT, kFwdOut><<<grid, kChunkThreads, 0, st>>>(a);
  else if (mode == kFwdStore) state_fwd_kernel<E, D, C, DVT, kFwdStore><<<grid, kChunkThreads, 0, st>>>(a);
  else state_fwd_kernel<E, D, C, DVT, kFwdBoth><<<grid, kChunkThreads, 0, st>>>(a);
}

template <typename E, int D, int C, bool F8>
void launch_chunk_fwd_core(const ChunkArgs& args, hipStream_t st, int mode) {
  static_assert(!F8 || use_wide_state<E, D, C>(), "fp8 inputs: bf16, d = 128, chunk 64");
  constexpr int DVT = state_dvt<E, D>();
  // The state passes at bf16, d = 128, chunk 64 read the plain K^T (exact in
  // bf16) and apply the decay to W's rows: no K lo part to write, load or
  // multiply per chunk step.
  const int nc = use_wide_state<E, D, C>() ? state_columns(args, D, mode) : DVT;
  ChunkArgs a = args;
  a.kt_plain = use_wide_state<E, D, C>();
  // The 16-column pass (few chains) is bound by its operand loads, which are
  // fastest as 1 KB of consecutive bytes per instruction: the preparation
  // then also writes q in that order (long 65536: state pass 1.72 -> 1.53 ms
  // for 0.05 ms more preparation; the whole-state passes read q themselves).
  a.q_frag = use_wide_state<E, D, C>() && !F8 && mode == kFwdOut && nc == 16;
  static const char* prep_name[4] = {"", "chunk_prep", "chunk_prep_bwd", "chunk_prep_save"};
  // the timing record names the state-pass variant that ran (whole or half
  // state per workgroup, or the column tile of the tiled pass)
  static const char* state_name[4][4] = {
      {"", "", "", ""},
      {"chunk_state_fwd:wide128", "chunk_state_fwd:wide64", "chunk_state_fwd:tiled16", "chunk_state_fwd:tiled32"},
      {"chunk_state_store:wide128", "chunk_state_store:wide64", "chunk_state_store:tiled16",
       "chunk_state_store:tiled32"},
      {"chunk_state_save:wide128", "chunk_state_save:wide64", "chunk_state_save:tiled16",
       "chunk_state_save:tiled32"}};
  const int variant = nc == 16 ? 2 : (use_wide_state<E, D, C>() ? (nc < D ? 1 : 0) : (DVT == 16 ? 2 : 3));
  // The preparation runs persistent: as many workgroups as fit at once (its
  // LDS use allows one per CU at d = 128, chunk 64), each walking its share of
  // items with the next one's loads in flight (long 65536: 1.69 -> 1.60 ms;
  // varlen: 0.87 -> 0.83 ms; the training workload's saving form 1.79 -> 1.68
  // ms since the reverse pass forms its transposed operands itself; when that
  // form still wrote them, one item per workgroup was faster).
  constexpr int per_cu = (160 * 1024) / (int)sizeof(PrepSmem<E, D, C>) >= 2 ? 2 : 1;
  const int64_t items = (int64_t)a.max_chunks * a.Hk;
  const int64_t resident = (int64_t)kNumCUs * per_cu;
  dim3 gprep((unsigned)(items > resident ? resident : items));
  {
    GDN_PROF(prep_name[mode], st);
    constexpr int NTH = D >= 64 ? 512 : kChunkThreads;  // 8 waves for the wide heads
    if constexpr (F8) prep_kernel<E, D, C, false, NTH, true><<<gprep, NTH, 0, st>>>(a);
    else if (mode == kFwdOut) prep_kernel<E, D, C, false, NTH><<<gprep, NTH, 0, st>>>(a);
    else prep_kernel<E, D, C, true, NTH><<<gprep, NTH, 0, st>>>(a);
  }
  GDN_PROF(state_name[mode][variant], st);
  if constexpr (use_wide_state<E, D, C>()) {
    if (nc == 16) launch_state_fwd_cols(a, st, mode, F8);
    else launch_state_fwd_wide(a, st, mode, nc < D, F8);
  } else {
    launch_state_fwd_tiled<E, D, C, DVT>(a, st, mode);  // reads K~^T in hi + lo
  }
}

// explicit instantiation helpers used by the dispatcher in chunk_bwd.hip
#define GDN_INST_FWD(E, D, C) template void launch_chunk_fwd_core<E, D, C, false>(const ChunkArgs&, hipStream_t, int);
template void launch_chunk_fwd_core<bf16, 128, 64, true>(const ChunkArgs&, hipStream_t, int);
GDN_INST_FWD(bf16, 16, 16) GDN_INST_FWD(bf16, 16, 32) GDN_INST_FWD(bf16, 16, 64)
GDN_INST_FWD(bf16, 32, 16) GDN_INST_FWD(bf16, 32, 32) GDN_INST_FWD(bf16, 32, 64)
GDN_INST_FWD(bf16, 64, 16) GDN_INST_FWD(bf16, 64, 32) GDN_INST_FWD(bf16, 64, 64)
GDN_INST_FWD(bf16, 128, 16) GDN_INST_FWD(bf16, 128, 32) GDN_INST_FWD(bf16, 128, 64)
GDN_INST_FWD(float, 16, 16) GDN_INST_FWD(float, 16, 32)
GDN_INST_FWD(float, 32, 16) GDN_INST_FWD(float, 32, 32)
GDN_INST_FWD(float, 64, 16) GDN_INST_FWD(float, 64, 32)
GDN_INST_FWD(float, 128, 16) GDN_INST_FWD(float, 128, 32)
#undef GDN_INST_FWD

}  // namespace gdn
