// Chunked gated delta rule, reverse mode, and the forward/backward dispatch.
//
// Pages: "[Qwen3.5 MoE] Add hybrid decoder model", Summary (GatedDeltaNet);
// "Support Qwen35 SFT", feature list (training with the layer).
//
// With H the state entering a chunk, dHn the gradient w.r.t. the state
// leaving it, dO' = scale * dO, K~ = diag(e) K (e_s = e^{gamma_last - gamma_s}):
//   dW  = P^T dO' + K~ dHn                      (state pass, reversed)
//   dH  = Gam_last dHn + (diag(Gam) Q)^T dO' - Wk^T dW
//   dWk = -dW H^T,  dT = dW (diag(beta) V)^T + dWk (diag(beta Gam) K)^T
//   dXu = T^T dW,  dXw = T^T dWk,  dA = strict_lower(-T^T dT T^T)
//   dV  = diag(beta) dXu
//   dS  = lower_incl(dO' W^T) * D
//   dQ  = diag(Gam) dO' H^T + dS K
//   dK  = diag(e) W dHn^T + diag(beta Gam) dXw + dS^T Q + A~ K + A~^T K,
//         A~ = dA * beta_r D_rs
//   dbeta_r = <dXu_r, v_r> + Gam_r <dXw_r, k_r> + sum_s dA_rs D_rs k_r.k_s
//   dgamma_r = <dQs_r, q_r> - <dKhn_r, k_r> + beta_r Gam_r <dXw_r, k_r>
//            + rows(dP*P) - cols(dP*P) + rows(dA*A) - cols(dA*A)
//   dgamma_last += Gam_last <H, dHn> + sum_r <dKhn_r, k_r>
//   dg_s = sum_{r >= s} dgamma_r   (within the chunk)
// Every sum has a fixed order; no floating-point atomics.
#include "chunk_common.cuh"
#include "profile.h"

namespace gdn {

template <typename E, int D, int C, bool F8 = false>
void launch_chunk_fwd_core(const ChunkArgs& a, hipStream_t st, int mode);

// ---------------------------------------------------------------------------
// Reverse state pass, one workgroup per (sequence, v-head, dv tile).
// fp32 operands that decide the result (P, Gam q, dW, dH) enter the bf16
// MFMAs as hi + lo parts; dO, Wk and K~ are used as stored.
// ---------------------------------------------------------------------------
template <typename E, int D, int C, int DVT>
struct StateBwdSmem {
  static constexpr int LO = Split<E>::on ? 1 : 0;
  static constexpr int LDQ = D + Pad<E>::E16;
  static constexpr int LDCE = C + Pad<E>::E16;
  static constexpr int LD2C = 2 * C + Pad<E>::E16;
  E Pt[C][LDCE];
  E Ptl[LO ? C : 1][LDCE];
  E Ktil[C][LDQ];
  E Ktill[LO ? C : 1][LDQ];  // lo part of K~
  E QW[D][LD2C];             // [ (Gam q)^T | Wk^T ]
  E Qlo[LO ? D : 1][LDCE];   // lo part of (Gam q)^T
  E Wklo[LO ? D : 1][LDCE];  // lo part of Wk^T
  E OW[DVT][LD2C];           // [ dO^T | dW^T ]
  E dWlo[LO ? DVT : 1][LDCE];
  E dHt[DVT][LDQ];
  E dHtl[LO ? DVT : 1][LDQ];
  float gam[C];
  float Gm[C];
};

template <typename E, int D, int C, int DVT>
__global__ __launch_bounds__(kChunkThreads) void state_bwd_kernel(ChunkArgs a) {
  using S = StateBwdSmem<E, D, C, DVT>;
  __shared__ S sm;
  constexpr bool LO = Split<E>::on;
  constexpr int NVT = D / DVT;
  constexpr int NCT = DVT / 16;
  constexpr int NHT = (D / 16) * NCT;
  constexpr int NHW = (NHT + kChunkWaves - 1) / kChunkWaves;
  constexpr int NWT = (C / 16) * NCT;
  int n, h, vt;
  if (!state_block(blockIdx.x, a.N, a.Hk, a.G, NVT, n, h, vt)) return;
  const int j = h / a.G;
  const int w = wave_id();
  const int col0 = vt * DVT;

  f32x4 dH[NHW];
#pragma unroll
  for (int i = 0; i < NHW; ++i) {
    const int t = w + kChunkWaves * i;
    dH[i] = zero4();
    if (t < NHT && a.dht) {
      const int rt = t / NCT, ct = t % NCT;
      const float* src = a.dht + ((int64_t)n * a.Hv + h) * D * D;
#pragma unroll
      for (int e = 0; e < 4; ++e) dH[i][e] = src[(rt * 16 + acc_row(e)) * D + col0 + ct * 16 + acc_col()];
    }
  }
  auto write_dHt = [&]() {
#pragma unroll
    for (int i = 0; i < NHW; ++i) {
      const int t = w + kChunkWaves * i;
      if (t < NHT) {
        const int rt = t / NCT, ct = t % NCT;
        const int c = ct * 16 + acc_col(), r = rt * 16 + acc_row(0);
        st4_split<E>(&sm.dHt[c][r], &sm.dHtl[0][0] + c * S::LDQ + r, dH[i]);
      }
    }
  };

  // next chunk's tiles, staged in registers (all pre-transposed by the
  // preparation pass except dO, which is gathered column-wise)
  TileRegs<float, C, C> pP;
  TileRegs<E, C, D> pKh, pKl;
  TileRegs<E, D, C> pWh, pWl, pQh, pQl;
  ColRegs<E, C, DVT> pO;
  TileRegs<float, 1, C> pG;
  // (first token, length) of chunk ci from cu_seqlens: no table load in front of the dO load
  // the sequence's bounds as scalars (buffer sizes formed from them stay uniform)
  const int c0 = __builtin_amdgcn_readfirstlane(a.seq_chunk0[n]);
  const int c1 = __builtin_amdgcn_readfirstlane(a.seq_chunk0[n + 1]);
  const int s0 = __builtin_amdgcn_readfirstlane(a.cu[n]), s1 = __builtin_amdgcn_readfirstlane(a.cu[n + 1]);
  int plen = 0;
  auto prefetch = [&](int ci) {
    const int tok0 = s0 + (ci - c0) * C;
    plen = min(C, s1 - tok0);
    const int64_t slot = (int64_t)ci * a.Hv + h;
    pP.load(a.Ptr + slot * C * C, C, C);
    pKh.load((const E*)a.Krh + slot * C * D, D, C);
    pWh.load((const E*)a.Wth + slot * D * C, C, D);
    pQh.load((const E*)a.Qth + slot * D * C, C, D);
    if constexpr (LO) {
      pKl.load((const E*)a.Krl + slot * C * D, D, C);
      pWl.load((const E*)a.Wtl + slot * D * C, C, D);
      pQl.load((const E*)a.Qtl + slot * D * C, C, D);
    }
    pO.load((const E*)a.d_o + (int64_t)tok0 * a.Hv * D + (int64_t)h * D + col0, (int64_t)a.Hv * D, plen);
    pG.load(a.gam + slot * C, C, 1);
  };

  if (c0 < c1) prefetch(c1 - 1);
  write_dHt();
  for (int ci = c1 - 1; ci >= c0; --ci) {
    const int len = plen;
    const int64_t slot = (int64_t)ci * a.Hv + h;
    __syncthreads();  // the previous chunk is done with the LDS tiles
    pP.template store_split<E>(&sm.Pt[0][0], LO ? &sm.Ptl[0][0] : nullptr, S::LDCE);
    pKh.store(&sm.Ktil[0][0], S::LDQ);
    pWh.store(&sm.QW[0][C], S::LD2C);
    pQh.store(&sm.QW[0][0], S::LD2C);
    if constexpr (LO) {
      pKl.store(&sm.Ktill[0][0], S::LDQ);
      pWl.store(&sm.Wklo[0][0], S::LDCE);
      pQl.store(&sm.Qlo[0][0], S::LDCE);
    }
    pO.store(&sm.OW[0][0], S::LD2C);
    pG.store(&sm.gam[0], C);
    {  // gradient w.r.t. the state leaving this chunk
      float* dst = a.dHn + slot * D * D;
#pragma unroll
      for (int i = 0; i < NHW; ++i) {
        const int t = w + kChunkWaves * i;
        if (t < NHT) store_tile<float>(dst, D, (t / NCT) * 16, col0 + (t % NCT) * 16, dH[i], D);
      }
    }
    __syncthreads();
    if (ci > c0) prefetch(ci - 1);  // in flight during this chunk's compute

    float* dWg = a.dW + slot * C * D;
    float* dWtg = a.dWt + slot * D * C;
    for (int t = w; t < NWT; t += kChunkWaves) {
      const int rt = t / NCT, ct = t % NCT;
      f32x4 p = mm_tile<E, C>(zero4(), &sm.Pt[rt * 16][0], S::LDCE, &sm.OW[ct * 16][0], S::LD2C);
      if constexpr (LO) p = mm_tile<E, C>(p, &sm.Ptl[rt * 16][0], S::LDCE, &sm.OW[ct * 16][0], S::LD2C);
      f32x4 kd = mm_tile<E, D>(zero4(), &sm.Ktil[rt * 16][0], S::LDQ, &sm.dHt[ct * 16][0], S::LDQ);
      if constexpr (LO) {
        kd = mm_tile<E, D>(kd, &sm.Ktil[rt * 16][0], S::LDQ, &sm.dHtl[ct * 16][0], S::LDQ);
        kd = mm_tile<E, D>(kd, &sm.Ktill[rt * 16][0], S::LDQ, &sm.dHt[ct * 16][0], S::LDQ);
      }
      f32x4 acc;
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] = a.scale * p[e] + kd[e];
      store_tile<float>(dWg, D, rt * 16, col0 + ct * 16, acc, C);
      store_tile_t(dWtg, C, rt * 16, col0 + ct * 16, acc);
      {
        const int c = ct * 16 + acc_col(), r = rt * 16 + acc_row(0);
        st4_split<E>(&sm.OW[c][C + r], &sm.dWlo[0][0] + c * S::LDCE + r, acc);
      }
    }
    __syncthreads();
    const float gl = __expf(sm.gam[len - 1]);
#pragma unroll
    for (int i = 0; i < NHW; ++i) {
      const int t = w + kChunkWaves * i;
      if (t < NHT) {
        const int rt = t / NCT, ct = t % NCT;
        f32x4 y1 = mm_tile<E, C>(zero4(), &sm.QW[rt * 16][0], S::LD2C, &sm.OW[ct * 16][0], S::LD2C);
        if constexpr (LO) y1 = mm_tile<E, C>(y1, &sm.Qlo[rt * 16][0], S::LDCE, &sm.OW[ct * 16][0], S::LD2C);
        f32x4 y2 = mm_tile<E, C>(zero4(), &sm.QW[rt * 16][C], S::LD2C, &sm.OW[ct * 16][C], S::LD2C);
        if constexpr (LO) {
          y2 = mm_tile<E, C>(y2, &sm.QW[rt * 16][C], S::LD2C, &sm.dWlo[ct * 16][0], S::LDCE);
          y2 = mm_tile<E, C>(y2, &sm.Wklo[rt * 16][0], S::LDCE, &sm.OW[ct * 16][C], S::LD2C);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) dH[i][e] = gl * dH[i][e] + a.scale * y1[e] - y2[e];
      }
    }
    write_dHt();  // the dW pass (the only reader of dHt) is over for every wave
  }
  if (a.dh0) {
    float* dst = a.dh0 + ((int64_t)n * a.Hv + h) * D * D;
#pragma unroll
    for (int i = 0; i < NHW; ++i) {
      const int t = w + kChunkWaves * i;
      if (t < NHT) {
        const int rt = t / NCT, ct = t % NCT;
#pragma unroll
        for (int e = 0; e < 4; ++e) dst[(rt * 16 + acc_row(e)) * D + col0 + ct * 16 + acc_col()] = dH[i][e];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Every contraction over d_v, one workgroup per (chunk, v-head), from operands
// staged in LDS (fp32 ones as hi + lo bf16):
//   dQs = scale diag(Gam) dO Hc^T        dWk = -dW Hc^T  (stored transposed)
//   dT  = dW (diag(beta) V)^T + dWk (diag(beta Gam) K)^T
//   dKh = diag(e) W dHn^T                dP  = scale dO W^T (lower-incl., rows < len)
//   hdot = <Hc, dHn>
// ---------------------------------------------------------------------------
template <typename E, int D, int C, int NTH>
struct GradASmem {
  static constexpr int LO = Split<E>::on ? 1 : 0;
  static constexpr int LDQ = D + Pad<E>::E16;
  static constexpr bool K_IN_HL = LO && D >= C;  // K's C rows fit the lo half of the H region
  E Hh[D][LDQ];                 // Hc, then dHn (hi)
  E Hl[LO ? D : 1][LDQ];        // lo parts; K while the H region is between uses (K_IN_HL)
  E Od[C][LDQ];                 // dO (read in (a) and (d))
  E Os[C][LDQ];                 // dWk hi
  E Xh[C][LDQ];                 // dW, then W (hi)
  E Xl[LO ? C : 1][LDQ];        // lo parts
  E Vs[C][LDQ];                 // V, then dWk lo
  E Ks[K_IN_HL ? 1 : C][LDQ];   // K, where it does not fit the H region
  float bs[C], gm[C], em[C];
  float red[NTH];
};

template <typename E, int D, int C, int NTH>
__global__ __launch_bounds__(NTH) void grad_a_kernel(ChunkArgs a) {
  using S = GradASmem<E, D, C, NTH>;
  __shared__ S sm;
  constexpr bool LO = Split<E>::on;
  constexpr int NT = C / 16, ND = D / 16;
  constexpr int NW = NTH / kWave;
  constexpr int RT = NT >= 2 ? 2 : 1;                           // block rows (C side)
  constexpr int CD = ND >= 4 ? (NW > kChunkWaves ? 2 : 4) : ND;  // block cols on the D side
  constexpr int CC = NT >= 2 && NW <= kChunkWaves ? 2 : 1;      // block cols on the C side
  const int ci = blockIdx.x, h = blockIdx.y;
  const int4 ent = chunk_entry(a.table, ci);
  if (ent.x < 0) return;
  const int tok0 = ent.y, len = ent.z;
  const int j = h / a.G;
  const int tid = threadIdx.x;
  const int64_t slot = (int64_t)ci * a.Hv + h;
  const float* Hc = a.Hc + slot * D * D;
  const float* dHn = a.dHn + slot * D * D;
  const E* dog = (const E*)a.d_o + (int64_t)tok0 * a.Hv * D + (int64_t)h * D;
  const int64_t ldo = (int64_t)a.Hv * D;
  E* Hlo = LO ? &sm.Hl[0][0] : nullptr;
  E* Xlo = LO ? &sm.Xl[0][0] : nullptr;
  E* Kst = S::K_IN_HL ? &sm.Hl[0][0] : &sm.Ks[0][0];

  // dHn (read after (a)) and K (for (c)) are requested with the first tiles
  using DRegs = TileRegs<float, D, D, NTH>;
  DRegs rD;
  TileRegs<E, C, D, NTH> rK;
  {  // stage Hc, dO, dW, V
    TileRegs<float, D, D, NTH> rH;
    TileRegs<E, C, D, NTH> rO, rV;
    TileRegs<float, C, D, NTH> rW;
    // the whole-state reverse pass writes dW^T only: its rows are staged transposed here
    constexpr bool DW_T = use_wide_state<E, D, C>();
    TileRegs<float, D, C, NTH, true> rWt;
    rH.load(Hc, D, D);
    rO.load(dog, ldo, len);
    if constexpr (DW_T) rWt.load(a.dWt + slot * D * C, C, D);
    else rW.load(a.dW + slot * C * D, D, C);
    rV.load((const E*)a.v + (int64_t)tok0 * a.sv + (int64_t)h * D, a.sv, len);
    rD.load(dHn, D, D);
    rK.load((const E*)a.k + (int64_t)tok0 * a.sqk + (int64_t)j * D, a.sqk, len);
    rH.template store_split<E>(&sm.Hh[0][0], Hlo, S::LDQ);
    rO.store(&sm.Od[0][0], S::LDQ);
    if constexpr (DW_T) rWt.template store_t<E>(&sm.Xh[0][0], S::LDQ, Xlo, S::LDQ);
    else rW.template store_split<E>(&sm.Xh[0][0], Xlo, S::LDQ);
    rV.store(&sm.Vs[0][0], S::LDQ);
  }
  if (tid < C) {  // per-row gates; every load unconditional (clamped rows), so they issue together
    const int e = tid;
    const float g = a.gam[slot * C + e];
    const float gl = a.gam[slot * C + len - 1];
    const float bt = chunk_beta_fin(a, chunk_beta_raw(a, tok0 + min(e, len - 1), h));
    sm.bs[e] = e < len ? bt : 0.f;
    sm.gm[e] = __expf(g);
    sm.em[e] = e < len ? __expf(gl - g) : 0.f;
  }
  __syncthreads();

  // (a) dQs = scale Gam dO Hc^T (to workspace); dT1 = dW V^T kept for (c)
  // dQs^T tiles [D][C] (the layout the WY-gradient kernel accumulates in)
  for_blocks<ND, NT, CD, RT, NW>([&](int d0, int r0) {
    f32x4 acc[CD][RT];
    zero_blk(acc);
    mm_blk<E, D, CD, RT, LO, false>(acc, &sm.Hh[d0 * 16][0], LO ? &sm.Hl[d0 * 16][0] : nullptr, S::LDQ,
                                    &sm.Od[r0 * 16][0], nullptr, S::LDQ);
#pragma unroll
    for (int i = 0; i < CD; ++i)
#pragma unroll
      for (int jj = 0; jj < RT; ++jj) {
        const float sc = a.scale * sm.gm[(r0 + jj) * 16 + acc_col()];
        f32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = sc * acc[i][jj][e];
        store_acc(a.dQs + slot * C * D, NT, d0 + i, r0 + jj, v);
      }
  });
  constexpr int NBT = (NT / RT) * (NT / CC);
  constexpr int NBW = (NBT + NW - 1) / NW;
  f32x4 dT1[NBW][RT][CC];
#pragma unroll
  for (int bi = 0; bi < NBW; ++bi) {
    zero_blk(dT1[bi]);
    const int b = wave_id() + bi * NW;
    if (b < NBT) {
      const int r0 = (b / (NT / CC)) * RT, c0 = (b % (NT / CC)) * CC;
      mm_blk<E, D, RT, CC, LO, false>(dT1[bi], &sm.Xh[r0 * 16][0], LO ? &sm.Xl[r0 * 16][0] : nullptr, S::LDQ,
                                      &sm.Vs[c0 * 16][0], nullptr, S::LDQ);
    }
  }
  __syncthreads();  // dO and V are no longer read

  // <Hc, dHn> is formed from the staged parts of Hc (hi + lo, exact in fp32
  // mode) before they are overwritten, so Hc is read from HBM once

  // (b) dWk = -dW Hc^T: hi -> Os, lo -> Vs; transposed fp32 copy to workspace
  for_blocks<NT, ND, RT, CD, NW>([&](int r0, int c0) {
    f32x4 acc[RT][CD];
    zero_blk(acc);
    mm_blk<E, D, RT, CD, LO, LO>(acc, &sm.Xh[r0 * 16][0], LO ? &sm.Xl[r0 * 16][0] : nullptr, S::LDQ,
                                 &sm.Hh[c0 * 16][0], LO ? &sm.Hl[c0 * 16][0] : nullptr, S::LDQ);
#pragma unroll
    for (int i = 0; i < RT; ++i)
#pragma unroll
      for (int jj = 0; jj < CD; ++jj) {
        f32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[e] = -acc[i][jj][e];
          const int r = (r0 + i) * 16 + acc_row(e), c = (c0 + jj) * 16 + acc_col();
          split_store<E>(&sm.Os[r][c], &sm.Vs[r][c], v[e]);
        }
        store_tile_t(a.dWkt + slot * D * C, C, (r0 + i) * 16, (c0 + jj) * 16, v);
      }
  });
  {
    float hs = 0.f;
#pragma unroll
    for (int i = 0; i < DRegs::N; ++i) {
      const int e = tid + i * NTH;
      if (e < DRegs::TOTAL) {
        const int row = e / DRegs::PER_ROW, c = (e % DRegs::PER_ROW) * DRegs::V;
        const float* x = reinterpret_cast<const float*>(&rD.r[i]);
#pragma unroll
        for (int u = 0; u < DRegs::V; ++u) {
          float hc = to_f<E>(sm.Hh[row][c + u]);
          if constexpr (LO) hc += to_f<E>(sm.Hl[row][c + u]);
          hs += x[u] * hc;
        }
      }
    }
    sm.red[tid] = hs;
  }
  __syncthreads();  // Hc is no longer read
  rK.store(Kst, S::LDQ);
  __syncthreads();
  TileRegs<float, C, D, NTH> rW2;  // W for (d): in flight during (c)
  rW2.load(a.W + slot * C * D, D, C);

  // (c) dT = beta_s dT1 + beta_s Gam_s dWk K^T
#pragma unroll
  for (int bi = 0; bi < NBW; ++bi) {
    const int b = wave_id() + bi * NW;
    if (b < NBT) {
      const int r0 = (b / (NT / CC)) * RT, c0 = (b % (NT / CC)) * CC;
      f32x4 acc[RT][CC];
      zero_blk(acc);
      mm_blk<E, D, RT, CC, LO, false>(acc, &sm.Os[r0 * 16][0], LO ? &sm.Vs[r0 * 16][0] : nullptr, S::LDQ,
                                      Kst + c0 * 16 * S::LDQ, nullptr, S::LDQ);
#pragma unroll
      for (int i = 0; i < RT; ++i)
#pragma unroll
        for (int jj = 0; jj < CC; ++jj) {
          const int s = (c0 + jj) * 16 + acc_col();
          const float bsv = sm.bs[s], bg = bsv * sm.gm[s];
#pragma unroll
          for (int e = 0; e < 4; ++e)
            a.dT[slot * C * C + ((r0 + i) * 16 + acc_row(e)) * C + s] = bsv * dT1[bi][i][jj][e] + bg * acc[i][jj][e];
        }
    }
  }
  __syncthreads();  // dWk and K are no longer read

  // stage dHn, W (dO is still staged)
  rD.template store_split<E>(&sm.Hh[0][0], Hlo, S::LDQ);
  rW2.template store_split<E>(&sm.Xh[0][0], Xlo, S::LDQ);
  __syncthreads();
  if (wave_id() == 0) {  // <Hc, dHn>: the per-thread partials summed lane-strided, then across the wave
    float s = 0.f;
    for (int i = lane_id(); i < NTH; i += kWave) s += sm.red[i];
    s = wave_sum(s);
    if (lane_id() == 0) a.hdot[slot] = s;
  }
  // (d) dKh = e W dHn^T (as dKh^T tiles [D][C]);  dP = scale dO W^T
  for_blocks<ND, NT, CD, RT, NW>([&](int d0, int r0) {
    f32x4 acc[CD][RT];
    zero_blk(acc);
    mm_blk<E, D, CD, RT, LO, LO>(acc, &sm.Hh[d0 * 16][0], LO ? &sm.Hl[d0 * 16][0] : nullptr, S::LDQ,
                                 &sm.Xh[r0 * 16][0], LO ? &sm.Xl[r0 * 16][0] : nullptr, S::LDQ);
#pragma unroll
    for (int i = 0; i < CD; ++i)
#pragma unroll
      for (int jj = 0; jj < RT; ++jj) {
        const float sc = sm.em[(r0 + jj) * 16 + acc_col()];
        f32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = sc * acc[i][jj][e];
        store_acc(a.dKh + slot * C * D, NT, d0 + i, r0 + jj, v);
      }
  });
  for_blocks<NT, NT, RT, CC, NW>([&](int r0, int c0) {
    f32x4 acc[RT][CC];
    zero_blk(acc);
    mm_blk<E, D, RT, CC, false, LO>(acc, &sm.Od[r0 * 16][0], nullptr, S::LDQ, &sm.Xh[c0 * 16][0],
                                    LO ? &sm.Xl[c0 * 16][0] : nullptr, S::LDQ);
#pragma unroll
    for (int i = 0; i < RT; ++i)
#pragma unroll
      for (int jj = 0; jj < CC; ++jj) {
        f32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = (r0 + i) * 16 + acc_row(e), c = (c0 + jj) * 16 + acc_col();
          v[e] = (c <= r && r < len) ? a.scale * acc[i][jj][e] : 0.f;
        }
        store_tile<float>(a.dP + slot * C * C, C, (r0 + i) * 16, (c0 + jj) * 16, v, C);
      }
  });
}

// ---------------------------------------------------------------------------
// WY-representation gradients, one workgroup per (chunk, k-head), looping
// over the k-head's v-heads; dq and dk accumulate in registers across them.
// Every operand is staged in LDS first (fp32 ones split on the fly into bf16
// hi + lo MFMA parts); K K^T is formed once per k-head.
// ---------------------------------------------------------------------------
// Workgroup size of the WY-gradient kernel: 8 waves where the tiles give each
// wave an r-tile and a d-strip of its own.
template <int D, int C>
constexpr int gb_threads() { return (D >= 64 && C >= 64) ? 2 * kChunkThreads : kChunkThreads; }
// Row partial sums over d: one slot per (wave along d, lane group of 16).
template <int D, int C>
constexpr int gb_slots() {
  constexpr int NWD = gb_threads<D, C>() / kWave / (C / 16), ND = D / 16;
  return (ND >= NWD ? NWD : ND) * 4;
}

template <typename E, int D, int C>
struct GradBSmem {
  static constexpr int LD2C = 2 * C + Pad<E>::E16;
  static constexpr int LDCE = C + Pad<E>::E16;
  static constexpr int LDCF = C + 4;
  static constexpr int NT = C / 16, ND = D / 16;
  static constexpr int LDV = D + Pad<E>::E16;
  E QKt[D][LD2C];      // [Q^T | K^T]
  float Skk[C][LDCF];  // K K^T
  union {
    float Am[C][LDCF];  // A (solve), later dA
    E Vs[C][LDV];       // v rows, between the two
  } av;
  union {
    struct {
      float Tm[C][LDCF];  // T, later P
      union {
        struct {
          E TtH[C][LDCE];  // T^T as MFMA operand parts (hi, lo)
          E TtL[Split<E>::on ? C : 1][LDCE];
        };
        float dPm[C][LDCF];  // dP', after T^T
      };
    };
    struct {
      E h[C][LD2C];
      E l[Split<E>::on ? C : 1][LD2C];
    } TS;  // [dS^T | A~ + A~^T] rows, hi + lo, after the C x C pass
  };
  union U {
    struct { E h[D][LDCE]; E l[Split<E>::on ? D : 1][LDCE]; } x;  // dW^T or dWk^T (hi, lo)
    struct { float dT[C][LDCF]; E M1h[C][LDCE]; E M1l[Split<E>::on ? C : 1][LDCE]; } m;  // dT, (dT T^T)^T
    struct { E dSh[C][LDCE]; E dSl[Split<E>::on ? C : 1][LDCE]; float At[C][LDCF]; } s;  // dS (hi, lo), A~
  } r;
  float gam[C], beta[C], Gm[C], em[C];
  float hdot;            // <H_c, dH_n> of the current v-head
  static constexpr int NPD = gb_slots<D, C>();
  float pCD[4][NPD][C];  // row partials over d: dXu.v, dXw.k, dQs.q, dKh.k
  float pCC[5][NT][C];   // dA D Skk rows, dA*A rows, dA*A cols, dP*P rows, dP*P cols
};

template <typename E, int D, int C, int NTH>
__global__ __launch_bounds__(NTH) void grad_b_kernel(ChunkArgs a) {
  using S = GradBSmem<E, D, C>;
  using M = Mma<E>;
  constexpr int KPL = M::KPL;
  constexpr bool LO = Split<E>::on;
  __shared__ S sm;
  constexpr int NT = S::NT, ND = S::ND;
  constexpr int NW = NTH / kWave;
  static_assert(NTH == gb_threads<D, C>(), "launch size");
  // The [C][D] results (dv, dq, dk and the row sums over d) are formed as
  // transposed [D][C] accumulator tiles, so a lane holds 4 consecutive d of
  // one chunk row r.  Each wave owns one r-tile and DT adjacent d-tiles: row
  // sums over d stay in-lane, one partial per (wave along d, lane group);
  // waves past the d-tiles idle.
  static_assert(NT <= NW, "one r-tile per wave");
  constexpr int NWR = NT, NWD = NW / NWR;         // waves along r / along d
  constexpr int DT = ND >= NWD ? ND / NWD : 1;   // d-tiles per wave
  const int w = wave_id(), lane = lane_id(), tid = threadIdx.x;
  const int rt = w % NWR, dt0 = (w / NWR) * DT;
  const bool act = dt0 < ND;
  const int pslot = (w / NWR) * 4 + (lane >> 4);  // this lane's row partial slot
  const int rrow = rt * 16 + (lane & 15);         // chunk row of this lane's accumulator column
  const int dl = 4 * (lane >> 4);                 // first of its 4 rows within a d-tile
  // Persistent: the workgroup walks items (chunk, k-head) = (it / Hk, it % Hk)
  // from blockIdx.x in steps of gridDim.x and requests the next item's q and k
  // rows before the current item's dq and dk leave, so that no item starts on
  // a cold round trip.  Padding chunks past the last one only zero their
  // shares of the gate sums.
  const int n_items = a.max_chunks * a.Hk;
  auto item_entry = [&](int it) {
    int4 e = it < n_items ? chunk_entry(a.table, it / a.Hk) : make_int4(-1, 0, 0, 0);
    // scalars: the buffer sizes formed from them stay scalar
    e.x = __builtin_amdgcn_readfirstlane(e.x);
    e.y = __builtin_amdgcn_readfirstlane(e.y);
    e.z = __builtin_amdgcn_readfirstlane(e.z);
    return e;
  };
  TileRegs<E, C, D, NTH, true> rq, rk;  // an item's q and k rows, requested one item ahead
  auto load_qk = [&](int it, int4 e) {   // zero-size reads for padding chunks and past the last item
    const int n = e.x >= 0 ? e.z : 0, tok = e.x >= 0 ? e.y : 0, jj = it % a.Hk;
    rq.load((const E*)a.q + (int64_t)tok * a.sqk + (int64_t)jj * D, a.sqk, n);
    rk.load((const E*)a.k + (int64_t)tok * a.sqk + (int64_t)jj * D, a.sqk, n);
  };
  int4 ent = item_entry(blockIdx.x);
  load_qk(blockIdx.x, ent);
  for (int it = blockIdx.x; it < n_items; it += gridDim.x) {
    const int ci = it / a.Hk, j = it % a.Hk;
    const int next = it + (int)gridDim.x;
    const int4 nent = item_entry(next);
    if (ent.x < 0) {  // padding entry past the last chunk: its shares of the gate sums are zero
      if (a.da)
        for (int i = threadIdx.x; i < a.G; i += NTH) {
          a.gpart[(int64_t)ci * a.Hv + j * a.G + i] = 0.f;
          a.gpart[((int64_t)a.max_chunks + ci) * a.Hv + j * a.G + i] = 0.f;
        }
      load_qk(next, nent);
      ent = nent;
      continue;
    }
    const int tok0 = ent.y, len = ent.z;
    // q and k rows, written transposed to LDS (every wave passed the previous
    // item's last barrier after its last read of them)
    rq.store_t_raw(&sm.QKt[0][0], S::LD2C);
    rk.store_t_raw(&sm.QKt[0][C], S::LD2C);
    __syncthreads();
    // K K^T (exact bf16 products, fp32 sums), shared by the k-head's v-heads
    for (int t = w; t < NT * NT; t += NW) {
      const int rt = t / NT, ct = t % NT;
      const f32x4 skk = mm_gen<E, D, false, false>(
          zero4(),
          [&](int r, int k, float* o) {
#pragma unroll
            for (int u = 0; u < KPL; ++u) o[u] = to_f<E>(sm.QKt[k + u][C + rt * 16 + r]);
          },
          [&](int c, int k, float* o) {
#pragma unroll
            for (int u = 0; u < KPL; ++u) o[u] = to_f<E>(sm.QKt[k + u][C + ct * 16 + c]);
          });
#pragma unroll
      for (int e = 0; e < 4; ++e) sm.Skk[rt * 16 + acc_row(e)][ct * 16 + acc_col()] = skk[e];
    }

    f32x4 dQ[DT][1], dK[DT][1];
    zero_blk(dQ);
    zero_blk(dK);

    for (int gi = 0; gi < a.G; ++gi) {
      const int h = j * a.G + gi;
      const int64_t slot = (int64_t)ci * a.Hv + h;
      const E* vg = (const E*)a.v + (int64_t)tok0 * a.sv + (int64_t)h * D;
      // Per-row gates, requested before the tiles so that wave 0, which writes
      // them to LDS, waits for these loads only.  Every thread loads those of row
      // tid % C (rows past len clamped): no load sits in a branch, where the
      // compiler would issue it after the tiles' or on its own.
      const int ge = tid & (C - 1), gr = min(ge, len - 1);
      const float gm = a.gam[slot * C + ge];
      const float gl = a.gam[slot * C + len - 1];
      const float braw = chunk_beta_raw(a, tok0 + gr, h);
      const float hd = a.hdot[slot];
      // fused gates: this row's raw a, A_log and dt_bias (zero-size reads without
      // them: a load under a branch is waited for in that branch)
      const int fz = a.ga ? 4 : 0;
      const float xa_raw = buf_load_f32(a.ga + (int64_t)tok0 * a.Hv + h, fz * len * a.Hv, gr * a.Hv * 4);
      const float alog = buf_load_f32(a.A_log + h, fz, 0), dtb = buf_load_f32(a.dt_bias + h, fz, 0);
      __builtin_amdgcn_sched_barrier(0);  // keep these loads ahead of the tiles'
      TileRegs<E, C, D, NTH> pV;  // v rows and T (from the preparation pass)
      TileRegs<float, C, C, NTH, true> pTm;  // rows first: also written transposed
      TileRegs<float, D, C, NTH> rXu, rXw;  // dW^T, and dWk^T (in flight during the dXu products)
      pV.load(vg, a.sv, len);
      pTm.load(a.Tw + slot * C * C, C, C);
      rXu.load(a.dWt + slot * D * C, C, D);
      rXw.load(a.dWkt + slot * D * C, C, D);
      // fused gates: this row's factors da / dg, db / dbeta and its g, kept for the row pass at the end
      float fa_r = 0.f, fb_r = 0.f, g_r = 0.f;
      if (tid < C) {
        if (a.ga) {
          // formed here, off the row pass's serial path (the expressions of gdn_gates_bwd)
          const float ea = __expf(alog), xa = xa_raw + dtb;
          fa_r = -ea * gate_sigmoid(xa);
          g_r = -ea * gate_softplus(xa);
          fb_r = gate_sigmoid(braw) * gate_sigmoid(-braw);
        }
        const float bt = chunk_beta_fin(a, braw);
        sm.gam[ge] = gm;
        sm.Gm[ge] = __expf(gm);
        sm.beta[ge] = ge < len ? bt : 0.f;
        sm.em[ge] = ge < len ? __expf(gl - gm) : 0.f;
        sm.hdot = hd;  // the same value from every lane: no branch for the load to sink into
      }
      pTm.store(&sm.Tm[0][0], S::LDCF);
      // fp32 operands of the products below are split into their MFMA parts once
      // here, not per tile
      E* const TtL = LO ? &sm.TtL[0][0] : nullptr;
      E* const XL = LO ? &sm.r.x.l[0][0] : nullptr;
      pTm.template store_t<E>(&sm.TtH[0][0], S::LDCE, TtL, S::LDCE);  // T^T, transposed here
      // dXu = T^T dW -> dv and <dXu, v>
      pV.store(&sm.av.Vs[0][0], S::LDV);
      rXu.template store_split<E>(&sm.r.x.h[0][0], XL, S::LDCE);
      __syncthreads();
      // tile (dt, rt) of (T^T X)^T = X^T T (X = dW^T or dWk^T staged in r.x)
      auto txt = [&](int dt) {
        f32x4 acc[1][1];
        zero_blk(acc);
        mm_blk<E, C, 1, 1, LO, LO>(acc, &sm.r.x.h[dt * 16][0], LO ? XL + dt * 16 * S::LDCE : nullptr, S::LDCE,
                                   &sm.TtH[rt * 16][0], LO ? TtL + rt * 16 * S::LDCE : nullptr, S::LDCE);
        return acc[0][0];
      };
      E* dvg = (E*)a.dv + (int64_t)tok0 * a.sv + (int64_t)h * D;
      if (act) {
        const float br = sm.beta[rrow];
        float pu = 0.f;
#pragma unroll
        for (int i = 0; i < DT; ++i) {
          const int d = (dt0 + i) * 16 + dl;
          const f32x4 xu = txt(dt0 + i);
          float vv[4];
          ld4<E>(&sm.av.Vs[rrow][d], vv);
          f32x4 dvv;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            dvv[e] = br * xu[e];
            pu += xu[e] * vv[e];
          }
          if (rrow < len) st4<E>(dvg + (int64_t)rrow * a.sv + d, dvv);
        }
        sm.pCD[0][pslot][rrow] = pu;
      }
      __syncthreads();
      // dXw = T^T dWk -> dK and <dXw, k>
      rXw.template store_split<E>(&sm.r.x.h[0][0], XL, S::LDCE);
      __syncthreads();
      // dT, P and dP' of the C x C passes: in flight during the dXw products
      TileRegs<float, C, C, NTH> rT, pP, pdP;
      rT.load(a.dT + slot * C * C, C, C);
      pP.load(a.P + slot * C * C, C, C);
      pdP.load(a.dP + slot * C * C, C, C);
      if (act) {
        const float bg = sm.beta[rrow] * sm.Gm[rrow];
        float pw = 0.f;
#pragma unroll
        for (int i = 0; i < DT; ++i) {
          const int d = (dt0 + i) * 16 + dl;
          const f32x4 xw = txt(dt0 + i);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            pw += xw[e] * to_f<E>(sm.QKt[d + e][C + rrow]);
            dK[i][0][e] += bg * xw[e];
          }
        }
        sm.pCD[1][pslot][rrow] = pw;
      }
      __syncthreads();
      // M1 = dT T^T (fp32 MFMA), stored transposed and split; dA = strict_lower(-T^T M1)
      rT.store(&sm.r.m.dT[0][0], S::LDCF);
      __syncthreads();
      for (int t = w; t < NT * NT; t += NW) {
        const int rt = t / NT, ct = t % NT;
        // fp32 operands fed as bf16 hi / lo parts (three products per k-step)
        // rather than to the fp32 matrix instruction, which does a quarter of
        // the work per cycle
        const f32x4 m = mm_gen<E, C, true, true>(
            zero4(), [&](int r, int k, float* o) { ld_row<float, KPL>(&sm.r.m.dT[rt * 16 + r][k], o); },
            [&](int c, int k, float* o) { ld_row<float, KPL>(&sm.Tm[ct * 16 + c][k], o); });
        E* const M1L = LO ? &sm.r.m.M1l[0][0] : nullptr;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int c = ct * 16 + acc_col(), r = rt * 16 + acc_row(e);
          split_store<E>(&sm.r.m.M1h[c][r], LO ? M1L + c * S::LDCE + r : nullptr, m[e]);
        }
      }
      __syncthreads();
      for (int t = w; t < NT * NT; t += NW) {
        const int rt = t / NT, ct = t % NT;
        f32x4 mb[1][1];
        zero_blk(mb);
        mm_blk<E, C, 1, 1, LO, LO>(mb, &sm.TtH[rt * 16][0], LO ? TtL + rt * 16 * S::LDCE : nullptr, S::LDCE,
                                   &sm.r.m.M1h[ct * 16][0], LO ? &sm.r.m.M1l[ct * 16][0] : nullptr, S::LDCE);
        const f32x4 m = mb[0][0];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = rt * 16 + acc_row(e), s = ct * 16 + acc_col();
          sm.av.Am[r][s] = (s < r && r < len) ? -m[e] : 0.f;
        }
      }
      __syncthreads();
      pP.store(&sm.Tm[0][0], S::LDCF);  // T is no longer needed
      pdP.store(&sm.dPm[0][0], S::LDCF);  // T^T is no longer needed
      __syncthreads();
      // C x C pass: A~, dS, and the dgamma / dbeta terms of A and P
      for (int t = w; t < NT * NT; t += NW) {
        const int rt = t / NT, ct = t % NT;
        float rb[4], ra[4], rp[4], ca = 0.f, cp = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = rt * 16 + acc_row(e), s = ct * 16 + acc_col();
          const float skk = sm.Skk[r][s];
          const float dd = (s <= r) ? __expf(sm.gam[r] - sm.gam[s]) : 0.f;
          const float dA = sm.av.Am[r][s];
          const float At = dA * sm.beta[r] * dd;
          const float AdA = At * skk;
          const float dP = sm.dPm[r][s];
          const float PdP = dP * sm.Tm[r][s];
          rb[e] = dA * dd * skk;
          ra[e] = AdA;
          rp[e] = PdP;
          ca += AdA;
          cp += PdP;
          split_store<E>(&sm.r.s.dSh[r][s], &sm.r.s.dSl[0][0] + r * S::LDCE + s, dP * dd);
          sm.r.s.At[r][s] = At;
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          rb[e] = group_sum<16>(rb[e]);
          ra[e] = group_sum<16>(ra[e]);
          rp[e] = group_sum<16>(rp[e]);
        }
        ca += __shfl_xor(ca, 16, kWave);
        ca += __shfl_xor(ca, 32, kWave);
        cp += __shfl_xor(cp, 16, kWave);
        cp += __shfl_xor(cp, 32, kWave);
        if ((lane & 15) == 0) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = rt * 16 + acc_row(e);
            sm.pCC[0][ct][r] = rb[e];
            sm.pCC[1][ct][r] = ra[e];
            sm.pCC[3][ct][r] = rp[e];
          }
        }
        if (lane < 16) {
          sm.pCC[2][rt][ct * 16 + lane] = ca;
          sm.pCC[4][rt][ct * 16 + lane] = cp;
        }
      }
      __syncthreads();
      // this lane's dKh and dQs tiles: in flight during the transpose below
      // (waves past the d-tiles load the last tile again and leave it unused)
      f32x4 khr[DT], qsr[DT];
#pragma unroll
      for (int i = 0; i < DT; ++i) {
        const int dtl = min(dt0 + i, ND - 1);
        khr[i] = load_acc(a.dKh + slot * C * D, NT, dtl, rt);
        qsr[i] = load_acc(a.dQs + slot * C * D, NT, dtl, rt);
      }
      // [dS^T | A~ + A~^T] as rows (P and dP' are consumed)
      for (int e = tid; e < C * C; e += NTH) {
        const int sr = e / C, r = e % C;
        sm.TS.h[sr][r] = sm.r.s.dSh[r][sr];
        if constexpr (LO) sm.TS.l[sr][r] = sm.r.s.dSl[r][sr];
        split_store<E>(&sm.TS.h[sr][C + r], &sm.TS.l[0][0] + sr * S::LD2C + C + r,
                       sm.r.s.At[sr][r] + sm.r.s.At[r][sr]);
      }
      __syncthreads();
      // dQ += dQs + dS K;   dK += dKh + [dS^T | A~ + A~^T] [Q ; K]   (transposed)
      if (act) {
        float pq = 0.f, pk = 0.f;
#pragma unroll
        for (int i = 0; i < DT; ++i) {
          const int d = (dt0 + i) * 16 + dl;
          const f32x4 qs = qsr[i];
          const f32x4 kh = khr[i];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            dQ[i][0][e] += qs[e];
            dK[i][0][e] += kh[e];
            pq += qs[e] * to_f<E>(sm.QKt[d + e][rrow]);
            pk += kh[e] * to_f<E>(sm.QKt[d + e][C + rrow]);
          }
        }
        sm.pCD[2][pslot][rrow] = pq;
        sm.pCD[3][pslot][rrow] = pk;
        mm_blk<E, C, DT, 1, false, LO>(dQ, &sm.QKt[dt0 * 16][C], nullptr, S::LD2C, &sm.r.s.dSh[rt * 16][0],
                                       LO ? &sm.r.s.dSl[0][0] + rt * 16 * S::LDCE : nullptr, S::LDCE);
        mm_blk<E, 2 * C, DT, 1, false, LO>(dK, &sm.QKt[dt0 * 16][0], nullptr, S::LD2C, &sm.TS.h[rt * 16][0],
                                           LO ? &sm.TS.l[0][0] + rt * 16 * S::LD2C : nullptr, S::LD2C);
      }
      __syncthreads();
      // per-row totals, then dg = reverse cumulative sum within the chunk
      if (w == 0) {
        const int r = lane;
        float dbeta = 0.f, dgam = 0.f, tk = 0.f;
        if (r < C) {
          float su = 0.f, sw = 0.f, sq = 0.f;
          for (int c = 0; c < S::NPD; ++c) {
            su += sm.pCD[0][c][r];
            sw += sm.pCD[1][c][r];
            sq += sm.pCD[2][c][r];
            tk += sm.pCD[3][c][r];
          }
          float rb = 0.f, ar = 0.f, ac = 0.f, pr = 0.f, pc = 0.f;
          for (int c = 0; c < NT; ++c) {
            rb += sm.pCC[0][c][r];
            ar += sm.pCC[1][c][r];
            ac += sm.pCC[2][c][r];
            pr += sm.pCC[3][c][r];
            pc += sm.pCC[4][c][r];
          }
          dbeta = su + sm.Gm[r] * sw + rb;
          dgam = sq - tk + sm.beta[r] * sm.Gm[r] * sw + (ar - ac) + (pr - pc);
          if (r >= len) dgam = tk = 0.f;
        }
        const float tks = wave_sum(tk);
        if (r == len - 1) dgam += sm.Gm[len - 1] * sm.hdot + tks;
        // reverse inclusive scan: dg_r = sum_{r' >= r} dgam_{r'}
        const float x = wave_suffix_sum(dgam);
        if (a.da) {
          // fused gates: da = -exp(A_log) sigmoid(a + dt_bias) dg, db = beta (1 - beta) dbeta,
          // and this chunk's shares of dA_log = sum dg g and ddt_bias = sum da
          float sA = 0.f, sdt = 0.f;
          if (r < len) {  // row r's factors: formed by this lane at the start of the v-head
            const int64_t e = (int64_t)(tok0 + r) * a.Hv + h;
            const float dav = fa_r * x;
            a.da[e] = dav;
            a.db[e] = fb_r * dbeta;
            sA = x * g_r;
            sdt = dav;
          }
          sA = wave_sum(sA);
          sdt = wave_sum(sdt);
          if (r == 0) {
            a.gpart[(int64_t)ci * a.Hv + h] = sA;
            a.gpart[((int64_t)a.max_chunks + ci) * a.Hv + h] = sdt;
          }
        } else if (r < len) {
          a.dg[(int64_t)(tok0 + r) * a.Hv + h] = x;
          a.dbeta[(int64_t)(tok0 + r) * a.Hv + h] = dbeta;
        }
      }
      __syncthreads();
    }
    load_qk(next, nent);  // in flight while this item's dq and dk leave
    E* dqg = (E*)a.dq + (int64_t)tok0 * a.sqk + (int64_t)j * D;
    E* dkg = (E*)a.dk + (int64_t)tok0 * a.sqk + (int64_t)j * D;
    if (act && rrow < len) {
#pragma unroll
      for (int i = 0; i < DT; ++i) {
        const int d = (dt0 + i) * 16 + dl;
        st4<E>(dqg + (int64_t)rrow * a.sqk + d, dQ[i][0]);
        st4<E>(dkg + (int64_t)rrow * a.sqk + d, dK[i][0]);
      }
    }
    ent = nent;
  }
}

// ---------------------------------------------------------------------------
// host side: workspace plan and dispatch
// ---------------------------------------------------------------------------
static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct WsPlan {
  size_t table, seq0, Wk, U, P, Kt, Ktl, gam, Qf, end_fwd;
  size_t Ptr, Tw, Krh, Krl, Wth, Wtl, Qth, Qtl, Hc, W, dHn, dW, dWt, dT, dWkt, dQs, dKh, dP, hdot, gpart, end_bwd;
};

static WsPlan plan(const gdn_shape* s) {
  const size_t M = (size_t)max_chunks(s), Hv = s->h_v, C = s->chunk, D = s->d_k;
  const size_t es = s->dtype == GDN_BF16 ? 2 : 4;
  WsPlan p;
  size_t o = 0;
  p.table = o; o = align256(o + M * 16);
  p.seq0 = o; o = align256(o + ((size_t)s->n_seqs + 1) * 4);
  p.Wk = o; o = align256(o + M * Hv * C * D * es);
  p.U = o; o = align256(o + M * Hv * C * D * 4);
  p.P = o; o = align256(o + M * Hv * C * C * 4);
  p.Kt = o; o = align256(o + M * Hv * D * C * es);
  // no K~ lo part where the state passes read the plain K^T (bf16, d = 128, chunk 64)
  const bool plain_k = es == 2 && D == 128 && C == 64;
  p.Ktl = o; o = align256(o + (es == 2 && !plain_k ? M * Hv * D * C * es : 0));
  p.gam = o; o = align256(o + M * Hv * C * 4);
  // q rows in fragment order, written and read by the inference forward only:
  // the backward's own buffers start at the same offset
  p.Qf = o;
  p.end_fwd = align256(o + (plain_k ? M * (size_t)s->h_qk * C * D * es : 0));
  // the whole-state reverse pass (plain_k) forms P^T, the K rows and (Gam q)^T
  // from P, k and q, and writes dW^T only
  const size_t tr = plain_k ? 0 : 1;
  p.Ptr = o; o = align256(o + tr * M * Hv * C * C * 4);
  p.Tw = o; o = align256(o + M * Hv * C * C * 4);
  p.Krh = o; o = align256(o + tr * M * Hv * C * D * es);
  p.Krl = o; o = align256(o + (plain_k ? 0 : M * Hv * C * D * es));
  p.Wth = o; o = align256(o + M * Hv * D * C * es);
  p.Wtl = o; o = align256(o + M * Hv * D * C * es);
  p.Qth = o; o = align256(o + tr * M * Hv * D * C * es);
  p.Qtl = o; o = align256(o + tr * M * Hv * D * C * es);
  p.Hc = o; o = align256(o + M * Hv * D * D * 4);
  p.W = o; o = align256(o + M * Hv * C * D * 4);
  p.dHn = o; o = align256(o + M * Hv * D * D * 4);
  p.dW = o; o = align256(o + tr * M * Hv * C * D * 4);
  p.dWt = o; o = align256(o + M * Hv * D * C * 4);
  p.dT = o; o = align256(o + M * Hv * C * C * 4);
  p.dWkt = o; o = align256(o + M * Hv * D * C * 4);
  p.dQs = o; o = align256(o + M * Hv * C * D * 4);
  p.dKh = o; o = align256(o + M * Hv * C * D * 4);
  p.dP = o; o = align256(o + M * Hv * C * C * 4);
  p.hdot = o; o = align256(o + M * Hv * 4);
  p.gpart = o; o = align256(o + 2 * M * Hv * 4);
  p.end_bwd = o;
  return p;
}

size_t chunk_fwd_ws_bytes(const gdn_shape* s) { return plan(s).end_fwd; }
size_t chunk_bwd_ws_bytes(const gdn_shape* s) { return plan(s).end_bwd; }

static void fill_ws(ChunkArgs& a, const gdn_shape* s, void* ws) {
  const WsPlan p = plan(s);
  char* b = (char*)ws;
  a.table = (const int32_t*)(b + p.table);
  a.seq_chunk0 = (const int32_t*)(b + p.seq0);
  a.Wk = b + p.Wk;
  a.U = (float*)(b + p.U);
  a.P = (float*)(b + p.P);
  a.Kt = b + p.Kt;
  a.Ktl = b + p.Ktl;
  a.Qf = b + p.Qf;
  a.gam = (float*)(b + p.gam);
  a.Ptr = (float*)(b + p.Ptr);
  a.Tw = (float*)(b + p.Tw);
  a.Krh = b + p.Krh;
  a.Krl = b + p.Krl;
  a.Wth = b + p.Wth;
  a.Wtl = b + p.Wtl;
  a.Qth = b + p.Qth;
  a.Qtl = b + p.Qtl;
  a.Hc = (float*)(b + p.Hc);
  a.W = (float*)(b + p.W);
  a.dHn = (float*)(b + p.dHn);
  a.dW = (float*)(b + p.dW);
  a.dWt = (float*)(b + p.dWt);
  a.dT = (float*)(b + p.dT);
  a.dWkt = (float*)(b + p.dWkt);
  a.dQs = (float*)(b + p.dQs);
  a.dKh = (float*)(b + p.dKh);
  a.dP = (float*)(b + p.dP);
  a.hdot = (float*)(b + p.hdot);
  a.gpart = (float*)(b + p.gpart);
}

template <typename E, int D, int C>
constexpr bool fits() {
  constexpr size_t lim = 160 * 1024;
  return sizeof(PrepSmem<E, D, C>) <= lim && sizeof(StateSmem<E, D, C, (D >= 32 ? 32 : D), true>) <= lim &&
         sizeof(StateBwdSmem<E, D, C, (D >= 32 ? 32 : D)>) <= lim && sizeof(GradASmem<E, D, C, 2 * kChunkThreads>) <= lim &&
         sizeof(GradBSmem<E, D, C>) <= lim;
}

template <typename E, int D, int C>
static void launch_chunk_bwd_core(const ChunkArgs& a, hipStream_t st, bool recompute) {
  constexpr int DVT = D >= 32 ? 32 : D;
  if (recompute) launch_chunk_fwd_core<E, D, C, false>(a, st, kFwdStore);  // operands, Hc, W per chunk
  {
    // the whole-state reverse pass splits each chain's state into two 64-column
    // halves when there are fewer chains than CUs (the same arithmetic per
    // element, so the same bits)
    constexpr bool wide = use_wide_state<E, D, C>();
    const bool half = wide && a.N * a.Hv < kNumCUs;
    const char* name = wide ? (half ? "chunk_state_bwd:wide64" : "chunk_state_bwd:wide128")
                            : (DVT == 16 ? "chunk_state_bwd:tiled16" : "chunk_state_bwd:tiled32");
    GDN_PROF(name, st);
    if constexpr (use_wide_state<E, D, C>()) launch_state_bwd_wide(a, st, half);
    else state_bwd_kernel<E, D, C, DVT><<<dim3(state_grid(a.N, a.Hk, a.G, D / DVT)), kChunkThreads, 0, st>>>(a);
  }
  {
    GDN_PROF("chunk_grad_a", st);
    constexpr int GA_THREADS = (D >= 64 && C >= 64) ? 2 * kChunkThreads : kChunkThreads;
    grad_a_kernel<E, D, C, GA_THREADS><<<dim3(a.max_chunks, a.Hv), GA_THREADS, 0, st>>>(a);
  }
  GDN_PROF("chunk_grad_b", st);
  // 8 waves where the [C][D] tiles give each one a column strip of its own
  constexpr int GB_THREADS = gb_threads<D, C>();
  // persistent: as many workgroups as fit at once (one per CU at d = 128, chunk 64)
  constexpr int gb_per_cu = (160 * 1024) / (int)sizeof(GradBSmem<E, D, C>) >= 2 ? 2 : 1;
  const int64_t gb_items = (int64_t)a.max_chunks * a.Hk, gb_resident = (int64_t)kNumCUs * gb_per_cu;
  grad_b_kernel<E, D, C, GB_THREADS>
      <<<dim3((unsigned)(gb_items > gb_resident ? gb_resident : gb_items)), GB_THREADS, 0, st>>>(a);
}

// Calls f.template operator()<E, D, C>() for the runtime (dtype, d, chunk)
// when that combination fits in LDS; returns false otherwise.
template <typename F>
static bool dispatch(const gdn_shape* s, F&& f) {
#define GDN_CASE(E, D, C)                                       \
  if (s->d_k == D && s->chunk == C) {                           \
    if constexpr (fits<E, D, C>()) { f.template operator()<E, D, C>(); return true; } \
    return false;                                               \
  }
  if (s->dtype == GDN_BF16) {
    GDN_CASE(bf16, 16, 16) GDN_CASE(bf16, 16, 32) GDN_CASE(bf16, 16, 64)
    GDN_CASE(bf16, 32, 16) GDN_CASE(bf16, 32, 32) GDN_CASE(bf16, 32, 64)
    GDN_CASE(bf16, 64, 16) GDN_CASE(bf16, 64, 32) GDN_CASE(bf16, 64, 64)
    GDN_CASE(bf16, 128, 16) GDN_CASE(bf16, 128, 32) GDN_CASE(bf16, 128, 64)
  } else if (s->dtype == GDN_F32) {
    // float32 runs chunks of at most 32: at 64 the chunk backward's dg (a
    // reverse sum over the chunk of terms that largely cancel) reaches the
    // float32 bar of 1e-4 x RMS (measured 1.06e-4 at d = 32)
    GDN_CASE(float, 16, 16) GDN_CASE(float, 16, 32)
    GDN_CASE(float, 32, 16) GDN_CASE(float, 32, 32)
    GDN_CASE(float, 64, 16) GDN_CASE(float, 64, 32)
    GDN_CASE(float, 128, 16) GDN_CASE(float, 128, 32)
  }
#undef GDN_CASE
  return false;
}

bool chunk_supported(const gdn_shape* s) {
  return dispatch(s, [&]<typename E, int D, int C>() {});
}

static void set_gates(ChunkArgs& a, const gdn_gate_inputs* gi) {
  if (!gi) return;
  a.g = a.beta = nullptr;
  a.ga = gi->a; a.gb = gi->b; a.A_log = gi->A_log; a.dt_bias = gi->dt_bias;
}

bool run_chunk_fwd(const gdn_shape* s, const void* q, const void* k, const void* v, int64_t sqk, int64_t sv,
                   const float* g, const float* beta, const gdn_gate_inputs* gi, const int32_t* cu,
                   const float* h0, void* o, float* ht, void* ws, bool save, hipStream_t st) {
  ChunkArgs a = {};
  a.q = q; a.k = k; a.v = v; a.sqk = sqk; a.sv = sv; a.g = g; a.beta = beta; a.cu = cu; a.h0 = h0;
  set_gates(a, gi);
  a.o = o; a.ht = ht;
  a.N = s->n_seqs; a.T = s->total_tokens; a.Hk = s->h_qk; a.Hv = s->h_v; a.G = s->h_v / s->h_qk;
  a.max_chunks = (int)max_chunks(s); a.scale = s->scale;
  fill_ws(a, s, ws);
  run_chunk_index(s, cu, (int32_t*)a.table, (int32_t*)a.seq_chunk0, st);
  return dispatch(s, [&]<typename E, int D, int C>() {
    launch_chunk_fwd_core<E, D, C, false>(a, st, save ? kFwdBoth : kFwdOut);
  });
}

bool run_chunk_fwd_f8(const gdn_shape* s, const void* q, const void* k, const void* v, int64_t sqk, int64_t sv,
                      const float scales[3], const float* g, const float* beta, const int32_t* cu, const float* h0,
                      void* o, float* ht, void* ws, hipStream_t st) {
  if (s->dtype != GDN_BF16 || s->d_k != 128 || s->chunk != 64) return false;
  ChunkArgs a = {};
  a.q = q; a.k = k; a.v = v; a.sqk = sqk; a.sv = sv; a.g = g; a.beta = beta; a.cu = cu; a.h0 = h0;
  a.o = o; a.ht = ht;
  a.N = s->n_seqs; a.T = s->total_tokens; a.Hk = s->h_qk; a.Hv = s->h_v; a.G = s->h_v / s->h_qk;
  a.max_chunks = (int)max_chunks(s); a.scale = s->scale;
  for (int i = 0; i < 3; ++i) a.f8_scale[i] = scales[i];
  fill_ws(a, s, ws);
  run_chunk_index(s, cu, (int32_t*)a.table, (int32_t*)a.seq_chunk0, st);
  launch_chunk_fwd_core<bf16, 128, 64, true>(a, st, kFwdOut);
  return true;
}

bool run_chunk_bwd(const gdn_shape* s, const void* q, const void* k, const void* v, int64_t sqk, int64_t sv,
                   const float* g, const float* beta, const gdn_gate_inputs* gi, const int32_t* cu,
                   const float* h0, const void* d_o, const float* dht, void* dq, void* dk, void* dv, float* dg,
                   float* dbeta, const gdn_gate_grads* gg, float* dh0, void* ws, bool saved, hipStream_t st) {
  ChunkArgs a = {};
  a.q = q; a.k = k; a.v = v; a.sqk = sqk; a.sv = sv; a.g = g; a.beta = beta; a.cu = cu; a.h0 = h0;
  set_gates(a, gi);
  a.o = nullptr; a.ht = nullptr;
  a.d_o = d_o; a.dht = dht; a.dq = dq; a.dk = dk; a.dv = dv; a.dg = dg; a.dbeta = dbeta; a.dh0 = dh0;
  if (gg) {
    a.dg = a.dbeta = nullptr;
    a.da = gg->da; a.db = gg->db;
  }
  a.N = s->n_seqs; a.T = s->total_tokens; a.Hk = s->h_qk; a.Hv = s->h_v; a.G = s->h_v / s->h_qk;
  a.max_chunks = (int)max_chunks(s); a.scale = s->scale;
  fill_ws(a, s, ws);
  if (!saved) run_chunk_index(s, cu, (int32_t*)a.table, (int32_t*)a.seq_chunk0, st);
  if (!dispatch(s, [&]<typename E, int D, int C>() { launch_chunk_bwd_core<E, D, C>(a, st, !saved); }))
    return false;
  if (gg) {  // dA_log, ddt_bias: the per-chunk shares summed over chunks in a fixed order
    GDN_PROF("gates_dw_sum", st);
    launch_colsum(a.gpart, a.max_chunks, a.Hv, gg->dA_log, st);
    launch_colsum(a.gpart + (size_t)a.max_chunks * a.Hv, a.max_chunks, a.Hv, gg->ddt_bias, st);
  }
  return true;
}

}  // namespace gdn
