// Inter-chunk state passes for d = 128, chunk 64, bf16: one 512-thread
// workgroup (8 waves) per (sequence, v-head) carries the whole 128 x 128
// state, so at 8 sequences x 32 v-heads every workgroup is resident at once
// and each chunk's operands are read once per head.
//
// Pages: "[Qwen3.5 MoE] Add hybrid decoder model", Summary (GatedDeltaNet);
// "Support Qwen35 SFT", XTuner changes (varlen mode: the state restarts at
// every sequence).
//
// LDS holds only what several waves read: K~^T, H^T and W^T (forward);
// [dO^T | dW^T], dH^T and K~ rows (reverse), each bf16 hi + lo.  Operands that
// one row-tile of waves reads (Wk, q, U, P in the forward; P^T, (Gam q)^T,
// Wk^T in the reverse) are loaded straight into MFMA fragments from global
// memory (L2), and the next chunk's copies are requested right after the
// current chunk's last use.
//
// Forward, per chunk (H = state entering it):
//   W = U - Wk H;   o = scale (diag(Gam) Q H + P W);   H <- Gam_last H + K~^T W
// Reverse, per chunk (dH = gradient w.r.t. the state leaving it):
//   dW = scale P^T dO + K~ dH;   dH <- Gam_last dH + scale (diag(Gam) Q)^T dO - Wk^T dW
#include "chunk_common.cuh"
#include "profile.h"

namespace gdn {
namespace {

constexpr int kD = 128, kC = 64;
constexpr int kThreads = 512;
constexpr int kP1 = 4;            // phase-1 tiles per wave: one row tile, 4 column tiles
constexpr int kP2 = 8;            // state tiles per wave: one row tile, all 8 column tiles
constexpr int kKR = kD * kC / 8 / kThreads;  // 16-byte pieces of a [D][C] tile per thread
constexpr int kLDC = kC + 8;      // row stride of [.][C] tiles (elements), 16-byte pad
constexpr int kLDQ = kD + 8;      // row stride of [.][D] tiles
constexpr int kLD2C = 2 * kC + 8;

typedef bf16 E;
typedef Mma<bf16> M;

struct FwdSmem {
  E Kt[kD][kLDC];    // K~^T, K~ = diag(e) K
  E Ktl[kD][kLDC];
  E Ht[kD][kLDQ];    // H^T: Ht[c][r] = H[r][c]
  E Htl[kD][kLDQ];
  E Wt[kD][kLDC];    // W^T
  E Wtl[kD][kLDC];
  float gam[kC];
};

struct BwdSmem {
  E OW[kD][kLD2C];   // [ dO^T | dW^T ]
  E dWl[kD][kLDC];   // lo part of dW^T
  E dHt[kD][kLDQ];   // dH^T
  E dHtl[kD][kLDQ];
  E Kr[kC][kLDQ];    // rows of K~
  E Krl[kC][kLDQ];
  float gam[kC];
};

__device__ __forceinline__ M::frag fr(const E* p) { return M::load(p); }

// 8 floats -> bf16 hi and lo fragments (lo = x - hi)
__device__ __forceinline__ void split8(const float4& a, const float4& b, M::frag& hi, M::frag& lo) {
  const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  float l[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) l[i] = v[i] - bf2f(f2bf(v[i]));
  hi = M::from_floats(v);
  lo = M::from_floats(l);
}

__device__ __forceinline__ float4 ld4(const float* p) { return *reinterpret_cast<const float4*>(p); }

template <int MODE>
__global__ __launch_bounds__(kThreads) void state_fwd_wide_kernel(ChunkArgs a) {
  constexpr bool OUT = MODE & kFwdOut, STORE = MODE & kFwdStore;
  constexpr int D = kD, C = kC;
  __shared__ FwdSmem sm;
  int n, h, vt;
  if (!state_block(blockIdx.x, a.N, a.Hk, a.G, 1, n, h, vt)) return;
  const int j = h / a.G;
  const int tid = threadIdx.x, w = wave_id(), lane = lane_id();
  const int r16 = lane & 15, kq = (lane >> 4) * 8;
  const int rt1 = w & 3, cb = kP1 * (w >> 2);  // W / O tiles: row tile rt1, column tiles cb .. cb+3
  const int rt2 = w;                           // state tiles: row tile rt2, every column tile

  f32x4 Hr[kP2];
#pragma unroll
  for (int i = 0; i < kP2; ++i) {
    Hr[i] = zero4();
    if (a.h0) {
      const float* src = a.h0 + ((int64_t)n * a.Hv + h) * D * D;
#pragma unroll
      for (int e = 0; e < 4; ++e) Hr[i][e] = src[(rt2 * 16 + acc_row(e)) * D + i * 16 + acc_col()];
    }
  }
  auto write_Ht = [&]() {
#pragma unroll
    for (int i = 0; i < kP2; ++i) {
      const int c = i * 16 + acc_col(), r = rt2 * 16 + acc_row(0);
      st4_split<E>(&sm.Ht[c][r], &sm.Htl[c][r], Hr[i]);
    }
  };

  // staged operands of the next chunk
  uint4 kt_h[kKR], kt_l[kKR];   // this thread's pieces of K~^T (hi, lo)
  float g_r = 0.f;
  M::frag wkf[4], qf[4];
  f32x4 uf[kP1];
  float4 pf[2][2];
  auto load_shared = [&](int ci) {
    const int64_t slot = (int64_t)ci * a.Hv + h;
#pragma unroll
    for (int i = 0; i < kKR; ++i) {
      kt_h[i] = reinterpret_cast<const uint4*>((const E*)a.Kt + slot * D * C)[tid + i * kThreads];
      kt_l[i] = reinterpret_cast<const uint4*>((const E*)a.Ktl + slot * D * C)[tid + i * kThreads];
    }
    if (tid < C) g_r = a.gam[slot * C + tid];
  };
  auto load_p1 = [&](int ci, int tok0, int len) {
    const int64_t slot = (int64_t)ci * a.Hv + h;
    const E* wk = (const E*)a.Wk + slot * C * D + (rt1 * 16 + r16) * D + kq;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) wkf[ks] = fr(wk + ks * 32);
    if constexpr (OUT) {
      const int row = rt1 * 16 + r16;
      const E* qp = (const E*)a.q + (int64_t)(tok0 + (row < len ? row : 0)) * a.sqk + (int64_t)j * D + kq;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) qf[ks] = row < len ? fr(qp + ks * 32) : M::zero();
    }
    const float* up = a.U + slot * C * D;
#pragma unroll
    for (int i = 0; i < kP1; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) uf[i][e] = up[(rt1 * 16 + acc_row(e)) * D + (cb + i) * 16 + acc_col()];
  };
  auto load_p2 = [&](int ci) {
    const float* pp = a.P + ((int64_t)ci * a.Hv + h) * C * C + (rt1 * 16 + r16) * C + kq;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      pf[ks][0] = ld4(pp + ks * 32);
      pf[ks][1] = ld4(pp + ks * 32 + 4);
    }
  };

  const int c0 = a.seq_chunk0[n], c1 = a.seq_chunk0[n + 1];
  int4 ent = make_int4(0, 0, 0, 0);
  if (c0 < c1) {
    ent = chunk_entry(a.table, c0);
    load_shared(c0);
    load_p1(c0, ent.y, ent.z);
    if constexpr (OUT) load_p2(c0);
  }
  write_Ht();
  for (int ci = c0; ci < c1; ++ci) {
    const int tok0 = ent.y, len = ent.z;
    const int64_t slot = (int64_t)ci * a.Hv + h;
    __syncthreads();  // the previous chunk is done with K~^T and W^T, and H^T is written
#pragma unroll
    for (int i = 0; i < kKR; ++i) {
      const int e = tid + i * kThreads;  // 16-byte piece: row e / 8, columns (e % 8) * 8 ..
      *reinterpret_cast<uint4*>(&sm.Kt[e >> 3][(e & 7) * 8]) = kt_h[i];
      *reinterpret_cast<uint4*>(&sm.Ktl[e >> 3][(e & 7) * 8]) = kt_l[i];
    }
    if (tid < C) sm.gam[tid] = g_r;
    if constexpr (STORE) {  // state entering this chunk, for the backward pass
      float* Hg = a.Hc + slot * D * D;
#pragma unroll
      for (int i = 0; i < kP2; ++i) store_tile<float>(Hg, D, rt2 * 16, i * 16, Hr[i], D);
    }
    __syncthreads();
    const bool more = ci + 1 < c1;
    int4 nent = ent;
    if (more) {
      nent = chunk_entry(a.table, ci + 1);
      load_shared(ci + 1);
    }

    // phase 1: W = U - Wk H and diag(Gam) Q H on this wave's tiles
    f32x4 x[kP1], o[kP1];
#pragma unroll
    for (int i = 0; i < kP1; ++i) x[i] = o[i] = zero4();
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
      for (int i = 0; i < kP1; ++i) {
        const int c = (cb + i) * 16 + r16;
        const M::frag bh = fr(&sm.Ht[c][ks * 32 + kq]);
        const M::frag bl = fr(&sm.Htl[c][ks * 32 + kq]);
        x[i] = M::mma(wkf[ks], bh, x[i]);
        x[i] = M::mma(wkf[ks], bl, x[i]);
        if constexpr (OUT) {
          o[i] = M::mma(qf[ks], bh, o[i]);
          o[i] = M::mma(qf[ks], bl, o[i]);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < kP1; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) x[i][e] = uf[i][e] - x[i][e];  // x <- W
    if constexpr (OUT) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float gm = __expf(sm.gam[rt1 * 16 + acc_row(e)]);
#pragma unroll
        for (int i = 0; i < kP1; ++i) o[i][e] *= gm;
      }
    }
    if (more) load_p1(ci + 1, nent.y, nent.z);  // Wk, q, U of the next chunk
#pragma unroll
    for (int i = 0; i < kP1; ++i) {
      const int c = (cb + i) * 16 + acc_col(), r = rt1 * 16 + acc_row(0);
      st4_split<E>(&sm.Wt[c][r], &sm.Wtl[c][r], x[i]);
      if constexpr (STORE) store_tile<float>(a.W + slot * C * D, D, rt1 * 16, (cb + i) * 16, x[i], C);
    }
    __syncthreads();

    // phase 2: H <- Gam_last H + K~^T W;  o = scale (diag(Gam) Q H + P W)
    const float gl = __expf(sm.gam[len - 1]);
#pragma unroll
    for (int i = 0; i < kP2; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) Hr[i][e] *= gl;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const M::frag ah = fr(&sm.Kt[rt2 * 16 + r16][ks * 32 + kq]);
      const M::frag al = fr(&sm.Ktl[rt2 * 16 + r16][ks * 32 + kq]);
#pragma unroll
      for (int i = 0; i < kP2; ++i) {
        const int c = i * 16 + r16;
        const M::frag bh = fr(&sm.Wt[c][ks * 32 + kq]);
        const M::frag bl = fr(&sm.Wtl[c][ks * 32 + kq]);
        Hr[i] = M::mma(ah, bh, Hr[i]);
        Hr[i] = M::mma(ah, bl, Hr[i]);
        Hr[i] = M::mma(al, bh, Hr[i]);
      }
    }
    if constexpr (OUT) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        M::frag ph, pl;
        split8(pf[ks][0], pf[ks][1], ph, pl);
#pragma unroll
        for (int i = 0; i < kP1; ++i) {
          const int c = (cb + i) * 16 + r16;
          const M::frag bh = fr(&sm.Wt[c][ks * 32 + kq]);
          const M::frag bl = fr(&sm.Wtl[c][ks * 32 + kq]);
          o[i] = M::mma(ph, bh, o[i]);
          o[i] = M::mma(ph, bl, o[i]);
          o[i] = M::mma(pl, bh, o[i]);
        }
      }
      if (more) load_p2(ci + 1);
      E* og = (E*)a.o + (int64_t)tok0 * a.Hv * D + (int64_t)h * D;
#pragma unroll
      for (int i = 0; i < kP1; ++i) {
#pragma unroll
        for (int e = 0; e < 4; ++e) o[i][e] *= a.scale;
        store_tile<E>(og, (int64_t)a.Hv * D, rt1 * 16, (cb + i) * 16, o[i], len);
      }
    }
    write_Ht();  // phase 1 (the only reader of H^T) is over for every wave
    ent = nent;
  }
  if (a.ht) {
    float* dst = a.ht + ((int64_t)n * a.Hv + h) * D * D;
#pragma unroll
    for (int i = 0; i < kP2; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) dst[(rt2 * 16 + acc_row(e)) * D + i * 16 + acc_col()] = Hr[i][e];
  }
}

__global__ __launch_bounds__(kThreads) void state_bwd_wide_kernel(ChunkArgs a) {
  constexpr int D = kD, C = kC;
  __shared__ BwdSmem sm;
  int n, h, vt;
  if (!state_block(blockIdx.x, a.N, a.Hk, a.G, 1, n, h, vt)) return;
  const int tid = threadIdx.x, w = wave_id(), lane = lane_id();
  const int r16 = lane & 15, kq = (lane >> 4) * 8;
  const int rt1 = w & 3, cb = kP1 * (w >> 2);  // dW tiles
  const int rt2 = w;                           // dH tiles: row tile rt2, every column tile

  f32x4 dH[kP2];
#pragma unroll
  for (int i = 0; i < kP2; ++i) {
    dH[i] = zero4();
    if (a.dht) {
      const float* src = a.dht + ((int64_t)n * a.Hv + h) * D * D;
#pragma unroll
      for (int e = 0; e < 4; ++e) dH[i][e] = src[(rt2 * 16 + acc_row(e)) * D + i * 16 + acc_col()];
    }
  }
  auto write_dHt = [&]() {
#pragma unroll
    for (int i = 0; i < kP2; ++i) {
      const int c = i * 16 + acc_col(), r = rt2 * 16 + acc_row(0);
      st4_split<E>(&sm.dHt[c][r], &sm.dHtl[c][r], dH[i]);
    }
  };

  // staged operands of the next chunk (reverse order)
  uint4 kr_h[kKR], kr_l[kKR];       // this thread's pieces of the K~ rows
  ColRegs<E, C, D, kThreads> pO;    // dO of the chunk, gathered column-wise
  float g_r = 0.f;
  float4 ptf[2][2];                 // P^T rows of this wave's dW tiles
  M::frag qth[2], qtl[2], wth[2], wtl[2];  // (Gam q)^T and Wk^T rows of its dH tiles
  auto load_shared = [&](int ci, int tok0, int len) {
    const int64_t slot = (int64_t)ci * a.Hv + h;
#pragma unroll
    for (int i = 0; i < kKR; ++i) {
      kr_h[i] = reinterpret_cast<const uint4*>((const E*)a.Krh + slot * C * D)[tid + i * kThreads];
      kr_l[i] = reinterpret_cast<const uint4*>((const E*)a.Krl + slot * C * D)[tid + i * kThreads];
    }
    pO.load((const E*)a.d_o + (int64_t)tok0 * a.Hv * D + (int64_t)h * D, (int64_t)a.Hv * D, len);
    if (tid < C) g_r = a.gam[slot * C + tid];
  };
  auto load_p1 = [&](int ci) {
    const float* pp = a.Ptr + ((int64_t)ci * a.Hv + h) * C * C + (rt1 * 16 + r16) * C + kq;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      ptf[ks][0] = ld4(pp + ks * 32);
      ptf[ks][1] = ld4(pp + ks * 32 + 4);
    }
  };
  auto load_p2 = [&](int ci) {
    const int64_t off = ((int64_t)ci * a.Hv + h) * D * C + (rt2 * 16 + r16) * C + kq;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      qth[ks] = fr((const E*)a.Qth + off + ks * 32);
      qtl[ks] = fr((const E*)a.Qtl + off + ks * 32);
      wth[ks] = fr((const E*)a.Wth + off + ks * 32);
      wtl[ks] = fr((const E*)a.Wtl + off + ks * 32);
    }
  };

  const int c0 = a.seq_chunk0[n], c1 = a.seq_chunk0[n + 1];
  int4 ent = make_int4(0, 0, 0, 0);
  if (c0 < c1) {
    ent = chunk_entry(a.table, c1 - 1);
    load_shared(c1 - 1, ent.y, ent.z);
    load_p1(c1 - 1);
    load_p2(c1 - 1);
  }
  write_dHt();
  for (int ci = c1 - 1; ci >= c0; --ci) {
    const int len = ent.z;
    const int64_t slot = (int64_t)ci * a.Hv + h;
    __syncthreads();  // the previous chunk is done with [dO^T | dW^T] and K~, and dH^T is written
#pragma unroll
    for (int i = 0; i < kKR; ++i) {
      const int e = tid + i * kThreads;  // 16-byte piece: row e / 16, columns (e % 16) * 8 ..
      *reinterpret_cast<uint4*>(&sm.Kr[e >> 4][(e & 15) * 8]) = kr_h[i];
      *reinterpret_cast<uint4*>(&sm.Krl[e >> 4][(e & 15) * 8]) = kr_l[i];
    }
    pO.store(&sm.OW[0][0], kLD2C);
    if (tid < C) sm.gam[tid] = g_r;
    {  // gradient w.r.t. the state leaving this chunk
      float* dst = a.dHn + slot * D * D;
#pragma unroll
      for (int i = 0; i < kP2; ++i) store_tile<float>(dst, D, rt2 * 16, i * 16, dH[i], D);
    }
    __syncthreads();
    const bool more = ci > c0;
    int4 nent = ent;
    if (more) {
      nent = chunk_entry(a.table, ci - 1);
      load_shared(ci - 1, nent.y, nent.z);
    }

    // phase 1: dW = scale P^T dO + K~ dH on this wave's tiles
    f32x4 p[kP1], kd[kP1];
#pragma unroll
    for (int i = 0; i < kP1; ++i) p[i] = kd[i] = zero4();
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      M::frag ph, pl;
      split8(ptf[ks][0], ptf[ks][1], ph, pl);
#pragma unroll
      for (int i = 0; i < kP1; ++i) {
        const M::frag b = fr(&sm.OW[(cb + i) * 16 + r16][ks * 32 + kq]);
        p[i] = M::mma(ph, b, p[i]);
        p[i] = M::mma(pl, b, p[i]);
      }
    }
    if (more) load_p1(ci - 1);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const M::frag ah = fr(&sm.Kr[rt1 * 16 + r16][ks * 32 + kq]);
      const M::frag al = fr(&sm.Krl[rt1 * 16 + r16][ks * 32 + kq]);
#pragma unroll
      for (int i = 0; i < kP1; ++i) {
        const int c = (cb + i) * 16 + r16;
        const M::frag bh = fr(&sm.dHt[c][ks * 32 + kq]);
        const M::frag bl = fr(&sm.dHtl[c][ks * 32 + kq]);
        kd[i] = M::mma(ah, bh, kd[i]);
        kd[i] = M::mma(ah, bl, kd[i]);
        kd[i] = M::mma(al, bh, kd[i]);
      }
    }
#pragma unroll
    for (int i = 0; i < kP1; ++i) {
#pragma unroll
      for (int e = 0; e < 4; ++e) kd[i][e] += a.scale * p[i][e];  // kd <- dW
      store_tile<float>(a.dW + slot * C * D, D, rt1 * 16, (cb + i) * 16, kd[i], C);
      store_tile_t(a.dWt + slot * D * C, C, rt1 * 16, (cb + i) * 16, kd[i]);
      const int c = (cb + i) * 16 + acc_col(), r = rt1 * 16 + acc_row(0);
      st4_split<E>(&sm.OW[c][C + r], &sm.dWl[c][r], kd[i]);
    }
    __syncthreads();

    // phase 2: dH <- Gam_last dH + scale (diag(Gam) Q)^T dO - Wk^T dW
    const float gl = __expf(sm.gam[len - 1]);
#pragma unroll
    for (int i = 0; i < kP2; ++i) {
      const int c = i * 16 + r16;
      f32x4 y1 = zero4(), y2 = zero4();
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const M::frag bo = fr(&sm.OW[c][ks * 32 + kq]);
        const M::frag bw = fr(&sm.OW[c][C + ks * 32 + kq]);
        const M::frag bwl = fr(&sm.dWl[c][ks * 32 + kq]);
        y1 = M::mma(qth[ks], bo, y1);
        y1 = M::mma(qtl[ks], bo, y1);
        y2 = M::mma(wth[ks], bw, y2);
        y2 = M::mma(wth[ks], bwl, y2);
        y2 = M::mma(wtl[ks], bw, y2);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) dH[i][e] = gl * dH[i][e] + a.scale * y1[e] - y2[e];
    }
    if (more) load_p2(ci - 1);
    write_dHt();  // phase 1 (the only reader of dH^T) is over for every wave
    ent = nent;
  }
  if (a.dh0) {
    float* dst = a.dh0 + ((int64_t)n * a.Hv + h) * D * D;
#pragma unroll
    for (int i = 0; i < kP2; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) dst[(rt2 * 16 + acc_row(e)) * D + i * 16 + acc_col()] = dH[i][e];
  }
}

}  // namespace

void launch_state_fwd_wide(const ChunkArgs& a, hipStream_t st, int mode) {
  const dim3 grid(state_grid(a.N, a.Hk, a.G, 1));
  if (mode == kFwdOut) state_fwd_wide_kernel<kFwdOut><<<grid, kThreads, 0, st>>>(a);
  else if (mode == kFwdStore) state_fwd_wide_kernel<kFwdStore><<<grid, kThreads, 0, st>>>(a);
  else state_fwd_wide_kernel<kFwdBoth><<<grid, kThreads, 0, st>>>(a);
}

void launch_state_bwd_wide(const ChunkArgs& a, hipStream_t st) {
  state_bwd_wide_kernel<<<dim3(state_grid(a.N, a.Hk, a.G, 1)), kThreads, 0, st>>>(a);
}

}  // namespace gdn
