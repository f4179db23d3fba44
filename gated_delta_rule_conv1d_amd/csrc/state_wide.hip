// Inter-chunk state passes for d = 128, chunk 64, bf16: one 512-thread
// workgroup (8 waves) per (sequence, v-head) carries the whole 128 x 128
// state, so at 8 sequences x 32 v-heads every workgroup is resident at once
// and each chunk's operands are read once per head.
//
// Pages: "[Qwen3.5 MoE] Add hybrid decoder model", Summary (GatedDeltaNet);
// "Support Qwen35 SFT", XTuner changes (varlen mode: the state restarts at
// every sequence).
//
// LDS holds only what several waves read: K^T, H^T and W^T (forward; H and W
// as bf16 hi + lo); [dO^T | dW^T], dH^T and K~ rows (reverse, hi + lo).  Operands that
// one row-tile of waves reads (Wk, q, U, P in the forward, Wk, U and the
// inference P in the order the preparation wrote them; P^T and (Gam q)^T
// gathered from P and q, and Wk^T, in the reverse) are loaded straight into
// MFMA fragments from global memory (L2), and the next chunk's copies are
// requested right after the current chunk's last use, on every path (the
// last chunk loads itself again), so the compiler's wait counts stay exact.
//
// Forward, per chunk (H = state entering it):
//   W = U - Wk H;   o = scale (diag(Gam) Q H + P W);   H <- Gam_last H + K^T diag(e) W
// (K~^T W with the decay e_s = e^{gamma_last - gamma_s} moved onto W's rows,
// so the bf16 K needs no lo part)
// Reverse, per chunk (dH = gradient w.r.t. the state leaving it):
//   dW = scale P^T dO + K~ dH;   dH <- Gam_last dH + scale (diag(Gam) Q)^T dO - Wk^T dW
// (K~ dH as diag(e) (K dH): the bf16 K needs no lo part)
#include "chunk_common.cuh"
#include "profile.h"

namespace gdn {
namespace {

constexpr int kD = 128, kC = 64;
constexpr int kThreads = 512;
constexpr int kKR = kD * kC / 8 / kThreads;  // 16-byte pieces of a [D][C] tile per thread
constexpr int kLDC = kC + 8;      // row stride of [.][C] tiles (elements), 16-byte pad
constexpr int kLDQ = kD + 8;      // row stride of [.][D] tiles
constexpr int kLD2C = 2 * kC + 8;

typedef bf16 E;
typedef Mma<bf16> M;

template <int NC, bool OUT>  // state columns this workgroup carries; whether it forms o
struct FwdSmem {
  E Kt[kD][kLDC];    // K^T, exact in bf16
  E Ht[NC][kLDQ];    // H^T: Ht[c][r] = H[r][c]
  E Htl[NC][kLDQ];
  E Wt[NC][kLDC];    // W^T (with OUT, for P W), else (diag(e) W)^T
  E Wtl[NC][kLDC];
  E Ws[OUT ? NC : 1][kLDC];   // (diag(e) W)^T, e_r = e^{gamma_last - gamma_r}, for the state update
  E Wsl[OUT ? NC : 1][kLDC];
  float gam[kC];
};

template <int NC>  // state columns this workgroup carries
struct BwdSmem {
  E OW[NC][kLD2C];   // [ dO^T | dW^T ]
  E dWl[NC][kLDC];   // lo part of dW^T
  E dHt[NC][kLDQ];   // dH^T
  E dHtl[NC][kLDQ];
  E Kr[kC][kLDQ];    // rows of K (exact in bf16; the decay e_s goes onto K dH's rows)
  float gam[kC];
  float Gm[kC];      // Gam_s = e^{gamma_s}
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

// A buffer resource over [base, base + bytes): loads take a 32-bit offset
// (out-of-range offsets read zero), so the per-lane operand is a small
// loop-invariant offset instead of a 64-bit address the compiler may spill.
struct Buf {
  __amdgpu_buffer_rsrc_t r;
  __device__ __forceinline__ Buf(const void* base, int64_t bytes)
      : r(__builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000)) {}
  __device__ __forceinline__ uint4 u4(int off) const {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
  }
  __device__ __forceinline__ float4 f4(int off) const {
    return __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
  }
  __device__ __forceinline__ float f1(int off) const {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
  }
  __device__ __forceinline__ M::frag fr(int off) const { return __builtin_bit_cast(M::frag, u4(off)); }
  // stores: an offset at or past the end drops the store
  __device__ __forceinline__ void st_f32(int off, float v) const {
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, off, 0, 0);
  }
  __device__ __forceinline__ void st_b16(int off, bf16 v) const {
    __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, v), r, off, 0, 0);
  }
  // 8 e4m3 bytes at byte offset off, decoded exactly to a bf16 fragment
  __device__ __forceinline__ M::frag fr_f8(int off, float scale) const {
    const uint2 raw = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
    return __builtin_bit_cast(M::frag, fp8x8_to_bf16x8(raw.x, raw.y, scale));
  }
};

// NC = 128: the whole state; NC = 64: half of its columns (exact: the update
// multiplies the state from the left only), two workgroups per (sequence,
// v-head) with the same per-element arithmetic
template <int MODE, int NC, bool F8 = false>
__global__ __launch_bounds__(kThreads) void state_fwd_wide_kernel(ChunkArgs a) {
  constexpr bool OUT = MODE & kFwdOut, STORE = MODE & kFwdStore;
  constexpr int D = kD, C = kC;
  constexpr int P1 = NC / 32;  // phase-1 column tiles per wave
  constexpr int P2 = NC / 16;  // state column tiles per wave
  static_assert(NC == kD || NC == kD / 2, "whole or half state");
  __shared__ FwdSmem<NC, OUT> sm;
  int n, h, vt;
  if (!state_block(blockIdx.x, a.N, a.Hk, a.G, kD / NC, n, h, vt)) return;
  const int j = h / a.G;
  const int col0 = vt * NC;  // first state column of this workgroup
  const int tid = threadIdx.x, w = wave_id(), lane = lane_id();
  const int r16 = lane & 15, kq = (lane >> 4) * 8;
  const int rt1 = w & 3, cb = P1 * (w >> 2);  // W / O tiles: row tile rt1, column tiles cb .. cb+P1-1
  const int rt2 = w;                          // state tiles: row tile rt2, every column tile

  f32x4 Hr[P2];
#pragma unroll
  for (int i = 0; i < P2; ++i) {
    Hr[i] = zero4();
    if (a.h0) {
      const float* src = a.h0 + ((int64_t)n * a.Hv + h) * D * D;
#pragma unroll
      for (int e = 0; e < 4; ++e) Hr[i][e] = src[(rt2 * 16 + acc_row(e)) * D + col0 + i * 16 + acc_col()];
    }
  }
  auto write_Ht = [&]() {
#pragma unroll
    for (int i = 0; i < P2; ++i) {
      const int c = i * 16 + acc_col(), r = rt2 * 16 + acc_row(0);
      st4_split<E>(&sm.Ht[c][r], &sm.Htl[c][r], Hr[i]);
    }
  };

  // staged operands of the next chunk
  static_assert(kKR == 2, "two 16-byte pieces of each [D][C] tile per thread");
  uint4 kt_h0, kt_h1;  // this thread's pieces of K^T; named, so they stay in registers
  float g_r = 0.f;
  M::frag wkf[4], qf[4];
  f32x4 uf[P1];
  float4 pf[2][2];
  auto load_shared = [&](int ci) {
    const int64_t slot = (int64_t)ci * a.Hv + h;
    const Buf kh((const E*)a.Kt + ((int64_t)ci * a.Hk + j) * D * C, D * C * 2);  // one K^T per k-head
    kt_h0 = kh.u4(tid * 16);
    kt_h1 = kh.u4((tid + kThreads) * 16);
    g_r = Buf(a.gam + slot * C, C * 4).f1((tid & (C - 1)) * 4);  // every thread loads; threads < C use it
  };
  const int a_off = (rt1 * 4 * 64 + lane) * 16;   // lane's piece of Wk's fragment (rt1, 0), fragment order
  auto load_p1 = [&](int ci, int tok0, int len) {
    const int64_t slot = (int64_t)ci * a.Hv + h;
    const Buf wk((const E*)a.Wk + slot * C * D, C * D * 2);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) wkf[ks] = wk.fr(a_off + ks * 1024);
    if constexpr (OUT && F8) {  // e4m3 q rows, decoded exactly on load
      const Buf qb((const uint8_t*)a.q + (int64_t)tok0 * a.sqk + (int64_t)j * D, (int64_t)len * a.sqk);
      const int q_off = (int)((int64_t)(rt1 * 16 + r16) * a.sqk + kq);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) qf[ks] = qb.fr_f8(q_off + ks * 32, a.f8_scale[0]);
    } else if constexpr (OUT) {  // q rows of the chunk; rows past len fall outside the buffer and read zero
      const Buf qb((const E*)a.q + (int64_t)tok0 * a.sqk + (int64_t)j * D, (int64_t)len * a.sqk * 2);
      const int q_off = (int)(((int64_t)(rt1 * 16 + r16) * a.sqk + kq) * 2);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) qf[ks] = qb.fr(q_off + ks * 64);
    }
    const Buf ub(a.U + slot * C * D, C * D * 4);  // accumulator order
#pragma unroll
    for (int i = 0; i < P1; ++i) {
      const float4 u = ub.f4(((rt1 * (D / 16) + col0 / 16 + cb + i) * 64 + lane) * 16);
      uf[i] = f32x4{u.x, u.y, u.z, u.w};
    }
  };
  auto load_p2 = [&](int ci) {
    const Buf pb(a.P + ((int64_t)ci * a.Hv + h) * C * C, C * C * 4);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      if constexpr (MODE == kFwdOut) {  // fragment order (inference preparation)
        pf[ks][0] = pb.f4((((rt1 * 2 + ks) * 2) * 64 + lane) * 16);
        pf[ks][1] = pb.f4((((rt1 * 2 + ks) * 2 + 1) * 64 + lane) * 16);
      } else {
        const int p_off = ((rt1 * 16 + r16) * C + kq) * 4;
        pf[ks][0] = pb.f4(p_off + ks * 128);
        pf[ks][1] = pb.f4(p_off + ks * 128 + 16);
      }
    }
  };

  // the sequence's chunks are consecutive table entries: (first token, length)
  // follow from cu_seqlens, with no table load inside the serial loop
  // the sequence's bounds as scalars (buffer sizes formed from them stay uniform)
  const int c0 = __builtin_amdgcn_readfirstlane(a.seq_chunk0[n]);
  const int c1 = __builtin_amdgcn_readfirstlane(a.seq_chunk0[n + 1]);
  const int s0 = __builtin_amdgcn_readfirstlane(a.cu[n]), s1 = __builtin_amdgcn_readfirstlane(a.cu[n + 1]);
  auto entry = [&](int ci) {
    const int t = s0 + (ci - c0) * C;
    return make_int4(n, t, min(C, s1 - t), 0);
  };
  int4 ent = make_int4(0, 0, 0, 0);
  if (c0 < c1) {
    ent = entry(c0);
    load_shared(c0);
    load_p1(c0, ent.y, ent.z);
    if constexpr (OUT) load_p2(c0);
  }
  write_Ht();
  for (int ci = c0; ci < c1; ++ci) {
    const int tok0 = ent.y, len = ent.z;
    const int64_t slot = (int64_t)ci * a.Hv + h;
    __syncthreads();  // the previous chunk is done with K^T and W^T, and H^T is written
    {  // 16-byte piece e of K^T in fragment order: fragment e / 64 (row tile, k step), lane e % 64
      auto put = [&](int e, uint4 v) {
        const int f = e >> 6, l = e & 63;
        *reinterpret_cast<uint4*>(&sm.Kt[(f >> 1) * 16 + (l & 15)][(f & 1) * 32 + (l >> 4) * 8]) = v;
      };
      put(tid, kt_h0);
      put(tid + kThreads, kt_h1);
    }
    if (tid < C) sm.gam[tid] = g_r;
    __syncthreads();
    // the next chunk's operands, or this chunk's again after the last: loads
    // issued on every path keep the compiler's wait counts exact
    const int cn = ci + 1 < c1 ? ci + 1 : ci;
    const int4 nent = entry(cn);
    load_shared(cn);
    // Stores go after the prefetch loads: the wait for a load also waits for
    // every earlier vector-memory access of the wave.
    if constexpr (STORE) {  // state entering this chunk, for the backward pass
      float* Hg = a.Hc + slot * D * D;
#pragma unroll
      for (int i = 0; i < P2; ++i) store_tile<float>(Hg, D, rt2 * 16, col0 + i * 16, Hr[i], D);
    }

    // phase 1: W = U - Wk H and diag(Gam) Q H on this wave's tiles
    f32x4 x[P1], o[P1];
#pragma unroll
    for (int i = 0; i < P1; ++i) x[i] = o[i] = zero4();
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
      for (int i = 0; i < P1; ++i) {
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
    for (int i = 0; i < P1; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) x[i][e] = uf[i][e] - x[i][e];  // x <- W
    if constexpr (OUT) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float gm = __expf(sm.gam[rt1 * 16 + acc_row(e)]);
#pragma unroll
        for (int i = 0; i < P1; ++i) o[i][e] *= gm;
      }
    }
    load_p1(cn, nent.y, nent.z);  // Wk, q, U of the next chunk
    float dec[4];  // e^{gamma_last - gamma_r} of this lane's rows, 0 past len
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = rt1 * 16 + acc_row(e);
      dec[e] = r < len ? __expf(sm.gam[len - 1] - sm.gam[r]) : 0.f;
    }
#pragma unroll
    for (int i = 0; i < P1; ++i) {
      const int c = (cb + i) * 16 + acc_col(), r = rt1 * 16 + acc_row(0);
      f32x4 xs;
#pragma unroll
      for (int e = 0; e < 4; ++e) xs[e] = x[i][e] * dec[e];
      if constexpr (OUT) {
        st4_split<E>(&sm.Wt[c][r], &sm.Wtl[c][r], x[i]);
        st4_split<E>(&sm.Ws[c][r], &sm.Wsl[c][r], xs);
      } else {
        st4_split<E>(&sm.Wt[c][r], &sm.Wtl[c][r], xs);
      }
      if constexpr (STORE) store_tile<float>(a.W + slot * C * D, D, rt1 * 16, col0 + (cb + i) * 16, x[i], C);
    }
    __syncthreads();

    // phase 2: H <- Gam_last H + K^T diag(e) W;  o = scale (diag(Gam) Q H + P W)
    const float gl = __expf(sm.gam[len - 1]);
#pragma unroll
    for (int i = 0; i < P2; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) Hr[i][e] *= gl;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const M::frag ah = fr(&sm.Kt[rt2 * 16 + r16][ks * 32 + kq]);
#pragma unroll
      for (int i = 0; i < P2; ++i) {
        const int c = i * 16 + r16;
        const M::frag bh = fr(OUT ? &sm.Ws[c][ks * 32 + kq] : &sm.Wt[c][ks * 32 + kq]);
        const M::frag bl = fr(OUT ? &sm.Wsl[c][ks * 32 + kq] : &sm.Wtl[c][ks * 32 + kq]);
        Hr[i] = M::mma(ah, bh, Hr[i]);
        Hr[i] = M::mma(ah, bl, Hr[i]);
      }
    }
    if constexpr (OUT) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        M::frag ph, pl;
        split8(pf[ks][0], pf[ks][1], ph, pl);
#pragma unroll
        for (int i = 0; i < P1; ++i) {
          const int c = (cb + i) * 16 + r16;
          const M::frag bh = fr(&sm.Wt[c][ks * 32 + kq]);
          const M::frag bl = fr(&sm.Wtl[c][ks * 32 + kq]);
          o[i] = M::mma(ph, bh, o[i]);
          o[i] = M::mma(ph, bl, o[i]);
          o[i] = M::mma(pl, bh, o[i]);
        }
      }
      load_p2(cn);
      E* og = (E*)a.o + (int64_t)tok0 * a.Hv * D + (int64_t)h * D;
#pragma unroll
      for (int i = 0; i < P1; ++i) {
#pragma unroll
        for (int e = 0; e < 4; ++e) o[i][e] *= a.scale;
        store_tile<E>(og, (int64_t)a.Hv * D, rt1 * 16, col0 + (cb + i) * 16, o[i], len);
      }
    }
    write_Ht();  // phase 1 (the only reader of H^T) is over for every wave
    ent = nent;
  }
  if (a.ht) {
    float* dst = a.ht + ((int64_t)n * a.Hv + h) * D * D;
#pragma unroll
    for (int i = 0; i < P2; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) dst[(rt2 * 16 + acc_row(e)) * D + col0 + i * 16 + acc_col()] = Hr[i][e];
  }
}

// NC = 128: the whole state; NC = 64: half of its columns, two workgroups per
// (sequence, v-head) (exact: dW's and dH's columns are computed independently)
template <int NC>
__global__ __launch_bounds__(kThreads) void state_bwd_wide_kernel(ChunkArgs a) {
  constexpr int D = kD, C = kC;
  constexpr int P1 = NC / 32;  // dW column tiles per wave
  constexpr int P2 = NC / 16;  // dH column tiles per wave
  __shared__ BwdSmem<NC> sm;
  int n, h, vt;
  if (!state_block(blockIdx.x, a.N, a.Hk, a.G, D / NC, n, h, vt)) return;
  const int col0 = vt * NC;  // first state column of this workgroup
  const int tid = threadIdx.x, w = wave_id(), lane = lane_id();
  const int r16 = lane & 15, kq = (lane >> 4) * 8;
  const int rt1 = w & 3, cb = P1 * (w >> 2);  // dW tiles
  const int rt2 = w;                          // dH tiles: row tile rt2, every column tile

  f32x4 dH[P2];
#pragma unroll
  for (int i = 0; i < P2; ++i) {
    dH[i] = zero4();
    if (a.dht) {
      const float* src = a.dht + ((int64_t)n * a.Hv + h) * D * D;
#pragma unroll
      for (int e = 0; e < 4; ++e) dH[i][e] = src[(rt2 * 16 + acc_row(e)) * D + col0 + i * 16 + acc_col()];
    }
  }
  auto write_dHt = [&]() {
#pragma unroll
    for (int i = 0; i < P2; ++i) {
      const int c = i * 16 + acc_col(), r = rt2 * 16 + acc_row(0);
      st4_split<E>(&sm.dHt[c][r], &sm.dHtl[c][r], dH[i]);
    }
  };

  // staged operands of the next chunk (reverse order).  K, q and P come
  // straight from the layer's k and q rows and the forward's P: the rows of K
  // into LDS, q and P gathered column-wise into this wave's fragments of
  // (Gam q)^T and P^T (a 2- or 4-byte load per element, rows past the chunk's
  // end reading zero), Gam applied and the hi / lo parts split at use.
  const int j = h / a.G;
  uint4 kr_h0, kr_h1;                // this thread's pieces of the K rows (named: registers)
  ColRegs<E, C, NC, kThreads> pO;   // dO of the chunk (this workgroup's columns), gathered column-wise
  float g_r = 0.f;
  float ptf[2][8];                  // P^T rows of this wave's dW tiles
  uint32_t qraw[2][4];              // q columns of its dH tiles (bf16 pairs), Gam not yet applied
  M::frag wth[2], wtl[2];           // Wk^T rows of its dH tiles
  const int64_t lq = a.sqk * 2;     // byte stride of q / k rows
  auto load_shared = [&](int ci, int tok0, int len) {
    const int64_t slot = (int64_t)ci * a.Hv + h;
    // 16-byte piece e of the K rows: row e / 16, columns (e % 16) * 8 ..
    const Buf kb((const E*)a.k + (int64_t)tok0 * a.sqk + (int64_t)j * D, (int64_t)len * lq);
    kr_h0 = kb.u4((int)((tid >> 4) * lq) + (tid & 15) * 16);
    kr_h1 = kb.u4((int)(((tid + kThreads) >> 4) * lq) + (tid & 15) * 16);
    pO.load((const E*)a.d_o + (int64_t)tok0 * a.Hv * D + (int64_t)h * D + col0, (int64_t)a.Hv * D, len);
    g_r = Buf(a.gam + slot * C, C * 4).f1((tid & (C - 1)) * 4);  // every thread loads; threads < C use it
  };
  // P^T[c][s] = P[s][c]: this lane's column c = rt1 * 16 + r16, rows s = ks * 32 + kq + u
  auto load_p1 = [&](int ci) {
    const Buf pb(a.P + ((int64_t)ci * a.Hv + h) * C * C, C * C * 4);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int u = 0; u < 8; ++u) ptf[ks][u] = pb.f1(((ks * 32 + kq + u) * C + rt1 * 16 + r16) * 4);
  };
  // (Gam q)^T[d][s]: this lane's d = rt2 * 16 + r16, positions s = ks * 32 + kq + u
  auto load_p2 = [&](int ci, int tok0, int len) {
    const int64_t o = ((int64_t)ci * a.Hv + h) * D * C;
    const int t_off = ((rt2 * 16 + r16) * C + kq) * 2;  // lane's fragment offset in a [D][C] bf16 tile
    const Buf wh((const E*)a.Wth + o, D * C * 2), wl((const E*)a.Wtl + o, D * C * 2);
    const Buf qb((const E*)a.q + (int64_t)tok0 * a.sqk + (int64_t)j * D, (int64_t)len * lq);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      wth[ks] = wh.fr(t_off + ks * 64);
      wtl[ks] = wl.fr(t_off + ks * 64);
#pragma unroll
      for (int u = 0; u < 8; u += 2) {
        const int s = ks * 32 + kq + u, off = (rt2 * 16 + r16) * 2;
        const uint32_t x0 = __builtin_amdgcn_raw_buffer_load_b16(qb.r, (int)(s * lq) + off, 0, 0);
        const uint32_t x1 = __builtin_amdgcn_raw_buffer_load_b16(qb.r, (int)((s + 1) * lq) + off, 0, 0);
        qraw[ks][u / 2] = (x0 & 0xFFFFu) | (x1 << 16);
      }
    }
  };

  // the sequence's bounds as scalars (buffer sizes formed from them stay uniform)
  const int c0 = __builtin_amdgcn_readfirstlane(a.seq_chunk0[n]);
  const int c1 = __builtin_amdgcn_readfirstlane(a.seq_chunk0[n + 1]);
  const int s0 = __builtin_amdgcn_readfirstlane(a.cu[n]), s1 = __builtin_amdgcn_readfirstlane(a.cu[n + 1]);
  auto entry = [&](int ci) {
    const int t = s0 + (ci - c0) * C;
    return make_int4(n, t, min(C, s1 - t), 0);
  };
  int4 ent = make_int4(0, 0, 0, 0);
  if (c0 < c1) {
    ent = entry(c1 - 1);
    load_shared(c1 - 1, ent.y, ent.z);
    load_p1(c1 - 1);
    load_p2(c1 - 1, ent.y, ent.z);
  }
  write_dHt();
  for (int ci = c1 - 1; ci >= c0; --ci) {
    const int len = ent.z;
    const int64_t slot = (int64_t)ci * a.Hv + h;
    __syncthreads();  // the previous chunk is done with [dO^T | dW^T] and K~, and dH^T is written
    {  // 16-byte piece e: row e / 16, columns (e % 16) * 8 ..
      const int e0 = tid, e1 = tid + kThreads;
      *reinterpret_cast<uint4*>(&sm.Kr[e0 >> 4][(e0 & 15) * 8]) = kr_h0;
      *reinterpret_cast<uint4*>(&sm.Kr[e1 >> 4][(e1 & 15) * 8]) = kr_h1;
    }
    pO.store(&sm.OW[0][0], kLD2C);
    if (tid < C) {
      sm.gam[tid] = g_r;
      sm.Gm[tid] = __expf(g_r);
    }
    __syncthreads();
    // the next chunk's operands (the previous one), or this chunk's again
    // after the first: loads issued on every path keep the wait counts exact
    const int cn = ci > c0 ? ci - 1 : ci;
    const int4 nent = entry(cn);
    load_shared(cn, nent.y, nent.z);

    // phase 1: dW = scale P^T dO + diag(e) K dH on this wave's tiles, one tile at a time
    M::frag ph[2], pl[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
      split8(make_float4(ptf[ks][0], ptf[ks][1], ptf[ks][2], ptf[ks][3]),
             make_float4(ptf[ks][4], ptf[ks][5], ptf[ks][6], ptf[ks][7]), ph[ks], pl[ks]);
    load_p1(cn);  // P^T of the next chunk
    // Stores go after this chunk's prefetch loads: the wait for a load also
    // waits for every earlier vector-memory access of the wave.
    {  // gradient w.r.t. the state leaving this chunk
      float* dst = a.dHn + slot * D * D;
#pragma unroll
      for (int i = 0; i < P2; ++i) store_tile<float>(dst, D, rt2 * 16, col0 + i * 16, dH[i], D);
    }
    float dec[4];  // e^{gamma_last - gamma_s} of this lane's rows s, 0 past len
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = rt1 * 16 + acc_row(e);
      dec[e] = r < len ? __expf(sm.gam[len - 1] - sm.gam[r]) : 0.f;
    }
#pragma unroll
    for (int i = 0; i < P1; ++i) {
      const int c = (cb + i) * 16 + r16;
      f32x4 p = zero4(), kd = zero4();
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const M::frag b = fr(&sm.OW[c][ks * 32 + kq]);
        p = M::mma(ph[ks], b, p);
        p = M::mma(pl[ks], b, p);
      }
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const M::frag ah = fr(&sm.Kr[rt1 * 16 + r16][ks * 32 + kq]);
        const M::frag bh = fr(&sm.dHt[c][ks * 32 + kq]);
        const M::frag bl = fr(&sm.dHtl[c][ks * 32 + kq]);
        kd = M::mma(ah, bh, kd);
        kd = M::mma(ah, bl, kd);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) kd[e] = dec[e] * kd[e] + a.scale * p[e];  // kd <- dW
      store_tile_t(a.dWt + slot * D * C, C, rt1 * 16, col0 + (cb + i) * 16, kd);
      const int cc = (cb + i) * 16 + acc_col(), r = rt1 * 16 + acc_row(0);
      st4_split<E>(&sm.OW[cc][C + r], &sm.dWl[cc][r], kd);
      __builtin_amdgcn_sched_barrier(0);
    }
    __syncthreads();

    // phase 2: dH <- Gam_last dH + scale (diag(Gam) Q)^T dO - Wk^T dW
    const float gl = __expf(sm.gam[len - 1]);
    M::frag qth[2], qtl[2];  // (Gam q)^T, hi / lo (the values the preparation would store)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const float4 g0 = *reinterpret_cast<const float4*>(&sm.Gm[ks * 32 + kq]);
      const float4 g1 = *reinterpret_cast<const float4*>(&sm.Gm[ks * 32 + kq + 4]);
      const float gs[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const uint32_t b = (qraw[ks][u / 2] >> (16 * (u & 1))) & 0xFFFFu;
        v[u] = gs[u] * bf2f((bf16)b);
      }
      split8(make_float4(v[0], v[1], v[2], v[3]), make_float4(v[4], v[5], v[6], v[7]), qth[ks], qtl[ks]);
    }
#pragma unroll
    for (int i = 0; i < P2; ++i) {
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
      __builtin_amdgcn_sched_barrier(0);  // keep the next tile's fragment loads out of this one's registers
    }
    load_p2(cn, nent.y, nent.z);
    write_dHt();  // phase 1 (the only reader of dH^T) is over for every wave
    ent = nent;
  }
  if (a.dh0) {
    float* dst = a.dh0 + ((int64_t)n * a.Hv + h) * D * D;
#pragma unroll
    for (int i = 0; i < P2; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) dst[(rt2 * 16 + acc_row(e)) * D + col0 + i * 16 + acc_col()] = dH[i][e];
  }
}

}  // namespace

// ---------------------------------------------------------------------------
// Forward state pass over 16-column tiles of the state, for chains too few to
// fill the chip (a single long sequence): eight workgroups per (sequence,
// v-head), each carrying 16 state columns through the whole sequence with
// eight compute waves (and, without fp8 inputs, a ninth that prefetches into
// L2).  Every operand that one wave reads alone goes straight from global
// memory (L2) into matrix-core fragments, in the order the preparation wrote it:
// rows of Wk and the U tile (waves 0-3), rows of q and P (waves 4-7), K^T rows
// of state row tile w (wave w); only H^T and W^T, which all waves read, pass
// through LDS.  The next chunk's operands load into a second register set at
// the start of each chunk.  Same arithmetic as the whole-state pass, per
// element.
// ---------------------------------------------------------------------------
struct ColsSmem {
  E Ht[16][kLDQ];   // H^T: Ht[c][r] = H[r][c], this workgroup's 16 columns
  E Htl[16][kLDQ];
  E Wt[16][kLDC];   // W^T (with OUT, for P W), else (diag(e) W)^T
  E Wtl[16][kLDC];
  E Ws[16][kLDC];   // (diag(e) W)^T for the state update (OUT)
  E Wsl[16][kLDC];
  // per chunk, double-buffered (written one chunk ahead by wave 0):
  float eg[2][kC];  // e^{gamma_r}
  float es[2][kC];  // e^{gamma_last - gamma_r}, 0 past the chunk's length
  float gl[2];      // e^{gamma_last}
};

// one wave's operands of one chunk
struct ColsOps {
  M::frag af[4];    // rows of Wk (waves 0-3) or q (waves 4-7), row tile w & 3
  f32x4 uf;         // U on the accumulator tile (waves 0-3)
  float4 pf[2][2];  // P rows (waves 4-7)
  M::frag ktf[2];   // K^T rows of state tile w
  float g;          // gamma of row `lane`
};

// A ninth wave per workgroup reads one dword of each 64 bytes of the chain's
// operands kAhead chunks ahead, so the compute waves' own loads find them in L2
// (their fragment loads missing to HBM cost ~12% of the pass).  The compute
// waves could not do this themselves: the vector-memory counter retires in
// order, so each of their own next-chunk loads would wait for those misses.
// (Not with fp8 inputs: that form needs the registers a ninth wave would take.)
constexpr int kColsWaves = 8, kAhead = 3;
template <bool F8> constexpr int cols_threads() { return (kColsWaves + (F8 ? 0 : 1)) * kWave; }

template <int MODE, bool F8>
__global__ __launch_bounds__(cols_threads<F8>()) void state_fwd_cols_kernel(ChunkArgs a) {
  constexpr bool OUT = MODE & kFwdOut, STORE = MODE & kFwdStore;
  constexpr int D = kD, C = kC;
  constexpr int kOff = 0x40000000;  // a buffer offset past every buffer's end: the store is dropped
  __shared__ ColsSmem sm;
  int n, h, vt;
  if (!state_block(blockIdx.x, a.N, a.Hk, a.G, kD / 16, n, h, vt)) return;
  const int j = h / a.G;
  const int col0 = vt * 16;
  const int w = __builtin_amdgcn_readfirstlane(wave_id()), lane = lane_id();
  const int r16 = lane & 15, kq = (lane >> 4) * 8;
  // waves 0-3 form W = U - Wk H on row tile w; waves 4-7 form
  // diag(Gam) Q H + P W on row tile w - 4; wave w carries state row tile w
  const bool xw = w < 4;
  const int rt1 = w & 3;
  const int rs = w;

  if (!F8 && w == kColsWaves) {  // the prefetch wave: the same barriers, no other work
    const int pc0 = __builtin_amdgcn_readfirstlane(a.seq_chunk0[n]);
    const int pc1 = __builtin_amdgcn_readfirstlane(a.seq_chunk0[n + 1]);
    // the chain's lines of one chunk, 64 bytes each: Wk [0, 256), U [256, 768),
    // P [768, 1024), K^T [1024, 1280), q in load order [1280, 1536); this
    // workgroup takes 192 of them, 64 per instruction (one region each)
    auto touch = [&](uint32_t (&t)[3], int cj) {
      const bool ok = cj < pc1;
      const int64_t slot = (int64_t)cj * a.Hv + h, kslot = (int64_t)cj * a.Hk + j;
#pragma unroll
      for (int i = 0; i < 3; ++i) {
        const int L0 = vt * 192 + i * 64;  // a multiple of 64: one region per instruction
        const void* base;
        int bytes = 16384, r0;
        if (L0 < 256) { base = (const E*)a.Wk + slot * C * D; r0 = 0; }
        else if (L0 < 768) { base = a.U + slot * C * D; bytes = 32768; r0 = 256; }
        else if (L0 < 1024) { base = a.P + slot * C * C; bytes = OUT ? 16384 : 0; r0 = 768; }
        else if (L0 < 1280) { base = (const E*)a.Kt + kslot * D * C; r0 = 1024; }
        else { base = (const E*)a.Qf + kslot * C * D; bytes = a.q_frag ? 16384 : 0; r0 = 1280; }
        t[i] = __builtin_bit_cast(uint32_t, buf_load_f32((const float*)base, ok ? bytes : 0, (L0 - r0 + lane) * 64));
      }
    };
    auto consume = [](const uint32_t (&t)[3]) { asm volatile("" ::"v"(t[0]), "v"(t[1]), "v"(t[2])); };
    // chunk ci: the two barriers of the compute waves' chunk step, touches of
    // chunk ci + kAhead, and the touches of two chunks ago taken (long returned)
    auto pstep = [&](int ci, uint32_t (&issue)[3], const uint32_t (&old)[3]) {
      __syncthreads();
      touch(issue, ci + kAhead);
      __syncthreads();
      consume(old);
    };
    uint32_t g0[3] = {0u, 0u, 0u}, g1[3] = {0u, 0u, 0u}, g2[3] = {0u, 0u, 0u};
    for (int ci = pc0; ci < pc1; ci += 3) {
      pstep(ci, g0, g1);
      if (ci + 1 >= pc1) break;
      pstep(ci + 1, g1, g2);
      if (ci + 2 >= pc1) break;
      pstep(ci + 2, g2, g0);
    }
    consume(g0);
    consume(g1);
    consume(g2);
    return;
  }

  f32x4 Hr = zero4();
  if (a.h0) {
    const float* src = a.h0 + ((int64_t)n * a.Hv + h) * D * D;
#pragma unroll
    for (int e = 0; e < 4; ++e) Hr[e] = src[(rs * 16 + acc_row(e)) * D + col0 + acc_col()];
  }
  auto write_Ht = [&]() {
    const int c = acc_col(), r = rs * 16 + acc_row(0);
    st4_split<E>(&sm.Ht[c][r], &sm.Htl[c][r], Hr);
  };

  // the sequence's chunks are consecutive table entries: (first token, length)
  // follow from cu_seqlens
  // the sequence's bounds as scalars (buffer sizes formed from them stay uniform)
  const int c0 = __builtin_amdgcn_readfirstlane(a.seq_chunk0[n]);
  const int c1 = __builtin_amdgcn_readfirstlane(a.seq_chunk0[n + 1]);
  const int s0 = __builtin_amdgcn_readfirstlane(a.cu[n]), s1 = __builtin_amdgcn_readfirstlane(a.cu[n + 1]);
  auto entry = [&](int ci) {
    const int t = s0 + (ci - c0) * C;
    return make_int2(t, min(C, s1 - t));
  };

  // Every wave issues the same number of vector-memory instructions, in the
  // same order, on every path (loads of the last chunk repeat it; rows past a
  // chunk's end and the other role's stores go to an offset past the buffer's
  // end, which the hardware drops), so the compiler's wait counts are exact
  // and the next chunk's loads stay in flight through the current one.
  const int a_off = (rt1 * 4 * 64 + lane) * 16;   // lane's piece of Wk's fragment (rt1, 0), fragment order
  auto load = [&](ColsOps& op, int ci) {
    const int64_t slot = (int64_t)ci * a.Hv + h;
    const int2 en = entry(ci);
    op.g = Buf(a.gam + slot * C, C * 4).f1(lane * 4);
    const int64_t q0 = (int64_t)en.x * a.sqk + (int64_t)j * D;   // q rows past the chunk's length read zero
    const int q_row = (rt1 * 16 + r16) * (int)a.sqk + kq;        // element offset of the lane's q piece
    if constexpr (F8) {  // e4m3 q rows, decoded exactly on load; waves 0-3 keep the Wk fragments
      const Buf wk((const E*)a.Wk + slot * C * D, C * D * 2);
      const Buf qb((const uint8_t*)a.q + q0, (int64_t)en.y * a.sqk);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const M::frag fw = wk.fr(xw ? a_off + ks * 1024 : kOff);
        const M::frag fq = qb.fr_f8(xw ? kOff : q_row + ks * 32, a.f8_scale[0]);
        op.af[ks] = xw ? fw : fq;
      }
    } else if constexpr (MODE == kFwdOut) {  // q rows in fragment order, from the preparation (q_frag)
      const Buf ab(xw ? (const void*)((const E*)a.Wk + slot * C * D)
                      : (const void*)((const E*)a.Qf + ((int64_t)ci * a.Hk + j) * C * D), C * D * 2);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) op.af[ks] = ab.fr(a_off + ks * 1024);
    } else {
      const Buf ab(xw ? (const void*)((const E*)a.Wk + slot * C * D) : (const void*)((const E*)a.q + q0),
                   xw ? (int64_t)C * D * 2 : (OUT ? (int64_t)en.y * a.sqk * 2 : 0));
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) op.af[ks] = ab.fr(xw ? a_off + ks * 1024 : q_row * 2 + ks * 64);
    }
    const Buf ub(a.U + slot * C * D, C * D * 4);  // accumulator order
    const float4 u = ub.f4(xw ? ((rt1 * (D / 16) + vt) * 64 + lane) * 16 : kOff);
    op.uf = f32x4{u.x, u.y, u.z, u.w};
    const Buf pb(a.P + slot * C * C, OUT ? C * C * 4 : 0);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      if constexpr (MODE == kFwdOut) {  // fragment order (inference preparation)
        op.pf[ks][0] = pb.f4(xw ? kOff : (((rt1 * 2 + ks) * 2) * 64 + lane) * 16);
        op.pf[ks][1] = pb.f4(xw ? kOff : (((rt1 * 2 + ks) * 2 + 1) * 64 + lane) * 16);
      } else {
        const int p_off = xw ? kOff : ((rt1 * 16 + r16) * C + kq) * 4 + ks * 128;
        op.pf[ks][0] = pb.f4(p_off);
        op.pf[ks][1] = pb.f4(p_off + 16);
      }
    }
    const Buf kb((const E*)a.Kt + ((int64_t)ci * a.Hk + j) * D * C, D * C * 2);  // fragment order, one per k-head
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) op.ktf[ks] = kb.fr(((rs * 2 + ks) * 64 + lane) * 16);
  };
  auto put_g = [&](const ColsOps& op, int b, int len) {  // wave 0: a chunk's decay factors into buffer b
    const float g_last = __shfl(op.g, len - 1, kWave);
    sm.eg[b][lane] = __expf(op.g);
    sm.es[b][lane] = lane < len ? __expf(g_last - op.g) : 0.f;
    if (lane == 0) sm.gl[b] = __expf(g_last);
  };

  auto step = [&](int ci, const ColsOps& cur, ColsOps& nxt) {
    const int2 en = entry(ci);
    const int tok0 = en.x, len = en.y;
    const int b = (ci - c0) & 1;
    const int64_t slot = (int64_t)ci * a.Hv + h;
    const int cn = ci + 1 < c1 ? ci + 1 : ci;
    __syncthreads();  // H^T and this chunk's decay factors are written, and W^T is free
    load(nxt, cn);
    if constexpr (STORE) {  // state entering this chunk, for the backward pass
      const Buf hb(a.Hc + slot * D * D, D * D * 4);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        hb.st_f32(((rs * 16 + acc_row(e)) * D + col0 + acc_col()) * 4, Hr[e]);
    }

    // phase 1: W = U - Wk H (waves 0-3) or diag(Gam) Q H (waves 4-7) on row tile rt1
    f32x4 x = zero4();
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const M::frag bh = fr(&sm.Ht[r16][ks * 32 + kq]);
      const M::frag bl = fr(&sm.Htl[r16][ks * 32 + kq]);
      x = M::mma(cur.af[ks], bh, x);
      x = M::mma(cur.af[ks], bl, x);
    }
    if (xw) {
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = cur.uf[e] - x[e];  // x <- W
      const int c = acc_col(), r = rt1 * 16 + acc_row(0);
      f32x4 xs;  // rows of W times e^{gamma_last - gamma_r}, 0 past len
#pragma unroll
      for (int e = 0; e < 4; ++e) xs[e] = x[e] * sm.es[b][r + e];
      if constexpr (OUT) {
        st4_split<E>(&sm.Wt[c][r], &sm.Wtl[c][r], x);
        st4_split<E>(&sm.Ws[c][r], &sm.Wsl[c][r], xs);
      } else {
        st4_split<E>(&sm.Wt[c][r], &sm.Wtl[c][r], xs);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] *= sm.eg[b][rt1 * 16 + acc_row(e)];
    }
    __syncthreads();

    // phase 2: H <- Gam_last H + K^T diag(e) W;  o = scale (diag(Gam) Q H + P W)
    const float gl = sm.gl[b];
#pragma unroll
    for (int e = 0; e < 4; ++e) Hr[e] *= gl;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const M::frag bh = fr(OUT ? &sm.Ws[r16][ks * 32 + kq] : &sm.Wt[r16][ks * 32 + kq]);
      const M::frag bl = fr(OUT ? &sm.Wsl[r16][ks * 32 + kq] : &sm.Wtl[r16][ks * 32 + kq]);
      Hr = M::mma(cur.ktf[ks], bh, Hr);
      Hr = M::mma(cur.ktf[ks], bl, Hr);
    }
    if (OUT && !xw) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        M::frag ph, pl;
        split8(cur.pf[ks][0], cur.pf[ks][1], ph, pl);
        const M::frag bh = fr(&sm.Wt[r16][ks * 32 + kq]);
        const M::frag bl = fr(&sm.Wtl[r16][ks * 32 + kq]);
        x = M::mma(ph, bh, x);
        x = M::mma(ph, bl, x);
        x = M::mma(pl, bh, x);
      }
    }
    // tile stores, issued by every wave in the modes that have them: W (waves
    // 0-3, STORE) and o (waves 4-7, OUT); the other role's, and rows past the
    // chunk's end, go past the buffer's end
    if constexpr (STORE) {
      const Buf wb(a.W + slot * C * D, C * D * 4);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        wb.st_f32(xw ? ((rt1 * 16 + acc_row(e)) * D + col0 + acc_col()) * 4 : kOff, x[e]);
    }
    if constexpr (OUT) {
      const int ld = a.Hv * D;
      const Buf ob((E*)a.o + (int64_t)tok0 * ld + (int64_t)h * D, ((int64_t)(len - 1) * ld + D) * 2);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = rt1 * 16 + acc_row(e);
        ob.st_b16(!xw && r < len ? (r * ld + col0 + acc_col()) * 2 : kOff, f2bf(x[e] * a.scale));
      }
    }
    write_Ht();  // phase 1 (the only reader of H^T) is over for every wave
    if (w == 0 && ci + 1 < c1) put_g(nxt, b ^ 1, entry(ci + 1).y);  // read after the next barrier
  };

  ColsOps A, B;
  if (c0 < c1) {
    load(A, c0);
    if (w == 0) put_g(A, 0, entry(c0).y);
  }
  write_Ht();
  for (int ci = c0; ci < c1; ci += 2) {
    step(ci, A, B);
    if (ci + 1 >= c1) break;
    step(ci + 1, B, A);
  }
  if (a.ht) {
    float* dst = a.ht + ((int64_t)n * a.Hv + h) * D * D;
#pragma unroll
    for (int e = 0; e < 4; ++e) dst[(rs * 16 + acc_row(e)) * D + col0 + acc_col()] = Hr[e];
  }
}

template <int NC>
static void launch_fwd_nc(const ChunkArgs& a, hipStream_t st, int mode, bool f8) {
  const dim3 grid(state_grid(a.N, a.Hk, a.G, kD / NC));
  if (f8) state_fwd_wide_kernel<kFwdOut, NC, true><<<grid, kThreads, 0, st>>>(a);  // fp8 inputs: inference only
  else if (mode == kFwdOut) state_fwd_wide_kernel<kFwdOut, NC><<<grid, kThreads, 0, st>>>(a);
  else if (mode == kFwdStore) state_fwd_wide_kernel<kFwdStore, NC><<<grid, kThreads, 0, st>>>(a);
  else state_fwd_wide_kernel<kFwdBoth, NC><<<grid, kThreads, 0, st>>>(a);
}

void launch_state_fwd_wide(const ChunkArgs& a, hipStream_t st, int mode, bool half, bool f8) {
  if (half) launch_fwd_nc<kD / 2>(a, st, mode, f8);
  else launch_fwd_nc<kD>(a, st, mode, f8);
}

void launch_state_fwd_cols(const ChunkArgs& a, hipStream_t st, int mode, bool f8) {
  const dim3 grid(state_grid(a.N, a.Hk, a.G, kD / 16));
  if (f8) state_fwd_cols_kernel<kFwdOut, true><<<grid, cols_threads<true>(), 0, st>>>(a);  // fp8 inputs: inference only
  else if (mode == kFwdOut) state_fwd_cols_kernel<kFwdOut, false><<<grid, cols_threads<false>(), 0, st>>>(a);
  else if (mode == kFwdStore) state_fwd_cols_kernel<kFwdStore, false><<<grid, cols_threads<false>(), 0, st>>>(a);
  else state_fwd_cols_kernel<kFwdBoth, false><<<grid, cols_threads<false>(), 0, st>>>(a);
}

void launch_state_bwd_wide(const ChunkArgs& a, hipStream_t st, bool half) {
  if (half) state_bwd_wide_kernel<64><<<dim3(state_grid(a.N, a.Hk, a.G, 2)), kThreads, 0, st>>>(a);
  else state_bwd_wide_kernel<128><<<dim3(state_grid(a.N, a.Hk, a.G, 1)), kThreads, 0, st>>>(a);
}

}  // namespace gdn
