// Shared pieces of the chunked gated-delta-rule kernels (forward and backward).
#pragma once

#include <utility>

#include "gdn_common.cuh"
#include "gdn_internal.h"

namespace gdn {

constexpr int kChunkThreads = 256;  // 4 waves per workgroup
constexpr int kChunkWaves = kChunkThreads / kWave;
constexpr int kNumCUs = 256;        // MI355X: 8 XCDs x 32 compute units

// What a forward pass over the chunks produces: the output (o and the final
// states), the per-chunk products the backward reads (the preparation pass's
// pre-transposed operands, the entering states H_c and W), or both at once.
enum FwdMode { kFwdOut = 1, kFwdStore = 2, kFwdBoth = 3 };

struct ChunkArgs {
  // inputs
  const void* q;
  const void* k;
  const void* v;
  int64_t sqk, sv;
  const float* g;
  const float* beta;
  // raw gate inputs (the fused-gate entry points; g and beta are then NULL):
  // g = -exp(A_log[h]) softplus(ga + dt_bias[h]), beta = sigmoid(gb)
  const float* ga;       // [T][Hv]
  const float* gb;       // [T][Hv]
  const float* A_log;    // [Hv]
  const float* dt_bias;  // [Hv]
  const int32_t* cu;
  const float* h0;
  // forward outputs
  void* o;
  float* ht;
  // backward inputs / outputs
  const void* d_o;
  const float* dht;
  void* dq;
  void* dk;
  void* dv;
  float* dg;
  float* dbeta;
  float* dh0;
  // fused-gate backward: gradients w.r.t. the raw gate inputs (dg, dbeta NULL)
  float* da;             // [T][Hv]
  float* db;             // [T][Hv]
  float* gpart;          // workspace [2][max_chunks][Hv]: per-chunk sums of dg g and da
  // sizes
  int N, T, Hk, Hv, G, max_chunks;
  float scale;
  int kt_plain;  // the preparation writes Kt = k_s^T unscaled (bf16, d = 128, chunk 64: the wide and 16-column passes)
  float f8_scale[3];  // fp8 inputs: power-of-two scales of q, k and v (q, k, v then point to e4m3 bytes)
  // workspace
  const int32_t* table;       // [max_chunks][4]
  const int32_t* seq_chunk0;  // [N+1]
  // (bf16, d = 128, chunk 64: Wk and K^T in A-fragment order, U in accumulator
  // order and the inference P in split A-fragment order -- af_off, acc_off,
  // pf_off below -- and the plain K^T once per (chunk, k-head))
  void* Wk;                   // [slot][C][D]
  float* U;                   // [slot][C][D]
  float* P;                   // [slot][C][C]
  void* Kt;                   // [slot][D][C]  (e_s k_s)^T, e_s = e^{gamma_last - gamma_s}; k_s^T with kt_plain ([chunk * Hk + k-head])
  void* Ktl;                  //               its lo part (bf16 only; not written with kt_plain)
  void* Qf;                   // [chunk * Hk + k-head][C][D] q rows in fragment order (written when q_frag)
  int q_frag;                 // the inference forward's 16-column state pass reads q from Qf
  // backward only: operands of the reverse state pass, transposed once per chunk
  float* Ptr;                 // [slot][C][C]  P^T
  float* Tw;                  // [slot][C][C]  T = (I + A)^-1 (for the WY gradients)
  void* Krh;                  // [slot][C][D]  rows e_s k_s (hi); rows k_s with kt_plain
  void* Krl;                  //               (lo; not written with kt_plain)
  void* Wth;                  // [slot][D][C]  Wk^T (hi)
  void* Wtl;                  //               (lo)
  void* Qth;                  // [slot][D][C]  (Gam_r q_r)^T (hi)
  void* Qtl;                  //               (lo)
  float* gam;                 // [slot][C]
  float* Hc;                  // [slot][D][D]  state entering the chunk
  float* W;                   // [slot][C][D]  W = U - Wk Hc
  float* dHn;                 // [slot][D][D]  gradient w.r.t. the state leaving the chunk
  float* dW;                  // [slot][C][D]
  float* dWt;                 // [slot][D][C]  dW transposed
  float* dT;                  // [slot][C][C]
  float* dWkt;                // [slot][D][C]  dWk transposed
  float* dQs;                 // [slot][C][D]  scale diag(Gam) dO Hc^T
  float* dKh;                 // [slot][C][D]  diag(e) W dHn^T
  float* dP;                  // [slot][C][C]  scale dO W^T (lower-inclusive, rows < len)
  float* hdot;                // [slot]        <Hc, dHn>
};


// g and beta of token t, v-head h: the caller's arrays, or computed from the
// raw gate inputs (the same functions as gdn_gates).  In two steps: *_raw
// loads (the caller's value, or a / b) and *_fin finishes, at first use, so
// that a prefetched gate does not force a wait for the loads issued with it
// (the vector-memory counter retires in order).
struct GateRaw {  // the caller's g (A, dt unused), or a with A_log[h] and dt_bias[h]
  float x, A, dt;
};
// one float at byte offset off through a buffer over [base, base + bytes):
// offsets past the end read zero (bytes = 0: no memory access at all)
__device__ __forceinline__ float buf_load_f32(const float* base, int bytes, int off) {
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(base), 0, bytes, 0x00020000);
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}
__device__ __forceinline__ GateRaw chunk_g_raw(const ChunkArgs& a, int64_t t, int h) {
  if (a.ga) return GateRaw{a.ga[t * a.Hv + h], a.A_log[h], a.dt_bias[h]};
  return GateRaw{a.g[t * a.Hv + h], 0.f, 0.f};
}
__device__ __forceinline__ float chunk_g_fin(const ChunkArgs& a, const GateRaw& r) {
  return a.ga ? -__expf(r.A) * gate_softplus(r.x + r.dt) : r.x;
}
__device__ __forceinline__ float chunk_beta_raw(const ChunkArgs& a, int64_t t, int h) {
  return a.gb ? a.gb[t * a.Hv + h] : a.beta[t * a.Hv + h];
}
__device__ __forceinline__ float chunk_beta_fin(const ChunkArgs& a, float raw) {
  return a.gb ? gate_sigmoid(raw) : raw;
}

template <typename E> struct Pad {
  static constexpr int E16 = 16 / (int)sizeof(E);  // elements per 16 bytes
};

// bf16 operands carry a second "lo" part (x - bf16(x)) so that products that
// decide the output keep ~16 significant bits; float operands need none.
template <typename E> struct Split { static constexpr bool on = false; };
template <> struct Split<bf16> { static constexpr bool on = true; };

template <typename E>
__device__ __forceinline__ void split_store(E* hi, E* lo, float x) {
  const E h = from_f<E>(x);
  *hi = h;
  if constexpr (Split<E>::on) *lo = from_f<E>(x - to_f<E>(h));
}

// 4 consecutive elements: load as floats / store from floats.
template <typename E>
__device__ __forceinline__ void ld4(const E* p, float* o) {
  if constexpr (sizeof(E) == 2) {
    const uint2 u = *reinterpret_cast<const uint2*>(p);
    const E* e = reinterpret_cast<const E*>(&u);
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = to_f<E>(e[i]);
  } else {
    const float4 u = *reinterpret_cast<const float4*>(p);
    o[0] = u.x; o[1] = u.y; o[2] = u.z; o[3] = u.w;
  }
}
template <typename E>
__device__ __forceinline__ void st4(E* p, f32x4 v) {
  if constexpr (sizeof(E) == 2) {
    uint2 u;
    E* e = reinterpret_cast<E*>(&u);
#pragma unroll
    for (int i = 0; i < 4; ++i) e[i] = from_f<E>(v[i]);
    *reinterpret_cast<uint2*>(p) = u;
  } else {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  }
}

// Accumulator-tile layout, for fp32 tensors that one kernel writes and another
// reads back as the same 16x16 MFMA accumulator tiles: tile (rt, ct) of a grid
// with TPR tiles per row sits at ((rt * TPR + ct) * 64 + lane) * 4, so a lane
// moves its four values in one 16-byte access and a wave moves 1 KiB
// contiguous.
__device__ __forceinline__ void store_acc(float* base, int tpr, int rt, int ct, f32x4 v) {
  *reinterpret_cast<f32x4*>(base + ((int64_t)(rt * tpr + ct) * kWave + lane_id()) * 4) = v;
}
__device__ __forceinline__ f32x4 load_acc(const float* base, int tpr, int rt, int ct) {
  return *reinterpret_cast<const f32x4*>(base + ((int64_t)(rt * tpr + ct) * kWave + lane_id()) * 4);
}

// Element load/store of one accumulator tile straight to/from global memory.
template <typename E>
__device__ __forceinline__ void store_tile(E* base, int64_t ld, int r0, int c0, f32x4 v, int rows_valid) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = r0 + acc_row(i);
    if (r < rows_valid) base[(int64_t)r * ld + c0 + acc_col()] = from_f<E>(v[i]);
  }
}

// one accumulator tile stored transposed: dst[(c0 + col) * ld + r0 + row]
// (each lane writes 4 consecutive rows = one 16-byte vector for float)
__device__ __forceinline__ void store_tile_t(float* dst, int64_t ld, int r0, int c0, f32x4 v) {
  *reinterpret_cast<float4*>(dst + (int64_t)(c0 + acc_col()) * ld + r0 + acc_row(0)) = make_float4(v[0], v[1], v[2], v[3]);
}

// the 4 accumulator values of a lane (consecutive rows r..r+3 of one column)
// written to hi[0..3] (and lo[0..3]) -- one 8-byte (bf16) or 16-byte store each
template <typename E>
__device__ __forceinline__ void st4_split(E* hi, E* lo, f32x4 v) {
  if constexpr (sizeof(E) == 2) {
    uint2 h, l;
    uint16_t* hh = reinterpret_cast<uint16_t*>(&h);
    uint16_t* ll = reinterpret_cast<uint16_t*>(&l);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bf16 b = f2bf(v[i]);
      hh[i] = b;
      ll[i] = f2bf(v[i] - bf2f(b));
    }
    *reinterpret_cast<uint2*>(hi) = h;
    if constexpr (Split<E>::on) *reinterpret_cast<uint2*>(lo) = l;
  } else {
    *reinterpret_cast<float4*>(hi) = make_float4(v[0], v[1], v[2], v[3]);
  }
}

__device__ __forceinline__ int4 chunk_entry(const int32_t* table, int ci) {
  return reinterpret_cast<const int4*>(table)[ci];
}

template <typename E, int D, int C>
struct PrepSmem {
  static constexpr int LDQ = D + Pad<E>::E16;   // [C][LDQ]  E
  static constexpr int LDCE = C + Pad<E>::E16;  // [*][LDCE] E
  static constexpr int LDCF = C + 4;            // [C][LDCF] f32
  E Qs[C][LDQ];
  E Ks[C][LDQ];
  E Kt[D][LDCE];
  E Vt[D][LDCE];
  float Sk[C][LDCF];
  float Am[C][LDCF];
  float Tm[C][LDCF];
  float Tt[C][LDCF];
  E TB[C][LDCE];   // hi part of T diag(beta) / T diag(beta Gam)
  union {
    E TBl[Split<E>::on ? C : 1][LDCE];  // lo part
    float Xs[kChunkWaves][16][20];      // solve scratch
  };
  float gam[C];
  float beta[C];
};

// (I + A)^-1 for strictly lower A [C][C] (fp32 in LDS) into Tm and Tt = Tm^T.
// While wave 0 solves the 16 x 16 diagonal blocks, the other waves write the
// zero blocks above the diagonal (of Tm; below it of Tt) and then run
// other(first, count) (thread tid - 64 of NTH - 64); it must not touch Am, Tm,
// Tt, Xs nor wait at a barrier.  The blocks below the diagonal follow by
// doubling: the 32 x 32 diagonal blocks from their 16 x 16 halves
// (L^-1 = [[L11^-1, 0], [-L22^-1 L21 L11^-1, L22^-1]]), then the 64 x 64 from
// its 32 x 32 halves, each product on fp32 MFMA (4 barriers in all at C = 64).
// The caller's barrier before and this function's last barrier bracket it.
struct NoWork {
  __device__ void operator()(int, int) const {}
};
// the 16-byte pieces of a 16 x 16 strictly lower triangle, rows first: piece i
// is row diag_piece_row(i), columns 4 diag_piece_col(i) ...
constexpr int kDiagPieces = 36;  // sum over rows r of ceil(r / 4)
constexpr int diag_piece_row(int i) {
  int r = 1;
  while (i >= (r + 3) / 4) i -= (r++ + 3) / 4;
  return r;
}
constexpr int diag_piece_col(int i) {
  int r = 1;
  while (i >= (r + 3) / 4) i -= (r++ + 3) / 4;
  return i;
}
template <int C, int LDCF, int NTH = kChunkThreads, typename F = NoWork>
__device__ __forceinline__ void unit_lower_inverse(const float (*Am)[LDCF], float (*Tm)[LDCF], float (*Tt)[LDCF],
                                                   float (*Xs)[16][20], F&& other = F{}) {
  static_assert(C <= kWave && NTH > kWave, "diagonal solve in wave 0");
  constexpr int NB = C / 16;
  static_assert(NB == 1 || NB == 2 || NB == 4, "chunks of 16, 32 or 64");
  const int tid = threadIdx.x, w = wave_id();
  if (tid >= kWave) {
    for (int e = tid - kWave; e < C * C; e += NTH - kWave) {
      const int r = e / C, c = e % C;
      if (r / 16 < c / 16) Tm[r][c] = 0.f;
      if (r / 16 > c / 16) Tt[r][c] = 0.f;
    }
    other(tid - kWave, NTH - kWave);
  } else if (tid < C) {  // diagonal 16x16 blocks, one column per lane
    const int o = (tid >> 4) * 16, c = tid & 15;
    // Forward substitution over the block's lower-triangle entries, read as
    // 16-byte pieces (row r, columns 4q .. 4q+3 for 4q < r) three pieces ahead
    // of their use: read one at a time, each read was waited for at its
    // multiply-add.  Same summation order as row by row.
    float x[16], acc = 0.f;
    float4 buf[4];
    auto fetch = [&]<int I>() {
      constexpr int r = diag_piece_row(I), q = diag_piece_col(I);
      buf[I % 4] = *reinterpret_cast<const float4*>(&Am[o + r][o + 4 * q]);
    };
    auto solve_piece = [&]<int I>() {
      if constexpr (I + 3 < kDiagPieces) fetch.template operator()<I + 3>();
      constexpr int r = diag_piece_row(I), q = diag_piece_col(I);
      if constexpr (q == 0) acc = (r == c) ? 1.f : 0.f;
      const float4 v = buf[I % 4];
      const float av[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (4 * q + u < r) acc -= av[u] * x[4 * q + u];
      if constexpr (4 * q + 4 >= r) x[r] = acc;
    };
    fetch.template operator()<0>();
    fetch.template operator()<1>();
    fetch.template operator()<2>();
    x[0] = (c == 0) ? 1.f : 0.f;
    [&]<int... I>(std::integer_sequence<int, I...>) {
      (solve_piece.template operator()<I>(), ...);
    }(std::make_integer_sequence<int, kDiagPieces>{});
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      Tm[o + r][o + c] = x[r];
      Tt[o + c][o + r] = x[r];
    }
  }
  __syncthreads();
  // T_rc = -T_rr X for the tile X in Xs[slot] (stored transposed), into Tm and Tt
  auto finish = [&](int br, int bc, f32x4 acc) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = br * 16 + acc_row(e), c = bc * 16 + acc_col();
      Tm[r][c] = -acc[e];
      Tt[c][r] = -acc[e];
    }
  };
  auto park = [&](int slot, f32x4 acc) {
#pragma unroll
    for (int e = 0; e < 4; ++e) Xs[slot][acc_col()][acc_row(e)] = acc[e];
  };
  if constexpr (NB >= 2) {  // blocks (1, 0) and (3, 2): one wave each, X through its own Xs slot
    if (w < NB / 2) {
      const int b = 2 * w;
      park(w, mm_tile<float, 16>(zero4(), &Am[(b + 1) * 16][b * 16], LDCF, &Tt[b * 16][b * 16], LDCF));
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");  // the wave's own parked tile
      finish(b + 1, b, mm_tile<float, 16>(zero4(), &Tm[(b + 1) * 16][(b + 1) * 16], LDCF, &Xs[w][0][0], 20));
    }
    __syncthreads();
  }
  if constexpr (NB == 4) {  // rows 2..3, columns 0..1: -T[2:4][2:4] (A[2:4][0:2] T[0:2][0:2])
    if (w < 4) {  // X_ab = sum_{k = b}^{1} A_{2+a, k} T_{k, b}
      const int ra = w >> 1, cb = w & 1;
      f32x4 acc = zero4();
      for (int k = cb; k < 2; ++k)
        acc = mm_tile<float, 16>(acc, &Am[(2 + ra) * 16][k * 16], LDCF, &Tt[cb * 16][k * 16], LDCF);
      park(w, acc);
    }
    __syncthreads();
    if (w < 4) {  // T_{2+a, b} = -sum_{m = 0}^{a} T_{2+a, 2+m} X_mb
      const int ra = w >> 1, cb = w & 1;
      f32x4 acc = zero4();
      for (int m = 0; m <= ra; ++m)
        acc = mm_tile<float, 16>(acc, &Tm[(2 + ra) * 16][(2 + m) * 16], LDCF, &Xs[2 * m + cb][0][0], 20);
      finish(2 + ra, cb, acc);
    }
    __syncthreads();
  }
}

template <typename E, int D, int C, int DVT, bool OUT>
struct StateSmem {
  static constexpr int LDQ = D + Pad<E>::E16;
  static constexpr int LDCE = C + Pad<E>::E16;
  static constexpr int LDU = DVT + 4;
  static constexpr int LO = Split<E>::on ? 1 : 0;
  E Wk[C][LDQ];
  E Q[OUT ? C : 1][LDQ];
  E Kt[D][LDCE];
  E Ktl[LO ? D : 1][LDCE];
  E P[OUT ? C : 1][LDCE];
  E Pl[OUT && LO ? C : 1][LDCE];
  E Ht[DVT][LDQ];
  E Htl[LO ? DVT : 1][LDQ];
  E Wt[DVT][LDCE];
  E Wtl[LO ? DVT : 1][LDCE];
  float U[C][LDU];
  float gam[C];
};

// fp8 inputs (OCP e4m3: 1 sign, 4 exponent bits with bias 7, 3 mantissa bits;
// exponent field 0 is subnormal, m 2^-9).  Decoded exactly: normal values are
// (1 + m/8) 2^(e-7), i.e. float bits ((e + 120) << 23) | (m << 20).  Every
// e4m3 value times a power-of-two scale (within bf16's range) is a bf16 value,
// so the decoded tile is exactly the bf16 tile of the dequantised inputs.
// (The e4m3 NaN code, 0x7f / 0xff, is outside the supported inputs.)
__device__ __forceinline__ float fp8_e4m3_to_f32(uint32_t b) {
  const uint32_t e = (b >> 3) & 0xFu, m = b & 7u;
  const float mag = e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0x1p-9f;
  return __uint_as_float(__float_as_uint(mag) | ((b & 0x80u) << 24));
}

// 8 fp8 values (two little-endian words) -> 8 bf16 values times `scale` (a power of two)
__device__ __forceinline__ uint4 fp8x8_to_bf16x8(uint32_t lo, uint32_t hi, float scale) {
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t src = i < 2 ? lo : hi, sh = (i & 1) * 16;
    const float a = fp8_e4m3_to_f32((src >> sh) & 0xFFu) * scale;
    const float b = fp8_e4m3_to_f32((src >> (sh + 8)) & 0xFFu) * scale;
    w[i] = (__float_as_uint(a) >> 16) | (__float_as_uint(b) & 0xFFFF0000u);  // exact: <= 4 significant bits
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// Register staging of one [R][COLS] tile of T read from global memory (row
// stride ld elements, rows past rows_valid read as zero) by all threads of a
// workgroup with 16-byte loads; store() writes it to LDS afterwards.  Used to
// issue the next chunk's loads before the current chunk's compute.
// Piece e (16 bytes) is, by default, row e / PER_ROW, columns (e % PER_ROW) * V:
// adjacent lanes take adjacent pieces of a row.  With RF (rows first), 16
// adjacent lanes take the same columns of 16 adjacent rows: store_t then
// writes 16 consecutive elements of a transposed row per lane group instead of
// one element each of 16 rows a 16-byte piece apart (which fall in the same
// LDS banks), at the price of 64-byte instead of 256-byte runs per global load.
template <typename T, int R, int COLS, int NTH = kChunkThreads, bool RF = false, bool BUF = true>
struct TileRegs {
  static constexpr int V = 16 / (int)sizeof(T);
  static constexpr int PER_ROW = COLS / V;
  static constexpr int TOTAL = R * PER_ROW;
  static constexpr int N = (TOTAL + NTH - 1) / NTH;
  // every thread holds N whole pieces: no per-piece guard (a guard the compiler
  // cannot fold is a branch, and loads it sinks into it wait there one by one)
  static constexpr bool FULL = TOTAL % NTH == 0;
  static_assert(!RF || R % 16 == 0, "rows-first pieces come in groups of 16 rows");
  uint4 r[N];
  __device__ __forceinline__ static void pos(int e, int& row, int& c) {
    if constexpr (RF) {
      const int g = e >> 4;
      row = (g / PER_ROW) * 16 + (e & 15);
      c = (g % PER_ROW) * V;
    } else {
      row = e / PER_ROW;
      c = (e % PER_ROW) * V;
    }
  }
  // Buffer loads through a resource that covers rows [0, rows_valid): pieces
  // past it (and past the tile) read as zero in hardware, so every load issues
  // at once.  (Loads under a per-piece branch were each followed by a full wait
  // for the vector-memory counter: the compiler drains it at the branch join.)
  __device__ __forceinline__ void load(const T* g, int64_t ld, int rows_valid) {
    if constexpr (!BUF) {
      load_each(g, ld, rows_valid);
      return;
    }
    const int64_t bytes = (int64_t)rows_valid * ld * (int64_t)sizeof(T);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<T*>(g), 0, (int)(bytes < 0x7fffffff ? bytes : 0x7fffffff), 0x00020000);
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int e = threadIdx.x + i * NTH;
      int row, c;
      pos(e, row, c);
      const int off = e < TOTAL ? (int)(((int64_t)row * ld + c) * (int64_t)sizeof(T)) : 0x7fffffe0;
      r[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0));
    }
  }
  // The same tile from an fp8 (e4m3) source with a power-of-two scale: 8-byte
  // pieces (8 elements) through a buffer resource over rows [0, rows_valid),
  // decoded exactly into the bf16 registers load() would hold for the
  // dequantised tile.  ld is in elements (= bytes).
  __device__ __forceinline__ void load_f8(const uint8_t* g, int64_t ld, int rows_valid, float scale) {
    static_assert(sizeof(T) == 2 && V == 8, "bf16 tiles");
    const int64_t bytes = (int64_t)rows_valid * ld;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(g), 0, (int)(bytes < 0x7fffffff ? bytes : 0x7fffffff), 0x00020000);
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int e = threadIdx.x + i * NTH;
      int row, c;
      pos(e, row, c);
      const int off = e < TOTAL ? (int)((int64_t)row * ld + c) : 0x7fffffe0;
      const uint2 raw = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rs, off, 0, 0));
      r[i] = fp8x8_to_bf16x8(raw.x, raw.y, scale);
    }
  }
  // One guarded load per piece, each completed before the next is issued.
  // The tiled state pass (whose next-chunk prefetch competes with its own
  // serial chunk step) measured faster this way at a single 65536-token
  // sequence: 3.06 against 3.21 ms.
  __device__ __forceinline__ void load_each(const T* g, int64_t ld, int rows_valid) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int e = threadIdx.x + i * NTH;
      r[i] = make_uint4(0, 0, 0, 0);
      if (FULL || e < TOTAL) {
        int row, c;
        pos(e, row, c);
        if (row < rows_valid) r[i] = *reinterpret_cast<const uint4*>(g + (int64_t)row * ld + c);
      }
    }
  }
  __device__ __forceinline__ void store(T* s, int lds) const {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int e = threadIdx.x + i * NTH;
      if (FULL || e < TOTAL) {
        int row, c;
        pos(e, row, c);
        *reinterpret_cast<uint4*>(s + row * lds + c) = r[i];
      }
    }
  }
  // tile written transposed: hi[c * lds + row] (optionally scaled per row by
  // rs[i] for the i-th register slot, and split into hi / lo[c * lds_lo + row]
  // when lo != null)
  template <typename E>
  __device__ __forceinline__ void store_t(E* hi, int lds, E* lo = nullptr, int lds_lo = 0, const float* rs = nullptr,
                                          float mult = 1.f) const {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int e = threadIdx.x + i * NTH;
      if (FULL || e < TOTAL) {
        int row, c;
        pos(e, row, c);
        const T* f = reinterpret_cast<const T*>(&r[i]);
        const float sc = (rs ? rs[i] : 1.f) * mult;
#pragma unroll
        for (int u = 0; u < V; ++u) {
          const float x = to_f<T>(f[u]) * sc;
          if (lo) split_store<E>(hi + (c + u) * lds + row, lo + (c + u) * lds_lo + row, x);
          else hi[(c + u) * lds + row] = from_f<E>(x);
        }
      }
    }
  }
  __device__ __forceinline__ int row_of(int i) const {
    int row, c;
    pos(threadIdx.x + i * NTH, row, c);
    return row;
  }
  // tile written transposed as it is: s[c * lds + row]
  __device__ __forceinline__ void store_t_raw(T* s, int lds) const {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int e = threadIdx.x + i * NTH;
      if (FULL || e < TOTAL) {
        int row, c;
        pos(e, row, c);
        const T* f = reinterpret_cast<const T*>(&r[i]);
#pragma unroll
        for (int u = 0; u < V; ++u) s[(c + u) * lds + row] = f[u];
      }
    }
  }
  // float tile written as E hi (and lo) parts
  template <typename E>
  __device__ __forceinline__ void store_split(E* hi, E* lo, int lds) const {
    static_assert(sizeof(T) == 4, "split store takes a float tile");
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int e = threadIdx.x + i * NTH;
      if (FULL || e < TOTAL) {
        int row, c;
        pos(e, row, c);
        const float* f = reinterpret_cast<const float*>(&r[i]);
        st4_split<E>(hi + row * lds + c, lo + row * lds + c, f32x4{f[0], f[1], f[2], f[3]});
      }
    }
  }
};

// Register staging of a [R][COLS] tile read column-wise: each slot holds V
// consecutive rows of one column, so store() writes the transposed tile
// (dst[c * lds + r]) with one 16-byte store per slot, and the loads of a wave
// walk along rows (coalesced for COLS >= 32).
template <typename T, int R, int COLS, int NTH = kChunkThreads>
struct ColRegs {
  static constexpr int V = 16 / (int)sizeof(T);
  static constexpr int TOTAL = COLS * (R / V);
  static constexpr int N = (TOTAL + NTH - 1) / NTH;
  static constexpr bool FULL = TOTAL % NTH == 0;
  static_assert(sizeof(T) == 2 || sizeof(T) == 4, "16- or 32-bit elements");
  uint4 r[N];
  // Buffer loads through a resource that covers rows [0, rows_valid): rows
  // past it read as zero in hardware, so every load issues at once, with no
  // branch and no per-load address.
  __device__ __forceinline__ void load(const T* g, int64_t ld, int rows_valid) {
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<T*>(g), 0, (int)((int64_t)rows_valid * ld * (int64_t)sizeof(T)), 0x00020000);
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int e = threadIdx.x + i * NTH;
      T* v = reinterpret_cast<T*>(&r[i]);
      const int c = e % COLS, r0 = (e / COLS) * V;
      // one per-lane offset; the row step (uniform) goes in the scalar offset
      const int off = (int)(((int64_t)r0 * ld + c) * (int64_t)sizeof(T));
      const int step = (int)(ld * (int64_t)sizeof(T));
#pragma unroll
      for (int u = 0; u < V; ++u) {
        if constexpr (sizeof(T) == 2) {
          v[u] = __builtin_bit_cast(T, (uint16_t)__builtin_amdgcn_raw_buffer_load_b16(rs, off, u * step, 0));
        } else {
          v[u] = __builtin_bit_cast(T, (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rs, off, u * step, 0));
        }
      }
    }
  }
  __device__ __forceinline__ void store(T* s, int lds) const {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int e = threadIdx.x + i * NTH;
      if (FULL || e < TOTAL) {
        const int c = e % COLS, r0 = (e / COLS) * V;
        *reinterpret_cast<uint4*>(s + c * lds + r0) = r[i];
      }
    }
  }
};

// Workgroup -> (sequence, v-head, dv tile) so that the G * NVT workgroups that
// read one (sequence, k-head)'s chunk tiles share an XCD (blocks are dealt to
// the 8 XCDs round-robin) and hence its L2.  Returns false for padding blocks.
__device__ __forceinline__ bool state_block(int bid, int N, int Hk, int G, int NVT, int& n, int& h, int& vt) {
  const int per = G * NVT;
  const int xcd = bid & 7, q = bid >> 3;
  const int m = q % per;
  const int gidx = (q / per) * 8 + xcd;
  if (gidx >= N * Hk) return false;
  n = gidx / Hk;
  h = (gidx % Hk) * G + m / NVT;
  vt = m % NVT;
  return true;
}


// f(t) for t = first, first + STEP, ... below TOTAL (first < STEP): a fixed,
// unrolled count per thread, so that the compiler's wait counts over the
// stores inside stay exact (a loop whose trip count it cannot see makes it
// assume the fewest stores, and later loads then wait for all of them)
template <int TOTAL, int STEP, typename F>
__device__ __forceinline__ void for_strided(int first, F&& f) {
  constexpr int N = (TOTAL + STEP - 1) / STEP;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const int t = first + i * STEP;
    if constexpr (TOTAL % STEP == 0) f(t);
    else if (t < TOTAL) f(t);
  }
}

// visit the RT x CT blocks of an NR x NC tile grid owned by this wave
template <int NR, int NC, int RT, int CT, int NW = kChunkWaves, typename F>
__device__ __forceinline__ void for_blocks(F&& f) {
  static_assert(NR % RT == 0 && NC % CT == 0, "block shape must divide the tile grid");
  constexpr int NBC = NC / CT, NB = (NR / RT) * NBC;
  for_strided<NB, NW>(wave_id(), [&](int b) { f((b / NBC) * RT, (b % NBC) * CT); });
}

inline int state_grid(int N, int Hk, int G, int NVT) { return ((N * Hk + 7) / 8) * 8 * G * NVT; }

// State passes with one 512-thread workgroup per (sequence, v-head), for
// bf16, d = 128, chunk 64 (state_wide.hip).
// half: two workgroups per (sequence, v-head), 64 state columns each
void launch_state_fwd_wide(const ChunkArgs& a, hipStream_t st, int mode, bool half, bool f8 = false);
// 16-column tiles, eight 256-thread workgroups per (sequence, v-head)
void launch_state_fwd_cols(const ChunkArgs& a, hipStream_t st, int mode, bool f8);
// half: two workgroups per (sequence, v-head), 64 state columns each
void launch_state_bwd_wide(const ChunkArgs& a, hipStream_t st, bool half);
template <typename E, int D, int C>
constexpr bool use_wide_state() { return sizeof(E) == 2 && D == 128 && C == 64; }

// Workspace layouts of the preparation's outputs at those shapes, in the order
// the state passes load them, so that every load instruction of a wave reads
// 1 KB of consecutive bytes (a row-major tile read as matrix-core fragments
// touches 16 rows per instruction, which the load path serves at about half
// the rate).
// A-operand order of a [M][K] bf16 tile: fragment (row tile, k step of 32),
// lane 16 g + r holds row r, k = 8 g .. 8 g + 7 (Wk [C][D], K^T [D][C]).
__device__ __forceinline__ int af_off(int row, int k, int K) {
  return ((((row >> 4) * (K >> 5) + (k >> 5)) * 64 + ((k >> 3) & 3) * 16 + (row & 15)) << 3) + (k & 7);
}
// Accumulator order of a [M][N] fp32 tile: tile (row tile, column tile), lane
// 16 g + c holds rows 4 g .. 4 g + 3 of column c (U [C][D]).
__device__ __forceinline__ int acc_off(int row, int col, int N) {
  return ((((row >> 4) * (N >> 4) + (col >> 4)) * 64 + ((row >> 2) & 3) * 16 + (col & 15)) << 2) + (row & 3);
}
// A-operand order of a [M][K] fp32 tile, each lane's 8 values as two 4-value
// halves stored half by half (P [C][C] of the inference forward).
__device__ __forceinline__ int pf_off(int row, int k, int K) {
  return (((((row >> 4) * (K >> 5) + (k >> 5)) * 2 + ((k >> 2) & 1)) * 64 + ((k >> 3) & 3) * 16 + (row & 15)) << 2) +
         (k & 3);
}

}  // namespace gdn
