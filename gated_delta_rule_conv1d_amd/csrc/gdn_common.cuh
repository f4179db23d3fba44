// Device helpers shared by the gfx950 kernels: bf16 conversion, the 16x16
// MFMA tile primitive, wave reductions, and the per-chunk workspace layout.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gdn {

typedef uint16_t bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf2f(bf16 b) { return __uint_as_float(((uint32_t)b) << 16); }

// float -> bf16, round to nearest even (gfx950 converts natively:
// v_cvt_pk_bf16_f32); NaN stays NaN, infinities pass.
__device__ __forceinline__ bf16 f2bf(float f) { return __builtin_bit_cast(bf16, static_cast<__bf16>(f)); }

template <typename E> __device__ __forceinline__ float to_f(E v);
template <> __device__ __forceinline__ float to_f<float>(float v) { return v; }
template <> __device__ __forceinline__ float to_f<bf16>(bf16 v) { return bf2f(v); }

template <typename E> __device__ __forceinline__ E from_f(float v);
template <> __device__ __forceinline__ float from_f<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16 from_f<bf16>(float v) { return f2bf(v); }

// 16-byte vector of elements: 8 bf16 or 4 float.
template <typename E> struct Vec {
  static constexpr int N = 16 / (int)sizeof(E);
  __device__ static void load(const E* p, float* out) {
    uint4 raw = *reinterpret_cast<const uint4*>(p);
    const E* e = reinterpret_cast<const E*>(&raw);
#pragma unroll
    for (int i = 0; i < N; ++i) out[i] = to_f<E>(e[i]);
  }
  __device__ static void store(E* p, const float* in) {
    uint4 raw;
    E* e = reinterpret_cast<E*>(&raw);
#pragma unroll
    for (int i = 0; i < N; ++i) e[i] = from_f<E>(in[i]);
    *reinterpret_cast<uint4*>(p) = raw;
  }
};

// ---------------------------------------------------------------------------
// MFMA 16x16 tiles.  One wave computes D[16x16] += A[16xK] * B[Kx16] with
// A stored row-major (K contiguous, row stride lda) and B stored column by
// column (K contiguous, column stride ldb).  Both may live in LDS or global
// memory.  Accumulator layout: lane l holds rows 4*(l>>4)+i (i<4), column l&15.
// bf16 operands use v_mfma_f32_16x16x32_bf16 (8 k-values per lane), float
// operands v_mfma_f32_16x16x4_f32 (1 k-value per lane).  The k-values each
// lane supplies only have to agree between A and B, so any consistent k order
// gives the same contraction.
// ---------------------------------------------------------------------------
template <typename E> struct Mma;

template <> struct Mma<bf16> {
  static constexpr int KS = 32, KPL = 8;
  typedef bf16x8 frag;
  __device__ static frag load(const bf16* p) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p));
  }
  __device__ static frag from_floats(const float* v) {
    uint4 raw;
    bf16* e = reinterpret_cast<bf16*>(&raw);
#pragma unroll
    for (int i = 0; i < 8; ++i) e[i] = f2bf(v[i]);
    return __builtin_bit_cast(bf16x8, raw);
  }
  __device__ static frag zero() { return __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0)); }
  __device__ static f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};

template <> struct Mma<float> {
  static constexpr int KS = 4, KPL = 1;
  typedef float frag;
  __device__ static frag load(const float* p) { return *p; }
  __device__ static frag from_floats(const float* v) { return v[0]; }
  __device__ static frag zero() { return 0.f; }
  __device__ static f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
};

// Gates of the recurrence (see gates.hip): softplus(x) = max(x, 0) +
// log1p(e^{-|x|}) (no overflow, no loss for very negative x), and the logistic
// sigmoid.  The gate kernels and the chunk kernels that compute g and beta
// from their raw inputs share these, so both give the same bits.
__device__ __forceinline__ float gate_softplus(float x) { return fmaxf(x, 0.f) + log1pf(__expf(-fabsf(x))); }
__device__ __forceinline__ float gate_sigmoid(float x) { return 1.f / (1.f + __expf(-x)); }

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }
__device__ __forceinline__ int wave_id() { return threadIdx.x / kWave; }
// accumulator coordinates
__device__ __forceinline__ int acc_row(int i) { return 4 * (lane_id() >> 4) + i; }
__device__ __forceinline__ int acc_col() { return lane_id() & 15; }

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

template <typename E, int K>
__device__ __forceinline__ f32x4 mm_tile(f32x4 acc, const E* A, int lda, const E* B, int ldb) {
  const int lane = lane_id();
  const int r = lane & 15, kq = (lane >> 4) * Mma<E>::KPL;
  const E* a = A + r * lda + kq;
  const E* b = B + r * ldb + kq;
  if constexpr (K % Mma<E>::KS != 0) {
    // K smaller than one instruction's k-extent (bf16, K = 16): lanes whose
    // k-values lie past K feed zeros
    static_assert(K < Mma<E>::KS, "K must be a multiple of the MFMA k-extent or smaller");
    const bool kv = kq < K;
    const typename Mma<E>::frag fa = kv ? Mma<E>::load(a) : Mma<E>::zero();
    const typename Mma<E>::frag fb = kv ? Mma<E>::load(b) : Mma<E>::zero();
    return Mma<E>::mma(fa, fb, acc);
  } else {
#pragma unroll
    for (int k0 = 0; k0 < K; k0 += Mma<E>::KS)
      acc = Mma<E>::mma(Mma<E>::load(a + k0), Mma<E>::load(b + k0), acc);
    return acc;
  }
}

// Same contraction with float operands fed to the MFMA of type E: for E=bf16
// each lane converts its 8 float k-values to bf16 on the fly.
template <typename E, int K>
__device__ __forceinline__ f32x4 mm_tile_f(f32x4 acc, const float* A, int lda, const float* B, int ldb) {
  const int lane = lane_id();
  const int r = lane & 15, kq = (lane >> 4) * Mma<E>::KPL;
  const float* a = A + r * lda + kq;
  const float* b = B + r * ldb + kq;
  constexpr bool PART = K % Mma<E>::KS != 0;
  static_assert(!PART || K < Mma<E>::KS, "K must be a multiple of the MFMA k-extent or smaller");
  const bool kv = !PART || kq < K;
#pragma unroll
  for (int k0 = 0; k0 < K; k0 += Mma<E>::KS) {
    float av[Mma<E>::KPL], bv[Mma<E>::KPL];
#pragma unroll
    for (int i = 0; i < Mma<E>::KPL; ++i) {
      av[i] = kv ? a[k0 + i] : 0.f;
      bv[i] = kv ? b[k0 + i] : 0.f;
    }
    acc = Mma<E>::mma(Mma<E>::from_floats(av), Mma<E>::from_floats(bv), acc);
  }
  return acc;
}

// A from float storage (converted to the MFMA type of E on the fly), B from E.
template <typename E, int K>
__device__ __forceinline__ f32x4 mm_tile_fa(f32x4 acc, const float* A, int lda, const E* B, int ldb) {
  const int lane = lane_id();
  const int r = lane & 15, kq = (lane >> 4) * Mma<E>::KPL;
  const float* a = A + r * lda + kq;
  const E* b = B + r * ldb + kq;
  constexpr bool PART = K % Mma<E>::KS != 0;
  static_assert(!PART || K < Mma<E>::KS, "K must be a multiple of the MFMA k-extent or smaller");
  const bool kv = !PART || kq < K;
#pragma unroll
  for (int k0 = 0; k0 < K; k0 += Mma<E>::KS) {
    float av[Mma<E>::KPL];
#pragma unroll
    for (int i = 0; i < Mma<E>::KPL; ++i) av[i] = kv ? a[k0 + i] : 0.f;
    acc = Mma<E>::mma(Mma<E>::from_floats(av), kv ? Mma<E>::load(b + k0) : Mma<E>::zero(), acc);
  }
  return acc;
}

// Both operands from (global) row-major storage with row validity: A row r
// (0..15 of the tile) is read only if r < a_rows, B "row" (output column) n
// only if n < b_rows; others contribute zero.  Row strides are 64-bit.
template <typename E, int K>
__device__ __forceinline__ f32x4 mm_tile_rows(f32x4 acc, const E* A, int64_t lda, int a_rows, const E* B,
                                              int64_t ldb, int b_rows) {
  const int lane = lane_id();
  const int r = lane & 15, kq = (lane >> 4) * Mma<E>::KPL;
  constexpr bool PART = K % Mma<E>::KS != 0;
  static_assert(!PART || K < Mma<E>::KS, "K must be a multiple of the MFMA k-extent or smaller");
  const bool kv = !PART || kq < K;
  const bool va = r < a_rows && kv, vb = r < b_rows && kv;
  const E* a = A + (va ? r : 0) * lda + kq;
  const E* b = B + (vb ? r : 0) * ldb + kq;
  const typename Mma<E>::frag zf = Mma<E>::zero();
#pragma unroll
  for (int k0 = 0; k0 < K; k0 += Mma<E>::KS) {
    const typename Mma<E>::frag fa = va ? Mma<E>::load(a + k0) : zf;
    const typename Mma<E>::frag fb = vb ? Mma<E>::load(b + k0) : zf;
    acc = Mma<E>::mma(fa, fb, acc);
  }
  return acc;
}

// ---------------------------------------------------------------------------
// Split-precision tiles.  Operands are produced by loader callables
//   la(r, k, float* out)  -> out[0..KPL) = A[r][k .. k+KPL)   (r = 0..15 in tile)
//   lb(c, k, float* out)  -> out[0..KPL) = B[k .. k+KPL)[c]
// For bf16 MFMA an fp32 operand x is fed as hi = bf16(x) and lo = bf16(x - hi)
// (SA / SB say which operands need it); the tile sums hi*hi, hi*lo and lo*hi,
// so the products keep ~16 significant bits while running on bf16 MFMA.
// Operands that are exactly bf16 (inputs) skip the lo part.  With float
// operands this is one fp32 MFMA per k-step.
// ---------------------------------------------------------------------------
template <typename E, int K, bool SA, bool SB, typename LA, typename LB>
__device__ __forceinline__ f32x4 mm_gen(f32x4 acc, LA&& la, LB&& lb) {
  using M = Mma<E>;
  const int lane = lane_id();
  const int r = lane & 15, kq = (lane >> 4) * M::KPL;
  constexpr bool PART = K % M::KS != 0;
  static_assert(!PART || K < M::KS, "K must be a multiple of the MFMA k-extent or smaller");
  const bool kv = !PART || kq < K;
#pragma unroll
  for (int k0 = 0; k0 < K; k0 += M::KS) {
    float av[M::KPL], bv[M::KPL];
    if (kv) {
      la(r, k0 + kq, av);
      lb(r, k0 + kq, bv);
    } else {
#pragma unroll
      for (int i = 0; i < M::KPL; ++i) av[i] = bv[i] = 0.f;
    }
    if constexpr (M::KPL == 1) {
      acc = M::mma(M::from_floats(av), M::from_floats(bv), acc);
    } else {
      float al[M::KPL], bl[M::KPL];
#pragma unroll
      for (int i = 0; i < M::KPL; ++i) {
        al[i] = av[i] - bf2f(f2bf(av[i]));
        bl[i] = bv[i] - bf2f(f2bf(bv[i]));
      }
      const typename M::frag ah = M::from_floats(av), bh = M::from_floats(bv);
      acc = M::mma(ah, bh, acc);
      if constexpr (SB) acc = M::mma(ah, M::from_floats(bl), acc);
      if constexpr (SA) acc = M::mma(M::from_floats(al), bh, acc);
    }
  }
  return acc;
}

// ---------------------------------------------------------------------------
// Register-blocked tiles: one wave computes RT x CT output tiles of 16x16,
// loading each A fragment once per k-step for CT tiles and each B fragment once
// for RT tiles (LDS / L1 traffic per MFMA drops by ~RT*CT/(RT+CT)).  A: RT*16
// rows, K contiguous, row stride lda; B: CT*16 output columns, K contiguous,
// stride ldb.  Optional lo parts (same layout) add hi*lo and lo*hi products.
// ---------------------------------------------------------------------------
template <typename E, int K, int RT, int CT, bool ALO, bool BLO>
__device__ __forceinline__ void mm_blk(f32x4 (&acc)[RT][CT], const E* A, const E* Al, int lda, const E* B,
                                       const E* Bl, int ldb) {
  using M = Mma<E>;
  const int lane = lane_id();
  const int r = lane & 15, kq = (lane >> 4) * M::KPL;
  constexpr bool PART = K % M::KS != 0;
  static_assert(!PART || K < M::KS, "K must be a multiple of the MFMA k-extent or smaller");
  const bool kv = !PART || kq < K;
#pragma unroll
  for (int k0 = 0; k0 < K; k0 += M::KS) {
    typename M::frag fa[RT], fal[RT], fb[CT], fbl[CT];
#pragma unroll
    for (int i = 0; i < RT; ++i) {
      fa[i] = kv ? M::load(A + (i * 16 + r) * lda + kq + k0) : M::zero();
      if constexpr (ALO) fal[i] = kv ? M::load(Al + (i * 16 + r) * lda + kq + k0) : M::zero();
    }
#pragma unroll
    for (int j = 0; j < CT; ++j) {
      fb[j] = kv ? M::load(B + (j * 16 + r) * ldb + kq + k0) : M::zero();
      if constexpr (BLO) fbl[j] = kv ? M::load(Bl + (j * 16 + r) * ldb + kq + k0) : M::zero();
    }
#pragma unroll
    for (int i = 0; i < RT; ++i)
#pragma unroll
      for (int j = 0; j < CT; ++j) {
        acc[i][j] = M::mma(fa[i], fb[j], acc[i][j]);
        if constexpr (BLO) acc[i][j] = M::mma(fa[i], fbl[j], acc[i][j]);
        if constexpr (ALO) acc[i][j] = M::mma(fal[i], fb[j], acc[i][j]);
      }
  }
}

template <int RT, int CT>
__device__ __forceinline__ void zero_blk(f32x4 (&acc)[RT][CT]) {
#pragma unroll
  for (int i = 0; i < RT; ++i)
#pragma unroll
    for (int j = 0; j < CT; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
}

// loaders
template <typename T, int N>
__device__ __forceinline__ void ld_row(const T* p, float* out) {  // N consecutive values
  if constexpr (sizeof(T) * N == 16) {
    Vec<T>::load(p, out);
  } else if constexpr (sizeof(T) * N == 32) {
    Vec<T>::load(p, out);
    Vec<T>::load(p + 16 / sizeof(T), out + 16 / sizeof(T));
  } else {
#pragma unroll
    for (int i = 0; i < N; ++i) out[i] = to_f<T>(p[i]);
  }
}

// ---------------------------------------------------------------------------
// Reductions
// ---------------------------------------------------------------------------
// One DPP move of v within each row of 16 lanes (CDNA3/4 DPP controls:
// quad_perm 0x00-0xff, row_mirror 0x140, row_half_mirror 0x141).
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false));
}

// Sum over aligned groups of WIDTH lanes, the same value in every lane of a
// group.  Inside a row the partners come from DPP: lane ^ 1 and lane ^ 2 by
// quad permutes, then the mirrored lane of the half row and of the row, which
// holds the sum of the partner quad / half (all its lanes agree by then), so
// the addition tree is that of xor partners 1, 2, 4, 8.  Across rows the
// partners come through ds_bpermute.
template <int WIDTH>
__device__ __forceinline__ float group_sum(float v) {
  static_assert(WIDTH >= 1 && WIDTH <= kWave && (WIDTH & (WIDTH - 1)) == 0, "power-of-two group");
  if constexpr (WIDTH >= 2) v += dpp_f<0xb1>(v);   // quad_perm [1,0,3,2]
  if constexpr (WIDTH >= 4) v += dpp_f<0x4e>(v);   // quad_perm [2,3,0,1]
  if constexpr (WIDTH >= 8) v += dpp_f<0x141>(v);  // row_half_mirror
  if constexpr (WIDTH >= 16) v += dpp_f<0x140>(v); // row_mirror
#pragma unroll
  for (int off = 16; off < WIDTH; off <<= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

// Sum over the whole wave, the same value in every lane: row sums by DPP, then
// the four row totals read out lane by lane and added in row order.
__device__ __forceinline__ float wave_sum(float v) {
  v = group_sum<16>(v);
  const int b = __builtin_bit_cast(int, v);
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 0));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 16));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 32));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 48));
  return ((r0 + r1) + r2) + r3;
}

// Inclusive suffix sum over the wave: lane i gets the sum of lanes i..63.
// Inside each row of 16 a Hillis-Steele scan on DPP row_shl (lane i reads lane
// i + k of its row; past the row end the identity 0 comes in), then each lane
// adds the totals of the rows above its own, read out lane by lane.
template <int CTRL>
__device__ __forceinline__ float dpp_or_zero(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float wave_suffix_sum(float v) {
  v += dpp_or_zero<0x101>(v);  // row_shl:1
  v += dpp_or_zero<0x102>(v);  // row_shl:2
  v += dpp_or_zero<0x104>(v);  // row_shl:4
  v += dpp_or_zero<0x108>(v);  // row_shl:8
  const int b = __builtin_bit_cast(int, v);
  const float t1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 16));
  const float t2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 32));
  const float t3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 48));
  const float s2 = t3, s1 = t2 + t3, s0 = t1 + s1;
  const int row = lane_id() >> 4;
  return v + (row == 0 ? s0 : row == 1 ? s1 : row == 2 ? s2 : 0.f);
}

// sigmoid with the hardware reciprocal (v_rcp_f32, 1 ulp) instead of an IEEE
// division sequence; 1 + e^-x = inf gives 0, as it should.
__device__ __forceinline__ float sigmoidf_(float x) { return __builtin_amdgcn_rcpf(1.f + __expf(-x)); }


// ---------------------------------------------------------------------------
// Deterministic column sums of per-block partials: out[c] = sum_p part[p*n + c].
// Thread (g, cc) of a block adds parts g, g + PG, g + 2 PG, ... of column
// blockIdx.x * CW + cc; one thread per column then adds the PG group sums in
// order.  The order of every addition is fixed, so results are bit-identical
// run to run.
// ---------------------------------------------------------------------------
template <int CW, int PG>
__global__ __launch_bounds__(CW * PG) void colsum_kernel(const float* __restrict__ part, int nparts, int n,
                                                         float* __restrict__ out) {
  __shared__ float s[PG][CW + 1];
  const int cc = threadIdx.x % CW, g = threadIdx.x / CW;
  const int c = blockIdx.x * CW + cc;
  float acc = 0.f;
  if (c < n)
    for (int p = g; p < nparts; p += PG) acc += part[(size_t)p * n + c];
  s[g][cc] = acc;
  __syncthreads();
  if (g == 0 && c < n) {
    float t = 0.f;
    for (int i = 0; i < PG; ++i) t += s[i][cc];
    out[c] = t;
  }
}

inline void launch_colsum(const float* part, int nparts, int n, float* out, hipStream_t st) {
  if (n < 4096) colsum_kernel<4, 64><<<(n + 3) / 4, 256, 0, st>>>(part, nparts, n, out);
  else colsum_kernel<16, 16><<<(n + 15) / 16, 256, 0, st>>>(part, nparts, n, out);
}

}  // namespace gdn
