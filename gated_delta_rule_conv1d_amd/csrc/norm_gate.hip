// RMSNormGated epilogue and its backward.
//
// Page: "[Qwen3.5 MoE] Add hybrid decoder model", Summary (RMSNormGated in
// GatedDeltaNet).  Per row (token, v-head) of dv values:
//   r = rsqrt(mean(o^2) + eps),  y = o * r * w * z * sigmoid(z).
// Backward, with a = dy * w * SiLU(z):
//   do = r (a - o r^2 mean(a o)),  dz = dy o r w s (1 + z (1 - s)),
//   dw = sum over rows of dy o r SiLU(z)  (fixed-order two-stage sum).
//
// A lane owns 16 bytes of a row (8 bf16 / 4 float); LPR = dv / that lanes form
// a row group that reduces with xor shuffles.  Pure HBM streaming.
#include <mutex>

#include "gdn_common.cuh"
#include "gdn_internal.h"
#include "profile.h"

namespace gdn {

constexpr int kNormThreads = 256;
constexpr int kNormBwdBlocks = 1024;  // fixed grid of the backward (row-block stride)

// Scratch of the allocation-free backward (gdn_norm_gate_bwd_noalloc): the
// backward's per-block dw partials, kNormBwdBlocks x d_v floats for d_v <= 128
// (512 KiB on each device the library runs on, held until the process ends).
// Every block of the backward writes its whole row of partials before the
// column sum reads them, so nothing needs clearing between calls.
constexpr size_t kNormScratchFloats = (size_t)kNormBwdBlocks * 128;
static __device__ __align__(256) float scratch[kNormScratchFloats];

template <typename E, int DV>
__global__ __launch_bounds__(kNormThreads) void norm_fwd_kernel(const E* __restrict__ o, const E* __restrict__ z,
                                                                const E* __restrict__ w, float eps, long rows,
                                                                E* __restrict__ y) {
  constexpr int V = Vec<E>::N;
  constexpr int LPR = DV / V;                       // lanes per row
  constexpr int RPB = kNormThreads / LPR;           // rows per block
  const int sub = threadIdx.x % LPR;
  const long row = (long)blockIdx.x * RPB + threadIdx.x / LPR;
  float wv[V];
  Vec<E>::load(w + sub * V, wv);
  float ov[V], zv[V];
  const bool ok = row < rows;
  if (ok) {
    Vec<E>::load(o + row * DV + sub * V, ov);
    Vec<E>::load(z + row * DV + sub * V, zv);
  } else {
#pragma unroll
    for (int i = 0; i < V; ++i) ov[i] = zv[i] = 0.f;
  }
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < V; ++i) ss += ov[i] * ov[i];
  ss = group_sum<LPR>(ss);
  const float r = rsqrtf(ss * (1.f / DV) + eps);
  float out[V];
#pragma unroll
  for (int i = 0; i < V; ++i) out[i] = ov[i] * r * wv[i] * (zv[i] * sigmoidf_(zv[i]));
  if (ok) Vec<E>::store(y + row * DV + sub * V, out);
}

template <typename E, int DV>
__global__ __launch_bounds__(kNormThreads) void norm_bwd_kernel(const E* __restrict__ dy, const E* __restrict__ o,
                                                                const E* __restrict__ z, const E* __restrict__ w,
                                                                float eps, long rows, E* __restrict__ d_o,
                                                                E* __restrict__ dz, float* __restrict__ dw_part) {
  constexpr int V = Vec<E>::N;
  constexpr int LPR = DV / V;
  constexpr int RPB = kNormThreads / LPR;
  __shared__ float red[RPB][DV];
  const int sub = threadIdx.x % LPR;
  const int rin = threadIdx.x / LPR;
  float wv[V];
  Vec<E>::load(w + sub * V, wv);
  float dwacc[V];
#pragma unroll
  for (int i = 0; i < V; ++i) dwacc[i] = 0.f;
  for (long base = (long)blockIdx.x * RPB; base < rows; base += (long)gridDim.x * RPB) {
    const long row = base + rin;
    const bool ok = row < rows;
    float ov[V], zv[V], gv[V];
    if (ok) {
      Vec<E>::load(o + row * DV + sub * V, ov);
      Vec<E>::load(z + row * DV + sub * V, zv);
      Vec<E>::load(dy + row * DV + sub * V, gv);
    } else {
#pragma unroll
      for (int i = 0; i < V; ++i) ov[i] = zv[i] = gv[i] = 0.f;
    }
    float ss = 0.f, ao = 0.f;
    float sg[V], a[V];
#pragma unroll
    for (int i = 0; i < V; ++i) {
      sg[i] = sigmoidf_(zv[i]);
      a[i] = gv[i] * wv[i] * zv[i] * sg[i];
      ss += ov[i] * ov[i];
      ao += a[i] * ov[i];
    }
    ss = group_sum<LPR>(ss);
    ao = group_sum<LPR>(ao) * (1.f / DV);
    const float r = rsqrtf(ss * (1.f / DV) + eps);
    float dov[V], dzv[V];
#pragma unroll
    for (int i = 0; i < V; ++i) {
      dov[i] = r * (a[i] - ov[i] * r * r * ao);
      dzv[i] = gv[i] * ov[i] * r * wv[i] * sg[i] * (1.f + zv[i] * (1.f - sg[i]));
      dwacc[i] += gv[i] * ov[i] * r * zv[i] * sg[i];
    }
    if (ok) {
      Vec<E>::store(d_o + row * DV + sub * V, dov);
      Vec<E>::store(dz + row * DV + sub * V, dzv);
    }
  }
#pragma unroll
  for (int i = 0; i < V; ++i) red[rin][sub * V + i] = dwacc[i];
  __syncthreads();
  for (int c = threadIdx.x; c < DV; c += kNormThreads) {
    float s = 0.f;
    for (int k = 0; k < RPB; ++k) s += red[k][c];
    dw_part[(size_t)blockIdx.x * DV + c] = s;
  }
}


size_t norm_bwd_ws_bytes(const gdn_shape* s) { return (size_t)kNormBwdBlocks * s->d_v * sizeof(float); }

size_t norm_scratch_bytes() { return sizeof(scratch); }

// Device address of `scratch` on the current device.  In host code the array's
// name stands for a host-side shadow, not device memory, so kernels get this
// address instead; it is looked up once per device (with that device current)
// and kept.
void* norm_scratch_ptr() {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* ptr[kMaxDevices] = {};
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (!ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    ptr[dev] = p;
  }
  return ptr[dev];
}

template <typename E, int DV>
static void launch_norm_fwd(const gdn_shape* s, const void* o, const void* z, const void* w, float eps, void* y,
                            hipStream_t st) {
  constexpr int RPB = kNormThreads / (DV / Vec<E>::N);
  const long rows = (long)s->total_tokens * s->h_v;
  const long blocks = (rows + RPB - 1) / RPB;
  GDN_PROF("norm_fwd", st);
  norm_fwd_kernel<E, DV><<<dim3((unsigned)blocks), kNormThreads, 0, st>>>((const E*)o, (const E*)z,
                                                                          (const E*)w, eps, rows, (E*)y);
}

template <typename E, int DV>
static void launch_norm_bwd(const gdn_shape* s, const void* dy, const void* o, const void* z, const void* w,
                            float eps, void* d_o, void* dz, float* dw, void* ws, hipStream_t st) {
  const long rows = (long)s->total_tokens * s->h_v;
  float* part = (float*)ws;
  {
    GDN_PROF("norm_bwd", st);
    norm_bwd_kernel<E, DV><<<kNormBwdBlocks, kNormThreads, 0, st>>>((const E*)dy, (const E*)o, (const E*)z,
                                                                    (const E*)w, eps, rows, (E*)d_o, (E*)dz, part);
  }
  GDN_PROF("norm_dw_sum", st);
  launch_colsum(part, kNormBwdBlocks, DV, dw, st);
}

bool run_norm_fwd(const gdn_shape* s, const void* o, const void* z, const void* w, float eps, void* y,
                  hipStream_t st) {
  if (s->total_tokens == 0) return true;
#define GDN_NORM(E, D) \
  if (s->d_v == D) { launch_norm_fwd<E, D>(s, o, z, w, eps, y, st); return true; }
  if (s->dtype == GDN_BF16) {
    GDN_NORM(bf16, 16) GDN_NORM(bf16, 32) GDN_NORM(bf16, 64) GDN_NORM(bf16, 128)
  } else {
    GDN_NORM(float, 16) GDN_NORM(float, 32) GDN_NORM(float, 64) GDN_NORM(float, 128)
  }
#undef GDN_NORM
  return false;
}

bool run_norm_bwd(const gdn_shape* s, const void* dy, const void* o, const void* z, const void* w, float eps,
                  void* d_o, void* dz, float* dw, void* ws, hipStream_t st) {
#define GDN_NORM(E, D) \
  if (s->d_v == D) { launch_norm_bwd<E, D>(s, dy, o, z, w, eps, d_o, dz, dw, ws, st); return true; }
  if (s->dtype == GDN_BF16) {
    GDN_NORM(bf16, 16) GDN_NORM(bf16, 32) GDN_NORM(bf16, 64) GDN_NORM(bf16, 128)
  } else {
    GDN_NORM(float, 16) GDN_NORM(float, 32) GDN_NORM(float, 64) GDN_NORM(float, 128)
  }
#undef GDN_NORM
  return false;
}

}  // namespace gdn
