// Achievable-peak probes for the measurement: a streaming copy (HBM) and a
// loop of independent bf16 MFMAs (matrix cores).  Neither is part of the
// layer; the benchmark times them with HIP events to report what this chip
// reaches beside the published peaks it prices every kernel against.
#include <algorithm>

#include "gdn_common.cuh"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kProbeThreads = 256;

// grid-stride copy, 16 bytes per lane, four loads in flight per lane
__global__ __launch_bounds__(kProbeThreads) void probe_copy_kernel(const uint4* __restrict__ src,
                                                                   uint4* __restrict__ dst, size_t n) {
  const size_t stride = (size_t)gridDim.x * kProbeThreads;
  size_t i = (size_t)blockIdx.x * kProbeThreads + threadIdx.x;
  for (; i + 3 * stride < n; i += 4 * stride) {
    const uint4 a = src[i], b = src[i + stride], c = src[i + 2 * stride], d = src[i + 3 * stride];
    dst[i] = a;
    dst[i + stride] = b;
    dst[i + 2 * stride] = c;
    dst[i + 3 * stride] = d;
  }
  for (; i < n; i += stride) dst[i] = src[i];
}

// each wave: independent accumulator chains of bf16 matrix-core products,
// iters rounds; the sums leave through out so nothing is optimised away.
// SHAPE 0: v_mfma_f32_16x16x32_bf16 (8 chains, 16384 flops each);
// SHAPE 1: v_mfma_f32_32x32x16_bf16 (4 chains, 32768 flops each)
template <int SHAPE>
__global__ __launch_bounds__(kProbeThreads) void probe_mfma_kernel(float* __restrict__ out, int iters) {
  typedef Mma<bf16> M;
  const int lane = lane_id();
  float av[8], bv[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    av[i] = 1e-3f * (float)((lane + i) & 7);
    bv[i] = 1e-3f * (float)((lane * 3 + i) & 7);
  }
  const M::frag a = M::from_floats(av), b = M::from_floats(bv);
  float s = 0.f;
  if constexpr (SHAPE == 0) {
    f32x4 acc[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] = zero4();
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[c] = M::mma(a, b, acc[c]);
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) s += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
  } else {
    typedef float f32x16 __attribute__((ext_vector_type(16)));
    f32x16 acc[4];
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[c][e] = 0.f;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
    }
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int e = 0; e < 16; ++e) s += acc[c][e];
  }
  out[(size_t)blockIdx.x * kProbeThreads + threadIdx.x] = s;
}

}  // namespace
}  // namespace gdn

using namespace gdn;

extern "C" {

gdn_status gdn_probe_copy(const void* src, void* dst, size_t bytes, gdn_stream stream) {
  if (!src || !dst || bytes % 16 || ((uintptr_t)src & 15u) || ((uintptr_t)dst & 15u)) return GDN_ERR_INVALID_ARG;
  const size_t n = bytes / 16;
  if (n == 0) return GDN_OK;
  const unsigned blocks = (unsigned)std::min<size_t>((n + kProbeThreads - 1) / kProbeThreads, 4096);
  probe_copy_kernel<<<blocks, kProbeThreads, 0, (hipStream_t)stream>>>((const uint4*)src, (uint4*)dst, n);
  return hipGetLastError() == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

gdn_status gdn_probe_mfma(float* out, int32_t blocks, int32_t iters, int32_t shape, gdn_stream stream) {
  if (!out || blocks < 1 || iters < 1 || shape < 0 || shape > 1) return GDN_ERR_INVALID_ARG;
  if (shape == 0) probe_mfma_kernel<0><<<(unsigned)blocks, kProbeThreads, 0, (hipStream_t)stream>>>(out, iters);
  else probe_mfma_kernel<1><<<(unsigned)blocks, kProbeThreads, 0, (hipStream_t)stream>>>(out, iters);
  return hipGetLastError() == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

}  // extern "C"
