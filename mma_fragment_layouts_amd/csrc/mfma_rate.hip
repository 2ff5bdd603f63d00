// mfma_rate_probe: the rate at which the chip's matrix cores retire
// v_mfma_f32_16x16x32 when nothing else runs — no memory traffic, no LDS, no
// dependent vector work.  It is the measured ceiling that a GEMM kernel's rate
// is compared with, next to the published peak (256 CUs x 4096 flop/clock x
// 2.4 GHz), which assumes a clock that the chip does not hold under MFMA load.
#include "common.hpp"

namespace mfl {
namespace {

constexpr int kRateGroups = 2048;  // workgroups: eight per compute unit
constexpr int kRateThreads = 256;  // four waves
constexpr int kRateChains = 16;    // independent accumulators per wave
static_assert(kRateGroups * kRateThreads == MFL_RATE_PROBE_OUTPUTS, "output count in mfl.h");

// Two 16-bit operand values of lane `lane`, pair index e.  seed 0: both 1.0.
// Otherwise a per-lane hash sets the mantissa bits of values in [1, 2), so the
// multipliers see changing data.
template <int DT>
__device__ __forceinline__ uint32_t operand_pair(int lane, int e, uint32_t seed) {
  const uint32_t one = DT == MFL_BF16 ? 0x3F80u : 0x3C00u;
  if (seed == 0) return one | (one << 16);
  uint32_t h = (uint32_t)lane * 0x9E3779B1u ^ (uint32_t)e * 0x85EBCA77u ^ seed;
  h ^= h >> 15;
  h *= 0x2C1B3C6Du;
  h ^= h >> 12;
  const uint32_t mask = DT == MFL_BF16 ? 0x7Fu : 0x3FFu;
  return (one | (h & mask)) | ((one | ((h >> 16) & mask)) << 16);
}

template <int DT>
__global__ __launch_bounds__(kRateThreads) void mfma_rate_kernel(int iters, uint32_t seed, float* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  u32x4 a, b;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    a[e] = operand_pair<DT>(lane, e, seed);
    b[e] = operand_pair<DT>(lane, e + 4, seed);
  }
  // distinct starting values keep the chains distinct computations
  f32x4 acc[kRateChains];
#pragma unroll
  for (int c = 0; c < kRateChains; ++c) acc[c] = f32x4{(float)c, (float)c, (float)c, (float)c};
  for (int it = 0; it < iters; ++it)
#pragma unroll
    for (int c = 0; c < kRateChains; ++c) acc[c] = mfma<0, DT>(a, b, acc[c]);
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kRateChains; ++c) s += (acc[c][0] + acc[c][1]) + (acc[c][2] + acc[c][3]);
  out[blockIdx.x * kRateThreads + threadIdx.x] = s;
}

}  // namespace
}  // namespace mfl

using namespace mfl;

extern "C" int mfma_rate_probe(int dtype, int iters, uint32_t seed, float* out, void* stream) {
  if ((dtype != MFL_F16 && dtype != MFL_BF16) || iters < 0 || !out || ((uintptr_t)out & 3)) return MFL_EINVAL;
  hipStream_t s = (hipStream_t)stream;
  if (dtype == MFL_BF16)
    hipLaunchKernelGGL(mfma_rate_kernel<MFL_BF16>, dim3(kRateGroups), dim3(kRateThreads), 0, s, iters, seed, out);
  else
    hipLaunchKernelGGL(mfma_rate_kernel<MFL_F16>, dim3(kRateGroups), dim3(kRateThreads), 0, s, iters, seed, out);
  return launch_status();
}
