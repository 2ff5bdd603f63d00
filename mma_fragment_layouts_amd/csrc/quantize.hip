// Elementwise fp32 -> 16-bit rounding and hi/lo splitting on the device.
//
// Tensor-core layout explainer, paragraph on mixed precision: conversion to a
// 16-bit format changes the values that enter the multiply.  Strata PR #800,
// "What's going on": an fp32 value is carried as a 16-bit hi part plus a 16-bit
// lo part, hi = RNE(x), lo = RNE(x - hi) (x - hi is exact in fp32).
#include "common.hpp"

using namespace mfl;

namespace {

// Each thread converts 8 consecutive values per step (two 16-byte loads, one
// 16-byte store per output); a scalar loop finishes a ragged tail.
template <int DT, bool SPLIT>
__global__ __launch_bounds__(256) void convert_kernel(const float* __restrict__ x, uint16_t* __restrict__ hi,
                                                     uint16_t* __restrict__ lo, int64_t n) {
  const int64_t nvec = n / 8;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; v < nvec; v += stride) {
    const f32x4 p = *reinterpret_cast<const f32x4*>(x + v * 8);
    const f32x4 q = *reinterpret_cast<const f32x4*>(x + v * 8 + 4);
    float f[8] = {p[0], p[1], p[2], p[3], q[0], q[1], q[2], q[3]};
    uint16_t h[8], l[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      h[e] = to16<DT>(f[e]);
      if constexpr (SPLIT) l[e] = to16<DT>(f[e] - from16<DT>(h[e]));
    }
    u32x4 hv, lv;
    __builtin_memcpy(&hv, h, 16);
    *reinterpret_cast<u32x4*>(hi + v * 8) = hv;
    if constexpr (SPLIT) {
      __builtin_memcpy(&lv, l, 16);
      *reinterpret_cast<u32x4*>(lo + v * 8) = lv;
    }
  }
  for (int64_t i = nvec * 8 + (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    const uint16_t h = to16<DT>(x[i]);
    hi[i] = h;
    if constexpr (SPLIT) lo[i] = to16<DT>(x[i] - from16<DT>(h));
  }
}

template <int DT, bool SPLIT>
int launch(const float* x, void* hi, void* lo, int64_t n, hipStream_t s) {
  int64_t blocks = (n / 8 + 255) / 256;
  if (blocks < 1) blocks = 1;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL((convert_kernel<DT, SPLIT>), dim3((unsigned)blocks), dim3(256), 0, s, x, (uint16_t*)hi,
                     (uint16_t*)lo, n);
  return launch_status();
}

}  // namespace

extern "C" int quantize_fp32(int dtype, const float* x, void* out, int64_t n, void* stream) {
  if (dtype != MFL_F16 && dtype != MFL_BF16) return MFL_EINVAL;
  if (n < 0) return MFL_EINVAL;
  if (n == 0) return MFL_OK;
  if (!x || !out || !aligned16(x) || !aligned16(out)) return MFL_EINVAL;
  hipStream_t s = (hipStream_t)stream;
  return dtype == MFL_BF16 ? launch<MFL_BF16, false>(x, out, nullptr, n, s) : launch<MFL_F16, false>(x, out, nullptr, n, s);
}

extern "C" int split_fp32(int dtype, const float* x, void* hi, void* lo, int64_t n, void* stream) {
  if (dtype != MFL_F16 && dtype != MFL_BF16) return MFL_EINVAL;
  if (n < 0) return MFL_EINVAL;
  if (n == 0) return MFL_OK;
  if (!x || !hi || !lo || !aligned16(x) || !aligned16(hi) || !aligned16(lo)) return MFL_EINVAL;
  hipStream_t s = (hipStream_t)stream;
  return dtype == MFL_BF16 ? launch<MFL_BF16, true>(x, hi, lo, n, s) : launch<MFL_F16, true>(x, hi, lo, n, s);
}
