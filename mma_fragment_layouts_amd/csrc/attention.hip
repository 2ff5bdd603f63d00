// attention_split_fp32: the attention-shaped pair of split GEMMs of Strata PR
// #800 — algo 0 (below) materialises the scores; algo 1 is the fused kernel of
// attention_fused.hip ("What's going on": q is split for q.k, p is split for p.v, each into an
// FP16 hi and lo half; "The fix": hi and lo products in separate accumulators).
//
//   1. S = Q K^T           split GEMM, Q split into f16 hi/lo, K rounded once
//   2. m = rowmax S, P~ = exp(S - m), l = rowsum P~          (fp32, in place)
//   3. O_s = P~[:, slice s] V[slice s, :]   split GEMM over K slices, P~ split,
//                                           V rounded once
//   4. O = (sum_s O_s) / l  slices summed in a fixed order
//
// Normalisation is deferred to step 4: P~ lies in (0, 1] with its maximum
// exactly 1, whereas the normalised probabilities (about 1/nk) would fall in
// fp16's subnormal range and lose most of their lo half.  softmax(S) V equals
// (P~ V) / l exactly in real arithmetic.  This version materialises S / P~ in
// the caller's workspace (HBM-bound); it keeps every step on the device.
#include <mutex>

#include "attention_fused.hpp"
#include "gemm_split.hpp"

namespace mfl {

int64_t attn_fused_workspace(int64_t nq, int64_t nk, bool skv);
int launch_attn_fused(int64_t nq, int64_t nk, const float* q, const float* k, const float* v, int chains, bool skv,
                      float* o, void* workspace, hipStream_t st);

namespace {

constexpr int kSoftmaxThreads = 512;
constexpr int kSoftmaxVec = 16;  // f32x4 per thread: rows up to 32768 stay in registers
// P~ = exp(s - m) is taken as 2^((s - m) log2 e) with the hardware exp2.
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

// Block-wide reduction of one value per thread (kSoftmaxThreads threads).
template <bool MAX>
__device__ __forceinline__ float block_reduce(float x, float* red) {
  x = MAX ? wave_max(x) : wave_sum(x);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = x;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int i = 1; i < kSoftmaxThreads / 64; ++i) r = MAX ? fmaxf(r, red[i]) : r + red[i];
  return r;
}

// One workgroup per row; the row (n <= 32768, n % 4 == 0) is read once into
// registers (non-temporal loads: S is not read again), P~ written back in
// place, m and l written per row.  The row sum adds each thread's values in
// order, then the threads' partial sums.
__global__ __launch_bounds__(kSoftmaxThreads) void softmax_rows_regs(float* __restrict__ S, int64_t lds_, int n,
                                                                   float* __restrict__ m_out,
                                                                   float* __restrict__ l_out) {
  __shared__ float red[kSoftmaxThreads / 64];
  float* row = S + (int64_t)blockIdx.x * lds_;
  f32x4 v[kSoftmaxVec];
  float mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < kSoftmaxVec; ++i) {
    const int c = (i * kSoftmaxThreads + threadIdx.x) * 4;
    if (c < n) {
      v[i] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(row + c));
      mx = fmaxf(mx, fmaxf(fmaxf(v[i][0], v[i][1]), fmaxf(v[i][2], v[i][3])));
    }
  }
  mx = block_reduce<true>(mx, red);
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < kSoftmaxVec; ++i) {
    const int c = (i * kSoftmaxThreads + threadIdx.x) * 4;
    if (c < n) {
      f32x4 p;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        p[e] = __builtin_amdgcn_exp2f((v[i][e] - mx) * kLog2e);
        sum += p[e];
      }
      *reinterpret_cast<f32x4*>(row + c) = p;
    }
  }
  sum = block_reduce<false>(sum, red);
  if (threadIdx.x == 0) {
    m_out[blockIdx.x] = mx;
    l_out[blockIdx.x] = sum;
  }
}

// Rows longer than the register budget: one pass for the max, one for P~ and l.
__global__ __launch_bounds__(kSoftmaxThreads) void softmax_rows_2pass(float* __restrict__ S, int64_t lds_, int n,
                                                                    float* __restrict__ m_out,
                                                                    float* __restrict__ l_out) {
  __shared__ float red[kSoftmaxThreads / 64];
  float* row = S + (int64_t)blockIdx.x * lds_;
  float mx = -INFINITY;
  for (int c = threadIdx.x * 4; c < n; c += kSoftmaxThreads * 4) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(row + c);
    mx = fmaxf(mx, fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3])));
  }
  mx = block_reduce<true>(mx, red);
  float sum = 0.f;
  for (int c = threadIdx.x * 4; c < n; c += kSoftmaxThreads * 4) {
    f32x4 p = *reinterpret_cast<const f32x4*>(row + c);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      p[e] = __builtin_amdgcn_exp2f((p[e] - mx) * kLog2e);
      sum += p[e];
    }
    *reinterpret_cast<f32x4*>(row + c) = p;
  }
  sum = block_reduce<false>(sum, red);
  if (threadIdx.x == 0) {
    m_out[blockIdx.x] = mx;
    l_out[blockIdx.x] = sum;
  }
}

// O[r][c] = (sum over slices s = 0, 1, ... of part[s][r][c]) / l[r].
__global__ __launch_bounds__(256) void reduce_slices(const float* __restrict__ part, int splits, int64_t stride,
                                                   const float* __restrict__ l, float* __restrict__ O, int d,
                                                   int64_t total) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= total) return;
  float acc = 0.f;
  for (int s = 0; s < splits; ++s) acc += part[s * stride + i];
  O[i] = acc / l[i / d];
}

struct Workspace {
  int64_t s_off, m_off, l_off, part_off, total;
  int splits;
};

int64_t align256(int64_t x) { return (x + 255) & ~(int64_t)255; }

// Split count of the second GEMM: enough slices of K (multiples of 64 keys)
// for about 512 workgroups over its (nq/128) output tiles.
int choose_splits(int64_t nq, int64_t nk) {
  const int64_t tiles = nq / 128;
  int s = 1;
  while (s < 32 && tiles * s < 512 && nk % (2 * s * 64) == 0) s *= 2;
  return s;
}

Workspace plan(int64_t nq, int64_t nk, int64_t d) {
  Workspace w;
  w.splits = choose_splits(nq, nk);
  int64_t off = 0;
  w.s_off = off;
  off = align256(off + nq * nk * 4);
  w.m_off = off;
  off = align256(off + nq * 4);
  w.l_off = off;
  off = align256(off + nq * 4);
  w.part_off = off;
  off = align256(off + (int64_t)w.splits * nq * d * 4);
  w.total = off;
  return w;
}

bool valid_sizes(int64_t nq, int64_t nk, int64_t d) {
  return d == 128 && nq > 0 && nk > 0 && nq % 128 == 0 && nk % 128 == 0 && nq <= (1 << 24) && nk <= (1 << 24) &&
         nq * nk <= ((int64_t)1 << 34);
}

// The fused kernel addresses K16 and V16^T through buffer descriptors with a
// 32-bit byte extent (nk * 128 * 2 bytes).
bool fused_fits(int64_t nk) { return nk * kAttnD * 2 <= (int64_t)UINT32_MAX; }

}  // namespace
}  // namespace mfl

using namespace mfl;

namespace {

// Checks of everything but the workspace (host only, before any HIP call).
int attention_args(int64_t nq, int64_t nk, int64_t d, const float* q, const float* k, const float* v, int chains,
                   int algo, const float* o) {
  if (chains != 1 && chains != 2) return MFL_EINVAL;
  if (algo < 0 || algo > 2) return MFL_EINVAL;
  if (!valid_sizes(nq, nk, d)) return nq < 0 || nk < 0 || d < 0 ? MFL_EINVAL : MFL_EUNSUPPORTED;
  if (!q || !k || !v || !o) return MFL_EINVAL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return MFL_EINVAL;
  if (algo >= 1 && !fused_fits(nk)) return MFL_EUNSUPPORTED;
  return MFL_OK;
}

int64_t attention_need(int64_t nq, int64_t nk, int64_t d, int algo) {
  return algo == 0 ? plan(nq, nk, d).total : attn_fused_workspace(nq, nk, algo == 2);
}

// Launches the algorithm on a workspace of at least attention_need bytes
// (arguments already checked).
int attention_launch(int64_t nq, int64_t nk, int64_t d, const float* q, const float* k, const float* v, int chains,
                     int algo, float* o, void* workspace, hipStream_t s) {
  if (algo >= 1) return launch_attn_fused(nq, nk, q, k, v, chains, algo == 2, o, workspace, s);
  const Workspace w = plan(nq, nk, d);
  char* ws = (char*)workspace;
  float* S = (float*)(ws + w.s_off);
  float* m = (float*)(ws + w.m_off);
  float* l = (float*)(ws + w.l_off);
  float* part = (float*)(ws + w.part_off);
  const int NQ = (int)nq, NK = (int)nk, D = (int)d;
  int st;
  // 1. S = split(Q) . round(K)^T ; K (nk x d row-major) is B = K^T column-major.
  st = dispatch_split_modes<MFL_F16, true, true>(true, false, chains, false, q, d, k, d, S, nk, NQ, NK, D, 1, D, 0, 0,
                                                 s);
  if (st != MFL_OK) return st;
  // 2. row softmax pieces, P~ in place.
  if (nk <= (int64_t)kSoftmaxThreads * kSoftmaxVec * 4)
    hipLaunchKernelGGL(softmax_rows_regs, dim3(NQ), dim3(kSoftmaxThreads), 0, s, S, nk, NK, m, l);
  else
    hipLaunchKernelGGL(softmax_rows_2pass, dim3(NQ), dim3(kSoftmaxThreads), 0, s, S, nk, NK, m, l);
  if ((st = launch_status()) != MFL_OK) return st;
  // 3. partial O per K slice: split(P~) . round(V) ; V (nk x d row-major) is B row-major.
  const int kps = NK / w.splits;
  st = dispatch_split_modes<MFL_F16, true, false>(true, false, chains, false, S, nk, v, d, part, d, NQ, D, NK, w.splits,
                                                  kps, nq * d, 0, s);
  if (st != MFL_OK) return st;
  // 4. fixed-order sum of the slices, then divide by l.
  const int64_t total = nq * d;
  hipLaunchKernelGGL(reduce_slices, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, part, w.splits, nq * d, l,
                     o, D, total);
  return launch_status();
}

}  // namespace

extern "C" int attention_workspace_bytes(int64_t nq, int64_t nk, int64_t d, int algo, int64_t* bytes) {
  if (!bytes || algo < 0 || algo > 2) return MFL_EINVAL;
  if (!valid_sizes(nq, nk, d) || (algo >= 1 && !fused_fits(nk))) return MFL_EUNSUPPORTED;
  *bytes = attention_need(nq, nk, d, algo);
  return MFL_OK;
}

extern "C" int attention_split_fp32(int64_t nq, int64_t nk, int64_t d, const float* q, const float* k, const float* v,
                                    int chains, int algo, float* o, void* workspace, int64_t workspace_bytes,
                                    void* stream) {
  int st = attention_args(nq, nk, d, q, k, v, chains, algo, o);
  if (st != MFL_OK) return st;
  if (!workspace || ((uintptr_t)workspace & 255) != 0) return MFL_EINVAL;
  if (workspace_bytes < attention_need(nq, nk, d, algo)) return MFL_EINVAL;
  return attention_launch(nq, nk, d, q, k, v, chains, algo, o, workspace, (hipStream_t)stream);
}

// ---- allocation-free variant -------------------------------------------------
// The workspace lives in a file-scope device array, one copy per GPU.  Its
// name is a host-side stand-in in host code: the device address of this GPU's
// copy comes from hipGetSymbolAddress, taken once per device on the first call
// made with that device current, and only that address is handed to kernels.
namespace {

static __device__ __attribute__((aligned(256))) char scratch[MFL_ATTN_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

int device_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return MFL_EHIP;
  if (dev < 0 || dev >= kMaxDevices) return MFL_EUNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MFL_EHIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MFL_OK;
}

}  // namespace

extern "C" int attention_split_fp32_static(int64_t nq, int64_t nk, int64_t d, const float* q, const float* k,
                                           const float* v, int chains, int algo, float* o, void* stream) {
  const int st = attention_args(nq, nk, d, q, k, v, chains, algo, o);
  if (st != MFL_OK) return st;
  if (attention_need(nq, nk, d, algo) > MFL_ATTN_STATIC_SCRATCH_BYTES) return MFL_ESCRATCH;
  void* ws = nullptr;
  const int sp = device_scratch(&ws);
  if (sp != MFL_OK) return sp;
  return attention_launch(nq, nk, d, q, k, v, chains, algo, o, ws, (hipStream_t)stream);
}
