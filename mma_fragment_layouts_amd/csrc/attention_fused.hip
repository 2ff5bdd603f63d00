// Kernels of the fused split-precision attention (design notes in
// attention_fused.hpp): preparation of K and V^T in fp16, the fused per-slice
// kernel, and the fixed-order combine of the key slices.
#include "attention_fused.hpp"

namespace mfl {
namespace {

template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// K (nk x 128 fp32) -> K16 (nk x 128 fp16, round to nearest even); 8 values per thread.
__global__ __launch_bounds__(256) void attn_prep_k(const float* __restrict__ K, uint16_t* __restrict__ Kq,
                                                   int64_t n8) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n8) return;
  const f32x4 a = *reinterpret_cast<const f32x4*>(K + i * 8);
  const f32x4 b = *reinterpret_cast<const f32x4*>(K + i * 8 + 4);
  u32x4 o;
  o[0] = pack2(to16<MFL_F16>(a[0]), to16<MFL_F16>(a[1]));
  o[1] = pack2(to16<MFL_F16>(a[2]), to16<MFL_F16>(a[3]));
  o[2] = pack2(to16<MFL_F16>(b[0]), to16<MFL_F16>(b[1]));
  o[3] = pack2(to16<MFL_F16>(b[2]), to16<MFL_F16>(b[3]));
  *reinterpret_cast<u32x4*>(Kq + i * 8) = o;
}

// V (nk x 128 fp32) -> V16^T (128 x nk fp16), keys of each 32-key block stored at
// vt_key_pos(r).  One workgroup per 32-key block, transposed through LDS.
__global__ __launch_bounds__(256) void attn_prep_vt(const float* __restrict__ V, uint16_t* __restrict__ Vt, int nk) {
  __shared__ __attribute__((aligned(16))) uint16_t t[kAttnD * 32];
  const int blk = blockIdx.x, tid = threadIdx.x;
  {
    const int key = tid >> 3, d0 = (tid & 7) * 16;
    const float* src = V + ((int64_t)blk * 32 + key) * kAttnD + d0;
    const int pos = vt_key_pos(key);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(src + 4 * q);
#pragma unroll
      for (int e = 0; e < 4; ++e) t[(d0 + 4 * q + e) * 32 + pos] = to16<MFL_F16>(v[e]);
    }
  }
  __syncthreads();
  const int dim = tid >> 1, half = tid & 1;
  uint16_t* dst = Vt + (int64_t)dim * nk + (int64_t)blk * 32 + half * 16;
  *reinterpret_cast<u32x4*>(dst) = *reinterpret_cast<const u32x4*>(t + dim * 32 + half * 16);
  *reinterpret_cast<u32x4*>(dst + 8) = *reinterpret_cast<const u32x4*>(t + dim * 32 + half * 16 + 8);
}

// Grid: x = query blocks of 128, y = key slices of keys_per_split keys.
template <int CHAINS, int STAGES>
__global__ __launch_bounds__(256) void attn_fused_kernel(const float* __restrict__ Q, const uint16_t* __restrict__ Kq,
                                                         const uint16_t* __restrict__ Vt, float* __restrict__ Opart,
                                                         float* __restrict__ Mpart, float* __restrict__ Lpart, int nq,
                                                         int nk, int keys_per_split) {
  constexpr int BK = 64;                                  // LDS tile depth (dims for K16, keys for V16^T)
  constexpr int KT = kAttnKV * BK;                        // one K16 half tile: 64 keys x 64 dims
  constexpr int STAGE = 2 * KT + kAttnD * kAttnKV;        // K16 halves + V16^T tile (elements)
  constexpr int LOADS = 8;                                // 1 KiB wave loads per stage per wave (32 / 4)
  __shared__ __attribute__((aligned(1024))) uint16_t lds[STAGES * STAGE];

  const int sp = blockIdx.y;
  const int kbeg = sp * keys_per_split;
  const int nchunks = keys_per_split / kAttnKV;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lr = lane & 15, g = lane >> 4;
  const int qw = blockIdx.x * kAttnQ + wave * 32;

  // Q^T fragments (B operand of GEMM1), split once: lane supplies query
  // qw + 16*qt + lr, dims 32*d + 8*g .. +7.
  u32x4 qh[2][4], ql[2][4];
#pragma unroll
  for (int qt = 0; qt < 2; ++qt)
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const float* p = Q + (int64_t)(qw + 16 * qt + lr) * kAttnD + 32 * d + 8 * g;
      const f32x4 x0 = *reinterpret_cast<const f32x4*>(p), x1 = *reinterpret_cast<const f32x4*>(p + 4);
      uint16_t h[8], l[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = e < 4 ? x0[e] : x1[e - 4];
        h[e] = to16<MFL_F16>(x);
        l[e] = to16<MFL_F16>(x - from16<MFL_F16>(h[e]));
      }
      __builtin_memcpy(&qh[qt][d], h, 16);
      __builtin_memcpy(&ql[qt][d], l, 16);
    }

  // Stage fill: 32 wave loads of 1 KiB (8 rows of 128 bytes); this wave issues
  // blocks b = wave + 4*i.  Blocks 0-15: K16 half b/8, key rows 8*(b%8)..;
  // blocks 16-31: V16^T dim rows 8*(b-16)...  Physical chunk lane%8 of row
  // 8*blk + lane/8 receives logical chunk (lane%8) ^ swz(row).
  const rsrc_t rk = make_rsrc(Kq, (uint32_t)((int64_t)nk * kAttnD * 2));
  const rsrc_t rv = make_rsrc(Vt, (uint32_t)((int64_t)nk * kAttnD * 2));
  uint32_t voff[LOADS];
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int b = wave + 4 * i;  // wave-uniform
    const int blk = b < 16 ? (b & 7) : b - 16;
    const int row = 8 * blk + (lane >> 3);
    const int lch = (lane & 7) ^ swz<BK>(row);
    if (b < 16)
      voff[i] = (uint32_t)(row * kAttnD + 64 * (b >> 3) + lch * 8) * 2u;
    else
      voff[i] = (uint32_t)(row * nk + lch * 8) * 2u;
  }
  auto issue = [&](int stage, int key0) {
    uint16_t* base = lds + stage * STAGE;
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int b = wave + 4 * i;
      if (b < 16)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_ptr_t)(base + (b >> 3) * KT + (b & 7) * 8 * BK), 16,
                                                 voff[i], (uint32_t)key0 * kAttnD * 2u, 0, 0);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_ptr_t)(base + 2 * KT + (b - 16) * 8 * BK), 16, voff[i],
                                                 (uint32_t)key0 * 2u, 0, 0);
    }
  };

  const FragOffsets<0, BK> fo(0, lane);  // lane row lr, chunk 4*kk + g
  f32x4 oh[8][2], ol[8][2];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      oh[i][qt] = f32x4{0.f, 0.f, 0.f, 0.f};
      ol[i][qt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  float m[2] = {-INFINITY, -INFINITY}, lsum[2] = {0.f, 0.f};

#pragma unroll
  for (int s = 0; s < STAGES - 1; ++s)
    if (s < nchunks) issue(s, kbeg + s * kAttnKV);
  for (int c = 0; c < nchunks; ++c) {
    if (c + STAGES - 2 < nchunks)
      wait_vm<(STAGES - 2) * LOADS>();
    else
      wait_vm<0>();
    __syncthreads();
    if (c + STAGES - 1 < nchunks) issue((c + STAGES - 1) % STAGES, kbeg + (c + STAGES - 1) * kAttnKV);
    const uint16_t* st = lds + (c % STAGES) * STAGE;

    // GEMM1: S^T (keys x queries), 4 key tiles x 2 query tiles
    f32x4 sh[4][2], sl[4][2];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
        sh[kt][qt] = f32x4{0.f, 0.f, 0.f, 0.f};
        sl[kt][qt] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      u32x4 a[4];
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) a[kt] = lds_read16(st + (d >> 1) * KT, fo.off[d & 1] + kt * 16 * BK);
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) {
          sh[kt][qt] = mfma<0, MFL_F16>(a[kt], qh[qt][d], sh[kt][qt]);
          if constexpr (CHAINS == 2)
            sl[kt][qt] = mfma<0, MFL_F16>(a[kt], ql[qt][d], sl[kt][qt]);
          else
            sh[kt][qt] = mfma<0, MFL_F16>(a[kt], ql[qt][d], sh[kt][qt]);
        }
    }

    // online softmax on the accumulators; lanes lr, lr+16, lr+32, lr+48 share a query
    u32x4 ph[2][2], pl[2][2];
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      float cmax = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        if constexpr (CHAINS == 2) sh[kt][qt] = sh[kt][qt] + sl[kt][qt];
#pragma unroll
        for (int j = 0; j < 4; ++j) cmax = fmaxf(cmax, sh[kt][qt][j]);
      }
      cmax = fmaxf(cmax, __shfl_xor(cmax, 16, 64));
      cmax = fmaxf(cmax, __shfl_xor(cmax, 32, 64));
      const float mnew = fmaxf(m[qt], cmax);
      const float sc = expf(m[qt] - mnew);
      m[qt] = mnew;
      lsum[qt] *= sc;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        oh[i][qt] = oh[i][qt] * sc;
        if constexpr (CHAINS == 2) ol[i][qt] = ol[i][qt] * sc;
      }
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        uint16_t h[8], l[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float p = expf(sh[2 * t + (e >> 2)][qt][e & 3] - mnew);
          lsum[qt] += p;
          h[e] = to16<MFL_F16>(p);
          l[e] = to16<MFL_F16>(p - from16<MFL_F16>(h[e]));
        }
        __builtin_memcpy(&ph[t][qt], h, 16);
        __builtin_memcpy(&pl[t][qt], l, 16);
      }
    }

    // GEMM2: O^T (dims x queries) += V16^T . P~^T
    const uint16_t* sv = st + 2 * KT;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const u32x4 a = lds_read16(sv, fo.off[t] + i * 16 * BK);
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) {
          oh[i][qt] = mfma<0, MFL_F16>(a, ph[t][qt], oh[i][qt]);
          if constexpr (CHAINS == 2)
            ol[i][qt] = mfma<0, MFL_F16>(a, pl[t][qt], ol[i][qt]);
          else
            oh[i][qt] = mfma<0, MFL_F16>(a, pl[t][qt], oh[i][qt]);
        }
      }
  }

  // slice results: unnormalised O (chains added in fp32), m, and l summed over
  // the four lanes of each query
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    float lt = lsum[qt];
    lt += __shfl_xor(lt, 16, 64);
    lt += __shfl_xor(lt, 32, 64);
    const int q = qw + 16 * qt + lr;
    float* orow = Opart + ((int64_t)sp * nq + q) * kAttnD;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      f32x4 o = oh[i][qt];
      if constexpr (CHAINS == 2) o = o + ol[i][qt];
      *reinterpret_cast<f32x4*>(orow + 16 * i + 4 * g) = o;
    }
    if (g == 0) {
      Mpart[(int64_t)sp * nq + q] = m[qt];
      Lpart[(int64_t)sp * nq + q] = lt;
    }
  }
}

// O[q][d] = sum_s w_s O_s[q][d] / sum_s w_s l_s[q], w_s = exp(m_s - max_s m_s),
// slices taken in order s = 0, 1, ...
__global__ __launch_bounds__(256) void attn_combine(const float* __restrict__ Opart, const float* __restrict__ Mpart,
                                                    const float* __restrict__ Lpart, float* __restrict__ O, int nq,
                                                    int splits) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)nq * kAttnD) return;
  const int q = (int)(i / kAttnD);
  float mx = -INFINITY;
  for (int s = 0; s < splits; ++s) mx = fmaxf(mx, Mpart[(int64_t)s * nq + q]);
  float num = 0.f, den = 0.f;
  for (int s = 0; s < splits; ++s) {
    const float w = expf(Mpart[(int64_t)s * nq + q] - mx);
    num += w * Opart[(int64_t)s * nq * kAttnD + i];
    den += w * Lpart[(int64_t)s * nq + q];
  }
  O[i] = num / den;
}

}  // namespace

// Sizes of the fused path's workspace pieces (bytes, each 256-aligned).
int64_t attn_fused_splits(int64_t nq, int64_t nk) {
  const int64_t qblocks = nq / kAttnQ;
  int64_t s = 1;
  while (s < 32 && qblocks * s < 512 && nk % (2 * s * kAttnKV) == 0) s *= 2;
  return s;
}

int64_t attn_fused_workspace(int64_t nq, int64_t nk) {
  auto al = [](int64_t x) { return (x + 255) & ~(int64_t)255; };
  const int64_t s = attn_fused_splits(nq, nk);
  return al(nk * kAttnD * 2) * 2 + al(s * nq * kAttnD * 4) + 2 * al(s * nq * 4);
}

int launch_attn_fused(int64_t nq, int64_t nk, const float* q, const float* k, const float* v, int chains, float* o,
                      void* workspace, hipStream_t st) {
  auto al = [](int64_t x) { return (x + 255) & ~(int64_t)255; };
  const int64_t splits = attn_fused_splits(nq, nk);
  char* w = (char*)workspace;
  uint16_t* kq = (uint16_t*)w;
  w += al(nk * kAttnD * 2);
  uint16_t* vt = (uint16_t*)w;
  w += al(nk * kAttnD * 2);
  float* op = (float*)w;
  w += al(splits * nq * kAttnD * 4);
  float* mp = (float*)w;
  w += al(splits * nq * 4);
  float* lp = (float*)w;
  const int64_t n8 = nk * kAttnD / 8;
  hipLaunchKernelGGL(attn_prep_k, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, st, k, kq, n8);
  hipLaunchKernelGGL(attn_prep_vt, dim3((unsigned)(nk / 32)), dim3(256), 0, st, v, vt, (int)nk);
  const dim3 grid((unsigned)(nq / kAttnQ), (unsigned)splits);
  const int kps = (int)(nk / splits);
  if (chains == 2)
    hipLaunchKernelGGL((attn_fused_kernel<2, 3>), grid, dim3(256), 0, st, q, kq, vt, op, mp, lp, (int)nq, (int)nk, kps);
  else
    hipLaunchKernelGGL((attn_fused_kernel<1, 3>), grid, dim3(256), 0, st, q, kq, vt, op, mp, lp, (int)nq, (int)nk, kps);
  const int64_t total = nq * kAttnD;
  hipLaunchKernelGGL(attn_combine, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, op, mp, lp, o, (int)nq,
                     (int)splits);
  return launch_status();
}

}  // namespace mfl
