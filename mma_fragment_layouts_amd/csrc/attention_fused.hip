// Kernels of the fused split-precision attention (design notes in
// attention_fused.hpp): preparation of K and V in fp16, the fused per-slice
// kernel, and the fixed-order combine of the key slices.
#include "attention_fused.hpp"

namespace mfl {
namespace attn_detail {

// The same split with x - hi taken by v_fma_mix_f32 straight from the fp16 hi
// (x * 1 - hi in one instruction; the difference is exact, so the result is the
// same as converting hi back and subtracting: checked on the device for every
// fp32 value in [2^-40, 2^9), fp16-subnormal hi included).  Two vector
// instructions fewer per pair.
__device__ __forceinline__ Split2 split2_mix(float a, float b) {
  const h16x2 h = __builtin_convertvector(f32x2{a, b}, h16x2);
  const uint32_t hb = __builtin_bit_cast(uint32_t, h);
  float r0, r1;
  asm("v_fma_mix_f32 %0, %1, 1.0, -%2 op_sel_hi:[0,0,1]" : "=v"(r0) : "v"(a), "v"(hb));
  asm("v_fma_mix_f32 %0, %1, 1.0, -%2 op_sel:[0,0,1] op_sel_hi:[0,0,1]" : "=v"(r1) : "v"(b), "v"(hb));
  const h16x2 l = __builtin_convertvector(f32x2{r0, r1}, h16x2);
  return {hb, __builtin_bit_cast(uint32_t, l)};
}

// Elementwise preparation of K and V (both nk x 128 fp32, key-major) into
// K16 and V16 (fp16, round to nearest even, same layout); with SKV also the lo
// planes Kl and Vl, lo = RNE16(x - hi).  Thread t of workgroup b converts the
// 16 consecutive values 16*(256*b + t) .. +15 of each operand (four 16-byte
// loads, two 16-byte stores per plane); n16 = nk * 128 / 16 threads in all.
template <bool SKV>
__global__ __launch_bounds__(256) void attn_prep(const float* __restrict__ K, const float* __restrict__ V,
                                                 uint16_t* __restrict__ Kq, uint16_t* __restrict__ Vq,
                                                 uint16_t* __restrict__ Kl, uint16_t* __restrict__ Vl, int64_t n16) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= n16) return;
  const int64_t idx = t * 16;
#pragma unroll
  for (int op = 0; op < 2; ++op) {
    const float* X = op ? V : K;
    uint16_t* H = op ? Vq : Kq;
    uint16_t* L = op ? Vl : Kl;
    uint32_t wh[8], wl[8];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const f32x4 x = *reinterpret_cast<const f32x4*>(X + idx + 4 * q);
      const Split2 a = split2(x[0], x[1]), b = split2(x[2], x[3]);
      wh[2 * q] = a.hi;
      wh[2 * q + 1] = b.hi;
      wl[2 * q] = a.lo;
      wl[2 * q + 1] = b.lo;
    }
    u32x4 o;
    __builtin_memcpy(&o, wh, 16);
    *reinterpret_cast<u32x4*>(H + idx) = o;
    __builtin_memcpy(&o, wh + 4, 16);
    *reinterpret_cast<u32x4*>(H + idx + 8) = o;
    if constexpr (SKV) {
      __builtin_memcpy(&o, wl, 16);
      *reinterpret_cast<u32x4*>(L + idx) = o;
      __builtin_memcpy(&o, wl + 4, 16);
      *reinterpret_cast<u32x4*>(L + idx + 8) = o;
    }
  }
}

// Maximum over lanes l, l^16, l^32, l^48 without a round trip through the LDS:
// v_permlane16_swap (v_permlane32_swap) with the same value in both operands
// hands every lane the pair {x[l & ~16], x[l | 16]} ({x[l & ~32], x[l | 32]}),
// as a one-wave probe of the instructions shows.  The two results are copied
// to scalars before the bit cast: a bit cast taken straight from an element of
// the returned pair reads element 0 for both (and the max then vanishes).
__device__ __forceinline__ float swap_max(float x, bool by32) {
  const uint32_t b = __builtin_bit_cast(uint32_t, x);
  const auto r = by32 ? __builtin_amdgcn_permlane32_swap(b, b, false, false)
                      : __builtin_amdgcn_permlane16_swap(b, b, false, false);
  const uint32_t r0 = r[0], r1 = r[1];
  return fmaxf(__builtin_bit_cast(float, r0), __builtin_bit_cast(float, r1));
}
__device__ __forceinline__ float max_over_lane_groups(float x) { return swap_max(swap_max(x, false), true); }

// One workgroup: 128 queries (8 waves of 16) x one slice of keys_per_split keys.
// Scores are kept in base-2 units (Q is scaled by log2 e before its split), so
// P~ = 2^(s - mref).  mref is a per-query reference that only moves when a
// chunk's maximum exceeds it by more than kAttnSlack; P~ then stays in
// (0, 2^kAttnSlack] and the rescaling of O and l (by 2^(mref_old - mref_new))
// is skipped for most chunks.  Any reference gives the same O = sum P~ V / sum P~
// in real arithmetic.
//
//
// SKV: K and V are split too (hi planes Kq / Vq, lo planes Kl / Vl).  A stage
// then holds the lo tiles after the hi ones, and each GEMM adds the third
// product into the correction chain: S = Kh Qh | (Kh Ql + Kl Qh), O += Vh Ph |
// (Vh Pl + Vl Ph).
template <int CHAINS, int STAGES, bool SKV>
__global__ __launch_bounds__(512) void attn_fused_kernel(const float* __restrict__ Q, const uint16_t* __restrict__ Kq,
                                                         const uint16_t* __restrict__ Vq,
                                                         const uint16_t* __restrict__ Kl,
                                                         const uint16_t* __restrict__ Vl, float* __restrict__ Opart,
                                                         float* __restrict__ Mpart, float* __restrict__ Lpart, int nq,
                                                         int nk, int keys_per_split, int qblocks, int xcd_map) {
  static_assert(kAttnQ == 128 && kAttnKV == 64 && kAttnD == 128, "tiling below assumes 128 x 64 x 128");
  static_assert(STAGES >= 2, "at least double buffering");
  constexpr int BK = 64;                    // LDS tile depth of the K16 halves (dims)
  constexpr int KT = kAttnKV * BK;          // one K16 half tile: 64 keys x 64 dims
  constexpr int HALF = 2 * KT + kAttnD * kAttnKV;  // K16 halves + k-major V16 tile (elements)
  constexpr int STAGE = SKV ? 2 * HALF : HALF;     // hi tiles, then (SKV) lo tiles
  constexpr int NW = 8;                     // waves per workgroup, 16 queries each
  constexpr int LOADS = 32 / NW;            // 1 KiB wave loads per stage per wave
  __shared__ __attribute__((aligned(1024))) uint16_t lds[STAGES * STAGE];

  int qb, sp;
  attn_block_of(blockIdx.x, gridDim.x, qblocks, xcd_map, qb, sp);
  const int kbeg = sp * keys_per_split;
  const int nchunks = keys_per_split / kAttnKV;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lr = lane & 15, g = lane >> 4;
  const int qw = qb * kAttnQ + wave * 16;

  // Q^T fragments (B operand of GEMM1), scaled by log2 e and split once: lane
  // supplies query qw + lr, dims 32*d + 8*g .. +7.
  u32x4 qh[4], ql[4];
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const float* p = Q + (int64_t)(qw + lr) * kAttnD + 32 * d + 8 * g;
    const f32x4 x0 = *reinterpret_cast<const f32x4*>(p), x1 = *reinterpret_cast<const f32x4*>(p + 4);
    constexpr float kLog2e = 1.4426950408889634f;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const Split2 s0 = split2(x0[2 * e] * kLog2e, x0[2 * e + 1] * kLog2e);
      const Split2 s1 = split2(x1[2 * e] * kLog2e, x1[2 * e + 1] * kLog2e);
      qh[d][e] = s0.hi;
      ql[d][e] = s0.lo;
      qh[d][2 + e] = s1.hi;
      ql[d][2 + e] = s1.lo;
    }
  }

  // Stage fill: 32 wave loads of 1 KiB; this wave issues blocks b = wave + NW*i.
  // Blocks 0-15: K16 half b/8, key rows 8*(b%8) .. +7 (128 bytes each); physical
  // chunk lane%8 of row 8*blk + lane/8 receives logical chunk (lane%8) ^ swz(row).
  // Blocks 16-31: the V16 chunk as a k-major tile (64 key rows x 128 dims, the
  // kmaj_chunk layout of the 16x16x32 instruction), chunk 64*(b-16) + lane; its
  // K row p holds key 32*(p/32) + vt_pos_key(p%32), so that GEMM2's transpose
  // reads hand every lane the keys its P~ fragment holds.
  const rsrc_t rk = make_rsrc(Kq, (uint32_t)((int64_t)nk * kAttnD * 2));
  const rsrc_t rv = make_rsrc(Vq, (uint32_t)((int64_t)nk * kAttnD * 2));
  const rsrc_t rkl = make_rsrc(SKV ? Kl : Kq, (uint32_t)((int64_t)nk * kAttnD * 2));
  const rsrc_t rvl = make_rsrc(SKV ? Vl : Vq, (uint32_t)((int64_t)nk * kAttnD * 2));
  uint32_t voff[LOADS];
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int b = wave + NW * i;  // wave-uniform
    if (b < 16) {
      const int row = 8 * (b & 7) + (lane >> 3);
      const int lch = (lane & 7) ^ swz<BK>(row);
      voff[i] = (uint32_t)(row * kAttnD + 64 * (b >> 3) + lch * 8) * 2u;
    } else {
      int p = 0, d = 0;
      kmaj_coords<0>(64 * (b - 16) + lane, &p, &d);
      voff[i] = (uint32_t)((32 * (p >> 5) + vt_pos_key(p & 31)) * kAttnD + d) * 2u;
    }
  }
  // With 8 waves, wave loads 0-1 (b = wave, wave + 8) fill K16 and 2-3 fill V16.
  static_assert(NW == 8 && LOADS == 4, "K16 / V16^T split of the wave loads assumes 8 waves");
  auto issue = [&](int chunk) {
    const uint32_t key0 = (uint32_t)(kbeg + chunk * kAttnKV);
#pragma unroll
    for (int set = 0; set < (SKV ? 2 : 1); ++set) {
      uint16_t* base = lds + (chunk % STAGES) * STAGE + set * HALF;
      const rsrc_t& rks = set ? rkl : rk;
      const rsrc_t& rvs = set ? rvl : rv;
#pragma unroll
      for (int i = 0; i < LOADS; ++i) {
        const int b = wave + NW * i;
        if (i < 2)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rks, (lds_ptr_t)(base + i * KT + wave * 8 * BK), 16, voff[i],
                                                   key0 * kAttnD * 2u, 0, 0);
        else
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rvs, (lds_ptr_t)(base + 2 * KT + (b - 16) * 512), 16, voff[i],
                                                   key0 * kAttnD * 2u, 0, 0);
      }
    }
  };

  const FragOffsets<0, BK> fo(0, lane);  // K16 reads: lane row lr, chunk 4*kk + g
  const KmFrag<0, kAttnD, kAttnD, 8> fv(0, lane);  // V16 reads: 8 dim tiles, transpose reads

  float mref = -INFINITY, lsum = 0.f;  // per-query reference and row sum of P~

  // GEMM1 of one chunk: S^T (64 keys x 16 queries) = K16 . (log2e Q)^T, hi and
  // lo products in chains sh / sl (CHAINS == 2) or both in sh.  The hi chain
  // starts from -mref (0 on the first chunk, which has no reference yet), so
  // the chunk's scores come out relative to the reference.
  auto gemm1 = [&](int chunk, f32x4 (&sh)[4], f32x4 (&sl)[4]) {
    const uint16_t* st = lds + (chunk % STAGES) * STAGE;
    const float mb = chunk > 0 ? -mref : 0.f;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      sh[kt] = f32x4{mb, mb, mb, mb};
      sl[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      u32x4 a[4], al[4];
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        a[kt] = lds_read16(st + (d >> 1) * KT, fo.off[d & 1] + kt * 16 * BK);
        if constexpr (SKV) al[kt] = lds_read16(st + HALF + (d >> 1) * KT, fo.off[d & 1] + kt * 16 * BK);
      }
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        sh[kt] = mfma<0, MFL_F16>(a[kt], qh[d], sh[kt]);
        f32x4& corr = CHAINS == 2 ? sl[kt] : sh[kt];
        corr = mfma<0, MFL_F16>(a[kt], ql[d], corr);
        if constexpr (SKV) corr = mfma<0, MFL_F16>(al[kt], qh[d], corr);
      }
    }
  };

  f32x4 oh[8], ol[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    oh[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    ol[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // Online softmax, in two parts.  Lanes lr, lr+16, lr+32, lr+48 share a query.
  // (1) Chains added (giving t = s - mref, or s on the first chunk), chunk
  // max, and the move of the reference when the max passes it by more than
  // the slack (wave-uniform branch, taken on the first chunk and rarely
  // after): mref rises by the overshoot, t falls by it, O and l are rescaled.
  auto update_ref = [&](int chunk, f32x4 (&sh)[4], const f32x4 (&sl)[4]) {
    float cmax = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      if constexpr (CHAINS == 2) sh[kt] = sh[kt] + sl[kt];
#pragma unroll
      for (int j = 0; j < 4; ++j) cmax = fmaxf(cmax, sh[kt][j]);
    }
    cmax = max_over_lane_groups(cmax);
    if (chunk == 0 || __builtin_amdgcn_ballot_w64(cmax > kAttnSlack) != 0) {
      const float shift = chunk == 0 ? cmax : fmaxf(cmax, 0.f);
      const float mnew = (chunk == 0 ? 0.f : mref) + shift;
      const float sc = __builtin_amdgcn_exp2f(mref - mnew);  // 0 on the first chunk (mref = -inf)
      mref = mnew;
      lsum *= sc;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        oh[i] = oh[i] * sc;
        if constexpr (CHAINS == 2) ol[i] = ol[i] * sc;
      }
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) sh[kt] = sh[kt] - shift;
    }
  };
  // (2) P~ = 2^t, its row-sum contribution, and the split P~^T fragments of
  // GEMM2.
  auto exp_split = [&](const f32x4 (&s)[4], u32x4 (&ph)[2], u32x4 (&pl)[2]) {
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        // K positions 2e, 2e+1 of block t: keys of tile 2t (e < 2) or 2t+1
        const f32x4& x = s[2 * t + (e >> 1)];
        const float p0 = __builtin_amdgcn_exp2f(x[2 * (e & 1)]);
        const float p1 = __builtin_amdgcn_exp2f(x[2 * (e & 1) + 1]);
        lsum += p0;
        lsum += p1;
        const Split2 sp2 = split2_mix(p0, p1);
        ph[t][e] = sp2.hi;
        pl[t][e] = sp2.lo;
      }
  };

  // GEMM2 of one chunk: O^T (128 dims x 16 queries) += V16^T . P~^T, the V16^T
  // fragments (dims 16i.., K positions 32t + 8g + ..) read from the k-major V16
  // tile with the transpose read.
  auto gemm2 = [&](int chunk, const u32x4 (&ph)[2], const u32x4 (&pl)[2]) {
    const uint16_t* sv = lds + (chunk % STAGES) * STAGE + 2 * KT;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const u32x4 a = frag_read(sv, fv, t, i);
        oh[i] = mfma<0, MFL_F16>(a, ph[t], oh[i]);
        f32x4& corr = CHAINS == 2 ? ol[i] : oh[i];
        corr = mfma<0, MFL_F16>(a, pl[t], corr);
        if constexpr (SKV) corr = mfma<0, MFL_F16>(frag_read(sv + HALF, fv, t, i), ph[t], corr);
      }
  };

  // chunk c is waited for, then the stage of chunk c-1 is refilled with chunk
  // c+STAGES-1 (every wave has passed the barrier, so chunk c-1 is consumed)
#pragma unroll
  for (int s = 0; s < STAGES - 1; ++s)
    if (s < nchunks) issue(s);
  for (int c = 0; c < nchunks; ++c) {
    if (c + STAGES - 2 < nchunks)
      wait_vmcnt<(STAGES - 2) * LOADS>();
    else
      wait_vmcnt<0>();
    __syncthreads();
    if (c + STAGES - 1 < nchunks) issue(c + STAGES - 1);
    f32x4 sh[4], sl[4];
    gemm1(c, sh, sl);
    u32x4 ph[2], pl[2];
    update_ref(c, sh, sl);
    exp_split(sh, ph, pl);
    gemm2(c, ph, pl);
  }

  // slice results: unnormalised O (chains added in fp32), mref and l summed
  // over the four lanes of each query
  lsum += __shfl_xor(lsum, 16, 64);
  lsum += __shfl_xor(lsum, 32, 64);
  const int q = qw + lr;
  float* orow = Opart + ((int64_t)sp * nq + q) * kAttnD;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    f32x4 o = oh[i];
    if constexpr (CHAINS == 2) o = o + ol[i];
    *reinterpret_cast<f32x4*>(orow + 16 * i + 4 * g) = o;
  }
  if (g == 0) {
    Mpart[(int64_t)sp * nq + q] = mref;
    Lpart[(int64_t)sp * nq + q] = lsum;
  }
}

// O[q][d] = sum_s w_s O_s[q][d] / sum_s w_s l_s[q], w_s = 2^(m_s - max_s m_s)
// (m_s in base-2 units), slices taken in order s = 0, 1, ...  One thread per
// query and 4 consecutive dims; S (the slice count) is a template parameter so
// that all of a thread's loads are issued together.
template <int S>
__global__ __launch_bounds__(256) void attn_combine(const float* __restrict__ Opart, const float* __restrict__ Mpart,
                                                    const float* __restrict__ Lpart, float* __restrict__ O, int nq) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // f32x4 index
  if (i >= (int64_t)nq * (kAttnD / 4)) return;
  const int q = (int)(i / (kAttnD / 4));
  float m[S], l[S];
  f32x4 o[S];
#pragma unroll
  for (int s = 0; s < S; ++s) {
    m[s] = Mpart[(int64_t)s * nq + q];
    l[s] = Lpart[(int64_t)s * nq + q];
    o[s] = reinterpret_cast<const f32x4*>(Opart + (int64_t)s * nq * kAttnD)[i];
  }
  float mx = m[0];
#pragma unroll
  for (int s = 1; s < S; ++s) mx = fmaxf(mx, m[s]);
  f32x4 num = {0.f, 0.f, 0.f, 0.f};
  float den = 0.f;
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const float w = __builtin_amdgcn_exp2f(m[s] - mx);
    num += w * o[s];
    den += w * l[s];
  }
  reinterpret_cast<f32x4*>(O)[i] = num / den;
}

}  // namespace attn_detail

using namespace attn_detail;

// Sizes of the fused path's workspace pieces (bytes, each 256-aligned).
int64_t attn_fused_splits(int64_t nq, int64_t nk) {
  const int64_t qblocks = nq / kAttnQ;
  int64_t s = 1;
  while (s < 32 && qblocks * s < 256 && nk % (2 * s * kAttnKV) == 0) s *= 2;
  return s;
}

int64_t attn_fused_workspace(int64_t nq, int64_t nk, bool skv) {
  auto al = [](int64_t x) { return (x + 255) & ~(int64_t)255; };
  const int64_t s = attn_fused_splits(nq, nk);
  return al(nk * kAttnD * 2) * (skv ? 4 : 2) + al(s * nq * kAttnD * 4) + 2 * al(s * nq * 4);
}

int launch_attn_fused(int64_t nq, int64_t nk, const float* q, const float* k, const float* v, int chains, bool skv,
                      float* o, void* workspace, hipStream_t st) {
  auto al = [](int64_t x) { return (x + 255) & ~(int64_t)255; };
  const int64_t splits = attn_fused_splits(nq, nk);
  char* w = (char*)workspace;
  uint16_t* kq = (uint16_t*)w;
  w += al(nk * kAttnD * 2);
  uint16_t* vq = (uint16_t*)w;
  w += al(nk * kAttnD * 2);
  uint16_t* kl = nullptr;
  uint16_t* vl = nullptr;
  if (skv) {
    kl = (uint16_t*)w;
    w += al(nk * kAttnD * 2);
    vl = (uint16_t*)w;
    w += al(nk * kAttnD * 2);
  }
  float* op = (float*)w;
  w += al(splits * nq * kAttnD * 4);
  float* mp = (float*)w;
  w += al(splits * nq * 4);
  float* lp = (float*)w;
  const int64_t n16 = nk * kAttnD / 16;  // 16-value groups per operand
  const dim3 pgrid((unsigned)((n16 + 255) / 256)), pblock(256);
  if (skv)
    hipLaunchKernelGGL(attn_prep<true>, pgrid, pblock, 0, st, k, v, kq, vq, kl, vl, n16);
  else
    hipLaunchKernelGGL(attn_prep<false>, pgrid, pblock, 0, st, k, v, kq, vq, kl, vl, n16);
  const int qblocks = (int)(nq / kAttnQ);
  const int nwg = qblocks * (int)splits;
  const int xcd_map = nwg % 8 == 0;
  const int kps = (int)(nk / splits);
  const dim3 grid((unsigned)nwg), block(512);
  // two LDS stages: measured as fast as three, and a third adds nothing at
  // one workgroup per CU
#define MFL_ATTN_LAUNCH(CH, SK)                                                                                      \
  hipLaunchKernelGGL((attn_fused_kernel<CH, 2, SK>), grid, block, 0, st, q, kq, vq, kl, vl, op, mp, lp, (int)nq,      \
                     (int)nk, kps, qblocks, xcd_map)
  if (skv) {
    if (chains == 2)
      MFL_ATTN_LAUNCH(2, true);
    else
      MFL_ATTN_LAUNCH(1, true);
  } else {
    if (chains == 2)
      MFL_ATTN_LAUNCH(2, false);
    else
      MFL_ATTN_LAUNCH(1, false);
  }
#undef MFL_ATTN_LAUNCH
  const int64_t vec = nq * kAttnD / 4;
  const dim3 cgrid((unsigned)((vec + 255) / 256)), cblock(256);
  switch (splits) {
    case 1: hipLaunchKernelGGL(attn_combine<1>, cgrid, cblock, 0, st, op, mp, lp, o, (int)nq); break;
    case 2: hipLaunchKernelGGL(attn_combine<2>, cgrid, cblock, 0, st, op, mp, lp, o, (int)nq); break;
    case 4: hipLaunchKernelGGL(attn_combine<4>, cgrid, cblock, 0, st, op, mp, lp, o, (int)nq); break;
    case 8: hipLaunchKernelGGL(attn_combine<8>, cgrid, cblock, 0, st, op, mp, lp, o, (int)nq); break;
    case 16: hipLaunchKernelGGL(attn_combine<16>, cgrid, cblock, 0, st, op, mp, lp, o, (int)nq); break;
    case 32: hipLaunchKernelGGL(attn_combine<32>, cgrid, cblock, 0, st, op, mp, lp, o, (int)nq); break;
    default: return MFL_EUNSUPPORTED;  // the split chooser only returns powers of two up to 32
  }
  return launch_status();
}

}  // namespace mfl
