// attention_split_fp32: the attention-shaped pair of split GEMMs of Strata PR
// #800 — algo 0 (below) materialises the scores; algo 1 is the fused kernel of
// attention_fused.hip ("What's going on": q is split for q.k, p is split for p.v, each into an
// FP16 hi and lo half; "The fix": hi and lo products in separate accumulators).
//
//   1. S = Q K^T           Q split into f16 hi/lo, K rounded once
//   2. m = rowmax S, P~ = exp(S - m), l = rowsum P~           (fp32)
//   3. O_s = P~[:, slice s] V[slice s, :]   per key slice, P~ split, V rounded once
//   4. O = (sum_s O_s) / l  slices summed in a fixed order
//
// Step 2 has no kernel of its own.  The scores kernel keeps each key slice's
// row maxima as it stores S; the P~ V kernel takes m as the maximum of those,
// forms every P~ entry from S and m as it loads S (so P~ is never stored), and
// adds the entries it forms into the slice's row sum; the reduce adds the
// slices' sums into l.
//
// Normalisation is deferred to step 4: P~ lies in (0, 1] with its maximum
// exactly 1, whereas the normalised probabilities (about 1/nk) would fall in
// fp16's subnormal range and lose most of their lo half.  softmax(S) V equals
// (P~ V) / l exactly in real arithmetic.  This version materialises S in the
// caller's workspace (HBM-bound); it keeps every step on the device.
//
// Kernels: attn_prep_kvt rounds K into K16 (key-major) and V into V16T (one
// row of nk keys per dim); attn_scores computes S for 128 queries and one key
// slice, Q's hi/lo halves held in registers and K16 chunks of 64 keys streamed
// through LDS; attn_pv streams S and V16T chunks through LDS; reduce_slices
// sums the slices.  S is stored chunk-blocked, S[key / 64][q][key % 64]: the
// 128 queries x 64 keys a workgroup handles per chunk are 32 KiB of contiguous
// memory, written and read whole.
#include <algorithm>
#include <mutex>

#include "attention_fused.hpp"

namespace mfl {

int64_t attn_fused_workspace(int64_t nq, int64_t nk, bool skv);
int launch_attn_fused(int64_t nq, int64_t nk, const float* q, const float* k, const float* v, int chains, bool skv,
                      float* o, void* workspace, hipStream_t st);

namespace {

// P~ = exp(s - m) is taken as 2^((s - m) log2 e) with the hardware exp2.
constexpr float kLog2e = 1.4426950408889634f;
// One entry of P~ from its score and the row maximum.  The P~ V kernel forms
// each entry once and both feeds it to the MFMAs and adds it to the row sum l.
__device__ __forceinline__ float p_tilde(float s, float m) { return __builtin_amdgcn_exp2f((s - m) * kLog2e); }

// K16 = RNE16(K), key-major like K; V16T = RNE16(V) transposed, V16T[d][key].
// One workgroup of 512 threads per 64 keys: each thread rounds 16 consecutive
// values of the K block, and one pair of keys x 8 dims of the V block, whose
// halves it packs per dim into 32-bit words of an LDS tile (a dim row of 32
// key pairs, padded to 33 words); the tile leaves as 128-byte rows of V16T,
// four threads per row.
__global__ __launch_bounds__(512) void attn_prep_kvt(const float* __restrict__ K, const float* __restrict__ V,
                                                    uint16_t* __restrict__ Kq, uint16_t* __restrict__ VqT, int64_t nk) {
  constexpr int PADW = 33;
  __shared__ uint32_t t[kAttnD * PADW];
  const int64_t key0 = (int64_t)blockIdx.x * kAttnKV;
  const int tid = threadIdx.x;
  {
    const int64_t base = key0 * kAttnD + tid * 16;
    uint32_t w[8];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const f32x4 x = *reinterpret_cast<const f32x4*>(K + base + 4 * q);
      const Split2 a = split2(x[0], x[1]), b = split2(x[2], x[3]);
      w[2 * q] = a.hi;
      w[2 * q + 1] = b.hi;
    }
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      u32x4 o;
      __builtin_memcpy(&o, w + 4 * q, 16);
      *reinterpret_cast<u32x4*>(Kq + base + 8 * q) = o;
    }
  }
  {
    const int kp = tid >> 4, d0 = (tid & 15) * 8;
    const float* r0 = V + (key0 + 2 * kp) * kAttnD + d0;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const f32x4 a = *reinterpret_cast<const f32x4*>(r0 + 4 * q);
      const f32x4 b = *reinterpret_cast<const f32x4*>(r0 + kAttnD + 4 * q);
#pragma unroll
      for (int e = 0; e < 4; ++e) t[(d0 + 4 * q + e) * PADW + kp] = split2(a[e], b[e]).hi;  // keys 2kp | 2kp+1
    }
  }
  __syncthreads();
  const int d = tid >> 2, h = tid & 3;  // dim row d, keys 16 h .. +15
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const uint32_t* r = t + d * PADW + 8 * h + 4 * q;
    *reinterpret_cast<u32x4*>(VqT + d * nk + key0 + 16 * h + 8 * q) = u32x4{r[0], r[1], r[2], r[3]};
  }
}

// Keys [kbeg, kbeg + 64 * nchunks) of slice sp: slices of kps keys, the last
// one shorter when nk is not a multiple of kps.
__device__ __forceinline__ int slice_chunks(int sp, int kps, int64_t nk) {
  const int64_t kbeg = (int64_t)sp * kps;
  return (int)((min(nk, kbeg + kps) - kbeg) / kAttnKV);
}

// Step 1: S (chunk-blocked) for 128 queries (8 waves x 16) and one key slice.
// Each wave holds the B fragments of its 16 queries' hi and lo halves for the
// whole slice; per 64-key chunk it computes S^T (64 keys x 16 queries) =
// K16 . Q^T with the hi products in one chain and the lo products in a second
// (CHAINS == 2) or the same one, adds the chains in fp32, stores the tile and
// keeps the running maximum of its queries' scores, written per query and
// slice at the end (Ms[slice][q]).  K16 chunks arrive by direct-to-LDS loads,
// two stages.
template <int CHAINS, bool NT>
__global__ __launch_bounds__(512) void attn_scores(const float* __restrict__ Q, const uint16_t* __restrict__ Kq,
                                                   float* __restrict__ S, float* __restrict__ Ms, int nq, int64_t nk,
                                                   int kps, int qblocks, int xcd_map) {
  constexpr int BK = 64, KT = kAttnKV * BK, STAGE = 2 * KT, NW = 8, LOADS = 2;
  __shared__ __attribute__((aligned(1024))) uint16_t lds[2 * STAGE];
  int qb, sp;
  attn_block_of(blockIdx.x, gridDim.x, qblocks, xcd_map, qb, sp);
  const int64_t kbeg = (int64_t)sp * kps;
  const int nchunks = slice_chunks(sp, kps, nk);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lr = lane & 15, g = lane >> 4;
  const int qw = qb * kAttnQ + wave * 16;
  // Q^T fragments: lane supplies query qw + lr, dims 32*d + 8*g .. +7
  u32x4 qh[4], ql[4];
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const float* p = Q + (int64_t)(qw + lr) * kAttnD + 32 * d + 8 * g;
    const f32x4 x0 = *reinterpret_cast<const f32x4*>(p), x1 = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const Split2 s0 = split2(x0[2 * e], x0[2 * e + 1]);
      const Split2 s1 = split2(x1[2 * e], x1[2 * e + 1]);
      qh[d][e] = s0.hi;
      ql[d][e] = s0.lo;
      qh[d][2 + e] = s1.hi;
      ql[d][2 + e] = s1.lo;
    }
  }
  // Stage fill: 16 wave loads of 1 KiB, block b = wave + 8i: K16 half b / 8
  // (dims 64 (b / 8) ..), key rows 8 (b % 8) .. +7 (128 bytes each, chunk
  // lane % 8 of row 8 (b % 8) + lane / 8 receives logical chunk
  // (lane % 8) ^ swz(row)).
  uint32_t voff[LOADS];
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int b = wave + NW * i;
    const int row = 8 * (b & 7) + (lane >> 3);
    voff[i] = (uint32_t)(row * kAttnD + 64 * (b >> 3) + (((lane & 7) ^ swz<BK>(row)) * 8)) * 2u;
  }
  auto issue = [&](int chunk) {
    const rsrc_t rk = make_rsrc(Kq + (kbeg + (int64_t)chunk * kAttnKV) * kAttnD, kAttnKV * kAttnD * 2);
    uint16_t* base = lds + (chunk & 1) * STAGE;
#pragma unroll
    for (int i = 0; i < LOADS; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_ptr_t)(base + i * KT + wave * 8 * BK), 16, voff[i], 0, 0, 0);
    asm volatile("" ::: "memory");  // the loads stay ahead of the chunk's score stores
  };
  const FragOffsets<0, BK> fo(0, lane);
  // The lane holds keys 16 kt + 4 g .. +3 of each chunk for query qw + lr and
  // stores them as 16 bytes (each store instruction: 64-byte pieces of 16 rows,
  // which the L2 merges into lines).  Non-temporal stores (NT) bypass that
  // merge and would move each piece as a line of its own, so there the wave's
  // 16 x 64 tile goes through a wave-private LDS tile (rows padded to 68
  // floats) and each store instruction writes four whole 256-byte rows.
  __shared__ __attribute__((aligned(16))) float stg[NT ? NW : 1][16][68];
  float (*tile)[68] = stg[NT ? wave : 0];
  float* sblk = S + (kbeg >> 6) * (int64_t)nq * kAttnKV + (int64_t)qw * kAttnKV;
  float* srow = sblk + lr * kAttnKV + 4 * g;
  const int64_t cstride = (int64_t)nq * kAttnKV;
  float mrun = -INFINITY;  // maximum of the lane's scores of query qw + lr
  issue(0);
  for (int c = 0; c < nchunks; ++c) {
    // chunk c's loads were issued before chunk c-1's four score stores
    if (c > 0)
      wait_vmcnt<4>();
    else
      wait_vmcnt<0>();
    lds_barrier();
    if (c + 1 < nchunks) issue(c + 1);
    const uint16_t* st = lds + (c & 1) * STAGE;
    f32x4 sh[4], sl[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      sh[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
      sl[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      u32x4 a[4];
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) a[kt] = lds_read16(st + (d >> 1) * KT, fo.off[d & 1] + kt * 16 * BK);
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        sh[kt] = mfma<0, MFL_F16>(a[kt], qh[d], sh[kt]);
        f32x4& corr = CHAINS == 2 ? sl[kt] : sh[kt];
        corr = mfma<0, MFL_F16>(a[kt], ql[d], corr);
      }
    }
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      f32x4 s = sh[kt];
      if constexpr (CHAINS == 2) s = s + sl[kt];
      if constexpr (NT)
        *reinterpret_cast<f32x4*>(&tile[lr][16 * kt + 4 * g]) = s;
      else
        *reinterpret_cast<f32x4*>(srow + c * cstride + 16 * kt) = s;
      mrun = fmaxf(mrun, fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])));
    }
    if constexpr (NT) {
      // LDS operations of one wave complete in order: the reads below see the
      // writes above (the asm keeps the compiler from reordering them)
      asm volatile("" ::: "memory");
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 4 * i + (lane >> 4), col = 4 * (lane & 15);
        const f32x4 x = *reinterpret_cast<const f32x4*>(&tile[row][col]);
        __builtin_nontemporal_store(x, reinterpret_cast<f32x4*>(sblk + c * cstride + row * kAttnKV + col));
      }
      asm volatile("" ::: "memory");  // the tile's reads stay before the next chunk's writes
    }
  }
  // the four lanes lr + 16 g hold the slice's keys of one query
  mrun = fmaxf(mrun, __shfl_xor(mrun, 16, 64));
  mrun = fmaxf(mrun, __shfl_xor(mrun, 32, 64));
  if (g == 0) Ms[(int64_t)sp * nq + qw + lr] = mrun;
}

// Step 3 for 128 queries and one key slice: O_s^T (128 dims x 16 queries per
// wave) += V16T . P~^T, the P~ fragments formed from the scores and the row
// maximum m = max over slices of Ms (p_tilde) and split into f16 hi (one chain)
// and lo (a second chain, CHAINS == 2, or the same one); the slice's row sums
// of P~ go to Ls[slice][q].  Per 64-key chunk a stage holds the V16T tile
// (128 dim rows of 64 keys, 128-byte rows swizzled like a GEMM operand tile)
// and the chunk's S block (128 query rows of 64 fp32, 256-byte rows whose
// 16-byte chunks are XOR-swizzled by row % 16, so that the 16 rows one
// fragment read touches fall on distinct banks).  Three stages of
// direct-to-LDS loads keep two chunks in flight.
template <int CHAINS, bool NT>
__global__ __launch_bounds__(512) void attn_pv(const float* __restrict__ S, const float* __restrict__ Ms,
                                               const uint16_t* __restrict__ VqT, float* __restrict__ Opart,
                                               float* __restrict__ Ls, int nq, int64_t nk, int kps, int splits,
                                               int qblocks, int xcd_map) {
  constexpr int BK = 64, NST = 3, VST = kAttnD * BK, PST = kAttnQ * kAttnKV * 2;  // 16-bit elements
  constexpr int STAGE = VST + PST, NW = 8, VL = 2, PL = 4, PER = VL + PL;
  __shared__ __attribute__((aligned(1024))) uint16_t lds[NST * STAGE];
  int qb, sp;
  attn_block_of(blockIdx.x, gridDim.x, qblocks, xcd_map, qb, sp);
  const int64_t kbeg = (int64_t)sp * kps;
  const int nchunks = slice_chunks(sp, kps, nk);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lr = lane & 15, g = lane >> 4;
  // wave load i fills V16T dim rows 8 (wave + 8i) .. +7 and P~ rows 4 (wave + 8i) .. +3
  uint32_t voff[VL], poff[PL];
#pragma unroll
  for (int i = 0; i < VL; ++i) {
    const int row = 8 * (wave + NW * i) + (lane >> 3);
    voff[i] = (uint32_t)row * (uint32_t)nk * 2u + (uint32_t)(((lane & 7) ^ swz<BK>(row)) << 4);
  }
#pragma unroll
  for (int i = 0; i < PL; ++i) {
    const int row = 4 * (wave + NW * i) + (lane >> 4);
    poff[i] = (uint32_t)row * 256u + (uint32_t)(((lane & 15) ^ (row & 15)) << 4);
  }
  // V16T from key key0 on: 127 rows of nk keys plus 64 keys (< 2^32 bytes for nk <= 2^24)
  const uint32_t vbytes = (uint32_t)(((int64_t)(kAttnD - 1) * nk + kAttnKV) * 2);
  auto fetch = [&](int chunk) {
    uint16_t* base = lds + (chunk % NST) * STAGE;
    const int64_t key0 = kbeg + (int64_t)chunk * kAttnKV;
    const rsrc_t rv = make_rsrc(VqT + key0, vbytes);
#pragma unroll
    for (int i = 0; i < VL; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_ptr_t)(base + (wave + NW * i) * 512), 16, voff[i], 0, 0, 0);
    const rsrc_t rp = make_rsrc(S + ((key0 >> 6) * nq + qb * kAttnQ) * kAttnKV, PST * 2);
#pragma unroll
    for (int i = 0; i < PL; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rp, (lds_ptr_t)(base + VST + (wave + NW * i) * 512), 16, poff[i], 0, 0,
                                               NT ? 2 : 0);  // 2: the non-temporal (streaming) policy
  };
  const FragOffsets<0, BK> fo(0, lane);  // V16T fragments: dim row 16 i + lr, keys 32 t + 8 g ..
  // P~ fragments: query row wave * 16 + lr, keys 32 t + 8 g .. +7 = logical
  // 16-byte chunks 8 t + 2 g and 8 t + 2 g + 1 of the row
  int pcol[2][2];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int h = 0; h < 2; ++h) pcol[t][h] = (wave * 16 + lr) * 128 + (((8 * t + 2 * g + h) ^ lr) << 3);
  // m of the lane's query row: the maximum of the slices' maxima, loaded 16
  // slices at a time (one load per iteration would wait out each latency in
  // turn).  An empty asm consumes m once the first stages' loads are issued
  // (below), so its wait overlaps them; a first use inside the chunk loop would
  // wait for every load in flight at each chunk.
  const int row = qb * kAttnQ + wave * 16 + lr;
  float mq = -INFINITY;
#pragma unroll 16
  for (int s2 = 0; s2 < splits; ++s2) mq = fmaxf(mq, Ms[(int64_t)s2 * nq + row]);
  float lsum = 0.f;  // the lane's P~ values of this slice: per-chunk sums, added in chunk order
  f32x4 oh[8], ol[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    oh[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    ol[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int s = 0; s < NST - 1; ++s)
    if (s < nchunks) fetch(s);
  asm volatile("" : "+v"(mq));
  for (int c = 0; c < nchunks; ++c) {
    if (c + NST - 2 < nchunks)
      wait_vmcnt<(NST - 2) * PER>();
    else
      wait_vmcnt<0>();
    lds_barrier();
    if (c + NST - 1 < nchunks) fetch(c + NST - 1);
    const uint16_t* sv = lds + (c % NST) * STAGE;
    const uint16_t* spp = sv + VST;
    u32x4 ph[2], pl[2];
    float csum = 0.f;  // the lane's 16 P~ values of the chunk, in key order
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      f32x4 x0 = __builtin_bit_cast(f32x4, lds_read16(spp, pcol[t][0]));
      f32x4 x1 = __builtin_bit_cast(f32x4, lds_read16(spp, pcol[t][1]));
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x0[e] = p_tilde(x0[e], mq);
        x1[e] = p_tilde(x1[e], mq);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) csum += x0[e];
#pragma unroll
      for (int e = 0; e < 4; ++e) csum += x1[e];
      const Split2 a = split2(x0[0], x0[1]), b = split2(x0[2], x0[3]);
      const Split2 e = split2(x1[0], x1[1]), f = split2(x1[2], x1[3]);
      ph[t] = u32x4{a.hi, b.hi, e.hi, f.hi};
      pl[t] = u32x4{a.lo, b.lo, e.lo, f.lo};
    }
    lsum += csum;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const u32x4 a = frag_read(sv, fo, t, i);
        oh[i] = mfma<0, MFL_F16>(a, ph[t], oh[i]);
        f32x4& corr = CHAINS == 2 ? ol[i] : oh[i];
        corr = mfma<0, MFL_F16>(a, pl[t], corr);
      }
  }
  // l of the slice: the four lanes lr + 16 g hold its keys of one query
  lsum += __shfl_xor(lsum, 16, 64);
  lsum += __shfl_xor(lsum, 32, 64);
  if (g == 0) Ls[(int64_t)sp * nq + row] = lsum;
  // lane holds O_s^T dims 16 i + 4 g .. +3 of query qb*128 + wave*16 + lr
  float* orow = Opart + ((int64_t)sp * nq + row) * kAttnD;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    f32x4 o = oh[i];
    if constexpr (CHAINS == 2) o = o + ol[i];
    *reinterpret_cast<f32x4*>(orow + 16 * i + 4 * g) = o;
  }
}

// Step 4: O[r][c..c+3] = (sum over slices s = 0, 1, ... of part[s][r][c..]) / l[r],
// with l[r] = sum over slices s = 0, 1, ... of Ls[s][r].
__global__ __launch_bounds__(256) void reduce_slices(const float* __restrict__ part, int splits, int nq,
                                                   const float* __restrict__ Ls, float* __restrict__ O, int64_t total4) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // f32x4 index
  if (i >= total4) return;
  const int64_t r = i / (kAttnD / 4), stride = (int64_t)nq * kAttnD;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float l = 0.f;
  // unrolled so that the loads of several slices are in flight together; the
  // sums still run in slice order
#pragma unroll 8
  for (int s = 0; s < splits; ++s) {
    acc += reinterpret_cast<const f32x4*>(part + s * stride)[i];
    l += Ls[(int64_t)s * nq + r];
  }
  reinterpret_cast<f32x4*>(O)[i] = acc / l;
}

struct Workspace {
  int64_t s_off, m_off, l_off, part_off, k16_off, vt_off, total;
  int kps, splits;
};

int64_t align256(int64_t x) { return (x + 255) & ~(int64_t)255; }

// Key slices of steps 1 and 3: about one workgroup per CU over the nq / 128
// query blocks, whole 64-key chunks, the last slice possibly shorter.
void choose_slices(int64_t nq, int64_t nk, int* kps, int* splits) {
  const int64_t qblocks = nq / kAttnQ, chunks = nk / kAttnKV;
  const int64_t want = std::max<int64_t>(1, std::min<int64_t>((256 + qblocks - 1) / qblocks, chunks));
  const int64_t per = (chunks + want - 1) / want;
  *kps = (int)(per * kAttnKV);
  *splits = (int)((chunks + per - 1) / per);
}

Workspace plan(int64_t nq, int64_t nk, int64_t d) {
  Workspace w;
  choose_slices(nq, nk, &w.kps, &w.splits);
  int64_t off = 0;
  w.s_off = off;
  off = align256(off + nq * nk * 4);
  w.m_off = off;  // per slice and query: the slice's maximum score
  off = align256(off + (int64_t)w.splits * nq * 4);
  w.l_off = off;  // per slice and query: the slice's sum of P~
  off = align256(off + (int64_t)w.splits * nq * 4);
  w.part_off = off;
  off = align256(off + (int64_t)w.splits * nq * d * 4);
  w.k16_off = off;
  off = align256(off + nk * d * 2);
  w.vt_off = off;
  off = align256(off + nk * d * 2);
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
  uint16_t* k16 = (uint16_t*)(ws + w.k16_off);
  uint16_t* vt = (uint16_t*)(ws + w.vt_off);
  const int NQ = (int)nq, qblocks = (int)(nq / kAttnQ), nwg = qblocks * w.splits, xcd_map = nwg % 8 == 0;
  int st;
  hipLaunchKernelGGL(attn_prep_kvt, dim3((unsigned)(nk / kAttnKV)), dim3(512), 0, s, k, v, k16, vt, nk);
  // S of at least the 256 MB last-level cache (MALL) cannot stay in it between
  // the two kernels: it is then written and read with the non-temporal policy,
  // so that reading it does not first evict the score kernel's dirty lines.
  const bool nt = nq * nk * 4 >= ((int64_t)256 << 20);
  // 1. S = split(Q) . round(K)^T, chunk-blocked; each slice's row maxima
#define MFL_SCORES(C, NT) \
  hipLaunchKernelGGL((attn_scores<C, NT>), dim3(nwg), dim3(512), 0, s, q, k16, S, m, NQ, nk, w.kps, qblocks, xcd_map)
  if (chains == 2) {
    if (nt) MFL_SCORES(2, true); else MFL_SCORES(2, false);
  } else {
    if (nt) MFL_SCORES(1, true); else MFL_SCORES(1, false);
  }
#undef MFL_SCORES
  if ((st = launch_status()) != MFL_OK) return st;
  // 2 and 3. per key slice: the row maximum over all slices, P~ formed from S
  // as it is loaded, split(P~) . round(V) and the slice's row sums of P~
#define MFL_PV(C, NT)                                                                                            \
  hipLaunchKernelGGL((attn_pv<C, NT>), dim3(nwg), dim3(512), 0, s, S, m, vt, part, l, NQ, nk, w.kps, w.splits, \
                     qblocks, xcd_map)
  if (chains == 2) {
    if (nt) MFL_PV(2, true); else MFL_PV(2, false);
  } else {
    if (nt) MFL_PV(1, true); else MFL_PV(1, false);
  }
#undef MFL_PV
  if ((st = launch_status()) != MFL_OK) return st;
  // 4. fixed-order sum of the slices, then divide by l.
  const int64_t total4 = nq * d / 4;
  hipLaunchKernelGGL(reduce_slices, dim3((unsigned)((total4 + 255) / 256)), dim3(256), 0, s, part, w.splits, NQ, l, o,
                     total4);
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
