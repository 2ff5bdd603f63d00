// The tiled MFMA GEMM core: global -> swizzled LDS tile loaders, the LDS ->
// fragment -> MFMA step with register-resident accumulators, and the epilogue
// that stores each accumulator value once through the fragment layout.
//
// Warp issue #1965 ("Description", "Proposed change") names the two costs a
// shared-memory-operand GEMM pays — fragment loads from plain shared layouts hit
// bank conflicts, and C is read and written through shared memory on every call
// — and the cure: swizzled operand tiles plus an accumulator that lives in
// registers across the K loop and is materialised once.  These templates are
// that design for CDNA4 wavefronts of 64 lanes.
#pragma once
#include <utility>
#include "common.hpp"

namespace mfl {

// Loads one R x BK operand tile (16-bit elements) from global memory into
// registers and later writes it to the swizzled LDS tile.
//   KC = true : element (r, k) of the tile is at base[(r0 + r)*ld + k0 + k]
//               (row-major A or column-major B: K contiguous); 16-byte loads
//               along K, 16-byte LDS writes.
//   KC = false: element (r, k) is at base[(k0 + k)*ld + r0 + r] (K strided);
//               16-byte loads along R, 16-byte LDS writes into a k-major tile
//               (the kmaj_chunk layout of the 16x16x32 instruction, read with
//               the transpose read).
// EDGE enables masking: K positions >= k_total are zero (in both operands, so a
// NaN in padding never meets a zero), R positions past rows_total are zero (KC =
// false) or repeat the last row (KC = true) and are never stored by the
// epilogue.  A chunk that straddles the edge is read element by element, so no
// read leaves the operand's storage ((rows - 1) * ld + inner extent).
template <int R, int BK, int NT, bool KC, bool EDGE>
struct TileLoader {
  static constexpr int CHUNKS = R * BK / 8;
  static constexpr int PER = CHUNKS / NT;
  static_assert(CHUNKS % NT == 0, "tile chunks must divide evenly among threads");
  u32x4 reg[PER];

  __device__ __forceinline__ void load(const uint16_t* __restrict__ base, int64_t ld, int r0, int k0, int rows_total,
                                       int k_total, int tid) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int idx = tid + i * NT;
      if constexpr (KC) {
        const int r = idx / (BK / 8), c = idx % (BK / 8);
        int gr = r0 + r;
        const int kf = k0 + c * 8;
        if constexpr (EDGE) {
          gr = min(gr, rows_total - 1);
          if (kf + 8 <= k_total)
            reg[i] = gload16(base + (int64_t)gr * ld + kf);
          else
            reg[i] = gload_partial(base + (int64_t)gr * ld + kf, k_total - kf);
        } else {
          reg[i] = gload16(base + (int64_t)gr * ld + kf);
        }
      } else {
        const int k = idx / (R / 8), rc = idx % (R / 8);
        const int gk = k0 + k, gr = r0 + rc * 8;
        if (!EDGE || (gk < k_total && gr + 8 <= rows_total))
          reg[i] = gload16(base + (int64_t)gk * ld + gr);
        else if (gk < k_total)
          reg[i] = gload_partial(base + (int64_t)gk * ld + gr, rows_total - gr);
        else
          reg[i] = u32x4{0, 0, 0, 0};
      }
    }
  }

  __device__ __forceinline__ void store(uint16_t* lds, int tid) const {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int idx = tid + i * NT;
      if constexpr (KC) {
        const int r = idx / (BK / 8), c = idx % (BK / 8);
        lds_write16(lds, lds_chunk<BK>(r, c), reg[i]);
      } else {
        static_assert(BK == 64 && (R == 128 || R == 256), "k-major tile shape");
        const int k = idx / (R / 8), rc = idx % (R / 8);
        lds_write16(lds, lds_elemKM<0>(k, rc * 8), reg[i]);
      }
    }
  }
};

// Reads MFMA operand fragments from the swizzled LDS tiles.  Lane l takes row
// (l mod MN) of each MN-row fragment and the 16-byte chunk (l div MN) of the
// current MFMA K step.  The per-lane offsets of the BK/KM K steps are computed
// once; fragment i of the wave adds the immediate i*MN*BK.
template <int SHAPE, int BK>
struct FragOffsets {
  static constexpr int MN = Shape<SHAPE>::MN, KM = Shape<SHAPE>::K, CPK = KM / 8, KSTEPS = BK / KM;
  // lane row lane % MN, chunk lane / MN: the exported operand numeral (layout.hpp)
  static_assert(operand_layout(SHAPE).rows == MN && operand_layout(SHAPE).cols == KM,
                "fragment reads must follow the operand numeral of the instruction");
  int off[KSTEPS];
  struct Plain {};
  // Unswizzled rows (chunk c of a row at c*8): the plain LDS layout of the
  // block-repeat ablation.
  __device__ __forceinline__ FragOffsets(int row0, int lane, Plain) {
    const int lr = lane % MN, lk = lane / MN;
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) off[kk] = (row0 + lr) * BK + (kk * CPK + lk) * 8;
  }
  __device__ __forceinline__ FragOffsets(int row0, int lane) {
    const int lr = lane % MN, lk = lane / MN;
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) off[kk] = lds_chunk<BK>(row0 + lr, kk * CPK + lk);
  }
};

// Fragment reads from a k-major tile (K-strided operands) with two transpose
// reads.  Lane l of the 16-lane group g addresses K row kb(g) + ((l >> 2) & 3)
// + 4h and columns rb(g) + 4*(l & 3) .. +3 in read h = 0, 1, where
// kb(g) = 8*(16g div MN) and rb(g) = 16g mod MN; after the transpose lane l holds
// row (l mod MN) at K positions 8*(l div MN) + 4h .. +3, i.e. elements 4h .. 4h+3
// of the instruction's operand numeral (checked below).
template <int SHAPE>
MFL_HD constexpr int tr_k(int lane) {
  return 8 * ((16 * (lane >> 4)) / Shape<SHAPE>::MN) + ((lane >> 2) & 3);
}
template <int SHAPE>
MFL_HD constexpr int tr_r(int lane) {
  return (16 * (lane >> 4)) % Shape<SHAPE>::MN + 4 * (lane & 3);
}
template <int SHAPE>
constexpr bool tr_reads_match_numeral() {
  const AccLayout& L = operand_layout(SHAPE);
  for (int lane = 0; lane < 64; ++lane)
    for (int i = 0; i < 8; ++i) {
      const int src = tr_src_lane(lane, i & 3);
      const int k = tr_k<SHAPE>(src) + 4 * (i >> 2), r = tr_r<SHAPE>(src) + tr_src_elem(lane);
      if (r != acc_row(L, lane, i) || k != acc_col(L, lane, i)) return false;
    }
  return true;
}
static_assert(tr_reads_match_numeral<0>() && tr_reads_match_numeral<1>(),
              "transpose fragment reads disagree with the operand numerals");

// Offsets of the reads relative to a lane's base address: read h of fragment f
// in MFMA K step kk.  The bits they set are never set in a lane's base (k, r),
// so adding is exact (checked below).
template <int SHAPE>
MFL_HD constexpr int kmaj_step(int kk, int h, int f) {
  return lds_elemKM<SHAPE>(kk * Shape<SHAPE>::K + 4 * h, f * Shape<SHAPE>::MN);
}

// For every lane, K step, read and fragment of a wave whose NF fragments start
// at r0 (a multiple of WS): the read lands on the element the lane needs, at
// base + kmaj_step; and within each phase (lanes 0-31, 32-63) no two lanes
// touch one 4-byte bank at different addresses.
template <int SHAPE, int R, int WS, int NF>
constexpr bool kmaj_reads_ok() {
  constexpr int MN = Shape<SHAPE>::MN, KM = Shape<SHAPE>::K;
  for (int r0 = 0; r0 < R; r0 += WS)
    for (int lane = 0; lane < 64; ++lane) {
      const int k = tr_k<SHAPE>(lane), r = r0 + tr_r<SHAPE>(lane);
      for (int kk = 0; kk < 64 / KM; ++kk)
        for (int h = 0; h < 2; ++h)
          for (int f = 0; f < NF; ++f)
            if (lds_elemKM<SHAPE>(k + kk * KM + 4 * h, r + f * MN) !=
                lds_elemKM<SHAPE>(k, r) + kmaj_step<SHAPE>(kk, h, f))
              return false;
    }
  for (int r0 = 0; r0 < R; r0 += MN)
    for (int h = 0; h < 2; ++h)
      for (int phase = 0; phase < 2; ++phase) {
        int owner[64] = {};  // 1 + the dword address that each bank serves in this phase
        for (int lane = 32 * phase; lane < 32 * phase + 32; ++lane) {
          const int dw = lds_elemKM<SHAPE>(tr_k<SHAPE>(lane) + 4 * h, r0 + tr_r<SHAPE>(lane)) / 2;
          for (int d = dw; d < dw + 2; ++d) {
            if (owner[d % 64] != 0 && owner[d % 64] != d + 1) return false;
            owner[d % 64] = d + 1;
          }
        }
      }
  return true;
}
// Per-lane base offset of a wave's NF fragments in a k-major tile of R columns;
// fragment f covers columns row0 + f*MN .. +MN, row0 being a multiple of WS.
template <int SHAPE, int R, int WS, int NF>
struct KmFrag {
  static_assert(NF * Shape<SHAPE>::MN <= WS && kmaj_reads_ok<SHAPE, R, WS, NF>(),
                "k-major tile: transpose reads conflict or are not immediate offsets");
  int off;
  __device__ __forceinline__ KmFrag(int row0, int lane)
      : off(lds_elemKM<SHAPE>(tr_k<SHAPE>(lane), row0 + tr_r<SHAPE>(lane))) {}
};

// Operand fragment f of MFMA K step kk, from a K-contiguous or a k-major tile.
template <int SHAPE, int BK>
__device__ __forceinline__ u32x4 frag_read(const uint16_t* s, const FragOffsets<SHAPE, BK>& o, int kk, int f) {
  return lds_read16(s, o.off[kk] + f * Shape<SHAPE>::MN * BK);
}
template <int SHAPE, int R, int WS, int NF>
__device__ __forceinline__ u32x4 frag_read(const uint16_t* s, const KmFrag<SHAPE, R, WS, NF>& o, int kk, int f) {
  return lds_read_tr(s, o.off + kmaj_step<SHAPE>(kk, 0, f), kmaj_step<SHAPE>(0, 1, 0));
}

// ---- transpose reads the compiler does not see --------------------------------
// The compiler makes every ds_read_b64_tr_b16 that follows a direct-to-LDS load
// wait for that load (s_waitcnt vmcnt(0)): it cannot tell the two buffers apart.
// With a ring of stages that wait drains every prefetch at each K step.  The
// same reads issued as inline assembly are invisible to its load tracking, so
// the kernel waits for them itself (s_waitcnt lgkmcnt(0)) and then passes each
// fragment through an empty asm that the MFMAs depend on, so no MFMA is moved
// above the wait.  The stage a read uses is never a load's target before the
// next workgroup barrier, which waits for all LDS operations.
template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}
__device__ __forceinline__ uint32_t lds_address(const uint16_t* p) {
  return (uint32_t)(size_t)(const __attribute__((address_space(3))) uint16_t*)p;
}
template <int OFF>
__device__ __forceinline__ u32x2 lds_read_tr_asm(uint32_t addr) {
  static_assert(OFF >= 0 && OFF < 65536, "immediate LDS offset");
  u32x2 r;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "n"(OFF) : "memory");
  return r;
}
// Fragment F of MFMA K step KK from a k-major tile; base is the LDS byte
// address of the lane's base element (tile + KmFrag::off).
template <int SHAPE, int KK, int F>
__device__ __forceinline__ u32x4 frag_read_tr_asm(uint32_t base) {
  const u32x2 lo = lds_read_tr_asm<2 * kmaj_step<SHAPE>(KK, 0, F)>(base);
  const u32x2 hi = lds_read_tr_asm<2 * kmaj_step<SHAPE>(KK, 1, F)>(base);
  return u32x4{lo.x, lo.y, hi.x, hi.y};
}

// One BK-deep slab of the wave's TM x TN grid of MFMA tiles: for each MFMA K
// step, read the A and B fragments from LDS and accumulate into registers.
// MASKK: when kvalid < BK only the first kvalid (a multiple of 8) K positions of
// the slab are real; a lane whose 8 K positions (8*(lane div MN) + i of the K
// step) lie past them zeroes its A and B fragments, so whatever the LDS holds
// there never reaches C.
template <int SHAPE, int DT, int TM, int TN, int BK, bool MASKK = false, class RA, class RB>
__device__ __forceinline__ void mma_slab(const uint16_t* sA, const uint16_t* sB, const RA& fa, const RB& fb,
                                         typename Shape<SHAPE>::Acc (&acc)[TM][TN], int kvalid = BK) {
  constexpr int MN = Shape<SHAPE>::MN, KM = Shape<SHAPE>::K;
#pragma unroll
  for (int kk = 0; kk < BK / KM; ++kk) {
    u32x4 a[TM], b[TN];
#pragma unroll
    for (int i = 0; i < TM; ++i) a[i] = frag_read(sA, fa, kk, i);
#pragma unroll
    for (int j = 0; j < TN; ++j) b[j] = frag_read(sB, fb, kk, j);
    if constexpr (MASKK) {
      if (kvalid < BK && kk * KM + 8 * ((int)(threadIdx.x & 63) / MN) >= kvalid) {  // kvalid is wave-uniform
#pragma unroll
        for (int i = 0; i < TM; ++i) a[i] = u32x4{0, 0, 0, 0};
#pragma unroll
        for (int j = 0; j < TN; ++j) b[j] = u32x4{0, 0, 0, 0};
      }
    }
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] = mfma<SHAPE, DT>(a[i], b[j], acc[i][j]);
  }
}

// mma_slab for slabs with a k-major operand (AKM: A, BKM: B), its fragments
// read by frag_read_tr_asm; the other operand's by the ordinary 16-byte reads.
template <int SHAPE, int DT, int TM, int TN, int BK, bool AKM, bool BKM, bool MASKK, class RA, class RB>
__device__ __forceinline__ void mma_slab_tr_asm(const uint16_t* sA, const uint16_t* sB, const RA& fa, const RB& fb,
                                                typename Shape<SHAPE>::Acc (&acc)[TM][TN], int kvalid) {
  static_assert(AKM || BKM, "a k-major operand");
  constexpr int MN = Shape<SHAPE>::MN, KM = Shape<SHAPE>::K;
  uint32_t baseA = 0, baseB = 0;
  if constexpr (AKM) baseA = lds_address(sA + fa.off);
  if constexpr (BKM) baseB = lds_address(sB + fb.off);
  static_for<BK / KM>([&](auto kkc) {
    constexpr int kk = decltype(kkc)::value;
    u32x4 a[TM], b[TN];
    static_for<TM>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      if constexpr (AKM)
        a[i] = frag_read_tr_asm<SHAPE, kk, i>(baseA);
      else
        a[i] = frag_read(sA, fa, kk, i);
    });
    static_for<TN>([&](auto jc) {
      constexpr int j = decltype(jc)::value;
      if constexpr (BKM)
        b[j] = frag_read_tr_asm<SHAPE, kk, j>(baseB);
      else
        b[j] = frag_read(sB, fb, kk, j);
    });
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if constexpr (AKM) {
#pragma unroll
      for (int i = 0; i < TM; ++i) asm volatile("" : "+v"(a[i]));
    }
    if constexpr (BKM) {
#pragma unroll
      for (int j = 0; j < TN; ++j) asm volatile("" : "+v"(b[j]));
    }
    if constexpr (MASKK) {
      if (kvalid < BK && kk * KM + 8 * ((int)(threadIdx.x & 63) / MN) >= kvalid) {  // kvalid is wave-uniform
#pragma unroll
        for (int i = 0; i < TM; ++i) a[i] = u32x4{0, 0, 0, 0};
#pragma unroll
        for (int j = 0; j < TN; ++j) b[j] = u32x4{0, 0, 0, 0};
      }
    }
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] = mfma<SHAPE, DT>(a[i], b[j], acc[i][j]);
  });
}

// mma_slab with part of the slab's last MFMA K step carried over the next
// barrier: the MFMAs of the last CARRY fragment rows of the last K step are not
// issued here; their A fragments (ca) and the step's B fragments (cb) stay in
// registers, and the next call issues them (`pending`) right after its first
// fragment reads, so every wave has MFMAs ready while the reads that follow the
// barrier are in flight.  Each accumulator still receives its MFMAs in the same
// K order, so the result is bit-identical to mma_slab.  After the last slab the
// caller issues the carried MFMAs with mma_carried.
template <int SHAPE, int DT, int TM, int TN, int CARRY>
__device__ __forceinline__ void mma_carried(const u32x4 (&ca)[CARRY], const u32x4 (&cb)[TN],
                                            typename Shape<SHAPE>::Acc (&acc)[TM][TN]) {
#pragma unroll
  for (int c = 0; c < CARRY; ++c)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[TM - CARRY + c][j] = mfma<SHAPE, DT>(ca[c], cb[j], acc[TM - CARRY + c][j]);
}

template <int SHAPE, int DT, int TM, int TN, int BK, int CARRY, bool MASKK = false, class RA, class RB>
__device__ __forceinline__ void mma_slab_carry(const uint16_t* sA, const uint16_t* sB, const RA& fa, const RB& fb,
                                               typename Shape<SHAPE>::Acc (&acc)[TM][TN], u32x4 (&ca)[CARRY],
                                               u32x4 (&cb)[TN], bool pending, int kvalid = BK) {
  constexpr int MN = Shape<SHAPE>::MN, KM = Shape<SHAPE>::K, KS = BK / KM;
  static_assert(CARRY > 0 && CARRY < TM, "carry some but not all fragment rows");
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) {
    u32x4 a[TM], b[TN];
#pragma unroll
    for (int i = 0; i < TM; ++i) a[i] = frag_read(sA, fa, kk, i);
#pragma unroll
    for (int j = 0; j < TN; ++j) b[j] = frag_read(sB, fb, kk, j);
    if constexpr (MASKK) {
      if (kvalid < BK && kk * KM + 8 * ((int)(threadIdx.x & 63) / MN) >= kvalid) {  // kvalid is wave-uniform
#pragma unroll
        for (int i = 0; i < TM; ++i) a[i] = u32x4{0, 0, 0, 0};
#pragma unroll
        for (int j = 0; j < TN; ++j) b[j] = u32x4{0, 0, 0, 0};
      }
    }
    if (kk == 0 && pending) {
      // the empty asm statements are ordered after the barrier that precedes
      // this call, and the carried MFMAs depend on them
#pragma unroll
      for (int c = 0; c < CARRY; ++c) asm volatile("" : "+v"(ca[c]));
      mma_carried<SHAPE, DT, TM, TN, CARRY>(ca, cb, acc);
    }
    constexpr int last = KS - 1;
#pragma unroll
    for (int i = 0; i < TM; ++i)
      if (kk != last || i < TM - CARRY)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = mfma<SHAPE, DT>(a[i], b[j], acc[i][j]);
    if (kk == last) {
#pragma unroll
      for (int c = 0; c < CARRY; ++c) ca[c] = a[TM - CARRY + c];
#pragma unroll
      for (int j = 0; j < TN; ++j) cb[j] = b[j];
    }
  }
}

// mma_slab / mma_slab_carry calling `after_reads()` once the fragment reads of
// the slab's first MFMA K step are issued (before that step's MFMAs), for a
// caller that must not issue its next direct-to-LDS loads ahead of those
// reads.  Kept apart from the plain forms, whose code the extra parameter
// would perturb.
template <int SHAPE, int DT, int TM, int TN, int BK, bool MASKK, class RA, class RB, class Hook>
__device__ __forceinline__ void mma_slab_then(const uint16_t* sA, const uint16_t* sB, const RA& fa, const RB& fb,
                                              typename Shape<SHAPE>::Acc (&acc)[TM][TN], int kvalid,
                                              const Hook& after_reads) {
  constexpr int MN = Shape<SHAPE>::MN, KM = Shape<SHAPE>::K, KS = BK / KM;
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) {
    u32x4 a[TM], b[TN];
#pragma unroll
    for (int i = 0; i < TM; ++i) a[i] = frag_read(sA, fa, kk, i);
#pragma unroll
    for (int j = 0; j < TN; ++j) b[j] = frag_read(sB, fb, kk, j);
    if (kk == 0) after_reads();
    if constexpr (MASKK) {
      if (kvalid < BK && kk * KM + 8 * ((int)(threadIdx.x & 63) / MN) >= kvalid) {  // kvalid is wave-uniform
#pragma unroll
        for (int i = 0; i < TM; ++i) a[i] = u32x4{0, 0, 0, 0};
#pragma unroll
        for (int j = 0; j < TN; ++j) b[j] = u32x4{0, 0, 0, 0};
      }
    }
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] = mfma<SHAPE, DT>(a[i], b[j], acc[i][j]);
  }
}

template <int SHAPE, int DT, int TM, int TN, int BK, int CARRY, bool MASKK, class RA, class RB, class Hook>
__device__ __forceinline__ void mma_slab_carry_then(const uint16_t* sA, const uint16_t* sB, const RA& fa,
                                                    const RB& fb, typename Shape<SHAPE>::Acc (&acc)[TM][TN],
                                                    u32x4 (&ca)[CARRY], u32x4 (&cb)[TN], bool pending, int kvalid,
                                                    const Hook& after_reads) {
  constexpr int MN = Shape<SHAPE>::MN, KM = Shape<SHAPE>::K, KS = BK / KM;
  static_assert(CARRY > 0 && CARRY < TM, "carry some but not all fragment rows");
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) {
    u32x4 a[TM], b[TN];
#pragma unroll
    for (int i = 0; i < TM; ++i) a[i] = frag_read(sA, fa, kk, i);
#pragma unroll
    for (int j = 0; j < TN; ++j) b[j] = frag_read(sB, fb, kk, j);
    if (kk == 0) after_reads();
    if constexpr (MASKK) {
      if (kvalid < BK && kk * KM + 8 * ((int)(threadIdx.x & 63) / MN) >= kvalid) {  // kvalid is wave-uniform
#pragma unroll
        for (int i = 0; i < TM; ++i) a[i] = u32x4{0, 0, 0, 0};
#pragma unroll
        for (int j = 0; j < TN; ++j) b[j] = u32x4{0, 0, 0, 0};
      }
    }
    if (kk == 0 && pending) {
#pragma unroll
      for (int c = 0; c < CARRY; ++c) asm volatile("" : "+v"(ca[c]));
      mma_carried<SHAPE, DT, TM, TN, CARRY>(ca, cb, acc);
    }
    constexpr int last = KS - 1;
#pragma unroll
    for (int i = 0; i < TM; ++i)
      if (kk != last || i < TM - CARRY)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = mfma<SHAPE, DT>(a[i], b[j], acc[i][j]);
    if (kk == last) {
#pragma unroll
      for (int c = 0; c < CARRY; ++c) ca[c] = a[TM - CARRY + c];
#pragma unroll
      for (int j = 0; j < TN; ++j) cb[j] = b[j];
    }
  }
}

// Wait until at most N of this wave's vector-memory operations (the
// direct-to-LDS loads included) are outstanding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Workgroup barrier after this wave's LDS operations have completed.  Unlike
// __syncthreads it does not wait for outstanding vector-memory loads (its
// release fence would), so loads issued for later stages stay in flight; a
// stage's direct-to-LDS loads are waited for with wait_vmcnt before it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Direct-to-LDS loads of one operand's R x 64 slab per stage.
//   K-contiguous (A row-major, B column-major): R rows of 64 K values, 128 bytes
//     each, chunk XOR swz<64>(row); a load instruction fills 8 rows.
//   k-major (A column-major, B row-major): the kmaj_chunk layout; a load
//     instruction fills 64 consecutive chunks, 8 K rows x 128 contiguous bytes.
// Load instruction i of wave w fills bytes (i*NW + w)*1024 .. +1024 of the slab.
// EDGE: only `valid` (<= R) rows / columns of the tile exist, and K need not be a
// multiple of 64.  The buffer extent then ends at the last valid element —
// K-contiguous: at K in row `valid` - 1; k-major: at column `valid` of the last
// K row — and the loads return zeros from there on (the hardware checks every
// dword against the extent).  Other values past the edges come from
// neighbouring storage: rows / columns past M or N only feed outputs that are
// never stored, and K positions past K are zeroed in the registers (mma_slab).
template <int SHAPE, int R, int NW, bool KMAJOR, bool EDGE = false>
struct DmaOperand {
  static constexpr int INSTR = R / 8 / NW;
  static_assert(INSTR * 8 * NW == R, "slab must split into whole wave loads");
  // K-contiguous: every load instruction of a wave starts at the same row mod 16,
  // so the swizzle — and the per-lane offset — is the same for all of them.
  static_assert(KMAJOR || (NW * 8) % 16 == 0, "per-lane swizzle must be load-invariant");
  static_assert(!KMAJOR || ((NW & (NW - 1)) == 0 && (R == 128 || R == 256)), "k-major slab shape");
  rsrc_t rs;
  uint32_t voff, ld2;

  // X: the operand; r0: first M (or N) index of the tile; ld: leading dimension;
  // valid: M (or N) - r0, used when EDGE.  With EDGE a K-contiguous operand's
  // extent ends at K in its last valid row, so a last slab that reaches past K
  // reads no element past the operand's storage.
  __device__ __forceinline__ DmaOperand(const uint16_t* X, uint32_t ld, int r0, int K, int wave, int lane,
                                        int valid = R) {
    ld2 = ld * 2u;
    const uint32_t v = EDGE ? (uint32_t)min(valid, R) : (uint32_t)R;
    if constexpr (KMAJOR) {
      rs = make_rsrc(X + r0, EDGE ? ((uint32_t)(K - 1) * ld + v) * 2u : (uint32_t)K * ld2);
      // chunk (i*NW + wave)*64 + lane: the bits of i, wave and lane are disjoint
      // and the layout permutes bits, so their (k, r) offsets add.
      int k = 0, r = 0;
      kmaj_coords<SHAPE>(wave * 64 + lane, &k, &r);
      voff = (uint32_t)k * ld2 + (uint32_t)r * 2u;
    } else {
      rs = make_rsrc(X + (int64_t)r0 * ld, EDGE ? ((v - 1u) * ld + (uint32_t)K) * 2u : v * ld2);
      const int row = wave * 8 + (lane >> 3);
      voff = (uint32_t)row * ld2 + (uint32_t)(((lane & 7) ^ swz<64>(row)) << 4);
    }
  }
  __device__ __forceinline__ void issue(uint16_t* slab, int wave, int k0) const {
#pragma unroll
    for (int i = 0; i < INSTR; ++i) {
      uint32_t soff;
      if constexpr (KMAJOR) {
        int ki = 0, ri = 0;
        kmaj_coords<SHAPE>(i * NW * 64, &ki, &ri);
        soff = (uint32_t)(ki + k0) * ld2 + (uint32_t)ri * 2u;
      } else {
        soff = (uint32_t)(i * NW * 8) * ld2 + (uint32_t)k0 * 2u;
      }
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)(slab + (i * NW + wave) * 512), 16, voff, soff, 0, 0);
    }
  }
};

// Epilogue: every accumulator value goes to C[(row0+row)*ldc + col0+col] with
// (row, col) from the instruction's accumulator layout — one store per value.
// ACCUM adds to the existing C instead of overwriting it.
template <int SHAPE, int TM, int TN, bool EDGE, bool ACCUM>
__device__ __forceinline__ void store_acc_impl(float* __restrict__ C, int64_t ldc, int row0, int col0, int M, int N,
                                               int lane, const typename Shape<SHAPE>::Acc (&acc)[TM][TN]) {
  constexpr AccLayout L = acc_layout(SHAPE);
  constexpr int MN = Shape<SHAPE>::MN, J = Shape<SHAPE>::J;
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int v = 0; v < J; ++v) {
        const int r = row0 + i * MN + acc_row(L, lane, v);
        const int c = col0 + j * MN + acc_col(L, lane, v);
        if (!EDGE || (r < M && c < N)) {
          float* p = C + (int64_t)r * ldc + c;
          if constexpr (ACCUM)
            *p += acc[i][j][v];
          else
            *p = acc[i][j][v];
        }
      }
}

template <int SHAPE, int TM, int TN, bool EDGE>
__device__ __forceinline__ void store_acc(float* __restrict__ C, int64_t ldc, int row0, int col0, int M, int N,
                                          int lane, const typename Shape<SHAPE>::Acc (&acc)[TM][TN], int accumulate) {
  if (accumulate)
    store_acc_impl<SHAPE, TM, TN, EDGE, true>(C, ldc, row0, col0, M, N, lane, acc);
  else
    store_acc_impl<SHAPE, TM, TN, EDGE, false>(C, ldc, row0, col0, M, N, lane, acc);
}

// The accumulator numeral's j digits all sit at multiples of the tile width, so
// (row, col)(lane, j) = (row, col)(lane, 0) + (row(0, j), 0): a per-lane part and
// a part that is uniform across the wave.  The buffer-store epilogue relies on it.
constexpr bool acc_rows_separable(const AccLayout& L) {
  for (int lane = 0; lane < L.lanes; ++lane)
    for (int j = 0; j < L.per_lane; ++j)
      if (acc_col(L, lane, j) != acc_col(L, lane, 0) || acc_col(L, 0, j) != 0 ||
          acc_row(L, lane, j) != acc_row(L, lane, 0) + acc_row(L, 0, j))
        return false;
  return true;
}
static_assert(acc_rows_separable(kAcc16x16x32) && acc_rows_separable(kAcc32x32x16), "layout j digits must be rows");

// Epilogue through a buffer resource whose base is the wave tile's origin in C:
// one 32-bit per-lane offset, uniform row offsets from the j digits.
// EDGE: columns from ncols on (relative to the origin) are not stored; rows past
// the buffer's extent are dropped by the hardware.
template <int SHAPE, int TM, int TN, bool ACCUM, bool EDGE = false>
__device__ __forceinline__ void store_acc_rsrc(rsrc_t c, uint32_t ldc, int lane,
                                               const typename Shape<SHAPE>::Acc (&acc)[TM][TN], int ncols = 0) {
  constexpr AccLayout L = acc_layout(SHAPE);
  constexpr int MN = Shape<SHAPE>::MN, J = Shape<SHAPE>::J;
  const uint32_t voff = ((uint32_t)acc_row(L, lane, 0) * ldc + (uint32_t)acc_col(L, lane, 0)) * 4u;
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int v = 0; v < J; ++v) {
      const uint32_t srow = (uint32_t)(i * MN + acc_row(L, 0, v)) * ldc * 4u;
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        if constexpr (EDGE)
          if (acc_col(L, lane, 0) + j * MN >= ncols) continue;
        // the b32 buffer builtins move raw 32-bit patterns: bit-cast, never convert
        float x = acc[i][j][v];
        if constexpr (ACCUM)
          x += __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(c, voff + j * MN * 4, srow, 0));
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, x), c, voff + j * MN * 4, srow, 0);
      }
    }
}

template <int SHAPE, int TM, int TN>
__device__ __forceinline__ void zero_acc(typename Shape<SHAPE>::Acc (&acc)[TM][TN]) {
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int v = 0; v < Shape<SHAPE>::J; ++v) acc[i][j][v] = 0.f;
}

}  // namespace mfl
