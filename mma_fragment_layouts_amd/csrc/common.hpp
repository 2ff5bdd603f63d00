// Device building blocks shared by the gfx950 kernels: vector types, MFMA
// wrappers, 16-bit conversions, the swizzled LDS tile layout, and the launch
// helpers of the C ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/mfl.h"
#include "layout.hpp"

namespace mfl {

typedef __bf16 bf16;
typedef _Float16 f16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// ---- MFMA shapes -----------------------------------------------------------
// SHAPE 0: v_mfma_f32_16x16x32_{f16,bf16}; SHAPE 1: v_mfma_f32_32x32x16_{f16,bf16}.
// Operand fragments (both shapes, 8 16-bit values per lane): lane l supplies
// A row (l mod MN) and B column (l mod MN) at K positions KB*(l div MN) + i,
// i = 0..7, where MN is 16 or 32 and KB = 8.  Any K permutation shared by A and
// B leaves the product unchanged; only the row/column assignment matters.
template <int SHAPE> struct Shape;
template <> struct Shape<0> {
  using Acc = f32x4;
  static constexpr int MN = 16, K = 32, J = 4;
};
template <> struct Shape<1> {
  using Acc = f32x16;
  static constexpr int MN = 32, K = 16, J = 16;
};

template <int SHAPE, int DT>  // DT: MFL_F16 or MFL_BF16
__device__ __forceinline__ typename Shape<SHAPE>::Acc mfma(u32x4 a, u32x4 b, typename Shape<SHAPE>::Acc c) {
  if constexpr (SHAPE == 0 && DT == MFL_BF16)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  else if constexpr (SHAPE == 0)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  else if constexpr (DT == MFL_BF16)
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// ---- 16-bit conversions (round to nearest even, the hardware default) -------
template <int DT>
__device__ __forceinline__ uint16_t to16(float x) {
  if constexpr (DT == MFL_BF16)
    return __builtin_bit_cast(uint16_t, (bf16)x);
  else
    return __builtin_bit_cast(uint16_t, (f16)x);
}
template <int DT>
__device__ __forceinline__ float from16(uint16_t h) {
  if constexpr (DT == MFL_BF16)
    return (float)__builtin_bit_cast(bf16, h);
  else
    return (float)__builtin_bit_cast(f16, h);
}

// ---- swizzled LDS tile -----------------------------------------------------
// A tile of R rows (M or N index) by BK K-values of 16-bit data, K contiguous,
// stored row after row as BK/8 16-byte chunks.  The chunk index is XOR-ed with
// a function of (row mod 16).
//
// gfx950's LDS serves a 64-lane ds_read_b128 in four phases of 16 lanes
// (256 bytes, one 16-byte slot per 4 of the 64 banks): lane l belongs to phase
// 2*(l >> 5) + parity((l >> 2) & 7), i.e. lanes {0-3, 12-15, 20-23, 24-27},
// {4-11, 16-19, 28-31} and the same two sets plus 32.  A read is conflict free
// when the 16 lanes of each phase touch 16 different slots of a 256-byte window.
// For the MFMA fragment reads (lane l: row l mod 16 or l mod 32, chunk
// l div 16 or l div 32 of the K step) and for row-wise fills, XOR-ing the chunk
// with (row >> 1) & 7 (128-byte rows) or with 2*bit2(row) ^ 3*bit3(row)
// (64-byte rows) achieves that for both MFMA shapes.  (Phases and conflict
// cycles measured with the SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE counters.)
// Because the swizzle repeats every 16 rows, fragment i of a wave sits a fixed
// i*16*BK elements after fragment 0 (an immediate offset).
template <int BK>
MFL_HD constexpr int swz(int row) {
  if constexpr (BK == 64)
    return (row >> 1) & 7;
  else
    return (((row >> 2) & 1) * 2) ^ (((row >> 3) & 1) * 3);  // BK == 32
}
// The fragment addressing (immediate i*16*BK offsets) needs the swizzle to
// repeat every 16 rows.
template <int BK>
constexpr bool swz_period16() {
  for (int r = 0; r < 1024; ++r)
    if (swz<BK>(r) != swz<BK>(r & 15)) return false;
  return true;
}
static_assert(swz_period16<64>() && swz_period16<32>(), "LDS swizzle must depend on row mod 16 only");

// Element offset (in 16-bit units) of chunk `chunk` of row `row`.
template <int BK>
__device__ __forceinline__ int lds_chunk(int row, int chunk) {
  return row * BK + ((chunk ^ swz<BK>(row)) << 3);
}

// ---- k-major LDS tiles and the CDNA4 transpose read ---------------------------
// A K-strided operand (A column-major, B row-major) is staged as a k-major tile:
// 64 K rows of R consecutive M (or N) values (R = 128 or 256).
//
// ds_read_b64_tr_b16 (gfx950) reads 8 bytes per lane and transposes 16-bit
// elements inside each group of 16 lanes: lane 16g + 4q + e receives, as its
// element t, element e of the 8 bytes that lane 16g + 4t + q addressed (q, e, t
// in 0..3).  Measured on MI355X by reading an index-filled LDS under several
// address patterns; the mapping does not depend on the addresses.
MFL_HD constexpr int tr_src_lane(int lane, int t) { return (lane & ~15) + 4 * t + ((lane & 15) >> 2); }
MFL_HD constexpr int tr_src_elem(int lane) { return lane & 3; }

// Layout of the k-major tile: element (k, r) at 16-bit offset
// 8 * kmaj_chunk(k, r) + (r & 7), the 16-byte chunk index being a permutation of
// the bits of k and r.  ds_read_b64 and ds_read_b64_tr_b16 serve a wave in two
// phases, lanes 0-31 and 32-63 (measured with SQ_LDS_BANK_CONFLICT on lane
// pairs); a fragment read touches, per phase, 8 K rows x 32 bytes (16x16x32:
// k bits 0, 1, 3 and r bit 3 vary) or 4 K rows x 64 bytes (32x32x16: k bits 0,
// 1 and r bits 3, 4 vary).  Those bits become chunk bits 0-3 — the 16 bank slots
// of 256 bytes — so every phase is conflict free.  The bits that step a read
// (the second read of a fragment: k bit 2; the MFMA K step: k bit 5, or bits 4
// and 5; the fragment: r bits 4-5, or bit 5) sit above them, so every read is an
// immediate offset from one per-lane address.  A direct-to-LDS load
// instruction fills 64 consecutive chunks: its lanes fetch 8 K rows x 128
// contiguous bytes, and instruction and wave indices map to fixed (k, r)
// offsets — uniform scalar offsets.
template <int SHAPE>
MFL_HD constexpr int kmaj_chunk(int k, int r) {
  const int k0 = k & 1, k1 = (k >> 1) & 1, k2 = (k >> 2) & 1, k3 = (k >> 3) & 1, k4 = (k >> 4) & 1, k5 = (k >> 5) & 1;
  const int r3 = (r >> 3) & 1, r4 = (r >> 4) & 1, r5 = (r >> 5) & 1, rh = r >> 6;
  if (SHAPE == 0)
    return r3 | k0 << 1 | k1 << 2 | k3 << 3 | r4 << 4 | r5 << 5 | k2 << 6 | k4 << 7 | k5 << 8 | rh << 9;
  return r3 | k0 << 1 | k1 << 2 | r4 << 3 | r5 << 4 | k3 << 5 | k2 << 6 | k4 << 7 | k5 << 8 | rh << 9;
}
// Inverse of kmaj_chunk: the (k, r) of the first element of chunk c.
template <int SHAPE>
MFL_HD constexpr void kmaj_coords(int c, int* k, int* r) {
  auto bit = [c](int i) { return (c >> i) & 1; };
  if (SHAPE == 0) {
    *k = bit(1) | bit(2) << 1 | bit(6) << 2 | bit(3) << 3 | bit(7) << 4 | bit(8) << 5;
    *r = (bit(0) << 3) | (bit(4) << 4) | (bit(5) << 5) | ((c >> 9) << 6);
  } else {
    *k = bit(1) | bit(2) << 1 | bit(6) << 2 | bit(5) << 3 | bit(7) << 4 | bit(8) << 5;
    *r = (bit(0) << 3) | (bit(3) << 4) | (bit(4) << 5) | ((c >> 9) << 6);
  }
}
template <int SHAPE>
MFL_HD constexpr int lds_elemKM(int k, int r) {
  return 8 * kmaj_chunk<SHAPE>(k, r) + (r & 7);
}
template <int SHAPE, int R>
constexpr bool kmaj_layout_ok() {
  for (int k = 0; k < 64; ++k)
    for (int r = 0; r < R; r += 8) {
      const int c = kmaj_chunk<SHAPE>(k, r);
      int k2 = -1, r2 = -1;
      kmaj_coords<SHAPE>(c, &k2, &r2);
      if (c < 0 || c >= 8 * R || k2 != k || r2 != r) return false;
    }
  return true;
}
static_assert(kmaj_layout_ok<0, 128>() && kmaj_layout_ok<0, 256>() && kmaj_layout_ok<1, 128>() &&
                  kmaj_layout_ok<1, 256>(),
              "k-major tile layout must be a bijection with the stated inverse");

// ---- buffer resources --------------------------------------------------------
// A raw buffer descriptor: base address, byte extent (accesses at or past it
// read 0 / are dropped), 32-bit dword format.  Per-lane 32-bit offsets plus
// uniform scalar offsets replace 64-bit per-lane addresses.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}
typedef __attribute__((address_space(3))) void* lds_ptr_t;

__device__ __forceinline__ u32x4 lds_read16(const uint16_t* lds, int elem_off) {
  return *reinterpret_cast<const u32x4*>(lds + elem_off);
}
__device__ __forceinline__ void lds_write16(uint16_t* lds, int elem_off, u32x4 v) {
  *reinterpret_cast<u32x4*>(lds + elem_off) = v;
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
// Two transpose reads, `step` elements apart, concatenated into one 8-element
// MFMA operand (elements 0-3 from the first read, 4-7 from the second).
__device__ __forceinline__ u32x4 lds_read_tr(const uint16_t* lds, int elem_off, int step) {
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(lds + elem_off));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(lds + elem_off + step));
  return __builtin_shufflevector(__builtin_bit_cast(u32x2, lo), __builtin_bit_cast(u32x2, hi), 0, 1, 2, 3);
}

__device__ __forceinline__ u32x4 gload16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

// The first n (may be <= 0 or >= 8) of 8 consecutive 16-bit values, read one
// by one, the rest zero: no read at or past p + n.
__device__ __forceinline__ u32x4 gload_partial(const uint16_t* p, int n) {
  uint16_t h[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) h[e] = e < n ? p[e] : (uint16_t)0;
  u32x4 v;
  __builtin_memcpy(&v, h, 16);
  return v;
}

// The first n (may be <= 0 or >= 4) of 4 consecutive fp32 values, read one by
// one, the rest zero: no read at or past p + n.
__device__ __forceinline__ f32x4 gload4_partial(const float* p, int n) {
  f32x4 v = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int e = 0; e < 4; ++e)
    if (e < n) v[e] = p[e];
  return v;
}

// ---- XCD-aware tile order --------------------------------------------------
// Workgroups are dealt round-robin to the 8 XCDs, each with its own L2.  Renumber
// so that the workgroups one XCD receives are consecutive, then walk tiles in
// groups of `group_m` tile rows so that consecutive ids share A and B panels.
__device__ __forceinline__ void tile_of(int bid, int nwg, int tiles_m, int tiles_n, int group_m, int* tm, int* tn) {
  if ((nwg & 7) == 0) bid = (bid & 7) * (nwg >> 3) + (bid >> 3);
  const int per_group = group_m * tiles_n;
  const int g = bid / per_group;
  const int first_m = g * group_m;
  const int gsize = min(tiles_m - first_m, group_m);
  const int in_g = bid - g * per_group;
  *tm = first_m + in_g % gsize;
  *tn = in_g / gsize;
}

// ---- host helpers ------------------------------------------------------------
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }
inline int launch_status() { return hipGetLastError() == hipSuccess ? MFL_OK : MFL_EHIP; }

}  // namespace mfl
