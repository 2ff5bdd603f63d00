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
__device__ __forceinline__ uint32_t pack2(uint16_t lo, uint16_t hi) { return (uint32_t)lo | ((uint32_t)hi << 16); }

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
template <int BK>
__device__ __forceinline__ int lds_elem(int row, int k) {
  return lds_chunk<BK>(row, k >> 3) + (k & 7);
}

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

__device__ __forceinline__ u32x4 gload16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

// Zero the 16-bit lanes of a chunk whose K index (k_first + e) is >= k_end.
__device__ __forceinline__ u32x4 mask_tail(u32x4 v, int k_first, int k_end) {
  uint16_t h[8];
  __builtin_memcpy(h, &v, 16);
#pragma unroll
  for (int e = 0; e < 8; ++e)
    if (k_first + e >= k_end) h[e] = 0;
  __builtin_memcpy(&v, h, 16);
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
