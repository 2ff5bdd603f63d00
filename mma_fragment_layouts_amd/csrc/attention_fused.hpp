// Fused split-precision attention (one head, head dim 128): the kernel shape of
// Strata PR #800 ("What's going on": q is split for q.k and p for p.v into an
// FP16 hi and lo half; "The fix": the halves accumulate in separate chains that
// are added in plain fp32), with the scores never leaving the compute unit.
//
// Work split: a workgroup owns 128 queries (8 waves x 16) and one slice of the
// keys.  Per 64-key chunk:
//   GEMM1  S^T (64 keys x 16 queries per wave) = K16 . Q^T, with Q's hi and lo
//          halves as B fragments held in registers for the whole kernel (two
//          chains, summed in fp32);
//   online softmax on the accumulators: per-query reference max (reduced
//          across the four lanes that share a query), P~ = exp(S - mref), the
//          output accumulators and the per-lane partial sum l rescaled when the
//          reference moves;
//   GEMM2  O^T (128 dims x 16 queries) += V16^T . P~^T, with P~ split into fp16
//          hi/lo B fragments built directly from the S^T accumulator registers
//          (two chains).
// Each slice writes its unnormalised O, mref and l; a combine kernel merges the
// slices with exp(m_s - max_s m_s) weights in a fixed order and divides by l.
// The exponentials are taken base 2 on scores pre-scaled by log2 e.
//
// Layout trick: the S^T accumulator gives lane l (query l mod 16, group
// g = l div 16) the keys 16*t' + 4g + j of each 16-key tile t'.  For GEMM2 the
// lane's 8 K positions 8g..8g+7 of 32-key block t are taken to be keys
// 32t + 4g + j (from tile 2t) and 32t + 16 + 4g + j (from tile 2t + 1).  V stays
// key-major in HBM (K16 and V16 are plain fp16 copies); the direct-to-LDS loads
// put key 32t + vt_pos_key(p) into K row 32t + p of a k-major V16 tile, and the
// gfx950 transpose read then hands every lane exactly those 8 keys for its 16
// dims.
#pragma once
#include "gemm_core.hpp"

namespace mfl {

constexpr int kAttnQ = 128;   // queries per workgroup
constexpr int kAttnKV = 64;   // keys per chunk
constexpr int kAttnD = 128;   // head dimension
// The reference max of a query moves only when a chunk's max (base-2 units)
// exceeds it by more than this, so P~ <= 2^kAttnSlack (well inside fp16).
constexpr float kAttnSlack = 8.f;

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 h16x2 __attribute__((ext_vector_type(2)));

// Packed hi/lo split of two fp32 values into fp16 pairs: hi = RNE16(x),
// lo = RNE16(x - hi), with x - hi exact in fp32.
struct Split2 {
  uint32_t hi, lo;
};
__device__ __forceinline__ Split2 split2(float a, float b) {
  const h16x2 h = __builtin_convertvector(f32x2{a, b}, h16x2);
  const f32x2 hf = __builtin_convertvector(h, f32x2);
  const h16x2 l = __builtin_convertvector(f32x2{a - hf.x, b - hf.y}, h16x2);
  return {__builtin_bit_cast(uint32_t, h), __builtin_bit_cast(uint32_t, l)};
}

// Workgroup -> (query block, key slice).  With xcd_map the workgroups that an
// XCD receives (hardware dispatch sends workgroup b to XCD b mod 8) cover a
// contiguous range of key slices for every query block, so each XCD's L2 holds
// only its own slices of K16 / V16^T.
__device__ __forceinline__ void attn_block_of(int b, int nwg, int qblocks, int xcd_map, int& qb, int& sp) {
  const int i = xcd_map ? (b & 7) * (nwg >> 3) + (b >> 3) : b;
  qb = i % qblocks;
  sp = i / qblocks;
}

// K row of key r (0..31) inside its 32-key block of the k-major V16 tile.
MFL_HD constexpr int vt_key_pos(int r) { return 8 * ((r & 15) >> 2) + 4 * (r >> 4) + (r & 3); }

constexpr bool vt_perm_is_bijection() {
  int seen[32] = {};
  for (int r = 0; r < 32; ++r) seen[vt_key_pos(r)]++;
  for (int p = 0; p < 32; ++p)
    if (seen[p] != 1) return false;
  return true;
}
static_assert(vt_perm_is_bijection(), "V^T key permutation must be a bijection");

// Key stored at position p (0..31) of a 32-key block: the inverse of vt_key_pos.
MFL_HD constexpr int vt_pos_key(int p) { return 16 * ((p >> 2) & 1) + 4 * (p >> 3) + (p & 3); }

constexpr bool vt_pos_key_is_inverse() {
  for (int r = 0; r < 32; ++r)
    if (vt_pos_key(vt_key_pos(r)) != r) return false;
  return true;
}
static_assert(vt_pos_key_is_inverse(), "vt_pos_key must invert vt_key_pos");

}  // namespace mfl
