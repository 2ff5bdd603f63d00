// Accumulator-fragment layouts of the CDNA4 MFMA instructions, as mixed-radix
// numerals.
//
// cuda-oxide PR #474 ("derive the m16n8k16 accumulator fragment layout",
// section "The layout is a mixed-radix numeral") shows that the row-major offset
// of a fragment element, written as a function of (lane, j), regroups into a
// numeral whose digits are bit fields of lane and j and whose place values are
// the running product of the lower radices.  A numeral of that form is uniquely
// decodable, so when its span equals lanes*J the map is a bijection onto the
// tile.  This header writes the two CDNA4 accumulator layouts in that form and
// derives every other view from it:
//
//   V_MFMA_F32_16X16X32_{F16,BF16}: 64 lanes x 4 fp32, 16x16 tile
//     row = 4*(lane>>4) + j, col = lane & 15
//     offset = (lane&15)*1 + j*16 + (lane>>4)*64              span 256
//   V_MFMA_F32_32X32X16_{F16,BF16}: 64 lanes x 16 fp32, 32x32 tile
//     row = 8*(j>>2) + 4*(lane>>5) + (j&3), col = lane & 31
//     offset = (lane&31)*1 + (j&3)*32 + (lane>>5)*128 + (j>>2)*256   span 1024
//
// In the 32x32 layout j occupies two non-adjacent digits (places 32 and 256),
// the same phenomenon the page points out for m16n8k16: j 0->1 is one row, j 3->4
// is eight rows.
//
// The operand fragments of the same instructions (which lane supplies which A
// and B element; the page leaves them out of scope, "Scope" section) are
// numerals of the same kind over the K-contiguous storage of the operand tile
// (A row-major m*K + k, B column-major n*K + k): lane l supplies the 8
// consecutive K positions 8*(l div MN) + i of row (A) or column (B) l mod MN.
//   16x16x32: offset = i*1 + (lane>>4)*8 + (lane&15)*32          span 512
//   32x32x16: offset = i*1 + (lane>>5)*8 + (lane&31)*16          span 512
//
// Everything here is constexpr and usable from host and device code.
#pragma once
#include <stdint.h>

#if defined(__HIPCC__)
#define MFL_HD __host__ __device__
#else
#define MFL_HD
#endif

namespace mfl {

enum Src : int { kLane = 0, kJ = 1 };

// One digit: value = (source >> shift) & (radix - 1); radix is a power of two.
struct Digit {
  int src;
  int shift;
  int radix;
};

struct AccLayout {
  int lanes;      // lanes of the wave holding the tile
  int per_lane;   // values per lane (J for accumulators, 8 for operands)
  int rows, cols; // tile shape; offsets are row-major: row*cols + col
  int ndigits;
  Digit d[4];     // lowest place first
};

// Shape ids match the C ABI's mfl_shape.
constexpr AccLayout kAcc16x16x32 = {64, 4, 16, 16, 3, {{kLane, 0, 16}, {kJ, 0, 4}, {kLane, 4, 4}, {0, 0, 1}}};
constexpr AccLayout kAcc32x32x16 = {64, 16, 32, 32, 4, {{kLane, 0, 32}, {kJ, 0, 4}, {kLane, 5, 2}, {kJ, 2, 4}}};

MFL_HD constexpr const AccLayout& acc_layout(int shape) { return shape == 0 ? kAcc16x16x32 : kAcc32x32x16; }

// Operand numerals: rows = MN, cols = K of the K-contiguous storage (j = i).
constexpr AccLayout kOp16x16x32 = {64, 8, 16, 32, 3, {{kJ, 0, 8}, {kLane, 4, 4}, {kLane, 0, 16}, {0, 0, 1}}};
constexpr AccLayout kOp32x32x16 = {64, 8, 32, 16, 3, {{kJ, 0, 8}, {kLane, 5, 2}, {kLane, 0, 32}, {0, 0, 1}}};

MFL_HD constexpr const AccLayout& operand_layout(int shape) { return shape == 0 ? kOp16x16x32 : kOp32x32x16; }

MFL_HD constexpr int acc_span(const AccLayout& L) {
  int s = 1;
  for (int i = 0; i < L.ndigits; ++i) s *= L.d[i].radix;
  return s;
}

// Row-major offset of (lane, j) inside the tile, evaluated as the numeral.
MFL_HD constexpr int acc_offset(const AccLayout& L, int lane, int j) {
  int off = 0, place = 1;
  for (int i = 0; i < L.ndigits; ++i) {
    const int src = L.d[i].src == kLane ? lane : j;
    off += ((src >> L.d[i].shift) & (L.d[i].radix - 1)) * place;
    place *= L.d[i].radix;
  }
  return off;
}

// Position in the tile: the offset split into row and column.
MFL_HD constexpr int acc_row(const AccLayout& L, int lane, int j) { return acc_offset(L, lane, j) / L.cols; }
MFL_HD constexpr int acc_col(const AccLayout& L, int lane, int j) { return acc_offset(L, lane, j) % L.cols; }

// Inverse of acc_offset: read each digit back out of the offset and reassemble
// lane and j from their bit fields.
MFL_HD constexpr void acc_decode(const AccLayout& L, int off, int* lane, int* j) {
  int l = 0, jj = 0, place = 1;
  for (int i = 0; i < L.ndigits; ++i) {
    const int v = (off / place) & (L.d[i].radix - 1);
    if (L.d[i].src == kLane)
      l |= v << L.d[i].shift;
    else
      jj |= v << L.d[i].shift;
    place *= L.d[i].radix;
  }
  *lane = l;
  *j = jj;
}

// Compile-time sanity: span equals the number of (lane, j) points, and decode
// inverts offset on every point.
constexpr bool layout_self_consistent(const AccLayout& L) {
  if (acc_span(L) != L.lanes * L.per_lane || acc_span(L) != L.rows * L.cols) return false;
  for (int lane = 0; lane < L.lanes; ++lane)
    for (int j = 0; j < L.per_lane; ++j) {
      int l2 = -1, j2 = -1;
      acc_decode(L, acc_offset(L, lane, j), &l2, &j2);
      if (l2 != lane || j2 != j) return false;
    }
  return true;
}
static_assert(layout_self_consistent(kAcc16x16x32), "16x16x32 numeral is not a bijection");
static_assert(layout_self_consistent(kAcc32x32x16), "32x32x16 numeral is not a bijection");
static_assert(layout_self_consistent(kOp16x16x32), "16x16x32 operand numeral is not a bijection");
static_assert(layout_self_consistent(kOp32x32x16), "32x32x16 operand numeral is not a bijection");

// The GEMM kernels read a lane's operand fragment as one 16-byte chunk: row
// (or column) lane mod MN, K positions from 8*(lane div MN).  That is element
// i = 0 of the operand numeral, and the 8 elements of a lane are consecutive.
constexpr bool operand_chunks_match(const AccLayout& L) {
  for (int lane = 0; lane < L.lanes; ++lane) {
    if (acc_offset(L, lane, 0) != (lane % L.rows) * L.cols + 8 * (lane / L.rows)) return false;
    for (int i = 1; i < L.per_lane; ++i)
      if (acc_offset(L, lane, i) != acc_offset(L, lane, 0) + i) return false;
  }
  return true;
}
static_assert(operand_chunks_match(kOp16x16x32) && operand_chunks_match(kOp32x32x16),
              "kernel fragment reads disagree with the operand numerals");

}  // namespace mfl
