/*
 * mfl.h — C ABI of libmfl.so: MFMA fragment layouts and tiled mixed-precision
 * GEMMs for AMD Instinct MI355X (gfx950, CDNA4).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Return value: an mfl_status (0 on success, negative on error).  Nothing is
 *    thrown across the ABI and there is no global error state; errors are found
 *    before any HIP call is made, so a rejected call has no side effect.
 *  - Matrix pointers are DEVICE pointers owned by the caller.  The library never
 *    allocates or frees device memory; scratch space, where an operation needs
 *    it, is a caller-provided workspace whose size a query function returns
 *    (one variant, attention_split_fp32_static, uses a static device array of
 *    the library instead).
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *    Device calls only enqueue work and return; results are ready when the
 *    stream is synchronised.  Calls on one stream are ordered; calls on
 *    different streams that write the same memory race.  A device call
 *    launches kernels and nothing else (no allocation, copy, fill or
 *    synchronisation), so it may be captured in a HIP graph and replayed;
 *    a replay recomputes everything from the operands, the workspace
 *    included.
 *  - Matrices: A is M x K, B is K x N, C is M x N.  A row-major A stores
 *    A[m][k] at a[m*lda + k]; a column-major A stores it at a[k*lda + m].  A
 *    row-major B stores B[k][n] at b[k*ldb + n]; a column-major B at
 *    b[n*ldb + k].  C is always row-major: C[m][n] at c[m*ldc + n].  The leading
 *    dimension is the element distance between successive rows (row-major) or
 *    columns (column-major) and may exceed the visible extent (padding); each
 *    operand's storage must span (outer extent) x ld elements.  (Tensor-core
 *    layout explainer, paragraph on leading dimensions.)
 *  - 16-bit operands need 16-byte aligned base pointers and ld a multiple of 8;
 *    fp32 operands 16-byte aligned base pointers and ld a multiple of 4.
 *    C needs 4-byte alignment only.  Violations return MFL_EINVAL.
 *  - Any M, N, K >= 0 is accepted (ragged edges are masked); M or N = 0 is a
 *    no-op; K = 0 gives C = 0 (or leaves C unchanged when accumulating).
 */
#ifndef MFL_H
#define MFL_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__)
#define MFL_API __attribute__((visibility("default")))
#else
#define MFL_API
#endif

typedef enum {
  MFL_OK = 0,
  MFL_EINVAL = -1,        /* bad argument: null pointer, out-of-range index, bad ld/alignment */
  MFL_EOVERFLOW = -2,     /* the result would not fit (the cuda-oxide page's "None on overflow") */
  MFL_EUNSUPPORTED = -3,  /* valid request this build does not implement */
  MFL_EHIP = -4,          /* a HIP launch failed (hipGetLastError after enqueue) */
  MFL_ESCRATCH = -5       /* the call needs more than the library's static scratch array holds */
} mfl_status;

typedef enum { MFL_MFMA_16X16X32 = 0, MFL_MFMA_32X32X16 = 1 } mfl_shape;
typedef enum { MFL_F16 = 0, MFL_BF16 = 1 } mfl_dtype;
typedef enum { MFL_ROW_MAJOR = 0, MFL_COL_MAJOR = 1 } mfl_order;
typedef enum { MFL_ROUND = 0, MFL_SPLIT = 1 } mfl_opmode;

/* Human-readable name of a status code (static string, never NULL). */
MFL_API const char *mfl_status_string(int status);

/* Library version as 10000*major + 100*minor + patch. */
MFL_API int mfl_version(void);

/* ---------------------------------------------------------------------------
 * Accumulator-fragment layout (host only, pure functions, no HIP calls).
 *
 * cuda-oxide PR #474, section "API": position, row-major offset, strided
 * destination and inverse of an MMA accumulator fragment element, derived once
 * as a mixed-radix numeral (section "The layout is a mixed-radix numeral") so
 * call sites do not re-derive it.  Here the maps are those of the CDNA4
 * instructions, identical for f16 and bf16 operands:
 *   MFL_MFMA_16X16X32 (v_mfma_f32_16x16x32_{f16,bf16}): 64 lanes x J=4, 16x16
 *   MFL_MFMA_32X32X16 (v_mfma_f32_32x32x16_{f16,bf16}): 64 lanes x J=16, 32x32
 * A (lane, j) pair with lane outside [0,64) or j outside [0,J), an unknown
 * shape or a NULL output pointer returns MFL_EINVAL and writes nothing.
 * ------------------------------------------------------------------------- */

/* Tile geometry of `shape`: lanes (64), values per lane J, rows and cols. */
MFL_API int mfl_acc_info(int shape, int *lanes, int *per_lane, int *rows, int *cols);

/* Position (row, col) of accumulator value j of `lane` within the tile. */
MFL_API int acc_coords(int shape, int lane, int j, int *row, int *col);

/* Row-major offset row*cols + col of (lane, j), computed in numeral form. */
MFL_API int acc_offset(int shape, int lane, int j, int *offset);

/* Inverse of acc_offset: the (lane, j) that owns `offset` in [0, rows*cols).
 * Exported so a caller can round-trip a hand-written layout in a test. */
MFL_API int acc_decode(int shape, int offset, int *lane, int *j);

/* Strided destination of (lane, j) for a tile whose element origin is
 * (row0, col0) in a row-major matrix with leading dimension ld:
 *   *out = (row0 + row) * ld + (col0 + col).
 * MFL_EOVERFLOW (the page's None) when the value does not fit int64 or when
 * col0 + col >= ld (the element would spill into the next row, breaking
 * disjointness of strided placement).  Negative row0/col0 or ld <= 0:
 * MFL_EINVAL. */
MFL_API int acc_matrix_offset(int shape, int lane, int j, int64_t row0, int64_t col0, int64_t ld,
                      int64_t *out);

/* ---------------------------------------------------------------------------
 * Operand-fragment layout (host only, pure functions, no HIP calls).
 *
 * The other half of the layout contract: which lane supplies which element of
 * the A (MN x K) and B (K x MN) operands of one MFMA.  cuda-oxide PR #474,
 * section "Scope", leaves A/B fragments out of its accumulator API; the
 * Tensor-core layout explainer (paragraph on fragments) says each thread
 * holds specific pieces of A and B as well as of C.  These calls give them
 * the same API shape and the same numeral treatment as the accumulator:
 * lane l supplies the 8 consecutive K positions 8*(l div MN) + i (i = 0..7)
 * of row l mod MN of A and of column l mod MN of B; MN = 16, K = 32 for
 * MFL_MFMA_16X16X32 and MN = 32, K = 16 for MFL_MFMA_32X32X16, for f16 and
 * bf16 alike.  Offsets are in the K-contiguous storage of the tile (A
 * row-major m*K + k, B column-major n*K + k), the order the MFMA consumes.
 * Unknown shape or operand, lane outside [0,64), i outside [0,8) or a NULL
 * output pointer: MFL_EINVAL, nothing written.
 * ------------------------------------------------------------------------- */

typedef enum { MFL_OPERAND_A = 0, MFL_OPERAND_B = 1 } mfl_operand;

/* Geometry of the operand tile: lanes (64), elements per lane (8), rows and
 * cols of the operand as written (A: MN x K, B: K x MN). */
MFL_API int mfl_operand_info(int shape, int operand, int *lanes, int *per_lane, int *rows, int *cols);

/* Position of element i of `lane`: (m, k) for A, (k, n) for B. */
MFL_API int operand_coords(int shape, int operand, int lane, int i, int *row, int *col);

/* K-contiguous offset of (lane, i), computed in numeral form. */
MFL_API int operand_offset(int shape, int operand, int lane, int i, int *offset);

/* Inverse of operand_offset over [0, MN*K). */
MFL_API int operand_decode(int shape, int operand, int offset, int *lane, int *i);

/* Strided source of (lane, i) for an operand tile whose element origin is
 * (row0, col0) (same row/col convention as operand_coords) in a matrix with
 * leading dimension ld stored row-major (order MFL_ROW_MAJOR:
 * (row0+row)*ld + col0+col) or column-major (MFL_COL_MAJOR:
 * (col0+col)*ld + row0+row).  MFL_EOVERFLOW when the value does not fit int64
 * or the contiguous coordinate reaches ld (the reading acc_matrix_offset
 * uses); negative row0/col0, ld <= 0 or an unknown order: MFL_EINVAL. */
MFL_API int operand_matrix_offset(int shape, int operand, int lane, int i, int64_t row0, int64_t col0,
                                  int64_t ld, int order, int64_t *out);

/* ---------------------------------------------------------------------------
 * Device entry points.
 * ------------------------------------------------------------------------- */

/* Strided operand load (device): one wave gathers the fragment of `operand`
 * for an operand tile at element origin (row0, col0) of a 16-bit matrix m
 * (device memory, f16 or bf16 bits, leading dimension ld, order as in
 * operand_matrix_offset) into frag[lane*8 + i] (512 16-bit values, device
 * memory) — the load-side twin of acc_store_strided, and what mfma_probe
 * takes as a_frag / b_frag.  MFL_EOVERFLOW if the tile's contiguous extent
 * passes ld or its last element does not fit int64; MFL_EINVAL on NULL or
 * odd pointers, negative origins, ld <= 0, unknown shape, operand or order. */
MFL_API int operand_load_strided(int shape, int operand, const void *m, int64_t row0, int64_t col0,
                                 int64_t ld, int order, void *frag, void *stream);

/* Strided epilogue store (device): one wave scatters a lane-major accumulator
 * acc[lane*J + j] (64*J fp32, device memory) into C at element origin
 * (row0, col0) of a row-major fp32 matrix with leading dimension ldc, writing
 * C[(row0+row)*ldc + col0+col] = acc[lane*J + j] through the layout above —
 * one store per accumulator value (Warp issue #1965, "Proposed change": the
 * accumulator is materialised once).  MFL_EOVERFLOW if col0 + cols > ldc. */
MFL_API int acc_store_strided(int shape, const float *acc, float *c, int64_t row0, int64_t col0,
                      int64_t ldc, void *stream);

/* Single-instruction probe (device): one wave executes one MFMA of `shape` and
 * `dtype` (MFL_F16 or MFL_BF16).  a_frag and b_frag hold each lane's 8 16-bit
 * operand values lane-major (lane*8 + i); c_in holds the accumulator input
 * lane-major (lane*J + j), or is NULL for zeros; the raw accumulator registers
 * are written lane-major to acc (lane*J + j).  No layout logic runs on the
 * device: the caller gathers the operands and scatters the result, which is how
 * the layout is checked against hardware (cuda-oxide PR #474, "Verified against
 * hardware"), and how the rounding of the accumulation is measured. */
MFL_API int mfma_probe(int shape, int dtype, const void *a_frag, const void *b_frag, const float *c_in,
                       float *acc, void *stream);

/* MFMA rate microbenchmark (device): the ceiling a GEMM's MFMA rate is measured
 * against.  The pages time their kernels against a published peak (Warp issue
 * #1965, "Spike": a stated TF32 peak beside measured rates); the published
 * MI355X figure assumes a 2.4 GHz clock that the chip does not hold under
 * matrix load, so this call measures what the matrix cores sustain with no
 * memory or vector work: MFL_RATE_PROBE_OUTPUTS / 64 waves (eight 4-wave
 * workgroups per compute unit), each issuing `iters` rounds of 16 independent
 * v_mfma_f32_16x16x32 of `dtype` (MFL_F16 or MFL_BF16).  Work per call:
 * MFL_RATE_PROBE_OUTPUTS / 64 * iters * 16 * 16384 flop.  Operands: seed 0 sets
 * every operand to 1.0 (then out[t] = 480 + 2048 * iters exactly while that
 * stays below 2^24); any other seed gives per-lane values in [1, 2) from a hash
 * of (lane, seed).  out (device, fp32, 4-byte aligned) receives
 * MFL_RATE_PROBE_OUTPUTS values, one per thread: the sum of its accumulators.
 * MFL_EINVAL on an unknown dtype, iters < 0 or a NULL / misaligned out. */
#define MFL_RATE_PROBE_OUTPUTS (2048 * 256)
MFL_API int mfma_rate_probe(int dtype, int iters, uint32_t seed, float *out, void *stream);

/* Round n fp32 values to `dtype` (round-to-nearest-even; NaN stays NaN,
 * overflow gives +-inf).  out receives n 16-bit values.  Tensor-core layout
 * explainer, paragraph on mixed precision: conversion changes the values that
 * enter the multiply. */
MFL_API int quantize_fp32(int dtype, const float *x, void *out, int64_t n, void *stream);

/* Split n fp32 values into hi = RNE(x) and lo = RNE(x - hi), both `dtype`
 * (Strata PR #800, "What's going on"). */
MFL_API int split_fp32(int dtype, const float *x, void *hi, void *lo, int64_t n, void *stream);

/* Tiled mixed-precision GEMM: C = A*B (accumulate = 0) or C += A*B
 * (accumulate = 1) with `dtype` operands (MFL_F16 or MFL_BF16) and fp32
 * accumulation kept in registers across the whole K loop; each output tile is
 * stored once through the accumulator layout (Warp issue #1965, "Proposed
 * change" and "Design consequences").  Operand orders are free.  The fast path
 * takes K a multiple of 8, M a multiple of 8 when A is column-major and N a
 * multiple of 8 when B is row-major, and buffers within 4 GiB (256 rows of
 * lda / ldb / ldc; K rows of lda for column-major A, of ldb for row-major B);
 * M, N and K need not be tile multiples (the last tiles are clipped, the K
 * positions of the last slab past k are zeroed in registers, and nothing
 * outside the m x n block of C, padding included, is written).  A
 * column-major A or row-major B is staged K-major in LDS and read with the
 * gfx950 transpose read, with results bit-identical to the K-contiguous
 * orders.  The tile follows the problem size: 256 x 256 when that gives at
 * least 128 workgroups (192 x 192 instead, for K-contiguous operands, when
 * 256-tiles would fill only part of one round of one tile per compute unit
 * and 192-tiles fit in one), else 128 x 128, 64 x 64 or 32 x 32; every output element
 * sees the same MFMA sequence whatever the tile, so the bits do not depend on
 * it.  A size whose 256 x 256 tiles fill at least two whole rounds of
 * one tile per compute unit plus a partial one runs as two launches on the
 * stream, split by rows: whole rounds of 256-tiles, then one round of
 * 128-tiles.  The bits are the same as with one launch.
 * Other sizes take the generic path.  Reads never go past the
 * minimum storage of an operand, (rows - 1) * ld + the inner extent. */
MFL_API int gemm_tile_mma(int dtype, int64_t m, int64_t n, int64_t k,
                  const void *a, int64_t lda, int order_a,
                  const void *b, int64_t ldb, int order_b,
                  float *c, int64_t ldc, int accumulate, void *stream);

/* Block-GEMM repeat (Warp issue #1965, "Spike"): the output C (m x n, fp32,
 * row-major, ldc = n) is cut into tm x tn tiles; the workgroup of tile (bi, bj)
 * loads A[bi*tm.., 0..tk) (a: row-major m x tk, lda = tk) and
 * B[0..tk, bj*tn..) (b: column-major tk x n, ldb = tk) into LDS once and runs
 * `repeats` back-to-back tm x tn x tk block MMAs into one register accumulator,
 * reading the operand fragments from LDS on every repeat, then stores the tile
 * once: C = repeats * A*B.  Supported (tm, tn, tk, threads): (64,64,64, 64|128|256),
 * (32,32,32, 128), (128,128,32, 128|256); m % tm == 0 and n % tn == 0;
 * others return MFL_EUNSUPPORTED. */
MFL_API int gemm_block_repeat(int dtype, int tm, int tn, int tk, int threads, int repeats,
                      int64_t m, int64_t n, const void *a, const void *b, float *c,
                      void *stream);

/* The same workload through the other arm of Warp issue #1965's comparison,
 * the shared-memory pointer API ("Description"): A and B in plain
 * (unswizzled) LDS tiles, and C kept in an fp32 LDS tile that every repeat
 * reads into registers, updates with one block MMA and writes back, with a
 * workgroup barrier between repeats.  Same arguments, result, tiles and errors
 * as gemm_block_repeat; it exists to measure the bank conflicts and the C
 * round trip the issue attributes to that API. */
MFL_API int gemm_block_repeat_lds_api(int dtype, int tm, int tn, int tk, int threads, int repeats,
                      int64_t m, int64_t n, const void *a, const void *b, float *c,
                      void *stream);

/* Split-precision fp32 GEMM (Strata PR #800, "The fix"): A and B are fp32; an
 * operand in MFL_SPLIT mode is split on load into hi = RNE(x) and
 * lo = RNE(x - hi) of type `piece` (MFL_F16 or MFL_BF16), an operand in
 * MFL_ROUND mode is rounded once.  Products per K step: hi*hi, hi*lo, lo*hi
 * (those that exist for the modes), plus lo*lo if `lolo` and both are split.
 *   chains = 1: every product goes into one accumulator (the single-chain
 *               variant, kept for comparison);
 *   chains = 2: hi*hi in one accumulator, all correction products in a second;
 *   chains = 3: hi*hi, hi*lo and lo*hi(+lo*lo) in three (both operands split).
 * The chains are summed in plain fp32 once, at the end: hh + (hl + lh).
 * C = result (accumulate = 0) or C += result (accumulate = 1). */
MFL_API int gemm_split_fp32(int piece, int64_t m, int64_t n, int64_t k,
                    const float *a, int64_t lda, int order_a, int mode_a,
                    const float *b, int64_t ldb, int order_b, int mode_b,
                    int chains, int lolo, float *c, int64_t ldc, int accumulate,
                    void *stream);

/* Workspace for gemm_split_fp32_ws: the bytes of the four 16-bit planes
 * (hi and lo of A and of B, each in its operand's storage shape — A: m rows
 * row-major, k rows column-major; B: n rows column-major, k rows row-major —
 * of ld elements, 256-byte aligned) when the planes path applies — both
 * operands MFL_SPLIT, any orders, m, n, k > 0, k % 8 == 0, m % 8 == 0 when A
 * is column-major, n % 8 == 0 when B is row-major, lda % 8 == 0,
 * ldb % 8 == 0, buffers within 4 GiB (128 rows of lda / ldb; k rows for a
 * column-major A or row-major B; 64 rows of ldc) — and 0 otherwise (then
 * gemm_split_fp32_ws runs the split-on-load kernel, which needs none).  m and
 * n need not be multiples of the 128 x 128 tile, nor k of its 64-deep slab.
 * MFL_EINVAL on NULL or unknown orders / modes, MFL_EOVERFLOW if the size
 * does not fit int64. */
MFL_API int gemm_split_fp32_workspace_bytes(int64_t m, int64_t n, int64_t k, int64_t lda, int order_a,
                                            int mode_a, int64_t ldb, int order_b, int mode_b, int64_t ldc,
                                            int64_t *bytes);

/* gemm_split_fp32 with a caller workspace (device memory, 256-byte aligned,
 * at least gemm_split_fp32_workspace_bytes; owned by the caller, contents
 * overwritten): when the planes path applies, each operand is split once into
 * hi and lo planes in the workspace (Strata PR #800, "What's going on": the hi
 * and lo halves) and the GEMM streams the planes; otherwise it is exactly
 * gemm_split_fp32 and the workspace is not touched.  Same arguments, result
 * and errors as gemm_split_fp32, plus MFL_EINVAL for a missing, misaligned or
 * short workspace.  The two kernels issue the same MFMAs in the same order per
 * accumulator, so their results are bit-identical. */
MFL_API int gemm_split_fp32_ws(int piece, int64_t m, int64_t n, int64_t k,
                    const float *a, int64_t lda, int order_a, int mode_a,
                    const float *b, int64_t ldb, int order_b, int mode_b,
                    int chains, int lolo, float *c, int64_t ldc, int accumulate,
                    void *workspace, int64_t workspace_bytes, void *stream);

/* gemm_tile_mma with an explicit MFMA instruction for the fast path
 * (MFL_MFMA_16X16X32 or MFL_MFMA_32X32X16); gemm_tile_mma uses 16x16x32.  The
 * generic path (k not a multiple of 8, a k-major operand whose m or n is not a
 * multiple of 8, or buffers past 4 GiB) always uses 16x16x32. */
MFL_API int gemm_tile_mma_shape(int shape, int dtype, int64_t m, int64_t n, int64_t k,
                                const void *a, int64_t lda, int order_a,
                                const void *b, int64_t ldb, int order_b,
                                float *c, int64_t ldc, int accumulate, void *stream);

/* Bytes of device workspace attention_split_fp32 needs for these sizes and
 * `algo`. */
MFL_API int attention_workspace_bytes(int64_t nq, int64_t nk, int64_t d, int algo, int64_t *bytes);

/* Attention-shaped pair of split GEMMs, one head (Strata PR #800): q (nq x d),
 * k and v (nk x d), o (nq x d), all fp32 row-major with ld = d.
 *   S = Q K^T with Q split into f16 hi/lo and K rounded once to f16;
 *   m = rowmax S, P~ = exp(S - m), l = rowsum P~ (fp32);
 *   O = (P~ V) / l with P~ split into f16 hi/lo and V rounded once to f16.
 * `chains` (1 or 2) selects single-chain or separate hi/lo accumulators for
 * both products.  No causal mask and no 1/sqrt(d) scaling are applied.
 *   algo 0: S materialised in the workspace: scores per 128 queries and key
 *           slice, which also keep each slice's row maxima; P~ V per key
 *           slice, forming P~ from S and the row maximum as it is loaded and
 *           summing it per row; a fixed-order reduce of the slices' partial O
 *           and row sums;
 *   algo 1: fused — per 128 queries and key slice, both products and an online
 *           softmax (running max, rescaled accumulators) stay in registers and
 *           LDS; key slices are merged by their exp(m_s - m) weights;
 *   algo 2: fused, and K and V are split into f16 hi/lo as well (each product
 *           then has the three terms hi*hi, hi*lo, lo*hi; with chains = 2 the
 *           two corrections share the second chain), so every operand enters
 *           at fp32-input accuracy instead of K and V being rounded once.
 * Supported: d = 128, nq and nk multiples of 128, and for algo 1 and 2
 * nk < 2^24 (the fused kernel's 32-bit buffer extent); others return
 * MFL_EUNSUPPORTED.  `workspace` is device memory
 * of at least attention_workspace_bytes(..., algo) bytes, 256-byte aligned. */
MFL_API int attention_split_fp32(int64_t nq, int64_t nk, int64_t d, const float *q, const float *k,
                                 const float *v, int chains, int algo, float *o, void *workspace,
                                 int64_t workspace_bytes, void *stream);

/* attention_split_fp32 without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture that may not call
 * hipMalloc, serving loops that forbid allocation, harnesses without an
 * allocator): same arguments, algorithms, kernels and results (bit for bit) as
 * attention_split_fp32, and the call allocates nothing.  The workspace is a
 * static device array of MFL_ATTN_STATIC_SCRATCH_BYTES that the library holds
 * on every GPU it runs on until the process ends; the first call on a device
 * looks up that device's copy (hipGetSymbolAddress), later calls reuse it.
 * The copy used is the current device's (hipGetDevice at the call), so the
 * stream and every pointer must belong to that device.
 * Calls whose attention_workspace_bytes exceeds the array return MFL_ESCRATCH
 * before any device work: 64 MiB holds algo 1 (32.3 MiB) and algo 2 (48.3 MiB)
 * at 2048 queries x 32768 keys, while algo 0, which materialises the nq x nk
 * scores, fits only small sizes.  Every call on a GPU shares that GPU's array, and the
 * array keeps the last call's contents (no call relies on them: every step
 * writes its part of the workspace before reading it); calls that overlap on
 * one GPU — on different streams, or from different host threads — race. */
#define MFL_ATTN_STATIC_SCRATCH_BYTES ((int64_t)64 << 20)
MFL_API int attention_split_fp32_static(int64_t nq, int64_t nk, int64_t d, const float *q, const float *k,
                                        const float *v, int chains, int algo, float *o, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MFL_H */
