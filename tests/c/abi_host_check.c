/* Host-only use of libmfl.so from plain C99 through include/mfl.h: the layout
 * calls over every point (each map a bijection, decode its inverse), overflow
 * and argument errors, workspace sizes.  No device call is made, so it runs
 * without a GPU.  Exit status 0 on success; the first failure is printed. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "mfl.h"

#define CHECK(cond)                                                        \
  do {                                                                     \
    if (!(cond)) {                                                         \
      fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #cond); \
      return 1;                                                            \
    }                                                                      \
  } while (0)

static int check_acc(int shape) {
  int lanes, per_lane, rows, cols;
  CHECK(mfl_acc_info(shape, &lanes, &per_lane, &rows, &cols) == MFL_OK);
  CHECK(lanes * per_lane == rows * cols && rows * cols <= 1024);
  static int own[1024];
  memset(own, 0, sizeof own);
  for (int l = 0; l < lanes; ++l)
    for (int j = 0; j < per_lane; ++j) {
      int r, c, off, l2, j2;
      CHECK(acc_coords(shape, l, j, &r, &c) == MFL_OK);
      CHECK(r >= 0 && r < rows && c >= 0 && c < cols);
      own[r * cols + c]++;
      CHECK(acc_offset(shape, l, j, &off) == MFL_OK && off == r * cols + c);
      CHECK(acc_decode(shape, off, &l2, &j2) == MFL_OK && l2 == l && j2 == j);
    }
  for (int i = 0; i < rows * cols; ++i) CHECK(own[i] == 1);
  int64_t out;
  CHECK(acc_matrix_offset(shape, lanes - 1, per_lane - 1, 0, cols, 2 * cols - 1, &out) == MFL_EOVERFLOW);
  CHECK(acc_matrix_offset(shape, 0, 0, (int64_t)1 << 62, 0, 4, &out) == MFL_EOVERFLOW);
  CHECK(acc_coords(shape, lanes, 0, &rows, &cols) == MFL_EINVAL);
  return 0;
}

static int check_operand(int shape, int operand) {
  int lanes, per_lane, rows, cols;
  CHECK(mfl_operand_info(shape, operand, &lanes, &per_lane, &rows, &cols) == MFL_OK);
  CHECK(lanes == 64 && per_lane == 8 && rows * cols == 512);
  static int own[512];
  memset(own, 0, sizeof own);
  for (int l = 0; l < lanes; ++l)
    for (int i = 0; i < per_lane; ++i) {
      int r, c, off, l2, i2;
      CHECK(operand_coords(shape, operand, l, i, &r, &c) == MFL_OK);
      CHECK(r >= 0 && r < rows && c >= 0 && c < cols);
      own[r * cols + c]++;
      CHECK(operand_offset(shape, operand, l, i, &off) == MFL_OK);
      CHECK(operand_decode(shape, operand, off, &l2, &i2) == MFL_OK && l2 == l && i2 == i);
      int64_t row_major, col_major;
      CHECK(operand_matrix_offset(shape, operand, l, i, 3, 5, 1000, MFL_ROW_MAJOR, &row_major) == MFL_OK);
      CHECK(operand_matrix_offset(shape, operand, l, i, 3, 5, 1000, MFL_COL_MAJOR, &col_major) == MFL_OK);
      CHECK(row_major == (int64_t)(3 + r) * 1000 + 5 + c && col_major == (int64_t)(5 + c) * 1000 + 3 + r);
    }
  for (int i = 0; i < rows * cols; ++i) CHECK(own[i] == 1);
  return 0;
}

int main(void) {
  CHECK(mfl_version() >= 100);
  CHECK(strcmp(mfl_status_string(MFL_OK), "MFL_OK") == 0);
  for (int shape = MFL_MFMA_16X16X32; shape <= MFL_MFMA_32X32X16; ++shape) {
    if (check_acc(shape)) return 1;
    if (check_operand(shape, MFL_OPERAND_A) || check_operand(shape, MFL_OPERAND_B)) return 1;
  }
  int64_t bytes = -1;
  CHECK(attention_workspace_bytes(2048, 32768, 128, 1, &bytes) == MFL_OK && bytes > 0);
  CHECK(attention_workspace_bytes(2048, 32768, 96, 1, &bytes) == MFL_EUNSUPPORTED);
  CHECK(gemm_split_fp32_workspace_bytes(4096, 4096, 4096, 4096, MFL_ROW_MAJOR, MFL_SPLIT, 4096, MFL_COL_MAJOR,
                                        MFL_SPLIT, 4096, &bytes) == MFL_OK &&
        bytes == (int64_t)4 * 4096 * 4096 * 2);
  /* a device entry point rejects bad arguments before any device call */
  CHECK(gemm_tile_mma(7, 64, 64, 64, NULL, 64, MFL_ROW_MAJOR, NULL, 64, MFL_COL_MAJOR, NULL, 64, 0, NULL) ==
        MFL_EINVAL);
  printf("abi_host_check: ok\n");
  return 0;
}
