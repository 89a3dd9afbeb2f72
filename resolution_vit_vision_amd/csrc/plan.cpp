// Launch-shape decisions of the matrix products and attention: pure host
// arithmetic on the problem sizes, kept apart from the kernels so the host
// orchestration can be built and checked without device code.
#include <stdint.h>

#include "qv_internal.h"

namespace qv {

int attention_bf16_rows_per_wg(int64_t wgs_at_128) {
  // 128 query rows per workgroup when that alone gives a workgroup per CU,
  // else 64 (the key split doubles the workgroups)
  return wgs_at_128 >= 256 ? 128 : 64;
}

// Split-K for narrow outputs at small M: 128x160 tiles (warp-specialized)
// with the K range cut into `splits` runs, one workgroup per (tile, run),
// so the grid fills the 256 CUs where the plain tiling has 64 tiles.
int gemm_splitk_runs(int M, int N, int K) {
  if (N % 160 || K % 64) return 1;
  const int64_t tiles = (int64_t)((M + 127) / 128) * (N / 160);
  for (int s : {4, 2}) {
    const int kt = K / 64 / s;
    if ((K / 64) % s == 0 && tiles * s <= 256 && (kt == 20 || kt == 40)) return s;
  }
  return 1;
}

// Split-K for a product whose output alone leaves most CUs idle (the
// merger's two Linears at small M): 128 x 160 tiles when N allows, else
// 128 x 128; the float32 partial sums are reduced by launch_splitk_reduce.
int gemm_splitk_any_runs(int M, int N, int K) {
  if (K % 64) return 1;
  const int kt = K / 64;
  const int64_t mt = (M + 127) / 128;
  if (N % 160 == 0) {
    for (int s : {4, 2})
      if (kt % s == 0 && mt * (N / 160) * s <= 256 && (kt / s == 20 || kt / s == 40)) return s;
    return 1;
  }
  if (N % 128 == 0) {
    for (int s : {8, 4, 2})
      if (kt % s == 0 && mt * (N / 128) * s <= 256 && (kt / s == 10 || kt / s == 20 || kt / s == 40)) return s;
  }
  return 1;
}

// K runs for an int8-weight GEMM of N = 1280 (1 = no split): the largest of
// 4 and 2 whose workgroups still fit one per CU.
int gemm_i8w_runs(int M, int N, int K) {
  if (N % 160 || K % 64) return 1;
  const int64_t tiles = (int64_t)((M + 127) / 128) * (N / 160);
  const int kt = K / 64;
  for (int s : {4, 2})
    if (tiles * s <= 256 && kt % s == 0 && (kt / s == 20 || kt / s == 10 || kt / s == 5)) return s;
  return 1;
}

bool gemm_i8w_wide(int M, int N) {
  return (int64_t)((M + 255) / 256) * ((N + 255) / 256) >= 160;  // the bf16 rule in run_pipe
}

}  // namespace qv
