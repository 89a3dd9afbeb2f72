// Internal interfaces between the host orchestration and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <stddef.h>
#include <stdint.h>

namespace qv {

// Launch timing (diagnostics): while a launch class is being timed, the host
// points g_launch_timing at an event pair and every kernel launch of that
// class goes through hipExtLaunchKernelGGL, whose events take the dispatch's
// own begin / end timestamps (the first launch records `start`, every launch
// re-records `stop`).  Otherwise a plain launch.
struct LaunchTiming {
  hipEvent_t start;
  hipEvent_t stop;
  bool started;
};
extern thread_local LaunchTiming* g_launch_timing;

#define QV_KLAUNCH(kernel, grid, block, shm, stream, ...)                                                   \
  do {                                                                                                      \
    ::qv::LaunchTiming* t_ = ::qv::g_launch_timing;                                                         \
    if (t_) {                                                                                               \
      hipExtLaunchKernelGGL(kernel, grid, block, shm, stream, t_->started ? nullptr : t_->start, t_->stop, 0, \
                            __VA_ARGS__);                                                                   \
      t_->started = true;                                                                                   \
    } else {                                                                                                \
      hipLaunchKernelGGL(kernel, grid, block, shm, stream, __VA_ARGS__);                                    \
    }                                                                                                       \
  } while (0)


constexpr int kHeadDim = 80;       // attention kernels are written for 80-wide heads
constexpr int kRopeFreqs = kHeadDim / 4;
constexpr int kSeqAlign = 128;     // each image's rows in Q/K/V^T start on this multiple

// Per-image description computed on the host from grid_thw.
struct ImgDesc {
  int32_t row0;   // first packed row (cu_seqlens[i])
  int32_t n;      // patches T*gh*gw
  int32_t t, gh, gw;
  int32_t prow0;  // first row in the padded attention layout
  int32_t wbase;  // windowed attention: global index of the image's first window
  int32_t nwy, nwx;  // windows per frame along h and w
};

constexpr int kDescChunk = 32;
constexpr int kPlanChunk = 128;  // plan entries per setup launch (2 KB of kernel arguments)
struct DescChunk {
  int32_t count;
  int32_t first;  // index of d[0] in the full list
  ImgDesc d[kDescChunk];
};

// One entry of the attention work plan, segments sorted by length, longest
// first.  A segment is an image (packed rows row0 .. row0 + n, taken from
// the host's grid list, never from the caller's device cu_seqlens) or, for
// windowed blocks, one window (output rows through the out_row map).
struct PlanEntry {
  int32_t row0;       // image plans: first packed row; window plans: window index
  int32_t prow0;      // padded row start
  int32_t qtile0;     // first global q-tile of this segment
  int32_t n;          // rows of the segment (patches of the image, or of the window)
};

// Patchify: one image per chunk entry.
struct PatchImg {
  int64_t offset;
  int32_t frames, channels, height, width;
  int32_t t, gh, gw, row0;
};
constexpr int kPatchChunk = 16;
struct PatchChunk {
  int32_t count;
  PatchImg d[kPatchChunk];
};

enum class Act : int { None = 0, QuickGelu = 1, GeluErf = 2 };

// ---- launchers (return hipGetLastError()) ----
// Pixel transform and row shape of the patch gather.
struct PatchMode {
  int32_t fold;        // 1: one temporal slot (still images), rows C*patch^2 wide
  int32_t normalize;   // 1: (x - mean[c]) / std[c]
  int32_t width;       // elements written per row (zero beyond the patch vector)
  int32_t reserved;
  float mean[4], stdv[4];
};
hipError_t launch_fold_weight(const void* w, int dim, int channels, int patch, int temporal, int ld_in, void* out,
                              int ld_out, bool bf16, hipStream_t s);
hipError_t launch_patchify(const float* pixels, const PatchChunk& c, int patch, int temporal, void* out,
                           bool bf16, int ld, const PatchMode& m, int64_t rows_in_chunk_max, hipStream_t s);

hipError_t launch_setup_tokens(const DescChunk& c, int2* tokinfo, hipStream_t s);
// windowed attention: tokinfo_w[row] = {h | w << 16, padded row in the window
// layout (window index * kSeqAlign + place in the window)} and
// out_row[padded row] = packed row, for windows of `window` patches
hipError_t launch_setup_windows(const DescChunk& c, int window, int slot, int2* tokinfo_w, int32_t* out_row,
                                hipStream_t s);
hipError_t launch_setup_plan(const PlanEntry* host_plan_chunk, int count, int first, PlanEntry* plan,
                             hipStream_t s);
hipError_t launch_rope_table(float2* tab, int positions, float theta, hipStream_t s);
hipError_t launch_zero(void* p, size_t bytes, hipStream_t s);

// Static device workspace of the allocation-free forward: its device address
// on the current device (looked up once per device, then cached).
hipError_t scratch_buffer(void** ptr);

// Bytes a LayerNorm of few rows reads beside its rows, to bring the weight
// matrix of a later product into the Infinity Cache before that product
// runs (nothing is written; null / 0: none).
struct CacheWarm {
  const void* p = nullptr;
  size_t bytes = 0;
};
hipError_t launch_layernorm(const float* x, const float* g, const float* b, void* y, bool bf16, int rows,
                            int dim, float eps, hipStream_t s, CacheWarm warm = {});

// K of the bf16 path is stored key-tiled and chunk-major per head:
// [head][P / 32][10 chunks of 8 dims][32 keys][8 dims], so the 32 key rows an
// attention wave multiplies are, chunk by chunk, 32 consecutive 16-byte slots
// (conflict-free LDS reads), and a run of keys is one contiguous block of
// memory (whole-KB LDS-DMA copies).  Element offset of (head, key, dim):
__host__ __device__ __forceinline__ size_t kc_offset(int head, int P, int key, int d) {
  return ((((size_t)head * (P / 32) + (key >> 5)) * (kHeadDim / 8) + (d >> 3)) * 32 + (key & 31)) * 8 + (d & 7);
}

// C = A . B^T with an epilogue (bf16 operands, MFMA).
struct QkvOut {
  void* q;         // [heads][P][80]
  void* k;         // bf16: key-tiled (kc_offset); f32: [heads][P][80]
  void* vt;        // [heads][80][P]
  const int2* tokinfo;
  const float2* rope;  // [positions][20] (cos, sin)
  int P;           // padded rows
  int dim;         // q/k/v width (heads*80)
};

hipError_t gemm_bf16_store_f32(const void* A, int lda, const void* B, int ldb, int M, int N, int K,
                               const float* bias, float* C, int ldc, hipStream_t s);
hipError_t gemm_bf16_resid_f32(const void* A, int lda, const void* B, int ldb, int M, int N, int K,
                               const float* bias, float* Z, int ldz, hipStream_t s);
// int8 weights (one float32 scale per weight row), bf16 activations.
hipError_t gemm_i8w_qkv(const void* A, int lda, const int8_t* B, int ldb, const float* scale, int M, int K,
                        const float* bias, const QkvOut& o, hipStream_t s);
hipError_t gemm_i8w_act_bf16(const void* A, int lda, const int8_t* B, int ldb, const float* scale, int M, int N,
                             int K, const float* bias, Act act, void* C, int ldc, hipStream_t s);
int gemm_i8w_runs(int M, int N, int K);
hipError_t gemm_i8w_splitk_bf16(const void* A, int lda, const int8_t* B, int ldb, const float* scale, int M, int N,
                                int K, int splits, uint16_t* P, hipStream_t s);
hipError_t gemm_i8w_resid_f32(const void* A, int lda, const int8_t* B, int ldb, const float* scale, int M, int N,
                              int K, const float* bias, float* Z, int ldz, hipStream_t s);
hipError_t launch_quantize_i8(const void* w, int rows, int cols, int ld, bool bf16, int8_t* q, float* scale,
                              hipStream_t s);
// Large M (gemm_i8w_wide): codes widened to bf16 by launch_codes_bf16, then
// the 256 x 256 bf16 kernel with the row scales applied to the sums.
bool gemm_i8w_wide(int M, int N);
hipError_t launch_codes_bf16(const int8_t* q, int64_t n, void* out, hipStream_t s);
hipError_t gemm_i8w_wide_qkv(const void* A, int lda, const void* codes, int ldb, const float* scale, int M, int K,
                             const float* bias, const QkvOut& o, hipStream_t s);
hipError_t gemm_i8w_wide_act_bf16(const void* A, int lda, const void* codes, int ldb, const float* scale, int M,
                                  int N, int K, const float* bias, Act act, void* C, int ldc, hipStream_t s);
hipError_t gemm_i8w_wide_resid_f32(const void* A, int lda, const void* codes, int ldb, const float* scale, int M,
                                   int N, int K, const float* bias, float* Z, int ldz, hipStream_t s);
// Split-K with the reduction left to launch_layernorm_acc: returns the number
// of K runs that fills the GPU for this shape (1 = no split).
int gemm_splitk_runs(int M, int N, int K);
// Split-K for the merger's Linears at small M (any N that is a multiple of 128
// or 160), with the reduction, bias and activation in launch_splitk_reduce.
int gemm_splitk_any_runs(int M, int N, int K);
hipError_t gemm_bf16_splitk_any_f32(const void* A, int lda, const void* B, int ldb, int M, int N, int K, int splits,
                                    float* P, hipStream_t s);
hipError_t launch_splitk_reduce(const float* P, int splits, size_t stride, const float* bias, Act act, void* out,
                                int ldo, int M, int N, hipStream_t s);
// P[s][M][N] = A[:, s K/S .. (s+1) K/S) . B[:, same]^T, float32, no bias.
hipError_t gemm_bf16_splitk_f32(const void* A, int lda, const void* B, int ldb, int M, int N, int K, int splits,
                                float* P, hipStream_t s);
// The same with each run's sums rounded to bf16 (the tower's fc2).
hipError_t gemm_bf16_splitk_bf16(const void* A, int lda, const void* B, int ldb, int M, int N, int K, int splits,
                                 uint16_t* P, hipStream_t s);
// x += sum_s parts[s] + pb (bf16 partial rows widened to float32, added in
// that order); y = LN(x) if g is non-null.
hipError_t launch_layernorm_acc(float* x, const uint16_t* parts, size_t part_stride, int splits, const float* pb,
                                const float* g, const float* b, void* y, bool bf16, int rows, int dim, float eps,
                                hipStream_t s, CacheWarm warm = {});
hipError_t gemm_bf16_act_bf16(const void* A, int lda, const void* B, int ldb, int M, int N, int K,
                              const float* bias, Act act, void* C, int ldc, hipStream_t s);
hipError_t gemm_bf16_qkv(const void* A, int lda, const void* B, int ldb, int M, int K, const float* bias,
                         const QkvOut& o, hipStream_t s);

// float32 counterparts (correctness mode).
hipError_t gemm_f32_store(const float* A, int lda, const float* B, int ldb, int M, int N, int K,
                          const float* bias, float* C, int ldc, hipStream_t s);
hipError_t gemm_f32_resid(const float* A, int lda, const float* B, int ldb, int M, int N, int K,
                          const float* bias, float* Z, int ldz, hipStream_t s);
hipError_t gemm_f32_act(const float* A, int lda, const float* B, int ldb, int M, int N, int K,
                        const float* bias, Act act, float* C, int ldc, hipStream_t s);
hipError_t rope_scatter_f32(const float* qkv, int M, const float* bias_unused, const QkvOut& o,
                            hipStream_t s);

// Varlen attention over the padded layout; O packed [N][ldo].
struct AttnArgs {
  const void* q;
  const void* k;
  const void* vt;
  void* o;
  int ldo;
  const PlanEntry* plan;
  int n_img;                 // plan entries (images or windows)
  const int32_t* out_row;    // null: segments are images; else window plan, packed row of each padded row
  int P;
  int heads;
  int total_qtiles;
  int rows_per_wg;   // query rows per workgroup of the bf16 kernel (128, 64 or 32)
};
hipError_t attention_bf16(const AttnArgs& a, hipStream_t s);
// Windows of at most kWinSlot patches, each in a kWinSlot-row slot; plan in
// window order (entry i = window i), out_row required.
constexpr int kWinSlot = 64;
hipError_t attention_bf16_windows(const AttnArgs& a, hipStream_t s);
hipError_t attention_f32(const AttnArgs& a, hipStream_t s);
int attention_bf16_rows_per_wg(int64_t wgs_at_128);
constexpr int kAttnBQ_f32 = 64;

}  // namespace qv
