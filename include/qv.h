/*
 * qv.h - C ABI of the native-resolution ViT vision encoder for MI355X (gfx950).
 *
 * The encoder is the Qwen2-VL vision tower: images are smart-resized onto a
 * 28-pixel lattice, cut into 2x14x14x3 temporal patches listed so that every
 * 2x2 merge group is contiguous, projected 1176 -> 1280, run through pre-norm
 * rotary ViT blocks with full attention inside each image of a packed batch,
 * and folded 2x2 by the PatchMerger to the decoder width.
 * Sources (page title, section):
 *   - Qwen2-VL ZeroModels docs: intro (smart resize, image_grid_thw),
 *     Qwen2VLVisionModel and Qwen2VLImageProcessor argument tables;
 *   - Neurarch "Qwen2-VL (Native-Resolution VLM)" card: Structure table and the
 *     exported PatchMerger module;
 *   - Qwen2.5-VL-7B-Instruct record: VISION TOKENS (tokens = pixels / 784,
 *     budget 3,136 .. 12,845,056 pixels);
 *   - Qwen2-VL-2B LiteRT-LM card: Vision/Adapter rows and Conversion notes
 *     (packed patches with cu_seqlens, 2-D rope, Conv3d patch-embed with a
 *     duplicated still frame, the 2x2-block order of the merger).
 *
 * Conventions shared by every entry point
 *   - All calls return a qv_status.  Arguments are validated on the host
 *     before anything is enqueued: on a validation error (every status but
 *     QV_ERR_HIP) nothing was launched and no output was written.
 *     QV_ERR_HIP reports a failed launch or runtime call; work enqueued
 *     before it stays enqueued.  qv_last_error() gives a short text for the
 *     calling thread.
 *   - Device entry points are asynchronous and ordered on `stream` (a
 *     hipStream_t passed as void*; NULL is the default stream).  Inputs must
 *     stay valid, and outputs must not be read, until the caller has
 *     synchronised with that stream.
 *   - "host" pointers are read during the call only.  "device" pointers are
 *     HIP device allocations owned by the caller; the library never allocates
 *     or frees device memory in these calls and keeps no pointer after return.
 *   - Matrices are row-major.  Linear weights use the [out][in] layout;
 *     vectors (biases, LayerNorm gain/shift) are float32 in both dtypes.
 *   - Device faults surface at the caller's next synchronisation, as in any
 *     HIP library.
 *   - Calls that overlap on the same workspace race; use one workspace per
 *     stream.
 */
#ifndef QV_H
#define QV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QV_ABI_VERSION 4

typedef enum qv_status {
  QV_OK = 0,
  QV_ERR_NULL = 1,        /* a required pointer is NULL                         */
  QV_ERR_SHAPE = 2,       /* sizes inconsistent (odd grid, image != 14 * grid...) */
  QV_ERR_BUDGET = 3,      /* no lattice size inside [min_pixels, max_pixels]    */
  QV_ERR_WORKSPACE = 4,   /* workspace smaller than the *_workspace_size value  */
  QV_ERR_UNSUPPORTED = 5, /* a configuration the kernels do not implement       */
  QV_ERR_HIP = 6          /* a HIP runtime call or launch failed                */
} qv_status;

/* Element types.  qv_dtype is a plain 32-bit integer so that any value a
 * caller passes is well defined on the library side and an unknown one is
 * rejected with QV_ERR_UNSUPPORTED. */
typedef int32_t qv_dtype;
enum {
  QV_F32 = 0,  /* float32 operands and activations (correctness mode)         */
  QV_BF16 = 1, /* bf16 GEMM/attention operands, float32 accumulation,
                  residual stream, LayerNorm statistics and softmax            */
  QV_I8 = 2    /* weight format only: int8 codes [rows][cols] with one float32
                  scale per row (qv_quantize_i8)                               */
};

/* Text of the last non-OK status returned on the calling thread ("" if none). */
const char *qv_last_error(void);

/* QV_ABI_VERSION of the loaded library. */
int32_t qv_abi_version(void);

/* ------------------------------------------------------------------ grid */

/* Lattice parameters of the image processor (ZeroModels docs,
 * Qwen2VLImageProcessor table; Qwen2.5-VL-7B record, VISION TOKENS).
 * Defaults: patch 14, merge 2, temporal 2, min 3136, max 12845056. */
typedef struct qv_grid_params {
  int32_t patch;      /* patch side in pixels                       */
  int32_t merge;      /* spatial merge factor (2)                    */
  int32_t temporal;   /* frames per temporal patch (2)               */
  int32_t reserved;   /* must be 0                                   */
  int64_t min_pixels; /* smallest allowed H'W'                       */
  int64_t max_pixels; /* largest allowed H'W'                        */
} qv_grid_params;

/* Fill *p with the defaults above.  p: host, non-NULL. */
void qv_grid_params_default(qv_grid_params *p);

/* Smart resize: picks H', W' (multiples of f = patch*merge) for an image of
 * height x width pixels and `frames` frames, and its grid (T, H'/patch,
 * W'/patch) with T = ceil(frames / temporal).  Rule (the pages fix only the
 * constraints): each side to the nearest multiple of f, ties to even, at
 * least f; if H'W' > max_pixels both sides become
 * max(f, f*floor(side / (beta*f))) with beta = sqrt(height*width/max_pixels);
 * if H'W' < min_pixels both become f*ceil(side*beta/f) with
 * beta = sqrt(min_pixels/(height*width)).  Integer arithmetic plus IEEE
 * double in the rescale, in exactly that order.
 * Host only.  p may be NULL (defaults).  out_height/out_width may be NULL;
 * out_grid_thw (3 int32) must not be.
 * Errors: QV_ERR_SHAPE for non-positive sizes or frames, QV_ERR_BUDGET when
 * the result lies outside [min_pixels, max_pixels] (extreme aspect ratios). */
qv_status qv_smart_resize_grid(int64_t height, int64_t width, int32_t frames,
                               const qv_grid_params *p, int64_t *out_height,
                               int64_t *out_width, int32_t out_grid_thw[3]);

/* Sequence metadata of a packed batch (LiteRT-LM card, Conversion notes).
 * grid_thw: host [n_img][3] (T, gh, gw), gh and gw multiples of `merge`.
 * cu_seqlens: host out [n_img + 1]: 0, n_0, n_0 + n_1, ... (n_i = T gh gw).
 * pos_hw: host out [N][2] or NULL: (h, w) patch coordinates of each slot.
 * perm: host out [N] or NULL: raster index t*gh*gw + h*gw + w of each slot
 *   inside its image.  Slots enumerate (t, block row, block col, dy, dx) with
 *   dx fastest, so each merge x merge group is contiguous.
 * Errors: QV_ERR_NULL, QV_ERR_SHAPE (non-positive or non-multiple sizes,
 * total over INT32_MAX). */
qv_status qv_seq_meta(const int32_t *grid_thw, int32_t n_img, int32_t merge,
                      int32_t *cu_seqlens, int32_t *pos_hw, int32_t *perm);

/* -------------------------------------------------------------- patchify */

/* One image inside a device pixel buffer: float32 pixels at
 * pixels[offset + ((f*channels + c)*height + y)*width + x]. */
typedef struct qv_image {
  int64_t offset;
  int32_t frames, channels, height, width;
  int32_t reserved; /* must be 0 */
} qv_image;

/* Cut images into temporal patches in merge-group order (LiteRT-LM card,
 * Conversion notes: Conv3d patch-embed with the still frame duplicated; the
 * merger's 2x2-block order).  Row s of image i (rows cu_i .. cu_i + n_i) is
 * the patch at slot s (see qv_seq_meta); its element
 * ((c*temporal + tau)*patch + r)*patch + q is pixel
 * frame[min(temporal*t + tau, frames-1)][c][patch*h + r][patch*w + q].
 * pixels: device float32.  images, grid_thw: host [n_img].  p: host or NULL.
 * patches: device out [N][ld] in out_dtype (QV_BF16: round to nearest even;
 * QV_F32: copy).  ld >= channels*temporal*patch^2 and a multiple of 8;
 * columns beyond that width are not written.
 * Errors: QV_ERR_NULL; QV_ERR_SHAPE unless height == patch*gh,
 * width == patch*gw, T == ceil(frames/temporal), gh, gw multiples of merge
 * (no resampling happens here); QV_ERR_UNSUPPORTED for merge != 2 or
 * patch*patch*channels*temporal not a multiple of 8; QV_ERR_HIP. */
qv_status qv_patchify(const float *pixels, const qv_image *images, int32_t n_img,
                      const int32_t *grid_thw, const qv_grid_params *p, void *patches,
                      qv_dtype out_dtype, int32_t ld, void *stream);

/* Options of qv_patchify_ex.
 * fold: still images (every image has one frame, so T == 1) only.  The
 *   duplicated frame is folded into the weight (LiteRT-LM card, Conversion
 *   notes: Conv3d -> Conv2d fold): row element (c*patch + r)*patch + q is
 *   pixel frame[0][c][patch*h + r][patch*w + q], width channels*patch^2
 *   (588), then zeros up to the next multiple of 8 (592).  Pair it with a
 *   weight from qv_fold_patch_weight and qv_vision_cfg.patch_dim = 592.
 * normalize: each pixel becomes (x - mean[c]) / std[c] in float32 (one
 *   subtraction, one correctly rounded division) before the cast (ZeroModels
 *   docs, Qwen2VLImageProcessor table: image_mean, image_std; the CLIP values
 *   are QV_CLIP_MEAN / QV_CLIP_STD).  At most 4 channels; std > 0. */
typedef struct qv_patch_opts {
  int32_t fold;       /* 0 or 1 */
  int32_t normalize;  /* 0 or 1 */
  float mean[4];
  float std[4];
} qv_patch_opts;

#define QV_CLIP_MEAN {0.48145466f, 0.4578275f, 0.40821073f, 0.0f}
#define QV_CLIP_STD {0.26862954f, 0.26130258f, 0.27577711f, 1.0f}

/* qv_patchify with options (opts NULL = qv_patchify).  Same arguments,
 * layout and errors as qv_patchify; with fold, ld >= round_up(channels *
 * patch^2, 8) and the pad columns up to that width are written as zeros.
 * Extra errors: QV_ERR_SHAPE for fold with an image of more than one frame;
 * QV_ERR_UNSUPPORTED for normalize with more than 4 channels or a std <= 0
 * (or NaN), or flags other than 0/1. */
qv_status qv_patchify_ex(const float *pixels, const qv_image *images, int32_t n_img,
                         const int32_t *grid_thw, const qv_grid_params *p,
                         const qv_patch_opts *opts, void *patches, qv_dtype out_dtype,
                         int32_t ld, void *stream);

/* Fold a Conv3d patch-embed weight into the Conv2d weight of still images
 * (LiteRT-LM card, Conversion notes: Conv3d -> Conv2d fold).
 * w: device [dim][ld_in] in dtype, row = [channels][temporal][patch][patch];
 * out: device [dim][ld_out] in dtype, row element (c*patch + r)*patch + q =
 * sum over tau = 0..temporal-1 (in that order, float32) of
 * w[(c*temporal + tau)*patch + r)*patch + q], rounded to dtype (bf16: to
 * nearest even); columns channels*patch^2 .. ld_out-1 are zero.
 * ld_in >= channels*temporal*patch^2; ld_out >= channels*patch^2.
 * Errors: QV_ERR_NULL, QV_ERR_SHAPE (sizes), QV_ERR_UNSUPPORTED (dtype),
 * QV_ERR_HIP.  out must not overlap w. */
qv_status qv_fold_patch_weight(const void *w, int32_t dim, int32_t channels, int32_t patch,
                               int32_t temporal, int32_t ld_in, void *out, int32_t ld_out,
                               qv_dtype dtype, void *stream);

/* ---------------------------------------------------------- vision tower */

/* Device pointers of one block.  Matrices in the tower dtype (int8 when
 * qv_vision_cfg.weights is QV_I8), vectors f32.
 * qkv_w [3*dim][dim] rows = [q | k | v], each head-major (head h owns rows
 * 80h .. 80h+79 of its third); proj_w [dim][dim]; fc1_w [mlp][dim];
 * fc2_w [dim][mlp].  With int8 weights the matrices are dense int8 codes
 * (16-byte aligned) and qkv_s [3*dim], proj_s [dim], fc1_s [mlp],
 * fc2_s [dim] their float32 row scales (weight = code * scale of its row);
 * otherwise the four scale pointers are ignored and may be NULL. */
typedef struct qv_block_w {
  const void *ln1_w, *ln1_b, *qkv_w, *qkv_b, *proj_w, *proj_b;
  const void *ln2_w, *ln2_b, *fc1_w, *fc1_b, *fc2_w, *fc2_b;
  const float *qkv_s, *proj_s, *fc1_s, *fc2_s;
} qv_block_w;

/* patch_w: device [dim][patch_dim] (the Conv3d weight [dim][C][2][14][14]
 * flattened); patch_b: device [dim] f32 or NULL; blocks: host [depth]. */
typedef struct qv_vision_w {
  const void *patch_w;
  const void *patch_b;
  const qv_block_w *blocks;
} qv_vision_w;

typedef struct qv_vision_cfg {
  int32_t depth;      /* blocks to run (0 = patch-embed only)                  */
  int32_t dim;        /* width, 1280; a multiple of 256, at most 2048           */
  int32_t heads;      /* heads; dim / heads must be 80                          */
  int32_t mlp;        /* MLP width, 5120; a multiple of 64                      */
  int32_t patch_dim;  /* patch vector length, 1176; a multiple of 8             */
  int32_t ld;         /* row stride of `patches` in elements, >= patch_dim, %8  */
  int32_t merge;      /* 2                                                      */
  int32_t dtype;      /* qv_dtype                                               */
  float ln_eps;       /* 1e-6                                                   */
  float rope_theta;   /* 1e4                                                    */
  /* Windowed attention (Qwen2.5-VL-7B-Instruct record, TWO-PART MODEL: 112-px
   * windows, full attention only in four blocks).  window: side of a window
   * in patches, a positive multiple of merge and at most 10 (8 = 112 px);
   * windows tile each frame's patch grid from its top-left corner, edge
   * windows are truncated; 0 = every block attends over the whole image
   * (Qwen2-VL).  full_blocks: with window > 0, bit l set = block l attends
   * over the whole image (Qwen2.5-VL: bits 7, 15, 23, 31); blocks from 64
   * on are windowed.  full_blocks is ignored when window is 0.  Workspace:
   * every window gets a slot of 64 padded rows (W <= 8) or 128 (W = 10) in
   * the q/k/v layout, so small windows cost more q/k/v workspace than the
   * image layout (W = 8: none; W = 2: 16x). */
  int32_t window;
  /* Format of the four block matrices (LiteRT-LM card, model table, Vision
   * and Adapter rows: int8 weights): 0 = the tower dtype; QV_I8 = int8 codes
   * with a float32 scale per output row (qv_block_w).  An int8 product is
   * out[m][n] = scale[n] * sum_k a[m][k] * code[n][k]: bf16 activations
   * times the codes (exact in bf16), float32 accumulation, the scale applied
   * to the float32 sum.  QV_I8 needs dtype QV_BF16, dim 1280 and mlp 5120.
   * The patch-embed weight stays in the tower dtype. */
  int32_t weights;
  uint64_t full_blocks;
} qv_vision_cfg;

/* Bytes of device workspace qv_vision_forward needs for this grid list.
 * grid_thw: host [n_img][3].  Errors: QV_ERR_NULL, QV_ERR_SHAPE,
 * QV_ERR_UNSUPPORTED (also for a bf16 batch whose widest activation,
 * N x max(mlp, 3 dim) bf16, reaches 2 GiB: about 209,000 patches at width
 * 1280; split such a batch over several calls). */
qv_status qv_vision_workspace_size(const qv_vision_cfg *c, const int32_t *grid_thw,
                                   int32_t n_img, size_t *bytes);

/* Encoder forward over a packed batch (ZeroModels docs, Qwen2VLVisionModel:
 * patch-embed -> rotary blocks; LiteRT-LM card, Conversion notes: packed
 * patches, 2-D rope, cu_seqlens).
 *   hidden = patches . patch_w^T (+ patch_b); then per block
 *   a = LN1(hidden); [q|k|v] = a . qkv_w^T + qkv_b; q, k rotated by the 2-D
 *   rope of each patch's (h, w) (pair j couples elements j and j+40 of a
 *   head, pairs 0..19 turn by h * theta^(-j/20), pairs 20..39 by
 *   w * theta^(-(j-20)/20)); o = softmax(q k^T / sqrt(80)) v inside each image
 *   (inside each window in the windowed blocks, see qv_vision_cfg.window);
 *   hidden += o . proj_w^T + proj_b; a = LN2(hidden);
 *   hidden += QuickGELU(a . fc1_w^T + fc1_b) . fc2_w^T + fc2_b.
 * patches: device [N][ld] in cfg dtype, merge-group order (qv_patchify).
 * grid_thw: host [n_img][3].  cu_seqlens: device int32 [n_img + 1], the
 * prefix sums of T*gh*gw.  The kernels take every image's rows from
 * grid_thw, so a cu_seqlens that disagrees with it cannot move an access
 * out of bounds; set QV_DEBUG_VALIDATE=1 in the environment to have it
 * copied back and compared (QV_ERR_SHAPE on a mismatch; this synchronises).
 * hidden: device out float32 [N][dim] (the residual stream after the last
 * block, before the merger).  ws: device workspace of ws_bytes.
 * Errors: QV_ERR_NULL, QV_ERR_SHAPE, QV_ERR_UNSUPPORTED, QV_ERR_WORKSPACE,
 * QV_ERR_HIP. */
qv_status qv_vision_forward(const qv_vision_cfg *c, const qv_vision_w *w, const void *patches,
                            const int32_t *grid_thw, int32_t n_img, const int32_t *cu_seqlens,
                            float *hidden, void *ws, size_t ws_bytes, void *stream);

/* Size of the static device workspace behind qv_vision_forward_noalloc. */
#define QV_SCRATCH_BYTES ((size_t)64 << 20)

/* Encoder forward that allocates nothing, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Same computation, arguments, output and
 * errors as qv_vision_forward, without ws / ws_bytes: the workspace is a
 * static device array of QV_SCRATCH_BYTES (64 MiB) compiled into the
 * library, one copy on every GPU the library runs on, held until the process
 * ends.  A call whose qv_vision_workspace_size exceeds it returns
 * QV_ERR_WORKSPACE before anything is enqueued (a 448x448 image needs
 * 32.5 MiB, a 672x672 image 50.7 MiB; four packed 672x672 images do not
 * fit).  The array of the device current at the call is used, so `stream`
 * must belong to that device; its address is looked up on the first call on
 * each device.  Every call on one GPU shares that GPU's array and leaves its
 * own contents there; each call initialises everything it reads, so nothing
 * carries over, but two calls whose work overlaps on one GPU (two streams,
 * or two host threads) race on the array: serialise them.  No hipMalloc,
 * hipFree or other allocating call is made. */
qv_status qv_vision_forward_noalloc(const qv_vision_cfg *c, const qv_vision_w *w, const void *patches,
                                    const int32_t *grid_thw, int32_t n_img, const int32_t *cu_seqlens,
                                    float *hidden, void *stream);

/* Symmetric per-row int8 weights (LiteRT-LM card, model table, Vision and
 * Adapter rows: int8 weights; the grouping and rounding are this library's
 * choice): for each row r, in float32, scale[r] = max_c |w[r][c]| / 127
 * (1 when the row is all zeros) and q[r][c] = w[r][c] / scale[r] rounded
 * half to even and clamped to [-127, 127].
 * w: device [rows][ld] in dtype (QV_F32 or QV_BF16, read exactly);
 * q: device out int8 [rows][cols] (dense); scale: device out float32
 * [rows].  Errors: QV_ERR_NULL, QV_ERR_SHAPE (rows, cols <= 0 or
 * ld < cols), QV_ERR_UNSUPPORTED (dtype), QV_ERR_HIP.  Outputs must not
 * overlap w. */
qv_status qv_quantize_i8(const void *w, int32_t rows, int32_t cols, int32_t ld, qv_dtype dtype, int8_t *q,
                         float *scale, void *stream);

/* ---------------------------------------------------------- patch merger */

typedef struct qv_merger_cfg {
  int32_t dim;      /* encoder width, 1280 (a multiple of 256, <= 2048)        */
  int32_t merge;    /* 2: groups of merge^2 = 4 consecutive tokens              */
  int32_t hidden;   /* MLP width = dim * merge^2 = 5120                         */
  int32_t out_dim;  /* decoder width (1536, 3584)                               */
  int32_t dtype;    /* qv_dtype of weights, MLP operands and `out`             */
  float ln_eps;     /* 1e-6                                                     */
} qv_merger_cfg;

/* ln_w, ln_b: [dim] f32; fc1_w [hidden][hidden], fc1_b [hidden] f32;
 * fc2_w [out_dim][hidden], fc2_b [out_dim] f32 (all device). */
typedef struct qv_merger_w {
  const void *ln_w, *ln_b, *fc1_w, *fc1_b, *fc2_w, *fc2_b;
} qv_merger_w;

qv_status qv_merge_workspace_size(const qv_merger_cfg *c, int64_t n_tokens, size_t *bytes);

/* PatchMerger (Neurarch card, exported PatchMerger; LiteRT-LM card, Adapter
 * row): y = LN(hidden) per token; each run of merge^2 consecutive rows is
 * one row of width hidden; out = GELU_erf(y . fc1_w^T + fc1_b) . fc2_w^T +
 * fc2_b.  hidden: device float32 [n_tokens][dim]; out: device
 * [n_tokens / merge^2][out_dim] in cfg dtype.
 * Errors: QV_ERR_NULL; QV_ERR_SHAPE when n_tokens is not a positive multiple
 * of merge^2 or hidden != dim*merge^2; QV_ERR_UNSUPPORTED; QV_ERR_WORKSPACE;
 * QV_ERR_HIP. */
qv_status qv_patch_merge(const qv_merger_cfg *c, const qv_merger_w *w, const float *hidden,
                         int64_t n_tokens, void *out, void *ws, size_t ws_bytes, void *stream);

/* ------------------------------------------------------------ diagnostics */

/* Kernel classes the encoder launches, for the timing hooks below. */
typedef enum qv_kernel_class {
  QV_KC_PATCHIFY = 0,     /* patch gather / reorder                        */
  QV_KC_PATCH_EMBED = 1,  /* 1176 -> dim projection                        */
  QV_KC_LAYERNORM = 2,    /* every LayerNorm (two per block, one in merger) */
  QV_KC_QKV = 3,          /* q/k/v projection + bias + 2-D rope            */
  QV_KC_ATTENTION = 4,    /* varlen attention                              */
  QV_KC_PROJ = 5,         /* attention output projection + residual        */
  QV_KC_FC1 = 6,          /* MLP up-projection + QuickGELU                 */
  QV_KC_FC2 = 7,          /* MLP down-projection + residual                */
  QV_KC_MERGE_FC1 = 8,    /* merger Linear + GELU                          */
  QV_KC_MERGE_FC2 = 9,    /* merger output Linear                          */
  QV_KC_COUNT = 10
} qv_kernel_class;

/* Start recording a hipEvent pair on the launch stream around every launch of
 * kernel class `cls` made by later qv_* calls in this process.  Diagnostic
 * only: not thread-safe against concurrent qv_* calls from other threads.
 * Errors: QV_ERR_UNSUPPORTED for an unknown class; QV_ERR_HIP. */
qv_status qv_timing_start(int32_t cls);

/* Stop recording, wait for every recorded event, and return the summed
 * device time in milliseconds and the number of launches timed.
 * total_ms, launches: host, non-NULL.  Errors: QV_ERR_NULL, QV_ERR_HIP. */
qv_status qv_timing_stop(double *total_ms, int64_t *launches);

#ifdef __cplusplus
}
#endif

#endif /* QV_H */
