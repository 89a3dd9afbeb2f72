// Host side of the qv C ABI: grid selection, sequence metadata, argument
// validation, workspace planning and the launch sequence of the encoder.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <mutex>
#include <string>
#include <utility>
#include <vector>

#include "../../include/qv.h"
#include "qv_internal.h"

using namespace qv;

namespace {

thread_local std::string g_err;

qv_status fail(qv_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

#define QV_HIP(call)                                                                   \
  do {                                                                                 \
    hipError_t e_ = (call);                                                            \
    if (e_ != hipSuccess) return fail(QV_ERR_HIP, "%s: %s", #call, hipGetErrorString(e_)); \
  } while (0)

// ------------------------------------------------- launch timing (diagnostic)
}  // namespace
namespace qv {
thread_local LaunchTiming* g_launch_timing = nullptr;
}  // namespace qv
namespace {
struct Timing {
  std::mutex mu;
  std::atomic<int> cls{-1};  // read without the lock on every launch; written under it
  std::vector<std::pair<hipEvent_t, hipEvent_t>> pool;
  size_t used = 0;
};
Timing& timing() {
  static Timing t;
  return t;
}

// Returns the event pair to record around the next launch of class `cls`, or
// nullptr when that class is not being timed.
std::pair<hipEvent_t, hipEvent_t>* timing_slot(int cls) {
  Timing& t = timing();
  if (t.cls.load(std::memory_order_relaxed) != cls) return nullptr;
  std::lock_guard<std::mutex> g(t.mu);
  if (t.cls.load(std::memory_order_relaxed) != cls) return nullptr;
  if (t.used == t.pool.size()) {
    hipEvent_t a, b;
    if (hipEventCreate(&a) != hipSuccess) return nullptr;
    if (hipEventCreate(&b) != hipSuccess) {
      (void)hipEventDestroy(a);
      return nullptr;
    }
    t.pool.emplace_back(a, b);
  }
  return &t.pool[t.used++];
}

// Gives back the last slot when the timed call launched no kernel.
void timing_unslot() {
  Timing& t = timing();
  std::lock_guard<std::mutex> g(t.mu);
  if (t.used) --t.used;
}

// Points the kernel launches of one call at an event pair for its lifetime.
struct TimingScope {
  LaunchTiming lt;
  explicit TimingScope(std::pair<hipEvent_t, hipEvent_t>* s) : lt{s->first, s->second, false} {
    g_launch_timing = &lt;
  }
  ~TimingScope() { g_launch_timing = nullptr; }
};

#define QV_LAUNCH(cls, stream, call)                                       \
  do {                                                                     \
    auto* slot_ = timing_slot(cls);                                        \
    if (slot_) {                                                           \
      bool launched_ = false;                                              \
      {                                                                    \
        TimingScope ts_(slot_);                                            \
        QV_HIP(call);                                                      \
        launched_ = ts_.lt.started;                                        \
      }                                                                    \
      if (!launched_) timing_unslot();                                     \
    } else {                                                               \
      QV_HIP(call);                                                        \
    }                                                                      \
  } while (0)

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

struct Grid {
  int32_t t, gh, gw;
};

qv_status read_grids(const int32_t* grid_thw, int32_t n_img, int32_t merge, std::vector<Grid>& out, int64_t& total) {
  if (!grid_thw) return fail(QV_ERR_NULL, "grid_thw is NULL");
  if (n_img <= 0) return fail(QV_ERR_SHAPE, "n_img must be positive (got %d)", n_img);
  if (merge <= 0) return fail(QV_ERR_SHAPE, "merge must be positive");
  out.resize(n_img);
  total = 0;
  for (int i = 0; i < n_img; ++i) {
    Grid g{grid_thw[3 * i], grid_thw[3 * i + 1], grid_thw[3 * i + 2]};
    if (g.t <= 0 || g.gh <= 0 || g.gw <= 0)
      return fail(QV_ERR_SHAPE, "image %d: grid (%d,%d,%d) must be positive", i, g.t, g.gh, g.gw);
    if (g.gh % merge || g.gw % merge)
      return fail(QV_ERR_SHAPE, "image %d: grid sides (%d,%d) must be multiples of merge %d", i, g.gh, g.gw, merge);
    out[i] = g;
    total += (int64_t)g.t * g.gh * g.gw;
    if (total > INT32_MAX) return fail(QV_ERR_SHAPE, "more than INT32_MAX patches");
  }
  return QV_OK;
}

}  // namespace

extern "C" {

const char* qv_last_error(void) { return g_err.c_str(); }

int32_t qv_abi_version(void) { return QV_ABI_VERSION; }

void qv_grid_params_default(qv_grid_params* p) {
  if (!p) return;
  p->patch = 14;
  p->merge = 2;
  p->temporal = 2;
  p->reserved = 0;
  p->min_pixels = 3136;
  p->max_pixels = 12845056;
}

qv_status qv_smart_resize_grid(int64_t height, int64_t width, int32_t frames, const qv_grid_params* pin,
                               int64_t* out_height, int64_t* out_width, int32_t out_grid_thw[3]) {
  qv_grid_params p;
  if (pin) p = *pin; else qv_grid_params_default(&p);
  if (!out_grid_thw) return fail(QV_ERR_NULL, "out_grid_thw is NULL");
  if (height <= 0 || width <= 0 || frames <= 0)
    return fail(QV_ERR_SHAPE, "height, width and frames must be positive");
  if (p.patch <= 0 || p.merge <= 0 || p.temporal <= 0 || p.min_pixels < 0 || p.max_pixels < p.min_pixels)
    return fail(QV_ERR_SHAPE, "invalid grid parameters");
  if (height > (1LL << 26) || width > (1LL << 26)) return fail(QV_ERR_SHAPE, "image side too large");
  const int64_t f = (int64_t)p.patch * p.merge;
  // nearest multiple of f, ties to even (nearbyint in the default rounding mode)
  int64_t h = std::max<int64_t>(f, (int64_t)nearbyint((double)height / (double)f) * f);
  int64_t w = std::max<int64_t>(f, (int64_t)nearbyint((double)width / (double)f) * f);
  if (h * w > p.max_pixels) {
    const double beta = sqrt((double)(height * width) / (double)p.max_pixels);
    h = std::max<int64_t>(f, (int64_t)floor((double)height / (beta * (double)f)) * f);
    w = std::max<int64_t>(f, (int64_t)floor((double)width / (beta * (double)f)) * f);
  } else if (h * w < p.min_pixels) {
    const double beta = sqrt((double)p.min_pixels / (double)(height * width));
    h = (int64_t)ceil((double)height * beta / (double)f) * f;
    w = (int64_t)ceil((double)width * beta / (double)f) * f;
  }
  if (h * w < p.min_pixels || h * w > p.max_pixels)
    return fail(QV_ERR_BUDGET, "no grid inside the pixel budget for %lldx%lld", (long long)height, (long long)width);
  if (out_height) *out_height = h;
  if (out_width) *out_width = w;
  out_grid_thw[0] = (int32_t)((frames + p.temporal - 1) / p.temporal);
  out_grid_thw[1] = (int32_t)(h / p.patch);
  out_grid_thw[2] = (int32_t)(w / p.patch);
  return QV_OK;
}

qv_status qv_seq_meta(const int32_t* grid_thw, int32_t n_img, int32_t merge, int32_t* cu_seqlens, int32_t* pos_hw,
                      int32_t* perm) {
  if (!cu_seqlens) return fail(QV_ERR_NULL, "cu_seqlens is NULL");
  std::vector<Grid> g;
  int64_t total = 0;
  qv_status st = read_grids(grid_thw, n_img, merge, g, total);
  if (st != QV_OK) return st;
  int64_t s = 0;
  cu_seqlens[0] = 0;
  for (int i = 0; i < n_img; ++i) {
    const Grid& G = g[i];
    for (int t = 0; t < G.t; ++t)
      for (int bh = 0; bh < G.gh / merge; ++bh)
        for (int bw = 0; bw < G.gw / merge; ++bw)
          for (int dy = 0; dy < merge; ++dy)
            for (int dx = 0; dx < merge; ++dx, ++s) {
              const int h = merge * bh + dy, w = merge * bw + dx;
              if (pos_hw) {
                pos_hw[2 * s] = h;
                pos_hw[2 * s + 1] = w;
              }
              if (perm) perm[s] = t * G.gh * G.gw + h * G.gw + w;
            }
    cu_seqlens[i + 1] = (int32_t)s;
  }
  return QV_OK;
}

qv_status qv_patchify(const float* pixels, const qv_image* images, int32_t n_img, const int32_t* grid_thw,
                      const qv_grid_params* pin, void* patches, qv_dtype out_dtype, int32_t ld, void* stream) {
  return qv_patchify_ex(pixels, images, n_img, grid_thw, pin, nullptr, patches, out_dtype, ld, stream);
}

qv_status qv_patchify_ex(const float* pixels, const qv_image* images, int32_t n_img, const int32_t* grid_thw,
                         const qv_grid_params* pin, const qv_patch_opts* opts, void* patches, qv_dtype out_dtype,
                         int32_t ld, void* stream) {
  qv_grid_params p;
  if (pin) p = *pin; else qv_grid_params_default(&p);
  qv_patch_opts o{};
  if (opts) o = *opts;
  if (!pixels || !images || !patches) return fail(QV_ERR_NULL, "pixels, images and patches must be non-NULL");
  if (p.merge != 2) return fail(QV_ERR_UNSUPPORTED, "only merge 2 is implemented");
  if (out_dtype != QV_F32 && out_dtype != QV_BF16) return fail(QV_ERR_UNSUPPORTED, "unknown dtype %d", (int)out_dtype);
  if ((o.fold != 0 && o.fold != 1) || (o.normalize != 0 && o.normalize != 1))
    return fail(QV_ERR_UNSUPPORTED, "fold and normalize must be 0 or 1");
  std::vector<Grid> g;
  int64_t total = 0;
  qv_status st = read_grids(grid_thw, n_img, p.merge, g, total);
  if (st != QV_OK) return st;
  const int channels = images[0].channels;
  if (o.normalize) {
    if (channels > 4) return fail(QV_ERR_UNSUPPORTED, "normalize supports at most 4 channels, got %d", channels);
    for (int ch = 0; ch < channels; ++ch)
      if (!(o.std[ch] > 0.f) || !std::isfinite(o.mean[ch]))
        return fail(QV_ERR_UNSUPPORTED, "normalize: std[%d] must be > 0 and mean[%d] finite", ch, ch);
  }
  const int vec = channels * (o.fold ? 1 : p.temporal) * p.patch * p.patch;
  const int patch_dim = o.fold ? (vec + 7) / 8 * 8 : vec;
  if (patch_dim % 8) return fail(QV_ERR_UNSUPPORTED, "patch vector length %d is not a multiple of 8", patch_dim);
  if (ld < patch_dim || ld % 8) return fail(QV_ERR_SHAPE, "ld %d must be >= %d and a multiple of 8", ld, patch_dim);
  std::vector<PatchImg> d(n_img);
  int64_t row = 0;
  for (int i = 0; i < n_img; ++i) {
    const qv_image& im = images[i];
    if (im.channels != channels) return fail(QV_ERR_SHAPE, "image %d: all images must have the same channels", i);
    if (im.frames <= 0 || im.channels <= 0 || im.offset < 0)
      return fail(QV_ERR_SHAPE, "image %d: frames/channels must be positive, offset non-negative", i);
    if (im.height != p.patch * g[i].gh || im.width != p.patch * g[i].gw)
      return fail(QV_ERR_SHAPE, "image %d: %dx%d is not %d * grid (%d,%d)", i, im.height, im.width, p.patch, g[i].gh,
                  g[i].gw);
    if (g[i].t != (im.frames + p.temporal - 1) / p.temporal)
      return fail(QV_ERR_SHAPE, "image %d: T=%d but %d frames", i, g[i].t, im.frames);
    if (o.fold && im.frames != 1)
      return fail(QV_ERR_SHAPE, "image %d: the Conv2d fold needs a single frame, got %d", i, im.frames);
    d[i] = PatchImg{im.offset, im.frames, im.channels, im.height, im.width, g[i].t, g[i].gh, g[i].gw, (int32_t)row};
    row += (int64_t)g[i].t * g[i].gh * g[i].gw;
  }
  PatchMode m{};
  m.fold = o.fold;
  m.normalize = o.normalize;
  m.width = patch_dim;
  for (int ch = 0; ch < 4; ++ch) {
    m.mean[ch] = o.mean[ch];
    m.stdv[ch] = o.normalize ? o.std[ch] : 1.f;
  }
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  for (int c0 = 0; c0 < n_img; c0 += kPatchChunk) {
    PatchChunk c{};
    c.count = std::min(kPatchChunk, n_img - c0);
    int64_t nmax = 0;
    for (int i = 0; i < c.count; ++i) {
      c.d[i] = d[c0 + i];
      nmax = std::max<int64_t>(nmax, (int64_t)c.d[i].t * c.d[i].gh * c.d[i].gw);
    }
    QV_LAUNCH(QV_KC_PATCHIFY, s, launch_patchify(pixels, c, p.patch, p.temporal, patches, out_dtype == QV_BF16, ld, m, nmax, s));
  }
  return QV_OK;
}

qv_status qv_fold_patch_weight(const void* w, int32_t dim, int32_t channels, int32_t patch, int32_t temporal,
                               int32_t ld_in, void* out, int32_t ld_out, qv_dtype dtype, void* stream) {
  if (!w || !out) return fail(QV_ERR_NULL, "w and out must be non-NULL");
  if (dtype != QV_F32 && dtype != QV_BF16) return fail(QV_ERR_UNSUPPORTED, "unknown dtype %d", (int)dtype);
  if (dim <= 0 || channels <= 0 || patch <= 0 || temporal <= 0)
    return fail(QV_ERR_SHAPE, "dim, channels, patch and temporal must be positive");
  const int64_t vec_in = (int64_t)channels * temporal * patch * patch, vec_out = (int64_t)channels * patch * patch;
  if (ld_in < vec_in || ld_out < vec_out)
    return fail(QV_ERR_SHAPE, "ld_in %d must be >= %lld and ld_out %d >= %lld", ld_in, (long long)vec_in, ld_out,
                (long long)vec_out);
  if ((int64_t)dim * std::max(ld_in, ld_out) > INT32_MAX) return fail(QV_ERR_SHAPE, "weight too large");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  QV_HIP(launch_fold_weight(w, dim, channels, patch, temporal, ld_in, out, ld_out, dtype == QV_BF16, s));
  return QV_OK;
}

qv_status qv_quantize_i8(const void* w, int32_t rows, int32_t cols, int32_t ld, qv_dtype dtype, int8_t* q,
                         float* scale, void* stream) {
  if (!w || !q || !scale) return fail(QV_ERR_NULL, "w, q and scale must be non-NULL");
  if (dtype != QV_F32 && dtype != QV_BF16) return fail(QV_ERR_UNSUPPORTED, "w must be QV_F32 or QV_BF16, not %d", (int)dtype);
  if (rows <= 0 || cols <= 0 || ld < cols) return fail(QV_ERR_SHAPE, "rows %d, cols %d must be positive and ld %d >= cols",
                                                       rows, cols, ld);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  QV_HIP(launch_quantize_i8(w, rows, cols, ld, dtype == QV_BF16, q, scale, s));
  return QV_OK;
}

}  // extern "C"

// ------------------------------------------------------------------ encoder
namespace {

struct VisionPlan {
  int64_t N = 0;
  int64_t P = 0;
  int n_img = 0;
  int max_pos = 0;
  int total_qtiles = 0;
  int attn_rows = 0;  // query rows per attention workgroup
  bool padded = false;
  size_t es = 2;
  std::vector<ImgDesc> desc;
  std::vector<PlanEntry> plan;
  // windowed attention: a second padded layout with one kSeqAlign-row slot per window
  int split_fc2 = 1;   // split-K runs of fc2 (bf16, small M)
  int split_proj = 1;  // split-K runs of the out-projection (int8 weights, small M)
  bool i8 = false;     // int8 block matrices
  // int8 at large M: these products widen their codes to bf16 in off_codes
  // (one matrix at a time) and use the 256 x 256 bf16 kernel
  bool wide_qkv = false, wide_proj = false, wide_fc1 = false, wide_fc2 = false;
  size_t off_codes = 0;
  int window = 0;
  int win_slot = 0;  // padded rows per window: kWinSlot (64) for W <= 8, else kSeqAlign (128)
  int64_t n_win = 0, Pw = 0;
  int total_qtiles_w = 0;
  std::vector<PlanEntry> plan_w;
  size_t off_tok = 0, off_plan = 0, off_rope = 0, off_a = 0, off_q = 0, off_k = 0, off_vt = 0, off_vt_end = 0,
         off_o = 0, off_h = 0, off_qkv = 0, off_tokw = 0, off_outrow = 0, off_planw = 0, off_part = 0, total = 0;
};

qv_status check_vision_cfg(const qv_vision_cfg* c) {
  if (!c) return fail(QV_ERR_NULL, "cfg is NULL");
  if (c->dtype != QV_F32 && c->dtype != QV_BF16) return fail(QV_ERR_UNSUPPORTED, "unknown dtype %d", c->dtype);
  if (c->depth < 0) return fail(QV_ERR_SHAPE, "depth must be >= 0");
  const int nv = c->dim / 256;
  if (c->dim <= 0 || c->dim % 256 || !(nv == 4 || nv == 5 || nv == 6 || nv == 8))
    return fail(QV_ERR_UNSUPPORTED, "dim %d: LayerNorm kernels exist for 1024, 1280, 1536, 2048", c->dim);
  if (c->heads <= 0 || c->heads * kHeadDim != c->dim)
    return fail(QV_ERR_UNSUPPORTED, "dim / heads must be %d (dim %d, heads %d)", kHeadDim, c->dim, c->heads);
  if (c->mlp <= 0 || c->mlp % 64) return fail(QV_ERR_UNSUPPORTED, "mlp %d must be a positive multiple of 64", c->mlp);
  if (c->patch_dim <= 0 || c->patch_dim % 8)
    return fail(QV_ERR_UNSUPPORTED, "patch_dim %d must be a positive multiple of 8", c->patch_dim);
  if (c->ld < c->patch_dim || c->ld % 8) return fail(QV_ERR_SHAPE, "ld %d must be >= patch_dim and a multiple of 8", c->ld);
  if (c->merge != 2) return fail(QV_ERR_UNSUPPORTED, "only merge 2 is implemented");
  if (!(c->ln_eps >= 0.f) || !(c->rope_theta > 0.f)) return fail(QV_ERR_SHAPE, "ln_eps >= 0 and rope_theta > 0 required");
  if (c->window < 0 || c->window % c->merge || c->window > 10)
    return fail(QV_ERR_UNSUPPORTED, "window %d must be 0 or a multiple of merge %d in [2, 10]", c->window, c->merge);
  if (c->weights != 0 && c->weights != QV_I8)
    return fail(QV_ERR_UNSUPPORTED, "weights %d must be 0 or QV_I8", c->weights);
  if (c->weights == QV_I8 && (c->dtype != QV_BF16 || c->dim != 1280 || c->mlp != 5120))
    return fail(QV_ERR_UNSUPPORTED, "int8 weights need dtype QV_BF16, dim 1280 and mlp 5120");
  return QV_OK;
}

qv_status make_plan(const qv_vision_cfg* c, const int32_t* grid_thw, int32_t n_img, VisionPlan& vp) {
  qv_status st = check_vision_cfg(c);
  if (st != QV_OK) return st;
  std::vector<Grid> g;
  int64_t total = 0;
  st = read_grids(grid_thw, n_img, c->merge, g, total);
  if (st != QV_OK) return st;
  vp = VisionPlan{};
  vp.n_img = n_img;
  vp.N = total;
  vp.es = c->dtype == QV_BF16 ? 2 : 4;
  vp.desc.resize(n_img);
  int64_t row = 0, prow = 0;
  for (int i = 0; i < n_img; ++i) {
    if (g[i].gh > 65535 || g[i].gw > 65535) return fail(QV_ERR_UNSUPPORTED, "grid side above 65535");
    const int64_t n = (int64_t)g[i].t * g[i].gh * g[i].gw;
    vp.desc[i] = ImgDesc{(int32_t)row, (int32_t)n, g[i].t, g[i].gh, g[i].gw, (int32_t)prow, 0, 0, 0};
    if (n % kSeqAlign) vp.padded = true;
    row += n;
    prow += round_up(n, kSeqAlign);
    vp.max_pos = std::max(vp.max_pos, std::max(g[i].gh, g[i].gw));
  }
  vp.P = prow;
  if (vp.P > INT32_MAX / 2) return fail(QV_ERR_SHAPE, "batch too large");
  // bf16 matrix products address operands with 32-bit byte offsets: the
  // widest activation ([N][mlp] or [N][3 dim] bf16) must stay below 2 GiB
  if (c->dtype == QV_BF16 && (size_t)vp.N * std::max(c->mlp, 3 * c->dim) * 2 >= 0x7FFFFFFFu)
    return fail(QV_ERR_UNSUPPORTED, "batch of %lld patches too large for one call", (long long)vp.N);
  int64_t tiles128 = 0;
  for (int i = 0; i < n_img; ++i) tiles128 += (vp.desc[i].n + 127) / 128;
  vp.attn_rows = c->dtype == QV_BF16 ? attention_bf16_rows_per_wg(tiles128 * c->heads) : kAttnBQ_f32;
  const int bq = vp.attn_rows;
  // attention work plan: longest images first so the tail of the grid is short
  std::vector<int> order(n_img);
  for (int i = 0; i < n_img; ++i) order[i] = i;
  std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return vp.desc[a].n > vp.desc[b].n; });
  vp.plan.resize(n_img);
  int qt = 0;
  for (int k = 0; k < n_img; ++k) {
    const ImgDesc& d = vp.desc[order[k]];
    vp.plan[k] = PlanEntry{d.row0, d.prow0, qt, d.n};
    qt += (int)((d.n + bq - 1) / bq);
  }
  vp.total_qtiles = qt;
  if (c->window > 0) {
    // Every window gets a slot of padded rows: 64 when W <= 8 (the small-window
    // kernel, one workgroup per window and head, plan in window order), else
    // 128 (windows of up to 10 x 10 patches: the full-attention kernel with
    // 64-row q-tiles reading one 128-key stage, plan sorted largest first).
    const int W = c->window;
    vp.window = W;
    vp.win_slot = W * W <= kWinSlot ? kWinSlot : kSeqAlign;
    std::vector<int> wn;  // window sizes in global window order
    for (int i = 0; i < n_img; ++i) {
      ImgDesc& d = vp.desc[i];
      d.nwy = (d.gh + W - 1) / W;
      d.nwx = (d.gw + W - 1) / W;
      d.wbase = (int32_t)wn.size();
      for (int t = 0; t < d.t; ++t)
        for (int wy = 0; wy < d.nwy; ++wy)
          for (int wx = 0; wx < d.nwx; ++wx)
            wn.push_back(std::min(W, d.gh - wy * W) * std::min(W, d.gw - wx * W));
    }
    vp.n_win = (int64_t)wn.size();
    vp.Pw = vp.n_win * vp.win_slot;
    if (vp.Pw > INT32_MAX / 2) return fail(QV_ERR_SHAPE, "batch too large");
    const int bqw = c->dtype == QV_BF16 ? 64 : kAttnBQ_f32;
    std::vector<int> worder((size_t)vp.n_win);
    for (int64_t i = 0; i < vp.n_win; ++i) worder[i] = (int)i;
    if (vp.win_slot != kWinSlot)
      std::stable_sort(worder.begin(), worder.end(), [&](int a, int b) { return wn[a] > wn[b]; });
    vp.plan_w.resize((size_t)vp.n_win);
    int qtw = 0;
    for (int64_t k = 0; k < vp.n_win; ++k) {
      const int wi = worder[k];
      vp.plan_w[k] = PlanEntry{wi, wi * vp.win_slot, qtw, wn[wi]};
      qtw += (wn[wi] + bqw - 1) / bqw;
    }
    vp.total_qtiles_w = qtw;
  }
  const size_t N = (size_t)vp.N, P = (size_t)std::max(vp.P, vp.Pw), es = vp.es;
  size_t o = 0;
  vp.off_tok = o;  o = align_up(o + N * sizeof(int2));
  vp.off_plan = o; o = align_up(o + (size_t)n_img * sizeof(PlanEntry));
  vp.off_rope = o; o = align_up(o + (size_t)vp.max_pos * kRopeFreqs * sizeof(float2));
  vp.off_a = o;    o = align_up(o + N * c->dim * es);
  vp.off_q = o;    o = align_up(o + (size_t)c->heads * P * kHeadDim * es);
  vp.off_k = o;    o = align_up(o + (size_t)c->heads * P * kHeadDim * es);
  vp.off_vt = o;   o = align_up(o + (size_t)c->heads * kHeadDim * P * es);
  vp.off_vt_end = o;
  vp.off_o = o;    o = align_up(o + N * c->dim * es);
  vp.off_h = o;    o = align_up(o + N * c->mlp * es);
  vp.off_qkv = o;
  if (c->dtype == QV_F32) o = align_up(o + N * 3 * c->dim * sizeof(float));
  vp.i8 = c->weights == QV_I8;
  if (vp.i8 && c->depth > 0) {
    // int8 weights use 128 x 160 tiles: at small M the out-projection has
    // too few of them unsplit, so both it and fc2 leave partial sums
    vp.split_fc2 = gemm_i8w_runs((int)N, c->dim, c->mlp);
    vp.split_proj = gemm_i8w_runs((int)N, c->dim, c->dim);
  } else if (c->dtype == QV_BF16 && c->dim == 1280 && c->depth > 0) {
    // fc2 only: the out-projection's K = 1280 is too short for its split to
    // pay for the partial sums the LayerNorm reads back (measured 10.8 + 7.8
    // us against 11.9 + 4.2 us at 448x448)
    vp.split_fc2 = gemm_splitk_runs((int)N, c->dim, c->mlp);
  }
  vp.off_part = o;
  const int max_split = std::max(vp.split_fc2, vp.split_proj);
  if (max_split > 1) o = align_up(o + (size_t)max_split * N * c->dim * sizeof(uint16_t));
  if (vp.i8 && c->depth > 0) {
    const int n = (int)N;
    vp.wide_qkv = gemm_i8w_wide(n, 3 * c->dim);
    vp.wide_proj = vp.split_proj == 1 && gemm_i8w_wide(n, c->dim);
    vp.wide_fc1 = gemm_i8w_wide(n, c->mlp);
    vp.wide_fc2 = vp.split_fc2 == 1 && gemm_i8w_wide(n, c->dim);
    size_t codes = 0;
    if (vp.wide_qkv) codes = std::max(codes, (size_t)3 * c->dim * c->dim);
    if (vp.wide_proj) codes = std::max(codes, (size_t)c->dim * c->dim);
    if (vp.wide_fc1 || vp.wide_fc2) codes = std::max(codes, (size_t)c->mlp * c->dim);
    vp.off_codes = o;
    o = align_up(o + codes * 2);
  }
  if (vp.window) {
    vp.off_tokw = o;   o = align_up(o + N * sizeof(int2));
    vp.off_outrow = o; o = align_up(o + (size_t)vp.Pw * sizeof(int32_t));
    vp.off_planw = o;  o = align_up(o + (size_t)vp.n_win * sizeof(PlanEntry));
  }
  vp.total = o;
  return QV_OK;
}

qv_status check_block(const qv_block_w& b, int l, bool i8) {
  const void* p[] = {b.ln1_w, b.ln1_b, b.qkv_w, b.qkv_b, b.proj_w, b.proj_b, b.ln2_w, b.ln2_b,
                     b.fc1_w, b.fc1_b, b.fc2_w, b.fc2_b, b.qkv_s, b.proj_s, b.fc1_s, b.fc2_s};
  const int n = i8 ? 16 : 12;
  for (int i = 0; i < n; ++i)
    if (!p[i]) return fail(QV_ERR_NULL, "block %d: weight pointer %d is NULL", l, i);
  if (i8) {
    const void* m[] = {b.qkv_w, b.proj_w, b.fc1_w, b.fc2_w};
    for (const void* x : m)
      if (reinterpret_cast<uintptr_t>(x) & 15) return fail(QV_ERR_SHAPE, "block %d: int8 matrices must be 16-byte aligned", l);
  }
  return QV_OK;
}

}  // namespace

extern "C" {

qv_status qv_vision_workspace_size(const qv_vision_cfg* c, const int32_t* grid_thw, int32_t n_img, size_t* bytes) {
  if (!bytes) return fail(QV_ERR_NULL, "bytes is NULL");
  VisionPlan vp;
  qv_status st = make_plan(c, grid_thw, n_img, vp);
  if (st != QV_OK) return st;
  *bytes = vp.total;
  return QV_OK;
}

}  // extern "C"

namespace {
// Body of qv_vision_forward and qv_vision_forward_noalloc: validation, the
// plan, then every launch on `stream`.  use_scratch: the workspace is the
// library's static device array instead of the caller's ws.
qv_status vision_forward_impl(const qv_vision_cfg* c, const qv_vision_w* w, const void* patches,
                              const int32_t* grid_thw, int32_t n_img, const int32_t* cu_seqlens, float* hidden,
                              void* ws, size_t ws_bytes, bool use_scratch, void* stream) {
  if (!w || !patches || !cu_seqlens || !hidden || (!ws && !use_scratch))
    return fail(QV_ERR_NULL, "weights, patches, cu_seqlens, hidden and ws must be non-NULL");
  VisionPlan vp;
  qv_status st = make_plan(c, grid_thw, n_img, vp);
  if (st != QV_OK) return st;
  if (!w->patch_w) return fail(QV_ERR_NULL, "patch_w is NULL");
  if (c->depth > 0 && !w->blocks) return fail(QV_ERR_NULL, "blocks is NULL");
  for (int l = 0; l < c->depth; ++l) {
    st = check_block(w->blocks[l], l, vp.i8);
    if (st != QV_OK) return st;
  }
  if (use_scratch) {
    if (vp.total > QV_SCRATCH_BYTES)
      return fail(QV_ERR_WORKSPACE, "this batch needs %zu bytes of workspace, above the %zu-byte static scratch of "
                  "the allocation-free forward (use qv_vision_forward with a caller workspace)",
                  vp.total, (size_t)QV_SCRATCH_BYTES);
    void* p = nullptr;
    QV_HIP(scratch_buffer(&p));
    ws = p;
    ws_bytes = QV_SCRATCH_BYTES;
  }
  if (ws_bytes < vp.total)
    return fail(QV_ERR_WORKSPACE, "workspace %zu bytes, need %zu", ws_bytes, vp.total);
  if ((reinterpret_cast<uintptr_t>(ws) & 255) != 0) return fail(QV_ERR_SHAPE, "workspace must be 256-byte aligned");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);

  const char* dbg = getenv("QV_DEBUG_VALIDATE");
  if (dbg && dbg[0] == '1') {
    std::vector<int32_t> cu(n_img + 1);
    QV_HIP(hipMemcpyAsync(cu.data(), cu_seqlens, sizeof(int32_t) * (n_img + 1), hipMemcpyDeviceToHost, s));
    QV_HIP(hipStreamSynchronize(s));
    for (int i = 0; i <= n_img; ++i) {
      const int32_t want = i == 0 ? 0 : vp.desc[i - 1].row0 + vp.desc[i - 1].n;
      if (cu[i] != want) return fail(QV_ERR_SHAPE, "cu_seqlens[%d] = %d, grid_thw gives %d", i, cu[i], want);
    }
  }

  char* base = reinterpret_cast<char*>(ws);
  int2* tok = reinterpret_cast<int2*>(base + vp.off_tok);
  PlanEntry* plan = reinterpret_cast<PlanEntry*>(base + vp.off_plan);
  float2* rope = reinterpret_cast<float2*>(base + vp.off_rope);
  void* A = base + vp.off_a;
  void* O = base + vp.off_o;
  void* H = base + vp.off_h;
  int2* tokw = reinterpret_cast<int2*>(base + vp.off_tokw);
  int32_t* outrow = reinterpret_cast<int32_t*>(base + vp.off_outrow);
  PlanEntry* planw = reinterpret_cast<PlanEntry*>(base + vp.off_planw);
  void* codes = base + vp.off_codes;
  QkvOut qo{base + vp.off_q, base + vp.off_k, base + vp.off_vt, tok, rope, (int)vp.P, c->dim};
  QkvOut qow{base + vp.off_q, base + vp.off_k, base + vp.off_vt, tokw, rope, (int)vp.Pw, c->dim};

  for (int c0 = 0; c0 < n_img; c0 += kDescChunk) {
    DescChunk dc{};
    dc.count = std::min(kDescChunk, n_img - c0);
    dc.first = c0;
    for (int i = 0; i < dc.count; ++i) dc.d[i] = vp.desc[c0 + i];
    QV_HIP(launch_setup_tokens(dc, tok, s));
    QV_HIP(launch_setup_plan(vp.plan.data() + c0, dc.count, c0, plan, s));
  }
  QV_HIP(launch_rope_table(rope, vp.max_pos, c->rope_theta, s));
  if (vp.padded || vp.window) QV_HIP(launch_zero(base + vp.off_q, vp.off_vt_end - vp.off_q, s));
  if (vp.window) {
    for (int c0 = 0; c0 < n_img; c0 += kDescChunk) {
      DescChunk dc{};
      dc.count = std::min(kDescChunk, n_img - c0);
      dc.first = c0;
      for (int i = 0; i < dc.count; ++i) dc.d[i] = vp.desc[c0 + i];
      QV_HIP(launch_setup_windows(dc, vp.window, vp.win_slot, tokw, outrow, s));
    }
    for (int64_t c0 = 0; c0 < vp.n_win; c0 += kPlanChunk) {
      const int cnt = (int)std::min<int64_t>(kPlanChunk, vp.n_win - c0);
      QV_HIP(launch_setup_plan(vp.plan_w.data() + c0, cnt, (int)c0, planw, s));
    }
  }

  const int M = (int)vp.N, D = c->dim, F = c->mlp;
  // Few-row towers read each block's weights cold from HBM (they were last
  // touched a forward ago).  The first LayerNorm of a block (a five-wave,
  // latency-bound kernel at these sizes) also reads the out-projection's
  // weight, so that product, two launches later, finds it in the Infinity
  // Cache (448x448: out-projection 13.7 -> 11.6 us, LayerNorm +1.2 us).
  constexpr int64_t kWarmRows = 4096;
  const bool bf = c->dtype == QV_BF16;
  if (bf)
    QV_LAUNCH(QV_KC_PATCH_EMBED, s, gemm_bf16_store_f32(patches, c->ld, w->patch_w, c->patch_dim, M, D, c->patch_dim,
                               reinterpret_cast<const float*>(w->patch_b), hidden, D, s));
  else
    QV_LAUNCH(QV_KC_PATCH_EMBED, s, gemm_f32_store(reinterpret_cast<const float*>(patches), c->ld, reinterpret_cast<const float*>(w->patch_w),
                          c->patch_dim, M, D, c->patch_dim, reinterpret_cast<const float*>(w->patch_b), hidden, D, s));

  AttnArgs aa{qo.q, qo.k, qo.vt, O, D, plan, n_img, nullptr, (int)vp.P, c->heads, vp.total_qtiles,
              vp.attn_rows};
  AttnArgs aw{qo.q, qo.k, qo.vt, O, D, planw, (int)vp.n_win, outrow, (int)vp.Pw, c->heads,
              vp.total_qtiles_w, bf ? 64 : kAttnBQ_f32};
  // Split-K (small M): fc2 leaves float32 partial sums; the next block's
  // first LayerNorm adds them, the bias and the residual in a fixed order
  // (after the last block a residual-only pass does it).
  uint16_t* part = reinterpret_cast<uint16_t*>(base + vp.off_part);
  const size_t part_stride = (size_t)vp.N * c->dim;
  int pending = 0;
  const float* pending_bias = nullptr;
  auto layer_norm = [&](const void* g, const void* bta, CacheWarm warm) -> qv_status {
    if (pending) {
      QV_LAUNCH(QV_KC_LAYERNORM, s, launch_layernorm_acc(hidden, part, part_stride, pending, pending_bias,
                                                         (const float*)g, (const float*)bta, A, bf, (int)vp.N,
                                                         c->dim, c->ln_eps, s, warm));
      pending = 0;
    } else {
      QV_LAUNCH(QV_KC_LAYERNORM, s, launch_layernorm(hidden, (const float*)g, (const float*)bta, A, bf, (int)vp.N,
                                                     c->dim, c->ln_eps, s, warm));
    }
    return QV_OK;
  };
  for (int l = 0; l < c->depth; ++l) {
    const qv_block_w& b = w->blocks[l];
    // windowed block: q/k/v scattered into the window layout, attention per window
    const bool win = vp.window && !(l < 64 && ((c->full_blocks >> l) & 1u));
    const QkvOut& qb = win ? qow : qo;
    const AttnArgs& ab = win ? aw : aa;
    const bool warm_ok = bf && !vp.i8 && vp.N <= kWarmRows;
    qv_status lst = layer_norm(b.ln1_w, b.ln1_b,
                               warm_ok ? CacheWarm{b.proj_w, (size_t)D * D * 2} : CacheWarm{});
    if (lst != QV_OK) return lst;
    if (bf) {
      if (vp.wide_qkv) {
        QV_LAUNCH(QV_KC_QKV, s, launch_codes_bf16((const int8_t*)b.qkv_w, (int64_t)3 * D * D, codes, s));
        QV_LAUNCH(QV_KC_QKV, s, gemm_i8w_wide_qkv(A, D, codes, D, b.qkv_s, M, D, (const float*)b.qkv_b, qb, s));
      } else if (vp.i8)
        QV_LAUNCH(QV_KC_QKV, s, gemm_i8w_qkv(A, D, (const int8_t*)b.qkv_w, D, b.qkv_s, M, D, (const float*)b.qkv_b, qb, s));
      else
        QV_LAUNCH(QV_KC_QKV, s, gemm_bf16_qkv(A, D, b.qkv_w, D, M, D, (const float*)b.qkv_b, qb, s));
      if (win && vp.win_slot == kWinSlot)
        QV_LAUNCH(QV_KC_ATTENTION, s, attention_bf16_windows(aw, s));
      else
        QV_LAUNCH(QV_KC_ATTENTION, s, attention_bf16(ab, s));
      if (vp.i8 && vp.split_proj > 1) {
        QV_LAUNCH(QV_KC_PROJ, s, gemm_i8w_splitk_bf16(O, D, (const int8_t*)b.proj_w, D, b.proj_s, M, D, D, vp.split_proj,
                                                     part, s));
        pending = vp.split_proj;
        pending_bias = (const float*)b.proj_b;
      } else if (vp.wide_proj) {
        QV_LAUNCH(QV_KC_PROJ, s, launch_codes_bf16((const int8_t*)b.proj_w, (int64_t)D * D, codes, s));
        QV_LAUNCH(QV_KC_PROJ, s, gemm_i8w_wide_resid_f32(O, D, codes, D, b.proj_s, M, D, D, (const float*)b.proj_b,
                                                         hidden, D, s));
      } else if (vp.i8) {
        QV_LAUNCH(QV_KC_PROJ, s, gemm_i8w_resid_f32(O, D, (const int8_t*)b.proj_w, D, b.proj_s, M, D, D,
                                                    (const float*)b.proj_b, hidden, D, s));
      } else {
        QV_LAUNCH(QV_KC_PROJ, s, gemm_bf16_resid_f32(O, D, b.proj_w, D, M, D, D, (const float*)b.proj_b, hidden, D, s));
      }
    } else {
      float* qkv = reinterpret_cast<float*>(base + vp.off_qkv);
      QV_LAUNCH(QV_KC_QKV, s, gemm_f32_store((const float*)A, D, (const float*)b.qkv_w, D, M, 3 * D, D, (const float*)b.qkv_b, qkv,
                            3 * D, s));
      QV_LAUNCH(QV_KC_QKV, s, rope_scatter_f32(qkv, M, nullptr, qb, s));
      QV_LAUNCH(QV_KC_ATTENTION, s, attention_f32(ab, s));
      QV_LAUNCH(QV_KC_PROJ, s, gemm_f32_resid((const float*)O, D, (const float*)b.proj_w, D, M, D, D, (const float*)b.proj_b, hidden,
                            D, s));
    }
    lst = layer_norm(b.ln2_w, b.ln2_b, CacheWarm{});
    if (lst != QV_OK) return lst;
    if (bf && vp.i8) {
      if (vp.wide_fc1) {
        QV_LAUNCH(QV_KC_FC1, s, launch_codes_bf16((const int8_t*)b.fc1_w, (int64_t)F * D, codes, s));
        QV_LAUNCH(QV_KC_FC1, s, gemm_i8w_wide_act_bf16(A, D, codes, D, b.fc1_s, M, F, D, (const float*)b.fc1_b,
                                                       Act::QuickGelu, H, F, s));
      } else {
        QV_LAUNCH(QV_KC_FC1, s, gemm_i8w_act_bf16(A, D, (const int8_t*)b.fc1_w, D, b.fc1_s, M, F, D,
                                                  (const float*)b.fc1_b, Act::QuickGelu, H, F, s));
      }
      if (vp.wide_fc2) {
        QV_LAUNCH(QV_KC_FC2, s, launch_codes_bf16((const int8_t*)b.fc2_w, (int64_t)D * F, codes, s));
        QV_LAUNCH(QV_KC_FC2, s, gemm_i8w_wide_resid_f32(H, F, codes, F, b.fc2_s, M, D, F, (const float*)b.fc2_b,
                                                        hidden, D, s));
      } else if (vp.split_fc2 > 1) {
        QV_LAUNCH(QV_KC_FC2, s, gemm_i8w_splitk_bf16(H, F, (const int8_t*)b.fc2_w, F, b.fc2_s, M, D, F, vp.split_fc2,
                                                    part, s));
        pending = vp.split_fc2;
        pending_bias = (const float*)b.fc2_b;
      } else {
        QV_LAUNCH(QV_KC_FC2, s, gemm_i8w_resid_f32(H, F, (const int8_t*)b.fc2_w, F, b.fc2_s, M, D, F,
                                                   (const float*)b.fc2_b, hidden, D, s));
      }
    } else if (bf) {
      QV_LAUNCH(QV_KC_FC1, s, gemm_bf16_act_bf16(A, D, b.fc1_w, D, M, F, D, (const float*)b.fc1_b, Act::QuickGelu, H, F, s));
      if (vp.split_fc2 > 1) {
        QV_LAUNCH(QV_KC_FC2, s, gemm_bf16_splitk_bf16(H, F, b.fc2_w, F, M, D, F, vp.split_fc2, part, s));
        pending = vp.split_fc2;
        pending_bias = (const float*)b.fc2_b;
      } else {
        QV_LAUNCH(QV_KC_FC2, s, gemm_bf16_resid_f32(H, F, b.fc2_w, F, M, D, F, (const float*)b.fc2_b, hidden, D, s));
      }
    } else {
      QV_LAUNCH(QV_KC_FC1, s, gemm_f32_act((const float*)A, D, (const float*)b.fc1_w, D, M, F, D, (const float*)b.fc1_b,
                          Act::QuickGelu, (float*)H, F, s));
      QV_LAUNCH(QV_KC_FC2, s, gemm_f32_resid((const float*)H, F, (const float*)b.fc2_w, F, M, D, F, (const float*)b.fc2_b, hidden, D,
                            s));
    }
  }
  if (pending) {
    QV_LAUNCH(QV_KC_LAYERNORM, s, launch_layernorm_acc(hidden, part, part_stride, pending, pending_bias, nullptr,
                                                       nullptr, nullptr, bf, (int)vp.N, c->dim, c->ln_eps, s));
    pending = 0;
  }
  return QV_OK;
}
}  // namespace

extern "C" {

qv_status qv_vision_forward(const qv_vision_cfg* c, const qv_vision_w* w, const void* patches,
                            const int32_t* grid_thw, int32_t n_img, const int32_t* cu_seqlens, float* hidden,
                            void* ws, size_t ws_bytes, void* stream) {
  return vision_forward_impl(c, w, patches, grid_thw, n_img, cu_seqlens, hidden, ws, ws_bytes, false, stream);
}

qv_status qv_vision_forward_noalloc(const qv_vision_cfg* c, const qv_vision_w* w, const void* patches,
                                    const int32_t* grid_thw, int32_t n_img, const int32_t* cu_seqlens,
                                    float* hidden, void* stream) {
  return vision_forward_impl(c, w, patches, grid_thw, n_img, cu_seqlens, hidden, nullptr, 0, true, stream);
}

static qv_status check_merger_cfg(const qv_merger_cfg* c, int64_t n_tokens) {
  if (!c) return fail(QV_ERR_NULL, "cfg is NULL");
  if (c->dtype != QV_F32 && c->dtype != QV_BF16) return fail(QV_ERR_UNSUPPORTED, "unknown dtype %d", c->dtype);
  const int nv = c->dim / 256;
  if (c->dim <= 0 || c->dim % 256 || !(nv == 4 || nv == 5 || nv == 6 || nv == 8))
    return fail(QV_ERR_UNSUPPORTED, "dim %d: LayerNorm kernels exist for 1024, 1280, 1536, 2048", c->dim);
  if (c->merge != 2) return fail(QV_ERR_UNSUPPORTED, "only merge 2 is implemented");
  if (c->hidden != c->dim * c->merge * c->merge)
    return fail(QV_ERR_SHAPE, "hidden %d must equal dim * merge^2 = %d", c->hidden, c->dim * c->merge * c->merge);
  if (c->out_dim <= 0) return fail(QV_ERR_SHAPE, "out_dim must be positive");
  if (!(c->ln_eps >= 0.f)) return fail(QV_ERR_SHAPE, "ln_eps must be >= 0");
  const int g = c->merge * c->merge;
  if (n_tokens <= 0 || n_tokens % g) return fail(QV_ERR_SHAPE, "n_tokens %lld must be a positive multiple of %d",
                                                 (long long)n_tokens, g);
  if (n_tokens > INT32_MAX) return fail(QV_ERR_SHAPE, "n_tokens too large");
  return QV_OK;
}

qv_status qv_merge_workspace_size(const qv_merger_cfg* c, int64_t n_tokens, size_t* bytes) {
  if (!bytes) return fail(QV_ERR_NULL, "bytes is NULL");
  qv_status st = check_merger_cfg(c, n_tokens);
  if (st != QV_OK) return st;
  const size_t es = c->dtype == QV_BF16 ? 2 : 4;
  const size_t m = (size_t)n_tokens / (c->merge * c->merge);
  size_t part = 0;  // float32 partial sums of a split-K Linear (bf16, small M)
  if (c->dtype == QV_BF16) {
    const int s1 = gemm_splitk_any_runs((int)m, c->hidden, c->hidden);
    const int s2 = gemm_splitk_any_runs((int)m, c->out_dim, c->hidden);
    part = std::max(s1 > 1 ? (size_t)s1 * m * c->hidden : 0, s2 > 1 ? (size_t)s2 * m * c->out_dim : 0) * sizeof(float);
  }
  *bytes = align_up((size_t)n_tokens * c->dim * es) + align_up(m * c->hidden * es) + align_up(part);
  return QV_OK;
}

qv_status qv_patch_merge(const qv_merger_cfg* c, const qv_merger_w* w, const float* hidden, int64_t n_tokens,
                         void* out, void* ws, size_t ws_bytes, void* stream) {
  if (!w || !hidden || !out || !ws) return fail(QV_ERR_NULL, "weights, hidden, out and ws must be non-NULL");
  size_t need = 0;
  qv_status st = qv_merge_workspace_size(c, n_tokens, &need);
  if (st != QV_OK) return st;
  if (!w->ln_w || !w->ln_b || !w->fc1_w || !w->fc1_b || !w->fc2_w || !w->fc2_b)
    return fail(QV_ERR_NULL, "a merger weight pointer is NULL");
  if (ws_bytes < need) return fail(QV_ERR_WORKSPACE, "workspace %zu bytes, need %zu", ws_bytes, need);
  if ((reinterpret_cast<uintptr_t>(ws) & 255) != 0) return fail(QV_ERR_SHAPE, "workspace must be 256-byte aligned");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const bool bf = c->dtype == QV_BF16;
  const size_t es = bf ? 2 : 4;
  const int M = (int)(n_tokens / (c->merge * c->merge)), Hd = c->hidden;
  char* base = reinterpret_cast<char*>(ws);
  void* Y = base;
  void* G = base + align_up((size_t)n_tokens * c->dim * es);
  QV_LAUNCH(QV_KC_LAYERNORM, s, launch_layernorm(hidden, (const float*)w->ln_w, (const float*)w->ln_b, Y, bf, (int)n_tokens, c->dim,
                          c->ln_eps, s));
  if (bf) {
    // small M: split K so the grid fills the GPU; partials reduced in order
    float* part = reinterpret_cast<float*>(base + align_up((size_t)n_tokens * c->dim * es) + align_up((size_t)M * Hd * es));
    const int s1 = gemm_splitk_any_runs(M, Hd, Hd), s2 = gemm_splitk_any_runs(M, c->out_dim, Hd);
    if (s1 > 1) {
      QV_LAUNCH(QV_KC_MERGE_FC1, s, gemm_bf16_splitk_any_f32(Y, Hd, w->fc1_w, Hd, M, Hd, Hd, s1, part, s));
      QV_LAUNCH(QV_KC_MERGE_FC1, s, launch_splitk_reduce(part, s1, (size_t)M * Hd, (const float*)w->fc1_b, Act::GeluErf,
                                                          G, Hd, M, Hd, s));
    } else {
      QV_LAUNCH(QV_KC_MERGE_FC1, s, gemm_bf16_act_bf16(Y, Hd, w->fc1_w, Hd, M, Hd, Hd, (const float*)w->fc1_b, Act::GeluErf,
                                                        G, Hd, s));
    }
    if (s2 > 1) {
      QV_LAUNCH(QV_KC_MERGE_FC2, s, gemm_bf16_splitk_any_f32(G, Hd, w->fc2_w, Hd, M, c->out_dim, Hd, s2, part, s));
      QV_LAUNCH(QV_KC_MERGE_FC2, s, launch_splitk_reduce(part, s2, (size_t)M * c->out_dim, (const float*)w->fc2_b,
                                                          Act::None, out, c->out_dim, M, c->out_dim, s));
    } else {
      QV_LAUNCH(QV_KC_MERGE_FC2, s, gemm_bf16_act_bf16(G, Hd, w->fc2_w, Hd, M, c->out_dim, Hd, (const float*)w->fc2_b,
                                                        Act::None, out, c->out_dim, s));
    }
  } else {
    QV_LAUNCH(QV_KC_MERGE_FC1, s, gemm_f32_act((const float*)Y, Hd, (const float*)w->fc1_w, Hd, M, Hd, Hd, (const float*)w->fc1_b,
                        Act::GeluErf, (float*)G, Hd, s));
    QV_LAUNCH(QV_KC_MERGE_FC2, s, gemm_f32_store((const float*)G, Hd, (const float*)w->fc2_w, Hd, M, c->out_dim, Hd,
                          (const float*)w->fc2_b, (float*)out, c->out_dim, s));
  }
  return QV_OK;
}

qv_status qv_timing_start(int32_t cls) {
  if (cls < 0 || cls >= QV_KC_COUNT) return fail(QV_ERR_UNSUPPORTED, "unknown kernel class %d", cls);
  Timing& t = timing();
  std::lock_guard<std::mutex> g(t.mu);
  t.used = 0;
  t.cls = cls;
  return QV_OK;
}

qv_status qv_timing_stop(double* total_ms, int64_t* launches) {
  if (!total_ms || !launches) return fail(QV_ERR_NULL, "total_ms and launches must be non-NULL");
  Timing& t = timing();
  std::lock_guard<std::mutex> g(t.mu);
  t.cls = -1;
  double sum = 0.0;
  for (size_t i = 0; i < t.used; ++i) {
    QV_HIP(hipEventSynchronize(t.pool[i].second));
    float ms = 0.f;
    QV_HIP(hipEventElapsedTime(&ms, t.pool[i].first, t.pool[i].second));
    sum += ms;
  }
  *total_ms = sum;
  *launches = (int64_t)t.used;
  t.used = 0;
  return QV_OK;
}

}  // extern "C"
