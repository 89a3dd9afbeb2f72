// Memory-bound kernels of the encoder: patch gather, per-token metadata,
// rotary table, zero fill and LayerNorm.  All written for wave64 (gfx950).
#include <mutex>

#include "../../include/qv.h"
#include "qv_internal.h"

namespace qv {

// ------------------------------------------------------------------ scratch
// Workspace of qv_vision_forward_noalloc: one copy per GPU, allocated by the
// loader with the code object and held until the process ends.  Host code
// never passes `scratch` itself to a kernel (on the host that name is a
// stand-in, not a device address): scratch_buffer() resolves the device
// address once per device with hipGetSymbolAddress and every launch takes
// that pointer, exactly as it takes a caller's workspace.
static __device__ __align__(256) unsigned char scratch[QV_SCRATCH_BYTES];

hipError_t scratch_buffer(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> g(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p || (reinterpret_cast<uintptr_t>(p) & 255)) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

// float -> bf16 bits, round to nearest even (v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

// ------------------------------------------------------------------ patchify
// One thread writes 8 consecutive elements of one output row.  Rows of an
// image follow the merge-group order: slot s -> (t, block row, block col,
// dy, dx) with dx fastest; element e -> (channel, temporal slot, row, col),
// or (channel, row, col) of the single frame when the temporal slots are
// folded into the weight; elements past the patch vector are zero.
__global__ __launch_bounds__(256) void k_patchify(const float* __restrict__ pixels, PatchChunk c, int patch,
                                                  int temporal, void* __restrict__ out, int bf16, int ld,
                                                  PatchMode m) {
  const int img = blockIdx.y;
  if (img >= c.count) return;
  const PatchImg d = c.d[img];
  const int chunks = m.width / 8;
  const int64_t n = (int64_t)d.t * d.gh * d.gw;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= n * chunks) return;
  const int64_t s = gid / chunks;
  const int e0 = (int)(gid % chunks) * 8;
  const int hw = d.gh * d.gw;
  const int tt = (int)(s / hw);
  const int rem = (int)(s % hw);
  const int blk = rem >> 2, q = rem & 3;
  const int half_w = d.gw >> 1;
  const int h = 2 * (blk / half_w) + (q >> 1);
  const int w = 2 * (blk % half_w) + (q & 1);
  const int pp = patch * patch;
  const int slots = m.fold ? 1 : temporal;      // temporal slots in the row
  const int vec = d.channels * slots * pp;      // patch vector length
  float v[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int e = e0 + u;
    if (e >= vec) {
      v[u] = 0.f;
      continue;
    }
    const int ch = e / (slots * pp);
    const int r1 = e % (slots * pp);
    const int tau = r1 / pp;
    const int r2 = r1 % pp;
    const int i = r2 / patch, j = r2 % patch;
    int f = temporal * tt + tau;
    f = f < d.frames - 1 ? f : d.frames - 1;
    const int64_t src = d.offset + (((int64_t)f * d.channels + ch) * d.height + (int64_t)patch * h + i) * d.width +
                        (int64_t)patch * w + j;
    float x = pixels[src];
    if (m.normalize) x = (x - m.mean[ch]) / m.stdv[ch];
    v[u] = x;
  }
  const int64_t row = d.row0 + s;
  if (bf16) {
    uint4 pk;
    pk.x = f32_to_bf16_rne(v[0]) | ((uint32_t)f32_to_bf16_rne(v[1]) << 16);
    pk.y = f32_to_bf16_rne(v[2]) | ((uint32_t)f32_to_bf16_rne(v[3]) << 16);
    pk.z = f32_to_bf16_rne(v[4]) | ((uint32_t)f32_to_bf16_rne(v[5]) << 16);
    pk.w = f32_to_bf16_rne(v[6]) | ((uint32_t)f32_to_bf16_rne(v[7]) << 16);
    *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(out) + row * ld + e0) = pk;
  } else {
    float4* o = reinterpret_cast<float4*>(reinterpret_cast<float*>(out) + row * ld + e0);
    o[0] = make_float4(v[0], v[1], v[2], v[3]);
    o[1] = make_float4(v[4], v[5], v[6], v[7]);
  }
}

hipError_t launch_patchify(const float* pixels, const PatchChunk& c, int patch, int temporal, void* out, bool bf16,
                           int ld, const PatchMode& m, int64_t rows_in_chunk_max, hipStream_t s) {
  const int64_t threads = rows_in_chunk_max * (m.width / 8);
  if (threads == 0) return hipSuccess;
  dim3 grid((unsigned)((threads + 255) / 256), (unsigned)c.count);
  QV_KLAUNCH(k_patchify, grid, dim3(256), 0, s, pixels, c, patch, temporal, out, bf16 ? 1 : 0, ld, m);
  return hipGetLastError();
}

// Conv3d -> Conv2d weight fold: out[o][(c*p + r)*p + q] = sum over tau of
// w[o][((c*T + tau)*p + r)*p + q], accumulated in float32 in tau order and
// rounded once; columns past C*p*p are zero.  One thread per output element.
__global__ __launch_bounds__(256) void k_fold_weight(const void* __restrict__ w, int dim, int channels, int patch,
                                                     int temporal, int ld_in, void* __restrict__ out, int ld_out,
                                                     int bf16) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (int64_t)dim * ld_out) return;
  const int o = (int)(gid / ld_out), e = (int)(gid % ld_out);
  const int pp = patch * patch;
  float acc = 0.f;
  if (e < channels * pp) {
    const int ch = e / pp, r = e % pp;
    for (int tau = 0; tau < temporal; ++tau) {
      const int64_t src = (int64_t)o * ld_in + ((int64_t)ch * temporal + tau) * pp + r;
      const float x = bf16 ? __builtin_bit_cast(float, (uint32_t)reinterpret_cast<const uint16_t*>(w)[src] << 16)
                           : reinterpret_cast<const float*>(w)[src];
      acc = tau == 0 ? x : acc + x;
    }
  }
  if (bf16)
    reinterpret_cast<uint16_t*>(out)[gid] = f32_to_bf16_rne(acc);
  else
    reinterpret_cast<float*>(out)[gid] = acc;
}

hipError_t launch_fold_weight(const void* w, int dim, int channels, int patch, int temporal, int ld_in, void* out,
                              int ld_out, bool bf16, hipStream_t s) {
  const int64_t total = (int64_t)dim * ld_out;
  if (total == 0) return hipSuccess;
  QV_KLAUNCH(k_fold_weight, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, w, dim, channels, patch,
                     temporal, ld_in, out, ld_out, bf16 ? 1 : 0);
  return hipGetLastError();
}

// ------------------------------------------------------------- token metadata
// tokinfo[row] = { h | (w << 16), padded row } for every packed row.
__global__ __launch_bounds__(256) void k_setup_tokens(DescChunk c, int2* __restrict__ tokinfo) {
  const int img = blockIdx.y;
  if (img >= c.count) return;
  const ImgDesc d = c.d[img];
  const int s = blockIdx.x * blockDim.x + threadIdx.x;
  if (s >= d.n) return;
  const int hw = d.gh * d.gw;
  const int rem = s % hw;
  const int blk = rem >> 2, q = rem & 3;
  const int half_w = d.gw >> 1;
  const int h = 2 * (blk / half_w) + (q >> 1);
  const int w = 2 * (blk % half_w) + (q & 1);
  tokinfo[d.row0 + s] = make_int2(h | (w << 16), d.prow0 + s);
}

hipError_t launch_setup_tokens(const DescChunk& c, int2* tokinfo, hipStream_t s) {
  int nmax = 0;
  for (int i = 0; i < c.count; ++i) nmax = c.d[i].n > nmax ? c.d[i].n : nmax;
  if (nmax == 0) return hipSuccess;
  dim3 grid((unsigned)((nmax + 255) / 256), (unsigned)c.count);
  QV_KLAUNCH(k_setup_tokens, grid, dim3(256), 0, s, c, tokinfo);
  return hipGetLastError();
}

// Windowed attention layout.  Windows tile each frame's patch grid from the
// top-left corner in steps of `window` patches (edge windows are truncated);
// window (t, wy, wx) of image i is global window wbase + (t * nwy + wy) * nwx
// + wx and occupies padded rows [slot * global window, + its size).
// Inside a window the tokens keep their packed (merge-group) order: group
// (bh', bw') of the window's ww/2 groups per row, member q = 2 dy + dx.
__global__ __launch_bounds__(256) void k_setup_windows(DescChunk c, int window, int slot, int2* __restrict__ tokinfo_w,
                                                       int32_t* __restrict__ out_row) {
  const int img = blockIdx.y;
  if (img >= c.count) return;
  const ImgDesc d = c.d[img];
  const int s = blockIdx.x * blockDim.x + threadIdx.x;
  if (s >= d.n) return;
  const int hw = d.gh * d.gw;
  const int t = s / hw, rem = s % hw;
  const int blk = rem >> 2, q = rem & 3;
  const int half_w = d.gw >> 1;
  const int h = 2 * (blk / half_w) + (q >> 1);
  const int w = 2 * (blk % half_w) + (q & 1);
  const int wy = h / window, wx = w / window;
  const int ww = min(window, d.gw - wx * window);
  const int hl = h - wy * window, wl = w - wx * window;
  const int local = ((hl >> 1) * (ww >> 1) + (wl >> 1)) * 4 + q;
  const int gwin = d.wbase + (t * d.nwy + wy) * d.nwx + wx;
  const int prow = gwin * slot + local;
  tokinfo_w[d.row0 + s] = make_int2(h | (w << 16), prow);
  out_row[prow] = d.row0 + s;
}

hipError_t launch_setup_windows(const DescChunk& c, int window, int slot, int2* tokinfo_w, int32_t* out_row,
                                hipStream_t s) {
  int nmax = 0;
  for (int i = 0; i < c.count; ++i) nmax = c.d[i].n > nmax ? c.d[i].n : nmax;
  if (nmax == 0) return hipSuccess;
  dim3 grid((unsigned)((nmax + 255) / 256), (unsigned)c.count);
  QV_KLAUNCH(k_setup_windows, grid, dim3(256), 0, s, c, window, slot, tokinfo_w, out_row);
  return hipGetLastError();
}

struct PlanChunk {
  int32_t count;
  int32_t first;
  PlanEntry e[kPlanChunk];
};

__global__ void k_setup_plan(PlanChunk c, PlanEntry* __restrict__ plan) {
  const int i = threadIdx.x;
  if (i < c.count) plan[c.first + i] = c.e[i];
}

hipError_t launch_setup_plan(const PlanEntry* host_plan_chunk, int count, int first, PlanEntry* plan,
                             hipStream_t s) {
  PlanChunk c;
  c.count = count;
  c.first = first;
  for (int i = 0; i < count; ++i) c.e[i] = host_plan_chunk[i];
  QV_KLAUNCH(k_setup_plan, dim3(1), dim3(kPlanChunk), 0, s, c, plan);
  return hipGetLastError();
}

// rope[p][k] = (cos, sin)(p * theta^(-k/20)), evaluated in double, stored f32.
__global__ __launch_bounds__(256) void k_rope_table(float2* __restrict__ tab, int positions, double theta) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= positions * kRopeFreqs) return;
  const int p = i / kRopeFreqs, k = i % kRopeFreqs;
  const double omega = pow(theta, -(double)k / (double)kRopeFreqs);
  const double a = (double)p * omega;
  tab[i] = make_float2((float)cos(a), (float)sin(a));
}

hipError_t launch_rope_table(float2* tab, int positions, float theta, hipStream_t s) {
  const int n = positions * kRopeFreqs;
  QV_KLAUNCH(k_rope_table, dim3((n + 255) / 256), dim3(256), 0, s, tab, positions, (double)theta);
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void k_zero(uint4* __restrict__ p, size_t n16) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride) p[i] = make_uint4(0, 0, 0, 0);
}

hipError_t launch_zero(void* p, size_t bytes, hipStream_t s) {
  const size_t n16 = bytes / 16;  // callers pass 16-byte multiples
  if (n16 == 0) return hipSuccess;
  size_t blocks = (n16 + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  QV_KLAUNCH(k_zero, dim3((unsigned)blocks), dim3(256), 0, s, reinterpret_cast<uint4*>(p), n16);
  return hipGetLastError();
}

// ----------------------------------------------------------------- LayerNorm
// One wave64 per row of NV*256 floats (width 1280 at few rows takes the
// five-wave kernel below): each lane holds NV float4.  Statistics
// in float32: mean, then the mean of squared deviations (two passes over
// registers), y = (x - mean) * rsqrt(var + eps) * g + b.
template <int NV>
__global__ __launch_bounds__(256) void k_layernorm(const float* __restrict__ x, const float* __restrict__ g,
                                                   const float* __restrict__ b, void* __restrict__ y, int bf16,
                                                   int rows, float eps) {
  constexpr int D = NV * 256;
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const float4* xr = reinterpret_cast<const float4*>(x + (size_t)row * D);
  const float4* g4 = reinterpret_cast<const float4*>(g);
  const float4* b4 = reinterpret_cast<const float4*>(b);
  float4 v[NV], gg[NV], bb[NV];
  // every load (row, gain, bias) issued up front: one memory round trip
#pragma unroll
  for (int i = 0; i < NV; ++i) v[i] = xr[i * 64 + lane];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    gg[i] = g4[i * 64 + lane];
    bb[i] = b4[i * 64 + lane];
  }
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < NV; ++i) sum += (v[i].x + v[i].y) + (v[i].z + v[i].w);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) sum += __shfl_xor(sum, o, 64);
  const float mean = sum * (1.0f / D);
  float sq = 0.f;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    v[i].x -= mean; v[i].y -= mean; v[i].z -= mean; v[i].w -= mean;
    sq += (v[i].x * v[i].x + v[i].y * v[i].y) + (v[i].z * v[i].z + v[i].w * v[i].w);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) sq += __shfl_xor(sq, o, 64);
  const float rstd = rsqrtf(sq * (1.0f / D) + eps);
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const float o0 = v[i].x * rstd * gg[i].x + bb[i].x, o1 = v[i].y * rstd * gg[i].y + bb[i].y;
    const float o2 = v[i].z * rstd * gg[i].z + bb[i].z, o3 = v[i].w * rstd * gg[i].w + bb[i].w;
    if (bf16) {
      uint2 pk;
      pk.x = f32_to_bf16_rne(o0) | ((uint32_t)f32_to_bf16_rne(o1) << 16);
      pk.y = f32_to_bf16_rne(o2) | ((uint32_t)f32_to_bf16_rne(o3) << 16);
      reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(y) + (size_t)row * D)[i * 64 + lane] = pk;
    } else {
      reinterpret_cast<float4*>(reinterpret_cast<float*>(y) + (size_t)row * D)[i * 64 + lane] =
          make_float4(o0, o1, o2, o3);
    }
  }
}

// Four bf16 values (two packed words) widened to float32 (exact).
__device__ __forceinline__ float4 bf16x4_to_f32(uint2 w) {
  return make_float4(__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xFFFF0000u), __uint_as_float(w.y << 16),
                     __uint_as_float(w.y & 0xFFFF0000u));
}

// Residual update from split-K partial sums, then LayerNorm of the result:
// x = x + ((p_0 + p_1 + ... + p_{S-1}) + pb), the bf16 partial rows widened
// and summed in that order in float32, written back; then y = LN(x) as in
// k_layernorm when g is non-null.  Same one memory round trip: the row, the
// S partial rows, pb, g and b are loaded up front.
template <int NV, int S>
__global__ __launch_bounds__(256) void k_layernorm_acc(float* __restrict__ x, const uint16_t* __restrict__ parts,
                                                       size_t part_stride, const float* __restrict__ pb,
                                                       const float* __restrict__ g, const float* __restrict__ b,
                                                       void* __restrict__ y, int bf16, int rows, float eps) {
  constexpr int D = NV * 256;
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  float4* xr = reinterpret_cast<float4*>(x + (size_t)row * D);
  float4 v[NV], acc[NV], bias[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) v[i] = xr[i * 64 + lane];
#pragma unroll
  for (int i = 0; i < NV; ++i)
    acc[i] = bf16x4_to_f32(reinterpret_cast<const uint2*>(parts + (size_t)row * D)[i * 64 + lane]);
  float4 pp[S - 1][NV];
#pragma unroll
  for (int k = 1; k < S; ++k)
#pragma unroll
    for (int i = 0; i < NV; ++i)
      pp[k - 1][i] =
          bf16x4_to_f32(reinterpret_cast<const uint2*>(parts + k * part_stride + (size_t)row * D)[i * 64 + lane]);
#pragma unroll
  for (int i = 0; i < NV; ++i) bias[i] = reinterpret_cast<const float4*>(pb)[i * 64 + lane];
  float4 gg[NV], bb[NV];
  if (g) {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      gg[i] = reinterpret_cast<const float4*>(g)[i * 64 + lane];
      bb[i] = reinterpret_cast<const float4*>(b)[i * 64 + lane];
    }
  }
#pragma unroll
  for (int k = 0; k < S - 1; ++k)
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      acc[i].x += pp[k][i].x; acc[i].y += pp[k][i].y; acc[i].z += pp[k][i].z; acc[i].w += pp[k][i].w;
    }
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    v[i].x += acc[i].x + bias[i].x; v[i].y += acc[i].y + bias[i].y;
    v[i].z += acc[i].z + bias[i].z; v[i].w += acc[i].w + bias[i].w;
    xr[i * 64 + lane] = v[i];
  }
  if (!g) return;
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < NV; ++i) sum += (v[i].x + v[i].y) + (v[i].z + v[i].w);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) sum += __shfl_xor(sum, o, 64);
  const float mean = sum * (1.0f / D);
  float sq = 0.f;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    v[i].x -= mean; v[i].y -= mean; v[i].z -= mean; v[i].w -= mean;
    sq += (v[i].x * v[i].x + v[i].y * v[i].y) + (v[i].z * v[i].z + v[i].w * v[i].w);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) sq += __shfl_xor(sq, o, 64);
  const float rstd = rsqrtf(sq * (1.0f / D) + eps);
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const float o0 = v[i].x * rstd * gg[i].x + bb[i].x, o1 = v[i].y * rstd * gg[i].y + bb[i].y;
    const float o2 = v[i].z * rstd * gg[i].z + bb[i].z, o3 = v[i].w * rstd * gg[i].w + bb[i].w;
    if (bf16) {
      uint2 pk;
      pk.x = f32_to_bf16_rne(o0) | ((uint32_t)f32_to_bf16_rne(o1) << 16);
      pk.y = f32_to_bf16_rne(o2) | ((uint32_t)f32_to_bf16_rne(o3) << 16);
      reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(y) + (size_t)row * D)[i * 64 + lane] = pk;
    } else {
      reinterpret_cast<float4*>(reinterpret_cast<float*>(y) + (size_t)row * D)[i * 64 + lane] =
          make_float4(o0, o1, o2, o3);
    }
  }
}

// Width 1280 with five waves per row (one float4 per lane), for up to
// kLnFewRows rows: at 1024 rows one wave per row leaves four waves per CU and
// the kernel waits on a single round of loads per SIMD; five times the waves
// keep five times the loads in flight (448x448: 14.4 -> 13.8 us per block
// for the two LayerNorms).  With many rows the one-wave kernels have waves
// enough and the cross-wave reduction only costs (9216 rows: +9 %).
// The row sum and the sum of squared deviations are reduced per wave, then
// over the five waves through LDS in wave order.
constexpr int kLnFewRows = 4096;
__device__ __forceinline__ float row5_sum(float v, float* red, int wave, int lane) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  if (lane == 0) red[wave] = v;
  __syncthreads();
  return (((red[0] + red[1]) + red[2]) + red[3]) + red[4];
}

__device__ __forceinline__ void row5_norm_store(float4 v, float4 gg, float4 bb, void* y, int bf16, int row, int tid,
                                                float eps, float* red, int wave, int lane) {
  constexpr int D = 1280;
  const float mean = row5_sum((v.x + v.y) + (v.z + v.w), red, wave, lane) * (1.0f / D);
  v.x -= mean; v.y -= mean; v.z -= mean; v.w -= mean;
  const float sq = row5_sum((v.x * v.x + v.y * v.y) + (v.z * v.z + v.w * v.w), red + 8, wave, lane);
  const float rstd = rsqrtf(sq * (1.0f / D) + eps);
  const float o0 = v.x * rstd * gg.x + bb.x, o1 = v.y * rstd * gg.y + bb.y;
  const float o2 = v.z * rstd * gg.z + bb.z, o3 = v.w * rstd * gg.w + bb.w;
  if (bf16) {
    uint2 pk;
    pk.x = f32_to_bf16_rne(o0) | ((uint32_t)f32_to_bf16_rne(o1) << 16);
    pk.y = f32_to_bf16_rne(o2) | ((uint32_t)f32_to_bf16_rne(o3) << 16);
    reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(y) + (size_t)row * D)[tid] = pk;
  } else {
    reinterpret_cast<float4*>(reinterpret_cast<float*>(y) + (size_t)row * D)[tid] = make_float4(o0, o1, o2, o3);
  }
}

// Cache warming beside a few-row LayerNorm: the workgroups read n16 16-byte
// chunks of p grid-stride, issued after the row's own loads (so waiting for
// those, in order, never waits for these) and folded into one word that is
// stored only through a null pointer check the host never passes (sink is
// always null), which keeps the loads without writing anything.
struct WarmArgs {
  const uint4* p;
  size_t n16;
  uint32_t* sink;
};
__device__ __forceinline__ uint32_t warm_issue(const WarmArgs& w, int tid) {
  uint32_t acc = 0;
  const size_t stride = (size_t)gridDim.x * 320;
  // four loads in flight per round (a matrix of up to 4 x 16 B per thread of
  // the grid takes one round)
  for (size_t i0 = (size_t)blockIdx.x * 320 + tid; i0 < w.n16; i0 += 4 * stride) {
    uint4 v[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const size_t i = i0 + k * stride;
      v[k] = i < w.n16 ? w.p[i] : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) acc ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
  }
  return acc;
}
__device__ __forceinline__ void warm_retire(const WarmArgs& w, uint32_t acc) {
  if (w.sink && acc == 0x9E3779B9u) *w.sink = acc;
}

__global__ __launch_bounds__(320) void k_layernorm_r5(const float* __restrict__ x, const float* __restrict__ g,
                                                      const float* __restrict__ b, void* __restrict__ y, int bf16,
                                                      float eps, WarmArgs warm) {
  __shared__ float red[16];
  const int row = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float4 v = reinterpret_cast<const float4*>(x + (size_t)row * 1280)[tid];
  const float4 gg = reinterpret_cast<const float4*>(g)[tid];
  const float4 bb = reinterpret_cast<const float4*>(b)[tid];
  const uint32_t wacc = warm_issue(warm, tid);
  row5_norm_store(v, gg, bb, y, bf16, row, tid, eps, red, wave, lane);
  warm_retire(warm, wacc);
}

template <int S>
__global__ __launch_bounds__(320) void k_layernorm_acc_r5(float* __restrict__ x, const uint16_t* __restrict__ parts,
                                                          size_t part_stride, const float* __restrict__ pb,
                                                          const float* __restrict__ g, const float* __restrict__ b,
                                                          void* __restrict__ y, int bf16, float eps, WarmArgs warm) {
  __shared__ float red[16];
  const int row = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  float4* xr = reinterpret_cast<float4*>(x + (size_t)row * 1280);
  float4 v = xr[tid];
  float4 p[S];
#pragma unroll
  for (int k = 0; k < S; ++k)
    p[k] = bf16x4_to_f32(reinterpret_cast<const uint2*>(parts + k * part_stride + (size_t)row * 1280)[tid]);
  const float4 bias = reinterpret_cast<const float4*>(pb)[tid];
  float4 gg = make_float4(0.f, 0.f, 0.f, 0.f), bb = gg;
  if (g) {
    gg = reinterpret_cast<const float4*>(g)[tid];
    bb = reinterpret_cast<const float4*>(b)[tid];
  }
  const uint32_t wacc = warm_issue(warm, tid);
  float4 acc = p[0];
#pragma unroll
  for (int k = 1; k < S; ++k) {
    acc.x += p[k].x; acc.y += p[k].y; acc.z += p[k].z; acc.w += p[k].w;
  }
  v.x += acc.x + bias.x; v.y += acc.y + bias.y; v.z += acc.z + bias.z; v.w += acc.w + bias.w;
  xr[tid] = v;
  if (g) row5_norm_store(v, gg, bb, y, bf16, row, tid, eps, red, wave, lane);  // uniform over the workgroup
  warm_retire(warm, wacc);
}

hipError_t launch_layernorm_acc(float* x, const uint16_t* parts, size_t part_stride, int splits, const float* pb,
                                const float* g, const float* b, void* y, bool bf16, int rows, int dim, float eps,
                                hipStream_t s, CacheWarm warm) {
  if (dim != 1280) return hipErrorInvalidValue;
  if (rows <= 0) return hipSuccess;
  if (rows <= kLnFewRows) {
    const dim3 grid((unsigned)rows);
    const WarmArgs wa{reinterpret_cast<const uint4*>(warm.p), warm.p ? warm.bytes / 16 : 0, nullptr};
    switch (splits) {
      case 2: QV_KLAUNCH((k_layernorm_acc_r5<2>), grid, dim3(320), 0, s, x, parts, part_stride, pb, g, b, y,
                         bf16 ? 1 : 0, eps, wa); break;
      case 4: QV_KLAUNCH((k_layernorm_acc_r5<4>), grid, dim3(320), 0, s, x, parts, part_stride, pb, g, b, y,
                         bf16 ? 1 : 0, eps, wa); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  dim3 grid((unsigned)((rows + 3) / 4));
  switch (splits) {
    case 2: QV_KLAUNCH((k_layernorm_acc<5, 2>), grid, dim3(256), 0, s, x, parts, part_stride, pb, g, b, y,
                       bf16 ? 1 : 0, rows, eps); break;
    case 4: QV_KLAUNCH((k_layernorm_acc<5, 4>), grid, dim3(256), 0, s, x, parts, part_stride, pb, g, b, y,
                       bf16 ? 1 : 0, rows, eps); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_layernorm(const float* x, const float* g, const float* b, void* y, bool bf16, int rows, int dim,
                            float eps, hipStream_t s, CacheWarm warm) {
  if (rows <= 0) return hipSuccess;
  if (dim == 1280 && rows <= kLnFewRows) {
    const WarmArgs wa{reinterpret_cast<const uint4*>(warm.p), warm.p ? warm.bytes / 16 : 0, nullptr};
    QV_KLAUNCH(k_layernorm_r5, dim3((unsigned)rows), dim3(320), 0, s, x, g, b, y, bf16 ? 1 : 0, eps, wa);
    return hipGetLastError();
  }
  dim3 grid((unsigned)((rows + 3) / 4));
  const int nv = dim / 256;
  switch (nv) {
    case 4: QV_KLAUNCH(k_layernorm<4>, grid, dim3(256), 0, s, x, g, b, y, bf16 ? 1 : 0, rows, eps); break;
    case 5: QV_KLAUNCH(k_layernorm<5>, grid, dim3(256), 0, s, x, g, b, y, bf16 ? 1 : 0, rows, eps); break;
    case 6: QV_KLAUNCH(k_layernorm<6>, grid, dim3(256), 0, s, x, g, b, y, bf16 ? 1 : 0, rows, eps); break;
    case 8: QV_KLAUNCH(k_layernorm<8>, grid, dim3(256), 0, s, x, g, b, y, bf16 ? 1 : 0, rows, eps); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace qv
