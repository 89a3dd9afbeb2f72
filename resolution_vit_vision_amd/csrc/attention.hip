// Full bidirectional attention inside each image of a packed batch
// (block-diagonal by cu_seqlens), head_dim 80, flash-style: keys are
// streamed in tiles through LDS with an online softmax, so memory is linear
// in the sequence and nothing of size n^2 is stored.
//
// Layouts (written by the q/k/v projection epilogue):
//   Q, K  [heads][P][80]   bf16/f32, image i's rows start at prow0_i
//   V^T   [heads][80][P]   (transposed so P.V reads keys contiguously)
// prow0_i is a multiple of 128 and rows past an image's end are zero.
// Output O is packed [N][ldo] with head h in columns 80h .. 80h+79.
//
// bf16 kernel (gfx950 MFMA, wave64): each wave owns 32 query rows of one
// (image, head) and a share of the keys.  Per 32-key block a wave forms
// S^T = K . Q^T with v_mfma_f32_32x32x16_bf16 (5 k-steps over the 80 head
// elements, so no padding), which leaves each lane holding one query column.
// That register layout is directly the B operand of O^T = V^T . P^T, so P
// never leaves registers.  The P.V product pads the head to 96 rows (three
// 32-row MFMA blocks); row 80 of V^T is a row of ones, so O^T row 80
// accumulates the softmax denominator for free, with the same bf16-rounded P
// as the numerator.
#include "qv_internal.h"

namespace qv {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef float f32x16 __attribute__((ext_vector_type(16)));

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two floats to packed bf16, round to nearest even (one v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  const bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// The running reference of the online softmax only moves when a score
// exceeds it by more than 2^kLazyLog2 (scores in log2 units).  Numerator and
// denominator share the reference, so the result does not depend on it; the
// rescale of the 48 O accumulators then happens once or twice per row
// instead of every key block, and P stays <= 2^kLazyLog2 (safe in bf16/f32).
constexpr float kLazyLog2 = 8.0f;

__device__ __forceinline__ int find_plan(const PlanEntry* plan, int n_img, int gt) {
  int lo = 0, hi = n_img - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (plan[mid].qtile0 <= gt) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Work split.  A workgroup is 4 waves = QW query groups x KW key groups.
// Wave (qw, kw) owns query rows 32 qw .. 32 qw + 31 of the workgroup's tile
// and, in every iteration, the kw-th sub-tile of KT keys of the KW * KT keys
// staged in LDS.  With KW > 1 the partial (max, numerator, denominator) of
// the KW key groups are combined through LDS at the end, so short images
// still give the GPU enough workgroups.
//
// V^T keys are stored permuted inside each group of 16 (bits 2 and 3 of the
// key index swapped, done by the q/k/v epilogue): the 8 keys one lane of the
// P.V operand needs are then contiguous, one 16-byte LDS read.
template <int KT>
__device__ __forceinline__ int v_swz(int d, int chunk) {
  return KT == 32 ? (chunk ^ ((d >> 2) & 3)) : (chunk ^ ((d >> 1) & 7));
}

template <int KW, int KT>
__global__ __launch_bounds__(256) void k_attn_bf16(AttnArgs a, float scale_log2) {
  constexpr int QW = 4 / KW;
  constexpr int BQ = 32 * QW;
  constexpr int IK = KW * KT;             // keys staged per iteration
  constexpr int NCH = IK * kHeadDim / 8;  // 16-byte chunks of K (and of V^T) per iteration
  constexpr int PER_T = (NCH + 255) / 256;
  constexpr int SB = KT / 32;             // 32-key S^T blocks per wave sub-tile
  // LDS: K rows of 80 elements, then V^T as [kw][80][KT]; reused for the combine
  constexpr int K_ELEMS = IK * kHeadDim;
  constexpr int V_ELEMS = KW * kHeadDim * KT;
  constexpr int COMB_FLOATS = (KW > 1 ? (KW - 1) * QW * 49 * 64 : 1);
  constexpr int LDS_BYTES = (2 * (K_ELEMS + V_ELEMS) > 4 * COMB_FLOATS) ? 2 * (K_ELEMS + V_ELEMS) : 4 * COMB_FLOATS;
  __shared__ __attribute__((aligned(16))) char lds[LDS_BYTES];
  uint16_t* sK = reinterpret_cast<uint16_t*>(lds);
  uint16_t* sV = sK + K_ELEMS;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hlf = lane >> 5, l32 = lane & 31;
  const int qw = wave / KW, kw = wave % KW;
  // Flat grid over (head, q-tile).  Workgroup b runs on XCD b % 8; when the
  // heads divide evenly, XCD x gets heads [x*H/8, (x+1)*H/8) so each L2 keeps
  // the K and V of only its own heads.
  int head, gt;
  {
    const int b = blockIdx.x, T = a.total_qtiles;
    if (a.heads % 8 == 0) {
      const int hpx = a.heads / 8, local = b / 8;
      head = (b % 8) * hpx + local / T;
      gt = local % T;
    } else {
      head = b / T;
      gt = b % T;
    }
  }
  const PlanEntry pe = a.plan[find_plan(a.plan, a.n_img, gt)];
  const int row0 = a.cu_seqlens[pe.img];
  const int n = a.cu_seqlens[pe.img + 1] - row0;
  const int qbase = (gt - pe.qtile0) * BQ + qw * 32;

  const uint16_t* Qh = reinterpret_cast<const uint16_t*>(a.q) + (size_t)head * a.P * kHeadDim;
  const uint16_t* Kh = reinterpret_cast<const uint16_t*>(a.k) + (size_t)head * a.P * kHeadDim;
  const uint16_t* Vh = reinterpret_cast<const uint16_t*>(a.vt) + (size_t)head * kHeadDim * a.P;

  bf16x8 qf[5];
  {
    const uint16_t* qr = Qh + (size_t)(pe.prow0 + qbase + l32) * kHeadDim + 8 * hlf;
#pragma unroll
    for (int kk = 0; kk < 5; ++kk) qf[kk] = *reinterpret_cast<const bf16x8*>(qr + 16 * kk);
  }

  uint4 rk[PER_T], rv[PER_T];
#pragma unroll
  for (int i = 0; i < PER_T; ++i) rk[i] = rv[i] = make_uint4(0, 0, 0, 0);
#define QV_ATTN_GLOAD(IT)                                                                                  \
  {                                                                                                        \
    const int key0 = pe.prow0 + (IT) * IK;                                                                 \
    _Pragma("unroll") for (int i = 0; i < PER_T; ++i) {                                                    \
      const int c = tid + 256 * i;                                                                         \
      if (NCH % 256 == 0 || c < NCH) {                                                                     \
        rk[i] = *reinterpret_cast<const uint4*>(Kh + (size_t)(key0 + c / 10) * kHeadDim + (c % 10) * 8);  \
        const int d = c / (IK / 8), g = c % (IK / 8);                                                      \
        rv[i] = *reinterpret_cast<const uint4*>(Vh + (size_t)d * a.P + key0 + g * 8);                      \
      }                                                                                                    \
    }                                                                                                      \
  }
#define QV_ATTN_SSTORE()                                                                                   \
  {                                                                                                        \
    _Pragma("unroll") for (int i = 0; i < PER_T; ++i) {                                                    \
      const int c = tid + 256 * i;                                                                         \
      if (NCH % 256 == 0 || c < NCH) {                                                                     \
        *reinterpret_cast<uint4*>(&sK[(c / 10) * kHeadDim + (c % 10) * 8]) = rk[i];                        \
        const int d = c / (IK / 8), g = c % (IK / 8);                                                      \
        const int w = g / (KT / 8), cc = g % (KT / 8);                                                     \
        *reinterpret_cast<uint4*>(&sV[(w * kHeadDim + d) * KT + (v_swz<KT>(d, cc) << 3)]) = rv[i];         \
      }                                                                                                    \
    }                                                                                                      \
  }

  f32x16 o[3];
#pragma unroll
  for (int t = 0; t < 3; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[t][r] = 0.f;
  float m_run = -INFINITY;

  bf16x8 vconst;
  {
    const __bf16 one = __builtin_bit_cast(__bf16, (uint16_t)(l32 == 16 ? 0x3F80 : 0));
#pragma unroll
    for (int e = 0; e < 8; ++e) vconst[e] = one;
  }

  const int iters = (n + IK - 1) / IK;
  QV_ATTN_GLOAD(0)
  for (int it = 0; it < iters; ++it) {
    __syncthreads();
    QV_ATTN_SSTORE()
    __syncthreads();
    if (it + 1 < iters) QV_ATTN_GLOAD(it + 1)
    const int kb = it * IK + kw * KT;  // first key of this wave's sub-tile
    if (kb >= n) continue;             // wave-uniform: sub-tile entirely past the image

    f32x16 s[SB];
#pragma unroll
    for (int sb = 0; sb < SB; ++sb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[sb][r] = 0.f;
      const uint16_t* kr = &sK[(kw * KT + 32 * sb + l32) * kHeadDim + 8 * hlf];
#pragma unroll
      for (int kk = 0; kk < 5; ++kk)
        s[sb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8*>(kr + 16 * kk), qf[kk],
                                                         s[sb], 0, 0, 0);
    }
    if (kb + KT > n) {
#pragma unroll
      for (int sb = 0; sb < SB; ++sb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kb + 32 * sb + 8 * (r >> 2) + 4 * hlf + (r & 3);
          if (key >= n) s[sb][r] = -INFINITY;
        }
    }
    float mx = s[0][0];
#pragma unroll
    for (int sb = 0; sb < SB; ++sb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[sb][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float cand = mx * scale_log2;
    const bool grow = cand > m_run + kLazyLog2;  // first block: m_run = -inf
    if (__any(grow)) {
      const float m_new = grow ? cand : m_run;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);  // 0 on the first block, 1 where kept
      m_run = m_new;
#pragma unroll
      for (int t = 0; t < 3; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[t][r] *= alpha;
    }

#pragma unroll
    for (int sb = 0; sb < SB; ++sb)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        bf16x8 pb;
#pragma unroll
        for (int e = 0; e < 8; ++e)
          pb[e] = (__bf16)__builtin_amdgcn_exp2f(fmaf(s[sb][8 * s2 + e], scale_log2, -m_run));
        const int chunk = 4 * sb + 2 * s2 + hlf;
#pragma unroll
        for (int t = 0; t < 3; ++t) {
          const int d = 32 * t + l32;
          bf16x8 vf;
          if (t < 2 || l32 < kHeadDim - 64)
            vf = *reinterpret_cast<const bf16x8*>(&sV[(kw * kHeadDim + d) * KT + (v_swz<KT>(d, chunk) << 3)]);
          else
            vf = vconst;
          o[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pb, o[t], 0, 0, 0);
        }
      }
  }

  if constexpr (KW > 1) {
    // combine the KW key groups of each query group: O = sum_w 2^(m_w - M) O_w
    float* comb = reinterpret_cast<float*>(lds);
    __syncthreads();
    if (kw > 0) {
      float* dst = comb + ((kw - 1) * QW + qw) * 49 * 64;
#pragma unroll
      for (int t = 0; t < 3; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) dst[(t * 16 + r) * 64 + lane] = o[t][r];
      dst[48 * 64 + lane] = m_run;
    }
    __syncthreads();
    if (kw > 0) return;
    float mw[KW];
    mw[0] = m_run;
    float M = m_run;
#pragma unroll
    for (int w = 1; w < KW; ++w) {
      mw[w] = comb[((w - 1) * QW + qw) * 49 * 64 + 48 * 64 + lane];
      M = fmaxf(M, mw[w]);
    }
    const float s0 = __builtin_amdgcn_exp2f(mw[0] - M);
#pragma unroll
    for (int t = 0; t < 3; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[t][r] *= s0;
#pragma unroll
    for (int w = 1; w < KW; ++w) {
      const float sw = __builtin_amdgcn_exp2f(mw[w] - M);
      const float* src = comb + ((w - 1) * QW + qw) * 49 * 64;
#pragma unroll
      for (int t = 0; t < 3; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[t][r] = fmaf(src[(t * 16 + r) * 64 + lane], sw, o[t][r]);
    }
  }

  // O^T row 80 (block 2, local row 16) = register 8 of the lower half-wave
  const float lsum = __shfl(o[2][8], l32, 64);
  const float inv = 1.0f / lsum;
  const int q = qbase + l32;
  if (q < n) {
    uint16_t* orow = reinterpret_cast<uint16_t*>(a.o) + (size_t)(row0 + q) * a.ldo + head * kHeadDim;
#pragma unroll
    for (int t = 0; t < 3; ++t)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * t + 8 * g + 4 * hlf;
        if (d0 < kHeadDim) {
          uint2 pk;
          pk.x = pack_bf16(o[t][4 * g] * inv, o[t][4 * g + 1] * inv);
          pk.y = pack_bf16(o[t][4 * g + 2] * inv, o[t][4 * g + 3] * inv);
          *reinterpret_cast<uint2*>(orow + d0) = pk;
        }
      }
  }
#undef QV_ATTN_GLOAD
#undef QV_ATTN_SSTORE
}

int attention_bf16_rows_per_wg(int64_t wgs_at_128) {
  // enough workgroups for two per CU: split keys across waves when the
  // 128-row tiling leaves the GPU under-filled
  if (wgs_at_128 >= 512) return 128;
  if (wgs_at_128 * 2 >= 512) return 64;
  return 32;
}

hipError_t attention_bf16(const AttnArgs& a, hipStream_t s) {
  if (a.total_qtiles == 0) return hipSuccess;
  const float scale_log2 = 1.4426950408889634f / sqrtf((float)kHeadDim);
  const dim3 grid((unsigned)a.total_qtiles * (unsigned)a.heads);
  switch (a.rows_per_wg) {
    case 128: hipLaunchKernelGGL((k_attn_bf16<1, 64>), grid, dim3(256), 0, s, a, scale_log2); break;
    case 64: hipLaunchKernelGGL((k_attn_bf16<2, 32>), grid, dim3(256), 0, s, a, scale_log2); break;
    case 32: hipLaunchKernelGGL((k_attn_bf16<4, 32>), grid, dim3(256), 0, s, a, scale_log2); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// ============================================================ float32 mode
// One wave per (64 query rows, head); one query row per lane with the full
// head vector and accumulator in registers; 32-key tiles in LDS; exact exp.
constexpr int FBQ = 64, FBK = 32;

__global__ __launch_bounds__(64) void k_attn_f32(AttnArgs a, float scale) {
  __shared__ float sK[FBK][kHeadDim + 1];
  __shared__ float sV[kHeadDim][FBK + 1];
  const int lane = threadIdx.x;
  const int head = blockIdx.y, gt = blockIdx.x;
  const PlanEntry pe = a.plan[find_plan(a.plan, a.n_img, gt)];
  const int row0 = a.cu_seqlens[pe.img];
  const int n = a.cu_seqlens[pe.img + 1] - row0;
  const int q = (gt - pe.qtile0) * FBQ + lane;
  const float* Qh = reinterpret_cast<const float*>(a.q) + (size_t)head * a.P * kHeadDim;
  const float* Kh = reinterpret_cast<const float*>(a.k) + (size_t)head * a.P * kHeadDim;
  const float* Vh = reinterpret_cast<const float*>(a.vt) + (size_t)head * kHeadDim * a.P;
  float qv[kHeadDim], acc[kHeadDim];
#pragma unroll
  for (int d = 0; d < kHeadDim; ++d) {
    qv[d] = Qh[(size_t)(pe.prow0 + q) * kHeadDim + d] * scale;
    acc[d] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  for (int k0 = 0; k0 < n; k0 += FBK) {
    for (int i = lane; i < FBK * kHeadDim; i += 64) {
      const int r = i / kHeadDim, d = i % kHeadDim;
      sK[r][d] = Kh[(size_t)(pe.prow0 + k0 + r) * kHeadDim + d];
      const int dd = i / FBK, c = i % FBK;
      sV[dd][c] = Vh[(size_t)dd * a.P + pe.prow0 + k0 + c];
    }
    __syncthreads();
    const int nk = n - k0 < FBK ? n - k0 : FBK;
    float sc[FBK];
    float mt = -INFINITY;
    for (int c = 0; c < FBK; ++c) {
      float dot = 0.f;
#pragma unroll
      for (int d = 0; d < kHeadDim; ++d) dot = fmaf(qv[d], sK[c][d], dot);
      sc[c] = c < nk ? dot : -INFINITY;
      mt = fmaxf(mt, sc[c]);
    }
    const float mn = fmaxf(m, mt);
    const float corr = expf(m - mn);
    l *= corr;
#pragma unroll
    for (int d = 0; d < kHeadDim; ++d) acc[d] *= corr;
    for (int c = 0; c < FBK; ++c) {
      const float p = expf(sc[c] - mn);
      l += p;
#pragma unroll
      for (int d = 0; d < kHeadDim; ++d) acc[d] = fmaf(p, sV[d][c], acc[d]);
    }
    m = mn;
    __syncthreads();
  }
  if (q < n) {
    float* orow = reinterpret_cast<float*>(a.o) + (size_t)(row0 + q) * a.ldo + head * kHeadDim;
    const float inv = 1.0f / l;
#pragma unroll
    for (int d = 0; d < kHeadDim; ++d) orow[d] = acc[d] * inv;
  }
}

hipError_t attention_f32(const AttnArgs& a, hipStream_t s) {
  if (a.total_qtiles == 0) return hipSuccess;
  hipLaunchKernelGGL(k_attn_f32, dim3((unsigned)a.total_qtiles, (unsigned)a.heads), dim3(64), 0, s, a,
                     1.0f / sqrtf((float)kHeadDim));
  return hipGetLastError();
}

}  // namespace qv
