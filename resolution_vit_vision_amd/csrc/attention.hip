// Full bidirectional attention inside each image of a packed batch
// (block-diagonal by cu_seqlens), head_dim 80, flash-style: keys are
// streamed in tiles through LDS with an online softmax, so memory is linear
// in the sequence and nothing of size n^2 is stored.
//
// Layouts (written by the q/k/v projection epilogue):
//   Q     [heads][P][80]                    bf16 / f32
//   K     bf16: key-tiled [heads][P/32][10][32][8] (kc_offset); f32: [heads][P][80]
//   V^T   [heads][80][P]   (transposed so P.V reads keys contiguously)
// image i's rows start at prow0_i, a multiple of 128, and rows past an
// image's end are zero.  Output O is packed [N][ldo] with head h in columns
// 80h .. 80h+79.
//
// bf16 kernel (gfx950 MFMA, wave64): each wave owns 32 query rows of one
// (image, head) and a share of the keys.  Per 32-key tile a wave forms
// S^T = K . Q^T with v_mfma_f32_32x32x16_bf16 (5 k-steps over the 80 head
// elements, so no padding), which leaves each lane holding one query column.
// That register layout is directly the B operand of O^T = V^T . P^T, so P
// never leaves registers.  The P.V product pads the head to 96 rows (three
// 32-row MFMA blocks); row 80 of V^T is a row of ones, so O^T row 80
// accumulates the softmax denominator for free, with the same bf16-rounded P
// as the numerator.
#include "gemm_pipe.h"  // MFMA operand types, LDS-DMA pointer types, wait / barrier macros
#include "qv_internal.h"

namespace qv {

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

// Maximum of two scores.  IEEE maximum (NaN-propagating) needs no quieting of
// its inputs, unlike fmaxf, so a max of three costs one v_maximum3_f32; the
// scores are never NaN, so the result equals fmaxf's.
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }

__device__ __forceinline__ int find_plan(const PlanEntry* plan, int n_img, int gt) {
  int lo = 0, hi = n_img - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (plan[mid].qtile0 <= gt) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Work split.  A workgroup is 8 waves = QW query groups x KW key groups (two
// waves per SIMD, so one wave's softmax arithmetic overlaps the other's
// matrix work).  Wave (qw, kw) owns query rows 32 qw .. 32 qw + 31 of the
// workgroup's BQ = 32 QW rows and, of every stage of IK = 32 KW keys, the
// kw-th 32-key tile.  The partial (max, numerator, denominator) of the KW key
// groups are combined through LDS at the end.
//
// Keys stream through a ring of 4 LDS stages filled by LDS-DMA (every wave
// issues its share of each stage's 1 KB blocks three stages ahead).  A stage is
//   K   : IK / 32 key tiles x 10 chunks x 32 keys x 16 B, a verbatim copy of
//         the key-tiled global layout (kc_offset), so a wave's operand read
//         of one chunk is 32 consecutive 16-byte slots;
//   V^T : 80 dims x IK keys, 16-byte key chunks XOR-swizzled by dim so the
//         32 dims a half-wave reads land on distinct bank groups.
// V^T keys are stored permuted inside each group of 16 (bits 2 and 3 of the
// key index swapped, done by the q/k/v epilogue): the 8 keys one lane of the
// P.V operand needs are then contiguous, one 16-byte LDS read.
template <int IK>
__device__ __forceinline__ int v_swz(int d, int chunk) {
  return IK == 128 ? (chunk ^ (d & 15)) : (chunk ^ ((d >> 1) & 7));
}

template <int QW, int KW>
__global__ __launch_bounds__(512) void k_attn_bf16(AttnArgs a, float scale_log2) {
  constexpr int NWV = QW * KW;
  static_assert(NWV == 8, "eight waves");
  constexpr int BQ = 32 * QW;
  constexpr int IK = 32 * KW;                 // keys per stage
  static_assert(IK == 64 || IK == 128, "stage of 64 or 128 keys (images are padded to 128)");
  constexpr int K_SLOTS = IK * (kHeadDim / 8);    // 16-byte slots of K per stage
  constexpr int V_SLOTS = kHeadDim * (IK / 8);    // of V^T
  constexpr int STAGE_BYTES = (K_SLOTS + V_SLOTS) * 16;
  constexpr int BLKS = STAGE_BYTES / 1024;        // LDS-DMA instructions per stage
  static_assert(STAGE_BYTES % 1024 == 0, "whole KB per stage");
  constexpr int LW = BLKS / NWV;                  // per wave and stage, at least
  constexpr int LWMAX = (BLKS + NWV - 1) / NWV;
  constexpr int NST = 4;
  constexpr int COMB_FLOATS = (KW > 1 ? (KW - 1) * QW * 49 * 64 : 1);
  constexpr int LDS_BYTES = (NST * STAGE_BYTES > 4 * COMB_FLOATS) ? NST * STAGE_BYTES : 4 * COMB_FLOATS;
  __shared__ __attribute__((aligned(1024))) char lds[LDS_BYTES];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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
  const int row0 = a.out_row ? 0 : pe.row0;
  const int n = pe.n;
  const int qbase = (gt - pe.qtile0) * BQ + qw * 32;

  const uint16_t* Qh = reinterpret_cast<const uint16_t*>(a.q) + (size_t)head * a.P * kHeadDim;
  const char* Kt = reinterpret_cast<const char*>(a.k) + kc_offset(head, a.P, pe.prow0, 0) * 2;
  const char* Vh = reinterpret_cast<const char*>(a.vt) + (size_t)head * kHeadDim * a.P * 2;

  // this wave's LDS-DMA blocks of a stage: blocks wave, wave + 8, ..., as
  // byte offsets from this head's K and V^T (buffer_load ... lds: a FLAT
  // load that writes LDS would make the compiler wait for every LDS read of
  // the wave before each MFMA that needs one); the K part of a stage is a
  // whole number of 1 KB blocks, so each block is all K or all V^T
  static_assert((K_SLOTS * 16) % 1024 == 0, "K and V^T blocks do not mix");
  uint32_t goff[LWMAX];
  uint32_t ldst[LWMAX];
#pragma unroll
  for (int i = 0; i < LWMAX; ++i) {
    int blk = wave + NWV * i;
    blk = blk < BLKS ? blk : BLKS - 1;  // (only used when i < count)
    const int slot = blk * 64 + lane;
    if (slot < K_SLOTS) {
      goff[i] = (uint32_t)slot * 16;
    } else {
      const int sv = slot - K_SLOTS;
      const int d = sv / (IK / 8), p = sv % (IK / 8);
      const int c = v_swz<IK>(d, p);
      goff[i] = (uint32_t)(((size_t)d * a.P + pe.prow0 + 8 * c) * 2);
    }
    ldst[i] = (uint32_t)(blk * 1024);
  }
  const int nblk = (BLKS - wave + NWV - 1) / NWV;  // blocks this wave issues per stage
#if defined(__HIP_DEVICE_COMPILE__)
  const auto rk = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(Kt), (short)0, 0x7FFFFFFF, 0x00020000);
  const auto rv = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(Vh), (short)0, 0x7FFFFFFF, 0x00020000);
#define QV_ATTN_ISSUE(IT)                                                                                      \
  {                                                                                                            \
    char* stage_ = lds + ((IT) % NST) * STAGE_BYTES;                                                           \
    _Pragma("unroll") for (int i = 0; i < LWMAX; ++i) {                                                        \
      if (i < nblk) {                                                                                          \
        if ((int)ldst[i] < K_SLOTS * 16) /* K: IK keys x 160 B per stage, contiguous */                       \
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (las_ptr)(stage_ + ldst[i]), 16, goff[i],               \
                                                   (IT) * IK * 160, 0, 0);                                     \
        else /* V^T: IK keys along each row */                                                                 \
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (las_ptr)(stage_ + ldst[i]), 16, goff[i],               \
                                                   (IT) * IK * 2, 0, 0);                                       \
      }                                                                                                        \
    }                                                                                                          \
  }
#else
#define QV_ATTN_ISSUE(IT) {}
#endif


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

  // Software pipeline over stages: the scores S^T of stage it + 1 are formed
  // in the same basic block as the softmax and P.V of stage it, so their
  // MFMAs can overlap the exp work.  Tiles past the image are computed and
  // fully masked (they add exact zeros), which keeps every wave in one
  // instruction stream; the running max starts at a large finite negative
  // so a fully masked first tile yields p = 0, not NaN.
  // Ring of NST = 4 buffers, loads issued three stages ahead; the buffer of
  // stage it + 3 is that of stage it - 1, whose P.V every wave finished before
  // the barrier that publishes stage it + 1.
#define QV_ATTN_S(IT, SACC)                                                                                    \
  {                                                                                                            \
    const uint16_t* sK_ = reinterpret_cast<const uint16_t*>(lds + ((IT) % NST) * STAGE_BYTES) +               \
                          kw * (kHeadDim / 8) * 32 * 8;                                                        \
    _Pragma("unroll") for (int r = 0; r < 16; ++r) SACC[r] = 0.f;                                             \
    _Pragma("unroll") for (int kk = 0; kk < 5; ++kk) SACC = __builtin_amdgcn_mfma_f32_32x32x16_bf16(          \
        *reinterpret_cast<const bf16x8*>(sK_ + ((2 * kk + hlf) * 32 + l32) * 8), qf[kk], SACC, 0, 0, 0);    \
  }
#define QV_ATTN_MASK(IT, SACC)                                                                                 \
  {                                                                                                            \
    const int kb_ = (IT) * IK + kw * 32;                                                                       \
    if (kb_ + 32 > n) {                                                                                        \
      _Pragma("unroll") for (int r = 0; r < 16; ++r) {                                                        \
        const int key_ = kb_ + 8 * (r >> 2) + 4 * hlf + (r & 3);                                               \
        if (key_ >= n) SACC[r] = -INFINITY;                                                                    \
      }                                                                                                        \
    }                                                                                                          \
  }

  QV_ATTN_ISSUE(0)
  bf16x8 qf[5];
  {
    // stage 0 and this wave's q fragments are waited for together, before
    // stages 1 and 2 are issued, so the q registers are complete at a point
    // the compiler can see and no vmcnt wait for them lands in the loop
    // (where it would also drain the ring's loads)
    const uint16_t* qr = Qh + (size_t)(pe.prow0 + qbase + l32) * kHeadDim + 8 * hlf;
#pragma unroll
    for (int kk = 0; kk < 5; ++kk) qf[kk] = *reinterpret_cast<const bf16x8*>(qr + 16 * kk);
  }
  QV_WAIT_VM(0);
  QV_BARRIER();
  if (iters > 1) QV_ATTN_ISSUE(1)
  if (iters > 2) QV_ATTN_ISSUE(2)
  m_run = -1.0e30f;
  f32x16 s_cur, s_nxt;
  QV_ATTN_S(0, s_cur)
  for (int it = 0; it < iters; ++it) {
    if (it + 1 < iters) {
      if (it + 2 < iters) QV_WAIT_VM(LW);
      else QV_WAIT_VM(0);
      QV_BARRIER();
      if (it + 3 < iters) QV_ATTN_ISSUE(it + 3)
    }
    QV_ATTN_MASK(it, s_cur)
    float mx = s_cur[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = vmax(mx, s_cur[r]);
    mx = vmax(mx, __shfl_xor(mx, 32, 64));
    const float cand = mx * scale_log2;
    const bool grow = cand > m_run + kLazyLog2;
    if (__any(grow)) {
      const float m_new = grow ? cand : m_run;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);  // 0 on the first tile, 1 where kept
      m_run = m_new;
#pragma unroll
      for (int t = 0; t < 3; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[t][r] *= alpha;
    }
    // one basic block: exp of stage it, S^T of stage it + 1 (its buffer is
    // published, or unused data past the last stage), P.V of stage it
    bf16x8 pb[2];
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int e = 0; e < 8; ++e)
        pb[s2][e] = (__bf16)__builtin_amdgcn_exp2f(fmaf(s_cur[8 * s2 + e], scale_log2, -m_run));
    QV_ATTN_S(it + 1, s_nxt)
    const uint16_t* sV = reinterpret_cast<const uint16_t*>(lds + (it % NST) * STAGE_BYTES + K_SLOTS * 16);
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      const int chunk = 4 * kw + 2 * s2 + hlf;  // 8-key chunk of the stage's IK keys
#pragma unroll
      for (int t = 0; t < 3; ++t) {
        const int d = 32 * t + l32;
        bf16x8 vf;
        if (t < 2 || l32 < kHeadDim - 64)
          vf = *reinterpret_cast<const bf16x8*>(sV + d * IK + (v_swz<IK>(d, chunk) << 3));
        else
          vf = vconst;
        o[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pb[s2], o[t], 0, 0, 0);
      }
    }
    s_cur = s_nxt;
  }
#undef QV_ATTN_S
#undef QV_ATTN_MASK
#undef QV_ATTN_ISSUE

  if constexpr (KW > 1) {
    // combine the KW key groups of each query group: O = sum_w 2^(m_w - M) O_w
    float* comb = reinterpret_cast<float*>(lds);
    QV_BARRIER();  // every wave is done with the ring (all its loads were waited for)
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
    const int orow_i = a.out_row ? a.out_row[pe.prow0 + q] : row0 + q;
    uint16_t* orow = reinterpret_cast<uint16_t*>(a.o) + (size_t)orow_i * a.ldo + head * kHeadDim;
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
}

// ====================================================== long sequences
// Images of a few thousand patches and more (128 query rows per workgroup):
// NW = 4 waves of 32 queries, keys streamed 32 per stage through a 4-stage
// LDS-DMA ring (K tile 5 KB + V^T 5 KB + a 32-byte constant block holding the
// ones row, per stage), the stage index a compile-time constant of a loop
// unrolled by 4 so every LDS address is an immediate offset.  The VALU work
// of a step (16 exponentials, 8 bf16 packs, the next tile's max) is spread
// over its 11 MFMAs with sched_group_barrier: the first 8 exponentials of
// the current tile run beside the 5 score MFMAs of the next tile, the other
// 8 beside the P.V MFMAs of the first 16 keys, the max of the next tile
// beside those of the last 16 keys (2.4 % faster at n = 16,384 and 65,536
// than all 16 exponentials beside the score MFMAs, together with the
// quieting-free max).  V^T chunks are XOR-swizzled by (row >> 2) & 3 (64-byte
// rows): the 16 rows one pass of a 16-byte read touches cover all 64 banks.
// Measured against the 8-wave kernel at n = 9216 .. 65,536: +9-14 %
// (1.06-1.13 PFLOP/s).
// The occupancy request of 4 waves per SIMD is not met (168 VGPRs leave 3),
// but the schedule the compiler builds under it measured 8-10 % faster than
// with no request or a request of 3; the unmet-target warning is silenced.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Wpass-failed"
template <int NW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(4, 4))) void k_attn_long(AttnArgs a) {
  constexpr int BQ = 32 * NW;
  constexpr int IK = 32;
  constexpr int K_BYTES = IK * kHeadDim * 2;   // 5120: one 32-key tile of the key-tiled layout
  constexpr int V_BYTES = kHeadDim * IK * 2;   // 5120: V^T rows of 32 keys (64 B each)
  constexpr int CONST_OFF = K_BYTES + V_BYTES; // 32 B: eight bf16 ones, then eight zeros
  constexpr int STRIDE = CONST_OFF + 32;
  constexpr int NST = 4;
  constexpr int BLKS = (K_BYTES + V_BYTES) / 1024;  // 10 DMA blocks per stage
  constexpr int LWMAX = (BLKS + NW - 1) / NW;
  // one LDS object for the ring and the redo flags (NW ints past the ring):
  // a second __shared__ array makes the compiler wait for every LDS-DMA
  // load before each LDS read, which empties the ring
  __shared__ __attribute__((aligned(1024))) char lds[NST * STRIDE + 4 * NW];
  int* const redo_flag = reinterpret_cast<int*>(lds + NST * STRIDE);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hlf = lane >> 5, l32 = lane & 31;
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
  const int row0 = a.out_row ? 0 : pe.row0;
  const int n = pe.n;
  const int qbase = (gt - pe.qtile0) * BQ + wave * 32;

  const uint16_t* Qh = reinterpret_cast<const uint16_t*>(a.q) + (size_t)head * a.P * kHeadDim;
  const char* Kt = reinterpret_cast<const char*>(a.k) + kc_offset(head, a.P, pe.prow0, 0) * 2;
  const char* Vh = reinterpret_cast<const char*>(a.vt) + (size_t)head * kHeadDim * a.P * 2;

  // DMA sources of this wave's blocks (block wave + NW i of each stage), as
  // byte offsets from this head's K and V^T (buffer_load ... lds: a FLAT
  // load that writes LDS would make the compiler wait for every LDS read of
  // the wave before each MFMA that needs one).  K_BYTES is a whole number
  // of 1 KB blocks, so each block is all K or all V^T.
  static_assert(K_BYTES % 1024 == 0, "K and V^T blocks do not mix");
  uint32_t goff[LWMAX];
  int ldst[LWMAX];
  bool isk[LWMAX];
#pragma unroll
  for (int i = 0; i < LWMAX; ++i) {
    int blk = wave + NW * i;
    blk = blk < BLKS ? blk : BLKS - 1;
    const int slot = blk * 64 + lane;
    if (blk < K_BYTES / 1024) {  // whole blocks: the same for every lane
      goff[i] = (uint32_t)slot * 16;
      isk[i] = true;
    } else {
      const int sv = slot - K_BYTES / 16;
      const int d = sv >> 2, p = sv & 3;
      const int c = p ^ ((d >> 2) & 3);
      goff[i] = (uint32_t)(((size_t)d * a.P + pe.prow0 + 8 * c) * 2);
      isk[i] = false;
    }
    ldst[i] = blk * 1024;
  }
  const int nblk = (BLKS - wave + NW - 1) / NW;
#if defined(__HIP_DEVICE_COMPILE__)
  const auto rk = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(Kt), (short)0, 0x7FFFFFFF, 0x00020000);
  const auto rv = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(Vh), (short)0, 0x7FFFFFFF, 0x00020000);
#define QV_L_ISSUE(IT, ST)                                                                                   \
  {                                                                                                          \
    _Pragma("unroll") for (int i = 0; i < LWMAX; ++i) {                                                      \
      if (i < nblk) {                                                                                        \
        if (isk[i])                                                                                          \
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (las_ptr)(lds + (ST) * STRIDE + ldst[i]), 16, goff[i],  \
                                                   (IT) * K_BYTES, 0, 0);                                    \
        else                                                                                                 \
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (las_ptr)(lds + (ST) * STRIDE + ldst[i]), 16, goff[i],  \
                                                   (IT) * IK * 2, 0, 0);                                     \
      }                                                                                                      \
    }                                                                                                        \
  }
#else
#define QV_L_ISSUE(IT, ST) {}
#endif

  // per-lane LDS offsets (stage offsets are immediates)
  const int koff = (hlf * 32 + l32) * 16;
  int voff[2], voff2[2];
#pragma unroll
  for (int s2 = 0; s2 < 2; ++s2) {
    const int c = 2 * s2 + hlf;
    voff[s2] = K_BYTES + l32 * 64 + ((c ^ ((l32 >> 2) & 3)) << 4);
    voff2[s2] = l32 < 16 ? K_BYTES + (64 + l32) * 64 + ((c ^ ((l32 >> 2) & 3)) << 4)
                         : CONST_OFF + (l32 == 16 ? 0 : 16);
  }

  const int iters = (n + IK - 1) / IK;
  bf16x8 qf[5];

  // Ring prologue: stages 0..2 in flight, this wave's q fragments, the
  // constant block (eight bf16 ones, eight zeros) of every stage.
#define QV_L_PROLOGUE()                                                                                      \
  {                                                                                                          \
    QV_L_ISSUE(0, 0)                                                                                         \
    const uint16_t* qr = Qh + (size_t)(pe.prow0 + qbase + l32) * kHeadDim + 8 * hlf;                         \
    _Pragma("unroll") for (int kk = 0; kk < 5; ++kk) qf[kk] = *reinterpret_cast<const bf16x8*>(qr + 16 * kk); \
    if (wave == 0 && lane < 2 * NST) {                                                                       \
      const uint32_t w = (lane & 1) ? 0u : 0x3F803F80u;                                                      \
      *reinterpret_cast<uint4*>(lds + (lane >> 1) * STRIDE + CONST_OFF + 16 * (lane & 1)) =                  \
          make_uint4(w, w, w, w);                                                                            \
    }                                                                                                        \
    QV_WAIT_VM(0);                                                                                           \
    __syncthreads();                                                                                         \
    if (iters > 1) QV_L_ISSUE(1, 1)                                                                          \
    if (iters > 2) QV_L_ISSUE(2, 2)                                                                          \
  }

  f32x16 o[3];

#define QV_L_S(ST, SACC)                                                                                     \
  {                                                                                                          \
    _Pragma("unroll") for (int r = 0; r < 16; ++r) SACC[r] = 0.f;                                           \
    _Pragma("unroll") for (int kk = 0; kk < 5; ++kk) SACC = __builtin_amdgcn_mfma_f32_32x32x16_bf16(        \
        *reinterpret_cast<const bf16x8*>(lds + (ST) * STRIDE + kk * 1024 + koff), qf[kk], SACC, 0, 0, 0);   \
  }
#define QV_L_MASK(IT, SACC)                                                                                  \
  {                                                                                                          \
    const int kb_ = (IT) * IK;                                                                               \
    if (kb_ + IK > n) {                                                                                      \
      _Pragma("unroll") for (int r = 0; r < 16; ++r) {                                                      \
        const int key_ = kb_ + 8 * (r >> 2) + 4 * hlf + (r & 3);                                             \
        if (key_ >= n) SACC[r] = -INFINITY;                                                                  \
      }                                                                                                      \
    }                                                                                                        \
  }
#define QV_L_MAX(SACC, OUT)                                                                                  \
  {                                                                                                          \
    float m_ = vmax(vmax(SACC[0], SACC[1]), SACC[2]);                                                        \
    _Pragma("unroll") for (int r = 3; r < 16; r += 2) m_ = vmax(vmax(m_, SACC[r]), SACC[r + 1 < 16 ? r + 1 : r]);\
    const auto sw_ = __builtin_amdgcn_permlane32_swap(__float_as_uint(m_), __float_as_uint(m_), false, false);\
    OUT = vmax(__uint_as_float(sw_[0]), __uint_as_float(sw_[1]));                                            \
  }

  // q arrives pre-scaled by log2(e)/sqrt(80) (the q/k/v epilogue), so the
  // scores are in log2 units.  The S MFMA chain starts from C = -m_run
  // (negm: the same value in the 16 registers of a lane), so the exponent
  // argument leaves the matrix core ready for v_exp_f32.
  f32x16 s_cur, s_nxt, negm;
  float m_run;
#define QV_L_FIRST()                                                                                         \
  {                                                                                                          \
    _Pragma("unroll") for (int t = 0; t < 3; ++t)                                                            \
    _Pragma("unroll") for (int r = 0; r < 16; ++r) o[t][r] = 0.f;                                           \
    QV_L_S(0, s_cur)                                                                                         \
    QV_L_MASK(0, s_cur)                                                                                      \
    QV_L_MAX(s_cur, m_run)                                                                                   \
    _Pragma("unroll") for (int r = 0; r < 16; ++r) {                                                         \
      s_cur[r] -= m_run;                                                                                     \
      negm[r] = -m_run;                                                                                      \
    }                                                                                                        \
  }

  // one step: tile IT in stage ST (compile-time).  LAZY (compile-time): the
  // next tile's max is taken and the reference moves when a score exceeds
  // it by more than 2^kLazyLog2; otherwise the reference stays at the first
  // tile's maximum for the whole row.  Without the max the step's 24 VALU
  // instructions (16 exponentials, 8 packs) go two beside each of its 11
  // MFMAs (4 x 672x672: attention 133 -> 126 us against the schedule tuned
  // for the lazy step).
#define QV_L_STEP(IT, ST, LAZY)                                                                              \
  {                                                                                                          \
    const bool more_ = (IT) + 1 < iters;                                                                     \
    if (more_) {                                                                                             \
      if ((IT) + 2 < iters) {                                                                                \
        if (nblk == LWMAX) QV_WAIT_VM(LWMAX); else QV_WAIT_VM(LWMAX - 1);                                    \
      } else {                                                                                               \
        QV_WAIT_VM(0);                                                                                       \
      }                                                                                                      \
      QV_BARRIER();                                                                                          \
      if ((IT) + 3 < iters) QV_L_ISSUE((IT) + 3, ((ST) + 3) % NST)                                          \
    }                                                                                                        \
    bf16x8 kf_[5];                                                                                           \
    _Pragma("unroll") for (int kk = 0; kk < 5; ++kk)                                                        \
      kf_[kk] = *reinterpret_cast<const bf16x8*>(lds + (((ST) + 1) % NST) * STRIDE + kk * 1024 + koff);     \
    s_nxt = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf_[0], qf[0], negm, 0, 0, 0);                          \
    _Pragma("unroll") for (int kk = 1; kk < 5; ++kk)                                                        \
      s_nxt = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf_[kk], qf[kk], s_nxt, 0, 0, 0);                      \
    bf16x8 pb[2];                                                                                            \
    _Pragma("unroll") for (int e = 0; e < 8; ++e)                                                            \
      pb[0][e] = (__bf16)__builtin_amdgcn_exp2f(s_cur[e]);                                                   \
    bf16x8 vf_[6];                                                                                           \
    _Pragma("unroll") for (int s2 = 0; s2 < 2; ++s2)                                                         \
    _Pragma("unroll") for (int t = 0; t < 3; ++t)                                                            \
      vf_[3 * s2 + t] = *reinterpret_cast<const bf16x8*>(lds + (ST) * STRIDE +                               \
                                                       (t < 2 ? voff[s2] + t * 2048 : voff2[s2]));           \
    asm volatile("" ::"v"(pb[0]));                                                                           \
    if (LAZY) {                                                                                              \
      __builtin_amdgcn_sched_group_barrier(0x100, 5, 0);                                                     \
      __builtin_amdgcn_sched_group_barrier(0x402, 3, 0);                                                     \
      _Pragma("unroll") for (int g_ = 0; g_ < 3; ++g_) {                                                     \
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                                   \
        __builtin_amdgcn_sched_group_barrier(0x402, 3, 0);                                                   \
      }                                                                                                      \
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                                     \
      __builtin_amdgcn_sched_group_barrier(0x402, 4, 0);                                                     \
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                                     \
      __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);                                                     \
    } else {                                                                                                 \
      __builtin_amdgcn_sched_group_barrier(0x100, 5, 0);                                                     \
      __builtin_amdgcn_sched_group_barrier(0x402, 2, 0);                                                     \
      _Pragma("unroll") for (int g_ = 0; g_ < 5; ++g_) {                                                     \
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                                   \
        __builtin_amdgcn_sched_group_barrier(0x402, 2, 0);                                                   \
      }                                                                                                      \
      __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);                                                     \
    }                                                                                                        \
    if (more_) QV_L_MASK((IT) + 1, s_nxt)                                                                    \
    _Pragma("unroll") for (int t = 0; t < 3; ++t)                                                            \
      o[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf_[t], pb[0], o[t], 0, 0, 0);                          \
    _Pragma("unroll") for (int e = 0; e < 8; ++e)                                                            \
      pb[1][e] = (__bf16)__builtin_amdgcn_exp2f(s_cur[8 + e]);                                               \
    float cand_ = 0.f;                                                                                       \
    if (LAZY) QV_L_MAX(s_nxt, cand_)                                                                         \
    _Pragma("unroll") for (int t = 0; t < 3; ++t)                                                            \
      o[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf_[3 + t], pb[1], o[t], 0, 0, 0);                      \
    if (LAZY) {                                                                                              \
      _Pragma("unroll") for (int g_ = 0; g_ < 3; ++g_) {                                                     \
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                                   \
        __builtin_amdgcn_sched_group_barrier(0x402, 4, 0);                                                   \
      }                                                                                                      \
      _Pragma("unroll") for (int g_ = 0; g_ < 3; ++g_) {                                                     \
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                                   \
        __builtin_amdgcn_sched_group_barrier(0x402, 4, 0);                                                   \
      }                                                                                                      \
    } else {                                                                                                 \
      _Pragma("unroll") for (int g_ = 0; g_ < 6; ++g_) {                                                     \
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                                   \
        __builtin_amdgcn_sched_group_barrier(0x402, 2, 0);                                                   \
      }                                                                                                      \
    }                                                                                                        \
    if (LAZY) {                                                                                              \
      const bool grow_ = more_ && cand_ > kLazyLog2;                                                         \
      if (__any(grow_)) {                                                                                    \
        const float d_ = grow_ ? cand_ : 0.f;                                                                \
        const float alpha_ = __builtin_amdgcn_exp2f(-d_);                                                    \
        m_run += d_;                                                                                         \
        _Pragma("unroll") for (int t = 0; t < 3; ++t)                                                       \
        _Pragma("unroll") for (int r = 0; r < 16; ++r) o[t][r] *= alpha_;                                   \
        _Pragma("unroll") for (int r = 0; r < 16; ++r) {                                                    \
          s_nxt[r] -= d_;                                                                                    \
          negm[r] = -m_run;                                                                                  \
        }                                                                                                    \
      }                                                                                                      \
    }                                                                                                        \
    s_cur = s_nxt;                                                                                           \
  }
  // Steady step: the fast pass's step for a tile whose successor is a whole
  // tile and whose loads three tiles ahead exist (no mask, no bounds tests),
  // so the step's VALU work is its 16 exponentials and 8 packs alone and the
  // step after the barrier is one basic block for the scheduler (the general
  // step's mask test split it in two and cost two VALU instructions a step).
  // 65,536-patch block 18.30 -> 17.83 ms, 4 x 672x672 and the mixed batch
  // -2.5 %, output bit for bit the same.
#define QV_L_STEADY(IT, ST)                                                                                  \
  {                                                                                                          \
    if (nblk == LWMAX) QV_WAIT_VM(LWMAX); else QV_WAIT_VM(LWMAX - 1);                                        \
    QV_BARRIER();                                                                                            \
    QV_L_ISSUE((IT) + 3, ((ST) + 3) % NST)                                                                   \
    bf16x8 kf_[5];                                                                                           \
    _Pragma("unroll") for (int kk = 0; kk < 5; ++kk)                                                        \
      kf_[kk] = *reinterpret_cast<const bf16x8*>(lds + (((ST) + 1) % NST) * STRIDE + kk * 1024 + koff);     \
    s_nxt = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf_[0], qf[0], negm, 0, 0, 0);                          \
    _Pragma("unroll") for (int kk = 1; kk < 5; ++kk)                                                        \
      s_nxt = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf_[kk], qf[kk], s_nxt, 0, 0, 0);                      \
    bf16x8 pb[2];                                                                                            \
    _Pragma("unroll") for (int e = 0; e < 8; ++e)                                                            \
      pb[0][e] = (__bf16)__builtin_amdgcn_exp2f(s_cur[e]);                                                   \
    bf16x8 vf_[6];                                                                                           \
    _Pragma("unroll") for (int s2 = 0; s2 < 2; ++s2)                                                         \
    _Pragma("unroll") for (int t = 0; t < 3; ++t)                                                            \
      vf_[3 * s2 + t] = *reinterpret_cast<const bf16x8*>(lds + (ST) * STRIDE +                               \
                                                       (t < 2 ? voff[s2] + t * 2048 : voff2[s2]));           \
    asm volatile("" ::"v"(pb[0]));                                                                           \
    __builtin_amdgcn_sched_group_barrier(0x100, 5, 0);                                                       \
    __builtin_amdgcn_sched_group_barrier(0x402, 2, 0);                                                       \
    _Pragma("unroll") for (int g_ = 0; g_ < 5; ++g_) {                                                       \
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                                     \
      __builtin_amdgcn_sched_group_barrier(0x402, 2, 0);                                                     \
    }                                                                                                        \
    __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);                                                       \
    _Pragma("unroll") for (int t = 0; t < 3; ++t)                                                            \
      o[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf_[t], pb[0], o[t], 0, 0, 0);                          \
    _Pragma("unroll") for (int e = 0; e < 8; ++e)                                                            \
      pb[1][e] = (__bf16)__builtin_amdgcn_exp2f(s_cur[8 + e]);                                               \
    _Pragma("unroll") for (int t = 0; t < 3; ++t)                                                            \
      o[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf_[3 + t], pb[1], o[t], 0, 0, 0);                      \
    _Pragma("unroll") for (int g_ = 0; g_ < 6; ++g_) {                                                       \
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                                     \
      __builtin_amdgcn_sched_group_barrier(0x402, 2, 0);                                                     \
    }                                                                                                        \
    s_cur = s_nxt;                                                                                           \
  }
#define QV_L_LOOP_FAST()                                                                                     \
  {                                                                                                          \
    int it = 0;                                                                                              \
    for (; it + 7 <= iters; it += NST) {                                                                     \
      QV_L_STEADY(it, 0)                                                                                     \
      QV_L_STEADY(it + 1, 1)                                                                                 \
      QV_L_STEADY(it + 2, 2)                                                                                 \
      QV_L_STEADY(it + 3, 3)                                                                                 \
    }                                                                                                        \
    for (; it < iters; it += NST) {                                                                          \
      QV_L_STEP(it, 0, false)                                                                                \
      if (it + 1 >= iters) break;                                                                            \
      QV_L_STEP(it + 1, 1, false)                                                                            \
      if (it + 2 >= iters) break;                                                                            \
      QV_L_STEP(it + 2, 2, false)                                                                            \
      if (it + 3 >= iters) break;                                                                            \
      QV_L_STEP(it + 3, 3, false)                                                                            \
    }                                                                                                        \
  }
#define QV_L_LOOP(LAZY)                                                                                      \
  for (int it = 0; it < iters; it += NST) {                                                                  \
    QV_L_STEP(it, 0, LAZY)                                                                                   \
    if (it + 1 >= iters) break;                                                                              \
    QV_L_STEP(it + 1, 1, LAZY)                                                                               \
    if (it + 2 >= iters) break;                                                                              \
    QV_L_STEP(it + 2, 2, LAZY)                                                                               \
    if (it + 3 >= iters) break;                                                                              \
    QV_L_STEP(it + 3, 3, LAZY)                                                                               \
  }

  // Fast pass: the reference stays at the first key tile's maximum, so a
  // step needs no max and no rescale.  Exact up to rounding as long as no
  // exponent overflows: a score above the reference by 128 (log2 units) or
  // a sum past the float range shows up as inf / NaN in the accumulators,
  // and then the whole workgroup runs the rows again with the lazy running
  // maximum, which bounds every exponent.
  QV_L_PROLOGUE()
  QV_L_FIRST()
  QV_L_LOOP_FAST()
  {
    float chk = 0.f;
#pragma unroll
    for (int t = 0; t < 3; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) chk += o[t][r];
    const int bad = __any(!__builtin_isfinite(chk)) ? 1 : 0;  // every lane votes (not inside the lane-0 branch)
    if (lane == 0) redo_flag[wave] = bad;
    __syncthreads();
    int redo = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) redo |= redo_flag[w];
    if (redo) {
      __syncthreads();  // every wave has read the flags and finished with the ring
      QV_L_PROLOGUE()
      QV_L_FIRST()
      QV_L_LOOP(true)
    }
  }
#undef QV_L_LOOP
#undef QV_L_LOOP_FAST
#undef QV_L_STEADY
#undef QV_L_STEP
#undef QV_L_FIRST
#undef QV_L_PROLOGUE
#undef QV_L_S
#undef QV_L_MASK
#undef QV_L_MAX
#undef QV_L_ISSUE

  const float lsum = __shfl(o[2][8], l32, 64);
  const float inv = 1.0f / lsum;
  const int q = qbase + l32;
  if (q < n) {
    const int orow_i = a.out_row ? a.out_row[pe.prow0 + q] : row0 + q;
    uint16_t* orow = reinterpret_cast<uint16_t*>(a.o) + (size_t)orow_i * a.ldo + head * kHeadDim;
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
}


#pragma clang diagnostic pop


hipError_t attention_bf16(const AttnArgs& a, hipStream_t s) {
  if (a.total_qtiles == 0) return hipSuccess;
  if (a.P % 128) return hipErrorInvalidValue;
  const float scale_log2 = 1.0f;  // q is pre-scaled by log2(e)/sqrt(80)
  const dim3 grid((unsigned)a.total_qtiles * (unsigned)a.heads);
  switch (a.rows_per_wg) {
    case 128: QV_KLAUNCH((k_attn_long<4>), grid, dim3(256), 0, s, a); break;
    case 64: QV_KLAUNCH((k_attn_bf16<2, 4>), grid, dim3(512), 0, s, a, scale_log2); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// ======================================================= small windows
// Windowed blocks whose windows hold at most 64 patches (W <= 8): one
// workgroup of two waves per (window, head).  A window sits in a 64-row slot
// of the padded layout, so its keys are two 32-key tiles of the key-tiled K
// (10 KB, contiguous) and 64 columns of V^T (80 rows of 128 B, 16-byte key
// chunks XOR-swizzled by (row >> 1) & 7): one LDS-DMA round brings all of it.
// Each wave takes 32 queries, forms both score tiles with the same MFMA
// layout as the full-attention kernel, and runs an exact softmax over the 64
// scores of each query (no running max, no rescale); P.V again pads the head
// to 96 rows with row 80 a row of ones for the denominator.
__global__ __launch_bounds__(128) void k_attn_win(AttnArgs a, float scale_log2) {
  constexpr int K_BYTES = 2 * 32 * kHeadDim * 2;   // 10240
  constexpr int V_BYTES = kHeadDim * kWinSlot * 2;  // 10240
  constexpr int BLKS = (K_BYTES + V_BYTES) / 1024;  // 20 DMA blocks, 10 per wave
  __shared__ __attribute__((aligned(1024))) char lds[K_BYTES + V_BYTES];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hlf = lane >> 5, l32 = lane & 31;
  const int head = blockIdx.x % a.heads, win = blockIdx.x / a.heads;
  const PlanEntry pe = a.plan[win];  // window order
  const int n = pe.n;

  const char* Kt = reinterpret_cast<const char*>(a.k) + kc_offset(head, a.P, pe.prow0, 0) * 2;
  const char* Vh = reinterpret_cast<const char*>(a.vt) + ((size_t)head * kHeadDim * a.P + pe.prow0) * 2;
  // buffer_load ... lds, as in the kernels above (K_BYTES is whole blocks)
  static_assert(K_BYTES % 1024 == 0, "K and V^T blocks do not mix");
#if defined(__HIP_DEVICE_COMPILE__)
  const auto rk = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(Kt), (short)0, 0x7FFFFFFF, 0x00020000);
  const auto rv = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(Vh), (short)0, 0x7FFFFFFF, 0x00020000);
#pragma unroll
  for (int i = 0; i < BLKS / 2; ++i) {
    const int blk = wave + 2 * i;
    const int slot = blk * 64 + lane;  // 16-byte slot of the LDS image
    if (slot < K_BYTES / 16) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (las_ptr)(lds + blk * 1024), 16, (uint32_t)slot * 16, 0, 0, 0);
    } else {
      const int sv = slot - K_BYTES / 16;
      const int d = sv >> 3, p = sv & 7;
      const uint32_t off = (uint32_t)(((size_t)d * a.P + 8 * (p ^ ((d >> 1) & 7))) * 2);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (las_ptr)(lds + blk * 1024), 16, off, 0, 0, 0);
    }
  }
#endif
  const int q0 = 32 * wave;
  bf16x8 qf[5];
  {
    const uint16_t* qr = reinterpret_cast<const uint16_t*>(a.q) +
                         ((size_t)head * a.P + pe.prow0 + q0 + l32) * kHeadDim + 8 * hlf;
#pragma unroll
    for (int kk = 0; kk < 5; ++kk) qf[kk] = *reinterpret_cast<const bf16x8*>(qr + 16 * kk);
  }
  QV_WAIT_VM(0);
  __syncthreads();
  if (q0 >= n) return;  // no query rows for this wave (after the only barrier)

  f32x16 sc[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const uint16_t* sK = reinterpret_cast<const uint16_t*>(lds + t * (K_BYTES / 2));
#pragma unroll
    for (int r = 0; r < 16; ++r) sc[t][r] = 0.f;
#pragma unroll
    for (int kk = 0; kk < 5; ++kk)
      sc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
          *reinterpret_cast<const bf16x8*>(sK + ((2 * kk + hlf) * 32 + l32) * 8), qf[kk], sc[t], 0, 0, 0);
  }
  float mx = -INFINITY;
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = 32 * t + 8 * (r >> 2) + 4 * hlf + (r & 3);
      if (key >= n) sc[t][r] = -INFINITY;
      mx = vmax(mx, sc[t][r]);
    }
  mx = vmax(mx, __shfl_xor(mx, 32, 64));
  const float msc = mx * scale_log2;  // key 0 is always valid: mx is finite
  bf16x8 pb[2][2];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int e = 0; e < 8; ++e)
        pb[t][s2][e] = (__bf16)__builtin_amdgcn_exp2f(fmaf(sc[t][8 * s2 + e], scale_log2, -msc));

  bf16x8 vconst;
  {
    const __bf16 one = __builtin_bit_cast(__bf16, (uint16_t)(l32 == 16 ? 0x3F80 : 0));
#pragma unroll
    for (int e = 0; e < 8; ++e) vconst[e] = one;
  }
  f32x16 o[3];
#pragma unroll
  for (int t = 0; t < 3; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[t][r] = 0.f;
  const uint16_t* sV = reinterpret_cast<const uint16_t*>(lds + K_BYTES);
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      const int chunk = 4 * t + 2 * s2 + hlf;  // 8-key chunk of the 64 keys
#pragma unroll
      for (int tt = 0; tt < 3; ++tt) {
        const int d = 32 * tt + l32;
        bf16x8 vf;
        if (tt < 2 || l32 < kHeadDim - 64)
          vf = *reinterpret_cast<const bf16x8*>(sV + d * kWinSlot + ((chunk ^ ((d >> 1) & 7)) << 3));
        else
          vf = vconst;
        o[tt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pb[t][s2], o[tt], 0, 0, 0);
      }
    }
  const float lsum = __shfl(o[2][8], l32, 64);
  const float inv = 1.0f / lsum;
  const int q = q0 + l32;
  if (q < n) {
    uint16_t* orow = reinterpret_cast<uint16_t*>(a.o) + (size_t)a.out_row[pe.prow0 + q] * a.ldo + head * kHeadDim;
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
}

hipError_t attention_bf16_windows(const AttnArgs& a, hipStream_t s) {
  if (a.n_img == 0) return hipSuccess;
  if (a.P % kWinSlot || !a.out_row) return hipErrorInvalidValue;
  const float scale_log2 = 1.0f;  // q is pre-scaled by log2(e)/sqrt(80)
  QV_KLAUNCH(k_attn_win, dim3((unsigned)a.n_img * (unsigned)a.heads), dim3(128), 0, s, a, scale_log2);
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
  const int row0 = a.out_row ? 0 : pe.row0;
  const int n = pe.n;
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
    const int orow_i = a.out_row ? a.out_row[pe.prow0 + q] : row0 + q;
    float* orow = reinterpret_cast<float*>(a.o) + (size_t)orow_i * a.ldo + head * kHeadDim;
    const float inv = 1.0f / l;
#pragma unroll
    for (int d = 0; d < kHeadDim; ++d) orow[d] = acc[d] * inv;
  }
}

hipError_t attention_f32(const AttnArgs& a, hipStream_t s) {
  if (a.total_qtiles == 0) return hipSuccess;
  QV_KLAUNCH(k_attn_f32, dim3((unsigned)a.total_qtiles, (unsigned)a.heads), dim3(64), 0, s, a,
                     1.0f / sqrtf((float)kHeadDim));
  return hipGetLastError();
}

}  // namespace qv
