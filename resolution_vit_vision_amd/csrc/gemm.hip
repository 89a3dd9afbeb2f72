// C = A . B^T on gfx950 matrix cores (bf16 operands, f32 accumulation) with
// fused epilogues, plus a plain float32 tiled kernel for the correctness mode.
//
// A is [M][lda] (activations), B is [N][ldb] (a Linear weight, [out][in]);
// both are K-contiguous, so one 16-byte global load moves 8 consecutive k of
// one row.  The tower's K (1280 and 5120) runs on the multi-stage
// direct-to-LDS kernel of gemm_pipe.h; any other K (the 1176-wide patch
// embedding) on a register-staged kernel below that handles K tails: tiles of
// BK = 64 go through registers into a double-buffered LDS tile with the same
// chunk swizzle, loads for tile k+1 issued before the MFMAs of tile k.
#include <type_traits>

#include "gemm_pipe.h"
#include "qv_internal.h"

namespace qv {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// float -> bf16 bits, round to nearest even (hardware v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint16_t bf16_bits(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float act_apply(Act a, float u) {
  if (a == Act::QuickGelu) return u / (1.0f + __expf(-1.702f * u));
  if (a == Act::GeluErf) return 0.5f * u * (1.0f + erff(u * 0.70710678118654752440f));
  return u;
}

// Output position of accumulator register r of MFMA block (fm, fn) for `lane`.
#define QV_ACC_ROW(wm0, fm, r, lane) ((wm0) + (fm) * 32 + 8 * ((r) >> 2) + 4 * ((lane) >> 5) + ((r) & 3))
#define QV_ACC_COL(wn0, fn, lane) ((wn0) + (fn) * 32 + ((lane) & 31))

// ------------------------------------------------------------- epilogues
// Staged epilogue: each 32x32 MFMA block of a wave goes through a private
// 32 x 40-float LDS patch (row pitch 40 floats: the two half-waves' rows land
// 32 banks apart, and rows stay 16-byte aligned), then is read back so that
// a lane owns VEC consecutive columns of one row and writes them with one
// 16-byte (f32 x 4) or 8/16-byte (bf16) store.  Scattered 4-byte stores
// straight from the MFMA layout measured 4-8 B/clk per CU.
//
// Every global load of the epilogue (bias, residual) is issued before its
// first store.  On gfx9 the vector-memory counter covers stores as well as
// loads and completes in order, so a load issued after a store makes the
// wave wait for that store's write acknowledgement, a round trip that cost
// microseconds per 32x32 block when all workgroups store at once.
// Op interface: col_param(col) (per-column value, e.g. bias), pre(cp, v)
// (value to stage), row_param(row, col) (per-store value loaded up front,
// e.g. the residual) and store(row, col, v[VEC], rp).
struct NoRowParam {};

// Epilogue operands that do not depend on the accumulators (per-column bias,
// residual rows, token info, rotary entries) are loaded by the epilogue's
// prefetch() before the K loop when they fit in a few registers, so their
// memory latency hides under the main loop instead of opening the epilogue.
// With every epilogue load replaced by a constant the 1024-row GEMMs ran
// 0.7-1.1 us and the 65,536-row ones 20-60 us faster; the prefetch recovers
// most of that at 1024 rows and 10 us of the out-projection's 48 at 65,536.
// Where the row values do not fit, the first block's are prefetched when
// they take at most 32 registers and the next block's are loaded while the
// current block is staged and stored.  prefetch(..., active = false) loads
// nothing (waves that leave before the epilogue).
template <int VEC, class Op, int FM, int FN>
struct StagedPre {
  static constexpr int LPR = 32 / VEC;   // lanes per 32-column row
  static constexpr int RPP = 64 / LPR;   // rows per pass
  static constexpr int PASSES = 32 / RPP;
  static constexpr bool HAS_RP = Op::kRowParamFloats > 0;
  // every row value of the wave tile in at most 64 registers: all of them up front
  static constexpr bool ALL = HAS_RP && FM * FN * PASSES * Op::kRowParamFloats <= 64;
  // otherwise one block ahead, where two blocks' values leave the tile's
  // accumulators enough registers
  static constexpr bool AHEAD = HAS_RP && !ALL && FM <= 4;
  // and the first block's before the K loop when it takes at most 32 registers
  static constexpr bool FIRST = AHEAD && FN * PASSES * Op::kRowParamFloats <= 32;
  using RP = typename Op::RowParam;
  float cp[FN];
  RP rp[ALL ? FM : 1][FN][PASSES];   // AHEAD: the first block's
};

template <int VEC, class Op, int FM, int FN>
__device__ __forceinline__ void staged_rows(const Op& op, typename Op::RowParam (&dst)[FN][32 / (64 / (32 / VEC))],
                                            int rb, int wn0, int lane, int M, int N) {
  constexpr int LPR = 32 / VEC, RPP = 64 / LPR, PASSES = 32 / RPP;
  const int rl0 = lane / LPR, cl = (lane % LPR) * VEC;
#pragma unroll
  for (int fn = 0; fn < FN; ++fn)
#pragma unroll
    for (int pass = 0; pass < PASSES; ++pass) {
      const int row = rb + pass * RPP + rl0, col = wn0 + fn * 32 + cl;
      if (row < M && col < N) dst[fn][pass] = op.row_param(row, col);
    }
}

template <int VEC, class Op, int FM, int FN>
__device__ __forceinline__ StagedPre<VEC, Op, FM, FN> staged_prefetch(const Op& op, int wm0, int wn0, int lane, int M,
                                                                      int N, bool active) {
  using P = StagedPre<VEC, Op, FM, FN>;
  P p;
  if (!active) return p;
#pragma unroll
  for (int fn = 0; fn < FN; ++fn) {
    const int col = wn0 + fn * 32 + (lane & 31);
    p.cp[fn] = col < N ? op.col_param(col) : 0.f;
  }
  if constexpr (P::ALL) {
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) staged_rows<VEC, Op, FM, FN>(op, p.rp[fm], wm0 + fm * 32, wn0, lane, M, N);
  } else if constexpr (P::FIRST) {
    staged_rows<VEC, Op, FM, FN>(op, p.rp[0], wm0, wn0, lane, M, N);
  }
  return p;
}

template <int VEC, class Op, int FM, int FN>
__device__ __forceinline__ void staged_store(const Op& op, f32x16 (&acc)[FM][FN], float* wlds, int wm0, int wn0,
                                             int lane, int M, int N, const StagedPre<VEC, Op, FM, FN>& pre) {
  using P = StagedPre<VEC, Op, FM, FN>;
  using RP = typename Op::RowParam;
  constexpr int LD = 40;
  constexpr int LPR = P::LPR, RPP = P::RPP, PASSES = P::PASSES;
  const int rl0 = lane / LPR, cl = (lane % LPR) * VEC;
  RP rq[P::AHEAD ? 2 : 1][FN][PASSES];
  if constexpr (P::FIRST) {
#pragma unroll
    for (int fn = 0; fn < FN; ++fn)
#pragma unroll
      for (int pass = 0; pass < PASSES; ++pass) rq[0][fn][pass] = pre.rp[0][fn][pass];
  } else if constexpr (P::HAS_RP && !P::ALL) {
    staged_rows<VEC, Op, FM, FN>(op, rq[0], wm0, wn0, lane, M, N);
  }
#pragma unroll
  for (int fm = 0; fm < FM; ++fm) {
    // row values of the next block, issued before this block's first store
    if constexpr (P::AHEAD) {
      if (fm + 1 < FM) staged_rows<VEC, Op, FM, FN>(op, rq[(fm + 1) & 1], wm0 + (fm + 1) * 32, wn0, lane, M, N);
    } else if constexpr (P::HAS_RP && !P::ALL) {
      if (fm > 0) staged_rows<VEC, Op, FM, FN>(op, rq[0], wm0 + fm * 32, wn0, lane, M, N);
    }
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) {
      const int col0 = wn0 + fn * 32;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int rl = 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        wlds[rl * LD + (lane & 31)] = op.pre(pre.cp[fn], acc[fm][fn][r]);
      }
#pragma unroll
      for (int pass = 0; pass < PASSES; ++pass) {
        const int rl = pass * RPP + rl0;
        float v[VEC];
#pragma unroll
        for (int q = 0; q < VEC; q += 4) {
          const float4 t = *reinterpret_cast<const float4*>(&wlds[rl * LD + cl + q]);
          v[q] = t.x; v[q + 1] = t.y; v[q + 2] = t.z; v[q + 3] = t.w;
        }
        const int row = wm0 + fm * 32 + rl, col = col0 + cl;
        const RP& rp = P::ALL ? pre.rp[P::ALL ? fm : 0][fn][pass] : rq[P::AHEAD ? (fm & 1) : 0][fn][pass];
        if (row < M && col < N) op.store(row, col, v, rp);
      }
    }
  }
}

// The prefetch / apply pair of an epilogue whose values go through
// staged_store with VEC columns per lane.
#define QV_STAGED_EPILOGUE(SELF, VEC)                                                                          \
  template <int FM, int FN>                                                                                    \
  using Pre = StagedPre<VEC, SELF, FM, FN>;                                                                    \
  template <int FM, int FN, bool DEEP>                                                                         \
  __device__ __forceinline__ Pre<FM, FN> prefetch(int wm0, int wn0, int lane, int M, int N, bool active) const { \
    return staged_prefetch<VEC, SELF, FM, FN>(*this, wm0, wn0, lane, M, N, active);                            \
  }                                                                                                            \
  template <int FM, int FN>                                                                                    \
  __device__ __forceinline__ void apply_staged(f32x16 (&acc)[FM][FN], float* wlds, int wm0, int wn0, int lane,  \
                                               int M, int N, const Pre<FM, FN>& pre) const {                   \
    staged_store<VEC>(*this, acc, wlds, wm0, wn0, lane, M, N, pre);                                            \
  }

// QuickGELU for the bf16 path with a hardware reciprocal (1 ulp; the result
// is rounded to bf16).
__device__ __forceinline__ float act_apply_fast(Act a, float u) {
  // sigma(1.702 u) = 1 / (1 + 2^(-1.702 log2(e) u)); v_exp_f32 and v_rcp_f32
  if (a == Act::QuickGelu) return u * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-2.4554669595930157f * u));
  return act_apply(a, u);
}

struct EpiStoreF32 {
  static constexpr bool kStaged = true;
  static constexpr int kPatchFloats = 32 * 40;
  using RowParam = NoRowParam;
  static constexpr int kRowParamFloats = 0;
  float* C; int ldc; const float* bias;
  __device__ float col_param(int col) const { return bias ? bias[col] : 0.f; }
  __device__ float pre(float cp, float v) const { return v + cp; }
  __device__ RowParam row_param(int, int) const { return {}; }
  __device__ void store(int row, int col, const float (&v)[4], const RowParam&) const {
    *reinterpret_cast<float4*>(C + (size_t)row * ldc + col) = make_float4(v[0], v[1], v[2], v[3]);
  }
  QV_STAGED_EPILOGUE(EpiStoreF32, 4)
  template <int FM, int FN>
  __device__ void apply(f32x16 (&acc)[FM][FN], int wm0, int wn0, int lane, int M, int N) const {
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) {
      const int col = QV_ACC_COL(wn0, fn, lane);
      if (col >= N) continue;
      const float cp = col_param(col);
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = QV_ACC_ROW(wm0, fm, r, lane);
          if (row < M) C[(size_t)row * ldc + col] = pre(cp, acc[fm][fn][r]);
        }
    }
  }
};

// Split-K partial sums: run s of the K range stores its float32 tile (no
// bias) at C + s * stride; the sum over the runs, the bias and the residual
// are added later in a fixed order (launch_layernorm_acc).
struct EpiPartF32 {
  static constexpr bool kStaged = true;
  static constexpr int kPatchFloats = 32 * 40;
  using RowParam = NoRowParam;
  static constexpr int kRowParamFloats = 0;
  float* C; int ldc; size_t stride;
  __device__ float col_param(int) const { return 0.f; }
  __device__ float pre(float, float v) const { return v; }
  __device__ RowParam row_param(int, int) const { return {}; }
  __device__ void store(int row, int col, const float (&v)[4], const RowParam&) const {
    *reinterpret_cast<float4*>(C + (size_t)row * ldc + col) = make_float4(v[0], v[1], v[2], v[3]);
  }
  QV_STAGED_EPILOGUE(EpiPartF32, 4)
};

__device__ __forceinline__ EpiPartF32 epi_at_split(const EpiPartF32& e, int s) {
  EpiPartF32 r = e;
  r.C += (size_t)s * e.stride;
  return r;
}

// The same partial sums rounded once to bf16 (the tower's split-K products,
// whose runs launch_layernorm_acc adds): half the bytes written here and
// read back there.  Each run's sum is rounded as a bf16 Linear rounds its
// output; the runs, the bias and the residual are then added in float32.
struct EpiPartBf16 {
  static constexpr bool kStaged = true;
  static constexpr int kPatchFloats = 32 * 40;
  using RowParam = NoRowParam;
  static constexpr int kRowParamFloats = 0;
  uint16_t* C; int ldc; size_t stride;
  __device__ float col_param(int) const { return 0.f; }
  __device__ float pre(float, float v) const { return v; }
  __device__ RowParam row_param(int, int) const { return {}; }
  __device__ void store(int row, int col, const float (&v)[8], const RowParam&) const {
    uint4 pk;
    pk.x = pack_bf16(v[0], v[1]);
    pk.y = pack_bf16(v[2], v[3]);
    pk.z = pack_bf16(v[4], v[5]);
    pk.w = pack_bf16(v[6], v[7]);
    *reinterpret_cast<uint4*>(C + (size_t)row * ldc + col) = pk;
  }
  QV_STAGED_EPILOGUE(EpiPartBf16, 8)
};

__device__ __forceinline__ EpiPartBf16 epi_at_split(const EpiPartBf16& e, int s) {
  EpiPartBf16 r = e;
  r.C += (size_t)s * e.stride;
  return r;
}

struct EpiResidF32 {
  static constexpr bool kStaged = true;
  static constexpr int kPatchFloats = 32 * 40;
  using RowParam = float4;
  static constexpr int kRowParamFloats = 4;
  float* Z; int ldz; const float* bias;
  __device__ float col_param(int col) const { return bias[col]; }
  __device__ float pre(float cp, float v) const { return v + cp; }
  __device__ RowParam row_param(int row, int col) const {
    return *reinterpret_cast<const float4*>(Z + (size_t)row * ldz + col);
  }
  __device__ void store(int row, int col, const float (&v)[4], const RowParam& z) const {
    *reinterpret_cast<float4*>(Z + (size_t)row * ldz + col) =
        make_float4(z.x + v[0], z.y + v[1], z.z + v[2], z.w + v[3]);
  }
  QV_STAGED_EPILOGUE(EpiResidF32, 4)
  template <int FM, int FN>
  __device__ void apply(f32x16 (&acc)[FM][FN], int wm0, int wn0, int lane, int M, int N) const {
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) {
      const int col = QV_ACC_COL(wn0, fn, lane);
      if (col >= N) continue;
      const float cp = col_param(col);
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = QV_ACC_ROW(wm0, fm, r, lane);
          if (row < M) {
            float* p = Z + (size_t)row * ldz + col;
            *p = *p + pre(cp, acc[fm][fn][r]);
          }
        }
    }
  }
};

// The activation is a template parameter: a run-time switch compiled every
// activation (erf included) into each element's path.
template <Act ACT>
struct EpiActBf16 {
  static constexpr bool kStaged = true;
  static constexpr int kPatchFloats = 32 * 40;
  using RowParam = NoRowParam;
  static constexpr int kRowParamFloats = 0;
  uint16_t* C; int ldc; const float* bias;
  __device__ float col_param(int col) const { return bias[col]; }
  __device__ float pre(float cp, float v) const { return act_apply_fast(ACT, v + cp); }
  __device__ RowParam row_param(int, int) const { return {}; }
  __device__ void store(int row, int col, const float (&v)[8], const RowParam&) const {
    uint4 pk;
    pk.x = pack_bf16(v[0], v[1]);
    pk.y = pack_bf16(v[2], v[3]);
    pk.z = pack_bf16(v[4], v[5]);
    pk.w = pack_bf16(v[6], v[7]);
    *reinterpret_cast<uint4*>(C + (size_t)row * ldc + col) = pk;
  }
  QV_STAGED_EPILOGUE(EpiActBf16, 8)
  template <int FM, int FN>
  __device__ void apply(f32x16 (&acc)[FM][FN], int wm0, int wn0, int lane, int M, int N) const {
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) {
      const int col = QV_ACC_COL(wn0, fn, lane);
      if (col >= N) continue;
      const float cp = col_param(col);
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = QV_ACC_ROW(wm0, fm, r, lane);
          if (row < M) C[(size_t)row * ldc + col] = bf16_bits(pre(cp, acc[fm][fn][r]));
        }
    }
  }
};

// q/k/v projection.  The GEMM's virtual column v runs over [0, 3 dim).  In
// the q and k thirds every aligned group of 64 virtual columns holds 32
// rotation pairs: virtual column 64g + c (c < 32) is element j and 64g + 32 + c
// is element j + 40 of the same head, pair index 32g + c = 40 head + j.  The
// B-row loader applies the same map, so both halves of a pair land in the
// same lane (MFMA blocks fn and fn + 1) and the rotation needs no exchange.
// The v third is stored transposed per head ([head][80][P]) for the
// attention kernel's P.V product, with the keys of every aligned group of 16
// permuted by swapping bits 2 and 3 of the key index.
__device__ __forceinline__ int qkv_weight_row(int v, int dim) {
  if (v >= 2 * dim) return v;
  const int region = v >= dim ? 1 : 0;
  const int vv = v - region * dim;
  const int within = vv & 63;
  const int pair = ((vv >> 6) << 5) + (within & 31);
  const int head = pair / (kHeadDim / 2), j = pair % (kHeadDim / 2);
  return region * dim + head * kHeadDim + j + (within >> 5) * (kHeadDim / 2);
}

struct RowMapIdentity {
  __device__ int operator()(int r) const { return r; }
};
struct RowMapQkv {
  int dim;
  __device__ int operator()(int r) const { return qkv_weight_row(r, dim); }
};

// The rotation of a pair (x0, x1) by the angle with cs = (cos, sin), in
// explicitly fused forms: x0 cos - x1 sin and x1 cos + x0 sin each round one
// product and fuse the other, so the result does not depend on which
// product the compiler would contract in a given code layout.
__device__ __forceinline__ float rot0(float x0, float x1, float2 cs) {
#pragma clang fp contract(off)
  const float t = x1 * cs.y;
  return __builtin_fmaf(x0, cs.x, -t);
}
__device__ __forceinline__ float rot1(float x0, float x1, float2 cs) {
#pragma clang fp contract(off)
  const float t = x0 * cs.y;
  return __builtin_fmaf(x1, cs.x, t);
}

// q leaves the projection multiplied by log2(e)/sqrt(80), so the attention
// kernels' scores are already the exponent in base 2.
constexpr float kQScaleLog2 = 0.16129820911147802f;

struct EpiQkv {
  static constexpr bool kStaged = true;
  static constexpr int kPatchFloats = 32 * 72;  // q/k: 32 rows x (64 + 8) floats
  QkvOut o; const float* bias;

  // Values that do not depend on the accumulators, loaded before the K loop
  // (see staged_prefetch).  q/k waves: the bias of their rotation pairs and
  // the token info of the first 32-row block; with DEEP (waves that issue no
  // ring loads, so a dependent load costs the main loop nothing) and one
  // block per wave, that block's rotary entries too.  v waves: the bias and
  // every block's padded rows.
  template <int FM, int FN>
  struct Pre {
    static constexpr int NP = FN / 2 > 0 ? FN / 2 : 1;
    static constexpr bool TOK0 = FM <= 4;
    float b0[NP], b1[NP];
    int pos[16], prow[4];
    float2 cs[NP][16];
    float bb[FN];
    int pr[FM];
    bool has_cs;  // cs holds the first block's rotary entries (a constant once inlined)
  };

  // Rotation-pair geometry of 64-column group fp of a q/k wave tile.
  __device__ __forceinline__ void pair_at(int v0, int c, int& f0, int& fi, int& j, int& g) const {
    const int dim = o.dim;
    const int region = v0 >= dim ? 1 : 0;
    g = (v0 - region * dim) >> 6;
    const int pair = 32 * g + c;
    const int head = pair / (kHeadDim / 2);
    j = pair % (kHeadDim / 2);
    f0 = region * dim + head * kHeadDim + j;
    fi = j < kRopeFreqs ? j : j - kRopeFreqs;
  }
  __device__ __forceinline__ void load_tok(int rb, int lane, int M, int (&pos)[16], int (&prow)[4]) const {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = rb + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
      pos[r] = row < M ? o.tokinfo[row].x : 0;
    }
#pragma unroll
    for (int pass = 0; pass < 4; ++pass) {
      const int row = rb + ((pass * 64 + lane) >> 3);
      prow[pass] = row < M ? o.tokinfo[row].y : 0;
    }
  }
  template <int NP>
  __device__ __forceinline__ void load_cs(const int (&pos)[16], const int (&fi)[NP], const int (&jj)[NP],
                                          float2 (&cs)[NP][16]) const {
#pragma unroll
    for (int fp = 0; fp < NP; ++fp)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int p = jj[fp] < kRopeFreqs ? (pos[r] & 0xFFFF) : (pos[r] >> 16);
        cs[fp][r] = o.rope[p * kRopeFreqs + fi[fp]];
      }
  }

  template <int FM, int FN, bool DEEP>
  __device__ __forceinline__ Pre<FM, FN> prefetch(int wm0, int wn0, int lane, int M, int N, bool active) const {
    using P = Pre<FM, FN>;
    P p;
    if (!active) return p;
    const int c = lane & 31;
    if (wn0 < 2 * o.dim) {
      int fi[P::NP], jj[P::NP];
#pragma unroll
      for (int fp = 0; fp < P::NP; ++fp) {
        int f0, g;
        pair_at(wn0 + fp * 64, c, f0, fi[fp], jj[fp], g);
        p.b0[fp] = bias[f0];
        p.b1[fp] = bias[f0 + kHeadDim / 2];
      }
      if constexpr (P::TOK0) load_tok(wm0, lane, M, p.pos, p.prow);
      p.has_cs = DEEP && FM == 1;
      if constexpr (DEEP && FM == 1) load_cs<P::NP>(p.pos, fi, jj, p.cs);
    } else {
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) p.bb[fn] = bias[wn0 + fn * 32 + c];
#pragma unroll
      for (int fm = 0; fm < FM; ++fm) {
        const int row = wm0 + fm * 32 + 4 * (lane & 7);
        p.pr[fm] = row < M ? o.tokinfo[row].y : 0;
      }
    }
    return p;
  }

  // Staged: rotated q/k values of a 32-row block go to LDS as [row][half*32 + c]
  // and leave as 16-byte runs of 8 consecutive head elements (an aligned run
  // of 8 pairs never crosses a head, heads being 40 pairs); v goes to LDS
  // transposed [feature][row] and leaves as 8-byte runs of 4 consecutive keys
  // (a 4-aligned run of packed rows stays inside one image and maps to 4
  // contiguous key slots even after the bits-2/3 key permutation).
  // Every global load of a 32-row block is issued before that block's first
  // store, and the next block's token info before this block's rotary loads.
  template <int FM, int FN>
  __device__ __forceinline__ void apply_staged(f32x16 (&acc)[FM][FN], float* wlds, int wm0, int wn0, int lane, int M,
                                               int N, const Pre<FM, FN>& pre) const {
    using P = Pre<FM, FN>;
    const int dim = o.dim;
    const int c = lane & 31;
    if (wn0 < 2 * dim) {
      constexpr int NP = FN / 2;  // 64-column groups of rotation pairs
      int fi[NP], jj[NP], gg[NP];
#pragma unroll
      for (int fp = 0; fp < NP; ++fp) {
        int f0;
        pair_at(wn0 + fp * 64, c, f0, fi[fp], jj[fp], gg[fp]);
      }
      // token info one block ahead where two blocks' worth leaves the tile's
      // accumulators enough registers
      constexpr bool AHEAD = FM > 1 && FM <= 4;
      int pos[AHEAD ? 2 : 1][16], prow[AHEAD ? 2 : 1][4];
      if constexpr (P::TOK0) {
#pragma unroll
        for (int r = 0; r < 16; ++r) pos[0][r] = pre.pos[r];
#pragma unroll
        for (int q = 0; q < 4; ++q) prow[0][q] = pre.prow[q];
      } else {
        load_tok(wm0, lane, M, pos[0], prow[0]);
      }
#pragma unroll
      for (int fm = 0; fm < FM; ++fm) {
        const int rb = wm0 + fm * 32;
        const int cur = AHEAD ? (fm & 1) : 0;
        if constexpr (AHEAD) {
          if (fm + 1 < FM) load_tok(rb + 32, lane, M, pos[cur ^ 1], prow[cur ^ 1]);
        } else {
          if (fm > 0) load_tok(rb, lane, M, pos[0], prow[0]);
        }
        float2 cs[NP][16];
        if (FM == 1 && pre.has_cs) {
#pragma unroll
          for (int fp = 0; fp < NP; ++fp)
#pragma unroll
            for (int r = 0; r < 16; ++r) cs[fp][r] = pre.cs[fp][r];
        } else {
          load_cs<NP>(pos[cur], fi, jj, cs);
        }
#pragma unroll
        for (int fp = 0; fp < NP; ++fp) {
          const bool isk = wn0 + fp * 64 >= dim;
          uint16_t* base = reinterpret_cast<uint16_t*>(isk ? o.k : o.q);
          const float qs = isk ? 1.0f : kQScaleLog2;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int rl = 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
            const float x0 = acc[fm][2 * fp][r] + pre.b0[fp], x1 = acc[fm][2 * fp + 1][r] + pre.b1[fp];
            const bool ok = rb + rl < M;
            wlds[rl * 72 + c] = ok ? rot0(x0, x1, cs[fp][r]) * qs : 0.f;
            wlds[rl * 72 + 32 + c] = ok ? rot1(x0, x1, cs[fp][r]) * qs : 0.f;
          }
#pragma unroll
          for (int pass = 0; pass < 4; ++pass) {
            const int task = pass * 64 + lane;
            const int rl = task >> 3, h = (task >> 2) & 1, q = task & 3;
            const float4 a0 = *reinterpret_cast<const float4*>(&wlds[rl * 72 + 32 * h + 8 * q]);
            const float4 a1 = *reinterpret_cast<const float4*>(&wlds[rl * 72 + 32 * h + 8 * q + 4]);
            if (rb + rl < M) {
              const int p0 = 32 * gg[fp] + 8 * q;
              const int hd = p0 / (kHeadDim / 2), j0 = p0 % (kHeadDim / 2);
              uint4 pk;
              pk.x = pack_bf16(a0.x, a0.y);
              pk.y = pack_bf16(a0.z, a0.w);
              pk.z = pack_bf16(a1.x, a1.y);
              pk.w = pack_bf16(a1.z, a1.w);
              const int d0 = j0 + h * (kHeadDim / 2);  // 8 consecutive dims, one 16-byte chunk
              const size_t off = isk ? kc_offset(hd, o.P, prow[cur][pass], d0)
                                     : ((size_t)hd * o.P + prow[cur][pass]) * kHeadDim + d0;
              *reinterpret_cast<uint4*>(base + off) = pk;
            }
          }
        }
      }
    } else {
      uint16_t* vt = reinterpret_cast<uint16_t*>(o.vt);
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) {
        const int col0 = wn0 + fn * 32;
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) {
          const int rb = wm0 + fm * 32;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int rl = 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
            wlds[c * 36 + rl] = acc[fm][fn][r] + pre.bb[fn];
          }
          const int row = rb + 4 * (lane & 7);
          const int pp = (pre.pr[fm] & ~12) | ((pre.pr[fm] & 4) << 1) | ((pre.pr[fm] & 8) >> 1);
#pragma unroll
          for (int pass = 0; pass < 4; ++pass) {
            const int cf = pass * 8 + (lane >> 3);
            const float4 a = *reinterpret_cast<const float4*>(&wlds[cf * 36 + 4 * (lane & 7)]);
            if (row < M) {
              const int f = col0 + cf - 2 * dim;
              const int hd = f / kHeadDim, dd = f % kHeadDim;
              uint2 pk;
              pk.x = pack_bf16(a.x, a.y);
              pk.y = pack_bf16(a.z, a.w);
              *reinterpret_cast<uint2*>(vt + ((size_t)hd * kHeadDim + dd) * o.P + pp) = pk;
            }
          }
        }
      }
    }
  }
  // Direct (unstaged) form for the register-staged kernel, used when the
  // width is not one the pipelined kernel is instantiated for.
  template <int FM, int FN>
  __device__ void apply(f32x16 (&acc)[FM][FN], int wm0, int wn0, int lane, int M, int N) const {
    const int dim = o.dim;
    if (wn0 < 2 * dim) {
#pragma unroll
      for (int fp = 0; fp < FN; fp += 2) {
        const int v = QV_ACC_COL(wn0, fp, lane);
        const int region = v >= dim ? 1 : 0;
        const int vv = v - region * dim;
        const int pair = ((vv >> 6) << 5) + (vv & 31);
        const int head = pair / (kHeadDim / 2), j = pair % (kHeadDim / 2);
        const int f0 = region * dim + head * kHeadDim + j;
        const float b0 = bias[f0], b1 = bias[f0 + kHeadDim / 2];
        uint16_t* qdst = reinterpret_cast<uint16_t*>(o.q) + (size_t)head * o.P * kHeadDim + j;
        uint16_t* kdst = reinterpret_cast<uint16_t*>(o.k);
        const int fi = j < kRopeFreqs ? j : j - kRopeFreqs;
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int row = QV_ACC_ROW(wm0, fm, r, lane);
            if (row >= M) continue;
            const int2 ti = o.tokinfo[row];
            const int p = j < kRopeFreqs ? (ti.x & 0xFFFF) : (ti.x >> 16);
            const float2 cs = o.rope[p * kRopeFreqs + fi];
            const float x0 = acc[fm][fp][r] + b0, x1 = acc[fm][fp + 1][r] + b1;
            const float qs = region ? 1.0f : kQScaleLog2;
            const uint16_t y0 = bf16_bits(rot0(x0, x1, cs) * qs), y1 = bf16_bits(rot1(x0, x1, cs) * qs);
            if (region) {
              kdst[kc_offset(head, o.P, ti.y, j)] = y0;
              kdst[kc_offset(head, o.P, ti.y, j + kHeadDim / 2)] = y1;
            } else {
              uint16_t* d = qdst + (size_t)ti.y * kHeadDim;
              d[0] = y0;
              d[kHeadDim / 2] = y1;
            }
          }
      }
    } else {
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) {
        const int col = QV_ACC_COL(wn0, fn, lane);
        if (col >= N) continue;
        const int f = col - 2 * dim;
        const int head = f / kHeadDim, dd = f % kHeadDim;
        const float bb = bias[col];
        uint16_t* dst = reinterpret_cast<uint16_t*>(o.vt) + ((size_t)head * kHeadDim + dd) * o.P;
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int row = QV_ACC_ROW(wm0, fm, r, lane);
            if (row < M) {
              const int pr = o.tokinfo[row].y;
              const int pp = (pr & ~12) | ((pr & 4) << 1) | ((pr & 8) >> 1);
              dst[pp] = bf16_bits(acc[fm][fn][r] + bb);
            }
          }
      }
    }
  }
};

// ------------------------------------------------------------------ kernel
template <int BM, int BN, int WM, int WN, class Epi, class RowMap>
__global__ __launch_bounds__(256) void k_gemm_bf16(const uint16_t* __restrict__ A, int lda,
                                                   const uint16_t* __restrict__ B, int ldb, int M, int N, int K,
                                                   Epi epi, RowMap rmap) {
  constexpr int BK = 64;
  constexpr int TM = BM / WM, TN = BN / WN;
  constexpr int FM = TM / 32, FN = TN / 32;
  constexpr int ACH = BM * 8 / 256, BCH = BN * 8 / 256;
  static_assert(WM * WN == 4, "four waves");
  static_assert(FM >= 1 && FN >= 1 && ACH >= 1 && BCH >= 1, "tile too small");
  __shared__ __attribute__((aligned(16))) uint16_t sA[2][BM * BK];
  __shared__ __attribute__((aligned(16))) uint16_t sB[2][BN * BK];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int tiles_n = (N + BN - 1) / BN;
  const int tm = blockIdx.x / tiles_n, tn = blockIdx.x % tiles_n;
  const int m0 = tm * BM, n0 = tn * BN;

  const uint16_t* ap[ACH];
  int aoff[ACH], akc[ACH];
  bool aok[ACH];
#pragma unroll
  for (int i = 0; i < ACH; ++i) {
    const int id = tid + 256 * i, r = id >> 3, c = id & 7;
    const int g = m0 + r;
    aok[i] = g < M;
    ap[i] = A + (size_t)(aok[i] ? g : 0) * lda + c * 8;
    akc[i] = c * 8;
    aoff[i] = r * BK + (swz_chunk(r, c) << 3);
  }
  const uint16_t* bp[BCH];
  int boff[BCH], bkc[BCH];
  bool bok[BCH];
#pragma unroll
  for (int i = 0; i < BCH; ++i) {
    const int id = tid + 256 * i, r = id >> 3, c = id & 7;
    const int g = n0 + r;
    bok[i] = g < N;
    bp[i] = B + (size_t)rmap(bok[i] ? g : 0) * ldb + c * 8;
    bkc[i] = c * 8;
    boff[i] = r * BK + (swz_chunk(r, c) << 3);
  }

  uint4 ra[ACH], rb[BCH];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < ACH; ++i)
      ra[i] = (aok[i] && k0 + akc[i] < K) ? *reinterpret_cast<const uint4*>(ap[i] + k0) : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < BCH; ++i)
      rb[i] = (bok[i] && k0 + bkc[i] < K) ? *reinterpret_cast<const uint4*>(bp[i] + k0) : make_uint4(0, 0, 0, 0);
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < ACH; ++i) *reinterpret_cast<uint4*>(&sA[buf][aoff[i]]) = ra[i];
#pragma unroll
    for (int i = 0; i < BCH; ++i) *reinterpret_cast<uint4*>(&sB[buf][boff[i]]) = rb[i];
  };

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int KT = (K + BK - 1) / BK;
  gload(0);
  sstore(0);
  __syncthreads();
  const int arow = wm * TM + (lane & 31), brow = wn * TN + (lane & 31);
  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < KT) gload((kt + 1) * BK);
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      const int c = kk * 2 + (lane >> 5);
      bf16x8 a[FM], b[FN];
#pragma unroll
      for (int fm = 0; fm < FM; ++fm) {
        const int r = arow + fm * 32;
        a[fm] = *reinterpret_cast<const bf16x8*>(&sA[cur][r * BK + (swz_chunk(r, c) << 3)]);
      }
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) {
        const int r = brow + fn * 32;
        b[fn] = *reinterpret_cast<const bf16x8*>(&sB[cur][r * BK + (swz_chunk(r, c) << 3)]);
      }
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
          acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[fm], b[fn], acc[fm][fn], 0, 0, 0);
    }
    if (kt + 1 < KT) sstore(cur ^ 1);
    __syncthreads();
  }
  epi.apply(acc, m0 + wm * TM, n0 + wn * TN, lane, M, N);
}

// XCD cut of the tile grid over nx XCD groups (see tile_coords_in): the xgn
// in {1, 2, .., nx} whose rectangles need the fewest A + B rows per XCD, and
// the grid size (8 x the largest rectangle).
struct XcdCut {
  int xgn;
  unsigned grid;
};
static XcdCut xcd_cut(int tiles_m, int tiles_n, int BM, int BN, int nx = 8) {
  XcdCut best{1, 0};
  int64_t best_rows = -1;
  for (int xgn = 1; xgn <= nx; xgn *= 2) {
    const int xgm = nx / xgn;
    const int64_t rm = (tiles_m + xgm - 1) / xgm, rn = (tiles_n + xgn - 1) / xgn;
    const int64_t rows = rm * BM + rn * BN;
    if (best_rows < 0 || rows < best_rows) {
      best_rows = rows;
      best = XcdCut{xgn, (unsigned)(8 * rm * rn)};
    }
  }
  return best;
}

template <int BM, int BN, int WM, int WN, int ST, int KT, class Epi, class RowMap>
static hipError_t launch_pipe(const void* A, int lda, const void* B, int ldb, int M, int N, const Epi& epi,
                              RowMap rmap, hipStream_t s) {
  // the kernel addresses its operands with 32-bit byte offsets below 2 GiB
  if ((size_t)M * lda * 2 >= 0x7FFFFFFFu || (size_t)N * ldb * 2 >= 0x7FFFFFFFu) return hipErrorInvalidValue;
  const XcdCut cut = xcd_cut((M + BM - 1) / BM, (N + BN - 1) / BN, BM, BN);
  QV_KLAUNCH((k_gemm_pipe<BM, BN, WM, WN, ST, KT, Epi, RowMap>), dim3(cut.grid), dim3(WM * WN * 64),
                     0, s, reinterpret_cast<const uint16_t*>(A), lda, reinterpret_cast<const uint16_t*>(B), ldb, M, N,
                     cut.xgn, 8, epi, rmap);
  return hipGetLastError();
}

template <int BM, int BN, int WM, int WN, int ST, int KT, int NP, class Epi, class RowMap>
static hipError_t launch_ws(const void* A, int lda, const void* B, int ldb, int M, int N, const Epi& epi,
                            RowMap rmap, hipStream_t s, int splits = 1) {
  // runs that divide the 8 XCDs get XCDs of their own (one grid row);
  // otherwise the grid width is a multiple of 8, so workgroup (x, y) still
  // runs on XCD x % 8 and y is the run
  const bool xruns = splits > 1 && 8 % splits == 0;
  const XcdCut cut = xcd_cut((M + BM - 1) / BM, (N + BN - 1) / BN, BM, BN, xruns ? 8 / splits : 8);
  QV_KLAUNCH((k_gemm_ws<BM, BN, WM, WN, ST, KT, NP, Epi, RowMap>), dim3(cut.grid, xruns ? 1u : (unsigned)splits),
                     dim3((WM * WN + NP) * 64), 0,
                     s, reinterpret_cast<const uint16_t*>(A), lda, reinterpret_cast<const uint16_t*>(B), ldb, M, N,
                     cut.xgn, 8, xruns ? splits : 1, epi, rmap);
  return hipGetLastError();
}

// Tile shape by how many output tiles the problem has: 256x256 (8 waves,
// direct pipeline) when that already fills the GPU; 128x160 when N is a
// multiple of 160 and that tiling fills one wave of 256 workgroups (the
// 448x448 image's MLP up-projection: 8 x 32 tiles); 128x128 for other mid
// sizes; 64x128 when N is narrow and M small.  The 128x160, 128x128 and
// 64x128 tilings run warp-specialized (producer waves own the LDS-DMA),
// which measured 5-15% faster there; eight producers of 4 loads a stage
// each for 128x128 (q/k/v at 448x448: 21.1 us with two producers, 20.2 with
// four, 18.7 with eight), eight of 3 for 64x128 (the out-projection at
// 448x448: 14.2 us with the K range split over two groups of four waves
// that all load, 13.5 with four consumers and eight producers).  The q/k/v
// epilogue needs wave tiles whose width is a multiple of 64, which 32x160
// is not.
template <int KT, bool ALLOW160, class Epi, class RowMap>
static hipError_t run_pipe(const void* A, int lda, const void* B, int ldb, int M, int N, const Epi& epi,
                           RowMap rmap, hipStream_t s) {
  const int64_t t256 = (int64_t)((M + 255) / 256) * ((N + 255) / 256);
  const int64_t t128 = (int64_t)((M + 127) / 128) * ((N + 127) / 128);
  const int64_t t160 = (int64_t)((M + 127) / 128) * (N / 160);
  // 256 x 256 tiles keep the matrix pipes ~47 % busy against ~32 % for the
  // 128 x 128 warp-specialized kernel at these sizes, so one round of them
  // on 160 or more CUs beats about three rounds of the smaller tile
  // (4 x 672x672: fc2 5.25 -> 4.24 ms per forward at 180 tiles)
  if (t256 >= 160) {
    // Tile height 192, 256 or 320 rows (256 columns, 8 waves, 2 stages):
    // the one with the least rounds x rows x relative cost per flop, the
    // rounds counted over the 256 CUs.  Per-flop costs 1.25 / 1.00 / 0.96
    // are measured (a 192-row tile does 75 % of the work of a 256-row one in
    // 94 % of the time; a 320-row one 125 % in 120 %).  Measured choices:
    // four 672x672 images take 320 rows for q/k/v (108.6 against 113.1 us
    // with 192), 192 for the out-projection and fc2, 256 for fc1; the mixed
    // 16-image batch takes 320 everywhere (fc2 590 -> 530 us, fc1 520 ->
    // 492, step -4.5 %); 3584x3584 keeps 256.  Output bits do not depend on
    // the tiling.
    const int64_t tn = (N + 255) / 256;
    auto cost = [&](int bm, int64_t per_flop) {
      const int64_t rounds = ((M + bm - 1) / bm * tn + 255) / 256;
      return rounds * bm * per_flop;
    };
    const int64_t c192 = cost(192, 125), c256 = cost(256, 100), c320 = cost(320, 96);
    if (c192 < c256 && c192 <= c320) return launch_pipe<192, 256, 2, 4, 2, KT>(A, lda, B, ldb, M, N, epi, rmap, s);
    if (c320 < c256) return launch_pipe<320, 256, 2, 4, 2, KT>(A, lda, B, ldb, M, N, epi, rmap, s);
    return launch_pipe<256, 256, 2, 4, 2, KT>(A, lda, B, ldb, M, N, epi, rmap, s);
  }
  if constexpr (ALLOW160)
    if (N % 160 == 0 && t160 >= 192 && t160 <= 256)
      return launch_ws<128, 160, 4, 1, 4, KT, 4>(A, lda, B, ldb, M, N, epi, rmap, s);
  if (t128 >= 200) return launch_ws<128, 128, 4, 2, 4, KT, 8>(A, lda, B, ldb, M, N, epi, rmap, s);
  // few tiles: 64x128, four consumers of 32x64, eight producers
  return launch_ws<64, 128, 2, 2, 4, KT, 8>(A, lda, B, ldb, M, N, epi, rmap, s);
}

template <class Epi, class RowMap>
static hipError_t run_bf16(const void* A, int lda, const void* B, int ldb, int M, int N, int K, const Epi& epi,
                           RowMap rmap, hipStream_t s) {
  if (M <= 0 || N <= 0) return hipSuccess;
  // 16-byte rows for the LDS-DMA loads; whole 32-column groups for the staged 16-byte stores
  const bool aligned = (lda % 8 == 0) && (ldb % 8 == 0) && (N % 32 == 0);
  constexpr bool is_qkv = std::is_same<Epi, EpiQkv>::value;  // always K = dim = 1280
  if (aligned && K == 1280) return run_pipe<20, !is_qkv>(A, lda, B, ldb, M, N, epi, rmap, s);
  if constexpr (!is_qkv)
    if (aligned && K == 5120) return run_pipe<80, true>(A, lda, B, ldb, M, N, epi, rmap, s);
  // any other K (the 1176-wide patch embedding): register-staged kernel with K tails
  constexpr int BM = 128, BN = 128;
  const unsigned tiles = (unsigned)(((M + BM - 1) / BM) * ((N + BN - 1) / BN));
  QV_KLAUNCH((k_gemm_bf16<BM, BN, 2, 2, Epi, RowMap>), dim3(tiles), dim3(256), 0, s,
                     reinterpret_cast<const uint16_t*>(A), lda, reinterpret_cast<const uint16_t*>(B), ldb, M, N, K,
                     epi, rmap);
  return hipGetLastError();
}

hipError_t gemm_bf16_store_f32(const void* A, int lda, const void* B, int ldb, int M, int N, int K,
                               const float* bias, float* C, int ldc, hipStream_t s) {
  if (M <= 0 || N <= 0) return hipSuccess;
  const EpiStoreF32 e{C, ldc, bias};
  const uint16_t* a = reinterpret_cast<const uint16_t*>(A);
  const uint16_t* b = reinterpret_cast<const uint16_t*>(B);
  const unsigned t128 = (unsigned)(((M + 127) / 128) * ((N + 127) / 128));
  if (t128 >= 256) {
    QV_KLAUNCH((k_gemm_bf16<128, 128, 2, 2, EpiStoreF32, RowMapIdentity>), dim3(t128), dim3(256), 0, s, a, lda, b, ldb,
               M, N, K, e, RowMapIdentity{});
  } else {
    // too few 128 x 128 tiles to fill the GPU (the patch embedding of one
    // 448x448 image has 80): 64 x 64 tiles, several workgroups per CU
    const unsigned t64 = (unsigned)(((M + 63) / 64) * ((N + 63) / 64));
    QV_KLAUNCH((k_gemm_bf16<64, 64, 2, 2, EpiStoreF32, RowMapIdentity>), dim3(t64), dim3(256), 0, s, a, lda, b, ldb,
               M, N, K, e, RowMapIdentity{});
  }
  return hipGetLastError();
}
hipError_t gemm_bf16_resid_f32(const void* A, int lda, const void* B, int ldb, int M, int N, int K,
                               const float* bias, float* Z, int ldz, hipStream_t s) {
  return run_bf16(A, lda, B, ldb, M, N, K, EpiResidF32{Z, ldz, bias}, RowMapIdentity{}, s);
}


hipError_t gemm_bf16_splitk_f32(const void* A, int lda, const void* B, int ldb, int M, int N, int K, int splits,
                                float* P, hipStream_t s) {
  if (M <= 0 || N <= 0) return hipSuccess;
  if (splits < 1 || N % 160 || K % 64 || (K / 64) % splits || lda % 8 || ldb % 8) return hipErrorInvalidValue;
  const EpiPartF32 e{P, N, (size_t)M * N};
  // six producer waves (fc2 at 448x448: 21.5 -> 21.1 us against four); the
  // activation epilogues of the same tile keep four, which leaves their
  // consumers the registers they need without spilling
  switch (K / 64 / splits) {
    case 20: return launch_ws<128, 160, 4, 1, 4, 20, 6>(A, lda, B, ldb, M, N, e, RowMapIdentity{}, s, splits);
    case 40: return launch_ws<128, 160, 4, 1, 4, 40, 6>(A, lda, B, ldb, M, N, e, RowMapIdentity{}, s, splits);
    default: return hipErrorInvalidValue;
  }
}

hipError_t gemm_bf16_splitk_bf16(const void* A, int lda, const void* B, int ldb, int M, int N, int K, int splits,
                                 uint16_t* P, hipStream_t s) {
  if (M <= 0 || N <= 0) return hipSuccess;
  if (splits < 1 || N % 160 || K % 64 || (K / 64) % splits || lda % 8 || ldb % 8) return hipErrorInvalidValue;
  const EpiPartBf16 e{P, N, (size_t)M * N};
  switch (K / 64 / splits) {
    case 20: return launch_ws<128, 160, 4, 1, 4, 20, 6>(A, lda, B, ldb, M, N, e, RowMapIdentity{}, s, splits);
    case 40: return launch_ws<128, 160, 4, 1, 4, 40, 6>(A, lda, B, ldb, M, N, e, RowMapIdentity{}, s, splits);
    default: return hipErrorInvalidValue;
  }
}

hipError_t gemm_bf16_splitk_any_f32(const void* A, int lda, const void* B, int ldb, int M, int N, int K, int splits,
                                    float* P, hipStream_t s) {
  if (M <= 0 || N <= 0) return hipSuccess;
  if (N % 160 == 0) return gemm_bf16_splitk_f32(A, lda, B, ldb, M, N, K, splits, P, s);
  if (splits < 1 || N % 128 || K % 64 || (K / 64) % splits || lda % 8 || ldb % 8) return hipErrorInvalidValue;
  const EpiPartF32 e{P, N, (size_t)M * N};
  switch (K / 64 / splits) {
    case 10: return launch_ws<128, 128, 4, 2, 4, 10, 8>(A, lda, B, ldb, M, N, e, RowMapIdentity{}, s, splits);
    case 20: return launch_ws<128, 128, 4, 2, 4, 20, 8>(A, lda, B, ldb, M, N, e, RowMapIdentity{}, s, splits);
    case 40: return launch_ws<128, 128, 4, 2, 4, 40, 8>(A, lda, B, ldb, M, N, e, RowMapIdentity{}, s, splits);
    default: return hipErrorInvalidValue;
  }
}

// out[m][n] = bf16(act(sum over runs r = 0, 1, ... of P[r][m][n] + bias[n])),
// the runs added in index order; four columns per thread.
template <Act ACT>
__global__ __launch_bounds__(256) void k_splitk_reduce(const float* __restrict__ P, int splits, size_t stride,
                                                       const float* __restrict__ bias, uint16_t* __restrict__ out,
                                                       int ldo, int M, int N) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int n4 = N / 4;
  if (i >= (int64_t)M * n4) return;
  const int m = (int)(i / n4), c = (int)(i % n4) * 4;
  const size_t off = (size_t)m * N + c;
  float4 v = *reinterpret_cast<const float4*>(P + off);
  for (int r = 1; r < splits; ++r) {
    const float4 w = *reinterpret_cast<const float4*>(P + r * stride + off);
    v.x += w.x; v.y += w.y; v.z += w.z; v.w += w.w;
  }
  const float4 b = *reinterpret_cast<const float4*>(bias + c);
  uint2 pk;
  pk.x = pack_bf16(act_apply_fast(ACT, v.x + b.x), act_apply_fast(ACT, v.y + b.y));
  pk.y = pack_bf16(act_apply_fast(ACT, v.z + b.z), act_apply_fast(ACT, v.w + b.w));
  *reinterpret_cast<uint2*>(out + (size_t)m * ldo + c) = pk;
}

hipError_t launch_splitk_reduce(const float* P, int splits, size_t stride, const float* bias, Act act, void* out,
                                int ldo, int M, int N, hipStream_t s) {
  if (M <= 0 || N <= 0) return hipSuccess;
  if (N % 4 || ldo % 4 || !bias) return hipErrorInvalidValue;
  const int64_t n = (int64_t)M * (N / 4);
  const dim3 grid((unsigned)((n + 255) / 256));
  uint16_t* o = reinterpret_cast<uint16_t*>(out);
  switch (act) {
    case Act::GeluErf: QV_KLAUNCH(k_splitk_reduce<Act::GeluErf>, grid, dim3(256), 0, s, P, splits, stride, bias, o, ldo, M, N); break;
    case Act::QuickGelu: QV_KLAUNCH(k_splitk_reduce<Act::QuickGelu>, grid, dim3(256), 0, s, P, splits, stride, bias, o, ldo, M, N); break;
    default: QV_KLAUNCH(k_splitk_reduce<Act::None>, grid, dim3(256), 0, s, P, splits, stride, bias, o, ldo, M, N); break;
  }
  return hipGetLastError();
}

hipError_t gemm_bf16_act_bf16(const void* A, int lda, const void* B, int ldb, int M, int N, int K,
                              const float* bias, Act act, void* C, int ldc, hipStream_t s) {
  uint16_t* c = reinterpret_cast<uint16_t*>(C);
  switch (act) {
    case Act::QuickGelu:
      return run_bf16(A, lda, B, ldb, M, N, K, EpiActBf16<Act::QuickGelu>{c, ldc, bias}, RowMapIdentity{}, s);
    case Act::GeluErf:
      return run_bf16(A, lda, B, ldb, M, N, K, EpiActBf16<Act::GeluErf>{c, ldc, bias}, RowMapIdentity{}, s);
    default:
      return run_bf16(A, lda, B, ldb, M, N, K, EpiActBf16<Act::None>{c, ldc, bias}, RowMapIdentity{}, s);
  }
}
hipError_t gemm_bf16_qkv(const void* A, int lda, const void* B, int ldb, int M, int K, const float* bias,
                         const QkvOut& o, hipStream_t s) {
  return run_bf16(A, lda, B, ldb, M, 3 * o.dim, K, EpiQkv{o, bias}, RowMapQkv{o.dim}, s);
}

// ============================================== int8 weights (bf16 path)
// C[m][n] = scale[n] * sum_k A[m][k] q[n][k] with int8 q [N][ldb] and one
// float32 scale per row of q, through k_gemm_ws_i8 (codes converted to bf16
// by producer waves, scales applied to the accumulators).  Tilings: 128x128
// for q/k/v (the rotation epilogue needs 64-wide wave tiles), 128x160
// otherwise, two A-DMA and two B-convert waves each, with the K range split
// into runs when the tile count is small (the runs' partial sums then go to
// the next LayerNorm).
template <int BM, int BN, int WM, int WN, int ST, int KT, class Epi, class RowMap>
static hipError_t launch_ws_i8(const void* A, int lda, const int8_t* B, int ldb, const float* scale, int M, int N,
                               const Epi& epi, RowMap rmap, hipStream_t s, int splits = 1) {
  constexpr int NPA = 2, NPB = 2;
  // K runs spread over the XCDs as in launch_ws
  const bool xruns = splits > 1 && 8 % splits == 0;
  const XcdCut cut = xcd_cut((M + BM - 1) / BM, (N + BN - 1) / BN, BM, BN, xruns ? 8 / splits : 8);
  QV_KLAUNCH((k_gemm_ws_i8<BM, BN, WM, WN, ST, KT, NPA, NPB, Epi, RowMap>),
             dim3(cut.grid, xruns ? 1u : (unsigned)splits), dim3((WM * WN + NPA + NPB) * 64), 0, s,
             reinterpret_cast<const uint16_t*>(A), lda, B, ldb, scale, M, N, cut.xgn, 8, xruns ? splits : 1, epi,
             rmap);
  return hipGetLastError();
}

static bool i8_shape_ok(const void* A, int lda, int ldb, int N, int K, int nmul) {
  return A && lda % 8 == 0 && ldb % 16 == 0 && N % nmul == 0 && K % 64 == 0;
}

hipError_t gemm_i8w_qkv(const void* A, int lda, const int8_t* B, int ldb, const float* scale, int M, int K,
                        const float* bias, const QkvOut& o, hipStream_t s) {
  if (M <= 0) return hipSuccess;
  if (!i8_shape_ok(A, lda, ldb, 3 * o.dim, K, 128) || K != 1280) return hipErrorInvalidValue;
  return launch_ws_i8<128, 128, 4, 2, 4, 20>(A, lda, B, ldb, scale, M, 3 * o.dim, EpiQkv{o, bias},
                                                RowMapQkv{o.dim}, s);
}

hipError_t gemm_i8w_act_bf16(const void* A, int lda, const int8_t* B, int ldb, const float* scale, int M, int N,
                             int K, const float* bias, Act act, void* C, int ldc, hipStream_t s) {
  if (M <= 0 || N <= 0) return hipSuccess;
  if (!i8_shape_ok(A, lda, ldb, N, K, 160) || K != 1280 || act != Act::QuickGelu) return hipErrorInvalidValue;
  return launch_ws_i8<128, 160, 4, 1, 4, 20>(A, lda, B, ldb, scale, M, N,
                                                EpiActBf16<Act::QuickGelu>{(uint16_t*)C, ldc, bias},
                                                RowMapIdentity{}, s);
}


hipError_t gemm_i8w_splitk_bf16(const void* A, int lda, const int8_t* B, int ldb, const float* scale, int M, int N,
                                int K, int splits, uint16_t* P, hipStream_t s) {
  if (M <= 0 || N <= 0) return hipSuccess;
  if (!i8_shape_ok(A, lda, ldb, N, K, 160) || (splits != 2 && splits != 4) || (K / 64) % splits)
    return hipErrorInvalidValue;
  const EpiPartBf16 e{P, N, (size_t)M * N};
  switch (K / 64 / splits) {
    case 20: return launch_ws_i8<128, 160, 4, 1, 4, 20>(A, lda, B, ldb, scale, M, N, e, RowMapIdentity{}, s, splits);
    case 10: return launch_ws_i8<128, 160, 4, 1, 4, 10>(A, lda, B, ldb, scale, M, N, e, RowMapIdentity{}, s, splits);
    case 5: return launch_ws_i8<128, 160, 4, 1, 4, 5>(A, lda, B, ldb, scale, M, N, e, RowMapIdentity{}, s, splits);
    default: return hipErrorInvalidValue;
  }
}

hipError_t gemm_i8w_resid_f32(const void* A, int lda, const int8_t* B, int ldb, const float* scale, int M, int N,
                              int K, const float* bias, float* Z, int ldz, hipStream_t s) {
  if (M <= 0 || N <= 0) return hipSuccess;
  if (!i8_shape_ok(A, lda, ldb, N, K, 160)) return hipErrorInvalidValue;
  const EpiResidF32 e{Z, ldz, bias};
  switch (K / 64) {
    case 20: return launch_ws_i8<128, 160, 4, 1, 4, 20>(A, lda, B, ldb, scale, M, N, e, RowMapIdentity{}, s);
    case 80: return launch_ws_i8<128, 160, 4, 1, 4, 80>(A, lda, B, ldb, scale, M, N, e, RowMapIdentity{}, s);
    default: return hipErrorInvalidValue;
  }
}

// Large M: where bf16 uses 256 x 256 tiles (enough of them to fill the
// GPU), the int8 codes of one matrix are first widened to bf16 in workspace
// (exact) and multiplied by that kernel; the row scales go onto the float32
// sums through this wrapper, so the result is the same function as above.
template <class Inner, class RowMap>
struct EpiColScale {
  static constexpr bool kStaged = Inner::kStaged;
  static constexpr int kPatchFloats = Inner::kPatchFloats;
  Inner in;
  const float* scale;
  RowMap rm;
  template <int FM, int FN>
  __device__ __forceinline__ void scale_acc(f32x16 (&acc)[FM][FN], int wn0, int lane, int N) const {
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) {
      const int col = QV_ACC_COL(wn0, fn, lane);
      const float sc = col < N ? scale[rm(col)] : 0.f;
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[fm][fn][r] *= sc;
    }
  }
  // the column scales and the inner epilogue's values, before the K loop
  template <int FM, int FN>
  struct Pre {
    typename Inner::template Pre<FM, FN> in;
    float sc[FN];
  };
  template <int FM, int FN, bool DEEP>
  __device__ __forceinline__ Pre<FM, FN> prefetch(int wm0, int wn0, int lane, int M, int N, bool active) const {
    Pre<FM, FN> p;
    if (!active) return p;
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) {
      const int col = QV_ACC_COL(wn0, fn, lane);
      p.sc[fn] = col < N ? scale[rm(col)] : 0.f;
    }
    p.in = in.template prefetch<FM, FN, DEEP>(wm0, wn0, lane, M, N, true);
    return p;
  }
  template <int FM, int FN>
  __device__ __forceinline__ void apply_staged(f32x16 (&acc)[FM][FN], float* wlds, int wm0, int wn0, int lane, int M,
                                               int N, const Pre<FM, FN>& pre) const {
#pragma unroll
    for (int fn = 0; fn < FN; ++fn)
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[fm][fn][r] *= pre.sc[fn];
    in.apply_staged(acc, wlds, wm0, wn0, lane, M, N, pre.in);
  }
  template <int FM, int FN>
  __device__ __forceinline__ void apply(f32x16 (&acc)[FM][FN], int wm0, int wn0, int lane, int M, int N) const {
    scale_acc(acc, wn0, lane, N);
    in.apply(acc, wm0, wn0, lane, M, N);
  }
};


template <int KT, class Epi, class RowMap>
static hipError_t launch_i8_wide(const void* A, int lda, const void* codes, int ldb, const float* scale, int M, int N,
                                 const Epi& epi, RowMap rmap, hipStream_t s) {
  return launch_pipe<256, 256, 2, 4, 2, KT>(A, lda, codes, ldb, M, N, EpiColScale<Epi, RowMap>{epi, scale, rmap},
                                            rmap, s);
}

hipError_t gemm_i8w_wide_qkv(const void* A, int lda, const void* codes, int ldb, const float* scale, int M, int K,
                             const float* bias, const QkvOut& o, hipStream_t s) {
  if (M <= 0) return hipSuccess;
  if (!A || lda % 8 || ldb % 8 || K != 1280) return hipErrorInvalidValue;
  return launch_i8_wide<20>(A, lda, codes, ldb, scale, M, 3 * o.dim, EpiQkv{o, bias}, RowMapQkv{o.dim}, s);
}

hipError_t gemm_i8w_wide_act_bf16(const void* A, int lda, const void* codes, int ldb, const float* scale, int M,
                                  int N, int K, const float* bias, Act act, void* C, int ldc, hipStream_t s) {
  if (M <= 0 || N <= 0) return hipSuccess;
  if (!A || lda % 8 || ldb % 8 || N % 32 || K != 1280 || act != Act::QuickGelu) return hipErrorInvalidValue;
  return launch_i8_wide<20>(A, lda, codes, ldb, scale, M, N, EpiActBf16<Act::QuickGelu>{(uint16_t*)C, ldc, bias},
                            RowMapIdentity{}, s);
}

hipError_t gemm_i8w_wide_resid_f32(const void* A, int lda, const void* codes, int ldb, const float* scale, int M,
                                   int N, int K, const float* bias, float* Z, int ldz, hipStream_t s) {
  if (M <= 0 || N <= 0) return hipSuccess;
  if (!A || lda % 8 || ldb % 8 || N % 32) return hipErrorInvalidValue;
  const EpiResidF32 e{Z, ldz, bias};
  switch (K) {
    case 1280: return launch_i8_wide<20>(A, lda, codes, ldb, scale, M, N, e, RowMapIdentity{}, s);
    case 5120: return launch_i8_wide<80>(A, lda, codes, ldb, scale, M, N, e, RowMapIdentity{}, s);
    default: return hipErrorInvalidValue;
  }
}

// int8 codes -> bf16 (exact): 16 codes per thread.
__global__ __launch_bounds__(256) void k_codes_bf16(const int8_t* __restrict__ q, int64_t n16,
                                                    uint16_t* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n16) return;
  const uint4 w = reinterpret_cast<const uint4*>(q)[i];
  const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
  uint32_t pk[8];
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    pk[2 * d] = pack_bf16_pair((float)(int8_t)wd[d], (float)(int8_t)(wd[d] >> 8));
    pk[2 * d + 1] = pack_bf16_pair((float)(int8_t)(wd[d] >> 16), (float)((int32_t)wd[d] >> 24));
  }
  uint4* o = reinterpret_cast<uint4*>(out) + 2 * i;
  o[0] = make_uint4(pk[0], pk[1], pk[2], pk[3]);
  o[1] = make_uint4(pk[4], pk[5], pk[6], pk[7]);
}

hipError_t launch_codes_bf16(const int8_t* q, int64_t n, void* out, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  if (n % 16) return hipErrorInvalidValue;
  const int64_t n16 = n / 16;
  QV_KLAUNCH(k_codes_bf16, dim3((unsigned)((n16 + 255) / 256)), dim3(256), 0, s, q, n16,
             reinterpret_cast<uint16_t*>(out));
  return hipGetLastError();
}

// Symmetric per-row int8: scale = max|w| / 127 (1 for an all-zero row),
// q = round half to even of w / scale clamped to +-127, all in float32.
// One 256-thread workgroup per row.
__global__ __launch_bounds__(256) void k_quantize_i8(const void* __restrict__ w, int cols, int ld, int bf16,
                                                     int8_t* __restrict__ q, float* __restrict__ scale) {
  const int row = blockIdx.x;
  const int tid = threadIdx.x;
  auto load = [&](int c) -> float {
    const size_t i = (size_t)row * ld + c;
    return bf16 ? __builtin_bit_cast(float, (uint32_t)reinterpret_cast<const uint16_t*>(w)[i] << 16)
                : reinterpret_cast<const float*>(w)[i];
  };
  float amax = 0.f;
  for (int c = tid; c < cols; c += 256) amax = fmaxf(amax, fabsf(load(c)));
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
  __shared__ float wmax[4];
  if ((tid & 63) == 0) wmax[tid >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  const float sc = amax > 0.f ? amax / 127.0f : 1.0f;
  if (tid == 0) scale[row] = sc;
  for (int c = tid; c < cols; c += 256) {
    float v = __builtin_rintf(load(c) / sc);
    v = fminf(fmaxf(v, -127.f), 127.f);
    q[(size_t)row * cols + c] = (int8_t)(int)v;
  }
}

hipError_t launch_quantize_i8(const void* w, int rows, int cols, int ld, bool bf16, int8_t* q, float* scale,
                              hipStream_t s) {
  if (rows <= 0 || cols <= 0) return hipSuccess;
  QV_KLAUNCH(k_quantize_i8, dim3((unsigned)rows), dim3(256), 0, s, w, cols, ld, bf16 ? 1 : 0, q, scale);
  return hipGetLastError();
}

// =================================================== float32 (correctness)
// 64 x 64 output tile, 256 threads with 4 x 4 outputs each, BK = 16.
template <class Epi>
__global__ __launch_bounds__(256) void k_gemm_f32(const float* __restrict__ A, int lda, const float* __restrict__ B,
                                                  int ldb, int M, int N, int K, Epi epi) {
  __shared__ float sA[16][65];
  __shared__ float sB[16][65];
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int tiles_n = (N + 63) / 64;
  const int m0 = (blockIdx.x / tiles_n) * 64, n0 = (blockIdx.x % tiles_n) * 64;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += 16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int id = tid + 256 * i, r = id >> 4, k = id & 15;
      const int gm = m0 + r, gn = n0 + r, gk = k0 + k;
      sA[k][r] = (gm < M && gk < K) ? A[(size_t)gm * lda + gk] : 0.f;
      sB[k][r] = (gn < N && gk < K) ? B[(size_t)gn * ldb + gk] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) { a[i] = sA[k][ty + 16 * i]; b[i] = sB[k][tx + 16 * i]; }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = m0 + ty + 16 * i, col = n0 + tx + 16 * j;
      if (row < M && col < N) epi(row, col, acc[i][j]);
    }
}

struct F32Store {
  float* C; int ldc; const float* bias;
  __device__ void operator()(int r, int c, float v) const { C[(size_t)r * ldc + c] = v + (bias ? bias[c] : 0.f); }
};
struct F32Resid {
  float* Z; int ldz; const float* bias;
  __device__ void operator()(int r, int c, float v) const {
    float* p = Z + (size_t)r * ldz + c;
    *p = *p + (v + bias[c]);
  }
};
struct F32Act {
  float* C; int ldc; const float* bias; Act act;
  __device__ void operator()(int r, int c, float v) const { C[(size_t)r * ldc + c] = act_apply(act, v + bias[c]); }
};

template <class Epi>
static hipError_t run_f32(const float* A, int lda, const float* B, int ldb, int M, int N, int K, const Epi& e,
                          hipStream_t s) {
  if (M <= 0 || N <= 0) return hipSuccess;
  const unsigned tiles = (unsigned)(((M + 63) / 64) * ((N + 63) / 64));
  QV_KLAUNCH(k_gemm_f32<Epi>, dim3(tiles), dim3(256), 0, s, A, lda, B, ldb, M, N, K, e);
  return hipGetLastError();
}

hipError_t gemm_f32_store(const float* A, int lda, const float* B, int ldb, int M, int N, int K, const float* bias,
                          float* C, int ldc, hipStream_t s) {
  return run_f32(A, lda, B, ldb, M, N, K, F32Store{C, ldc, bias}, s);
}
hipError_t gemm_f32_resid(const float* A, int lda, const float* B, int ldb, int M, int N, int K, const float* bias,
                          float* Z, int ldz, hipStream_t s) {
  return run_f32(A, lda, B, ldb, M, N, K, F32Resid{Z, ldz, bias}, s);
}
hipError_t gemm_f32_act(const float* A, int lda, const float* B, int ldb, int M, int N, int K, const float* bias,
                        Act act, float* C, int ldc, hipStream_t s) {
  return run_f32(A, lda, B, ldb, M, N, K, F32Act{C, ldc, bias, act}, s);
}

// qkv [M][3 dim] (bias already added) -> rotated q, k and transposed v in the
// padded per-head layouts.  One thread per (row, pair) for q and k and per
// (row, element) for v.
__global__ __launch_bounds__(256) void k_rope_scatter_f32(const float* __restrict__ qkv, int M, QkvOut o) {
  const int dim = o.dim;
  const int per_row = 2 * dim;  // dim/2 pairs of q, dim/2 pairs of k, dim elements of v
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (int64_t)M * per_row) return;
  const int row = (int)(gid / per_row), c = (int)(gid % per_row);
  const int2 ti = o.tokinfo[row];
  const float* src = qkv + (size_t)row * 3 * dim;
  if (c < dim) {
    const int region = c / (dim / 2), pair = c % (dim / 2);
    const int head = pair / (kHeadDim / 2), j = pair % (kHeadDim / 2);
    const int f0 = region * dim + head * kHeadDim + j;
    const float x0 = src[f0], x1 = src[f0 + kHeadDim / 2];
    const int p = j < kRopeFreqs ? (ti.x & 0xFFFF) : (ti.x >> 16);
    const float2 cs = o.rope[p * kRopeFreqs + (j < kRopeFreqs ? j : j - kRopeFreqs)];
    float* dst = reinterpret_cast<float*>(region ? o.k : o.q) + ((size_t)head * o.P + ti.y) * kHeadDim + j;
    dst[0] = x0 * cs.x - x1 * cs.y;
    dst[kHeadDim / 2] = x1 * cs.x + x0 * cs.y;
  } else {
    const int f = c - dim;
    const int head = f / kHeadDim, dd = f % kHeadDim;
    reinterpret_cast<float*>(o.vt)[((size_t)head * kHeadDim + dd) * o.P + ti.y] = src[2 * dim + f];
  }
}

hipError_t rope_scatter_f32(const float* qkv, int M, const float*, const QkvOut& o, hipStream_t s) {
  const int64_t n = (int64_t)M * 2 * o.dim;
  if (n == 0) return hipSuccess;
  QV_KLAUNCH(k_rope_scatter_f32, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, qkv, M, o);
  return hipGetLastError();
}

}  // namespace qv
