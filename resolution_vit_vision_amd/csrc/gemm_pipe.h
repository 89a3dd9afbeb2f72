// Multi-stage C = A . B^T for gfx950 with direct global->LDS loads.
//
// Each stage holds a BM x 64 tile of A and a BN x 64 tile of B (bf16, row =
// 128 bytes of 8 16-byte chunks).  Tiles are fetched by LDS-DMA
// (buffer_load_dwordx4 ... lds, or global_load_lds_dwordx4 in waves that
// never read LDS): one instruction moves 64 lanes x 16 bytes into 1 KB of
// LDS at the wave-uniform base (lane l lands at base + 16 l), so the LDS
// layout is chosen by which global chunk each lane fetches.  The layout is
// row-major with the chunk index XOR-ed by (row >> 1) & 7: the operand reads
// of v_mfma_f32_32x32x16_bf16 (32 consecutive rows, one 16-byte chunk per
// lane, two chunks per wave) then hit 64 distinct banks per 16 lanes.
//
// STAGES buffers form a ring; loads for tile kt + STAGES - 1 are issued
// right after the barrier that opens tile kt, so STAGES - 1 tiles are in
// flight while one is consumed.  The waits are explicit vmcnt counts (each
// wave waits for its own loads of the tile, then the barrier publishes all
// waves' loads); the ring uses one __shared__ array per stage and a
// statically unrolled loop so that every LDS access names its stage.
#pragma once

#include "qv_internal.h"

namespace qv {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef const __attribute__((address_space(1))) void* gas_ptr;
typedef __attribute__((address_space(3))) void* las_ptr;

// s_waitcnt with vmcnt <= n and no constraint on the other counters (gfx9 encoding).
#define QV_WAIT_VM(n) \
  __builtin_amdgcn_s_waitcnt(((n) & 0xF) | 0x70 | 0xF00 | ((((n) >> 4) & 3) << 14))
// Workgroup barrier without the memory fence __syncthreads() implies (which
// would wait for every load in flight); compiler-level ordering is kept.
#define QV_BARRIER()                      \
  do {                                    \
    asm volatile("" ::: "memory");        \
    __builtin_amdgcn_s_barrier();         \
    asm volatile("" ::: "memory");        \
  } while (0)

__device__ __forceinline__ int swz_chunk(int row, int chunk) { return chunk ^ ((row >> 1) & 7); }

// WM x WN waves share one LDS ring of STAGES 64-deep k-tiles of A and B.
template <int BM_, int BN_, int WM, int WN, int STAGES>
struct PipeCfg {
  static constexpr int BM = BM_, BN = BN_;
  static constexpr int NW = WM * WN;
  static constexpr int NT = NW * 64;
  static constexpr int BK = 64;
  static constexpr int TM = BM_ / WM, TN = BN_ / WN;
  static constexpr int FM = TM / 32, FN = TN / 32;
  static constexpr int STAGE_ELEMS = (BM_ + BN_) * BK;        // bf16 elements per stage (A, then B)
  static constexpr int LOADS_A = BM_ * 8 / NT;                // 16-byte chunks per thread per stage
  static constexpr int LOADS_B = BN_ * 8 / NT;
  static constexpr int LOADS = LOADS_A + LOADS_B;             // vmcnt of one stage per wave
  static_assert(FM >= 1 && FN >= 1, "wave tile at least 32x32");
  static_assert(STAGES >= 2 && STAGES <= 8, "2..8 stages");
};

// The loads are buffer_load ... lds (MUBUF) rather than global_load_lds:
// the compiler counts a FLAT instruction that writes LDS as both a memory
// and an LDS access, and while one is in flight it waits for every LDS read
// of the wave (lgkmcnt(0)) before the first MFMA of a step; with the buffer
// form the waits name only the fragments each MFMA needs.  Offsets are
// 32-bit bytes from each matrix's base (every operand is below 2 GiB; the
// host checks).
template <class C>
struct PipeState {
  uint32_t voff[C::LOADS];      // byte offset of this thread's chunk at step 0 from its matrix's base
  uint32_t ldst[C::LOADS];      // wave-uniform LDS byte offset of the 1 KB block inside a stage
  uint32_t amask;               // bit i: load i reads A (wave-uniform)
  const void* abase;
  const void* bbase;
};

template <class C, class RowMap>
__device__ __forceinline__ void pipe_setup(PipeState<C>& ps, const uint16_t* A, int lda, const uint16_t* B, int ldb,
                                           int M, int N, int m0, int n0, RowMap rmap, int wave, int lane) {
  static_assert(C::BM * 8 % C::NT == 0 && C::BN * 8 % C::NT == 0, "whole 1 KB chunks per wave");
#pragma unroll
  for (int i = 0; i < C::LOADS; ++i) {
    // 1 KB block index inside the stage: A blocks first, then B blocks
    const int blk = i * C::NW + wave;
    const int p = blk * 64 + lane;              // 16-byte slot inside the stage
    const bool isA = p < C::BM * 8;
    const int q = isA ? p : p - C::BM * 8;
    const int r = q >> 3;                       // tile row
    const int c = swz_chunk(r, q & 7);          // logical k chunk stored at this slot
    if (isA) {
      int g = m0 + r;
      g = g < M ? g : M - 1;
      ps.voff[i] = (uint32_t)(((size_t)g * lda + c * 8) * 2);
    } else {
      int g = n0 + r;
      g = g < N ? g : N - 1;
      ps.voff[i] = (uint32_t)(((size_t)rmap(g) * ldb + c * 8) * 2);
    }
    ps.ldst[i] = (uint32_t)(blk * 1024);
  }
  uint32_t am = 0;
#pragma unroll
  for (int i = 0; i < C::LOADS; ++i)
    if ((i * C::NW + wave) * 64 < C::BM * 8) am |= 1u << i;
  ps.amask = am;
  ps.abase = A;
  ps.bbase = B;
}

template <class C>
__device__ __forceinline__ void pipe_issue(const PipeState<C>& ps, uint16_t* stage, int kt) {
  // device pass only: the buffer-resource type exists for the GPU target alone
#if defined(__HIP_DEVICE_COMPILE__)
  const auto ra = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(ps.abase), (short)0, 0x7FFFFFFF, 0x00020000);
  const auto rb = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(ps.bbase), (short)0, 0x7FFFFFFF, 0x00020000);
#pragma unroll
  for (int i = 0; i < C::LOADS; ++i) {
    char* dst = reinterpret_cast<char*>(stage) + ps.ldst[i];
    if ((ps.amask >> i) & 1u)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (las_ptr)dst, 16, ps.voff[i], kt * 128, 0, 0);
    else
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (las_ptr)dst, 16, ps.voff[i], kt * 128, 0, 0);
  }
#endif
}

// Operand fragments are software-pipelined: the LDS reads of k-step kk + 1
// are issued before the MFMAs of k-step kk (the scheduler is fenced so it
// cannot hoist the MFMAs above them), so LDS latency overlaps matrix work.
template <class C>
__device__ __forceinline__ void pipe_read(const uint16_t* stage, bf16x8 (&a)[C::FM], bf16x8 (&b)[C::FN], int kk,
                                          int arow, int brow, int lane) {
  const uint16_t* sA = stage;
  const uint16_t* sB = stage + C::BM * C::BK;
  const int c = kk * 2 + (lane >> 5);
#pragma unroll
  for (int fm = 0; fm < C::FM; ++fm) {
    const int r = arow + fm * 32;
    a[fm] = *reinterpret_cast<const bf16x8*>(&sA[r * C::BK + (swz_chunk(r, c) << 3)]);
  }
#pragma unroll
  for (int fn = 0; fn < C::FN; ++fn) {
    const int r = brow + fn * 32;
    b[fn] = *reinterpret_cast<const bf16x8*>(&sB[r * C::BK + (swz_chunk(r, c) << 3)]);
  }
}

template <class C>
__device__ __forceinline__ void pipe_compute(const uint16_t* stage, f32x16 (&acc)[C::FM][C::FN], int wm, int wn,
                                             int lane) {
  const int arow = wm * C::TM + (lane & 31), brow = wn * C::TN + (lane & 31);
  constexpr int KS = C::BK / 16;
  bf16x8 a[2][C::FM], b[2][C::FN];
  pipe_read<C>(stage, a[0], b[0], 0, arow, brow, lane);
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) {
    if (kk + 1 < KS) pipe_read<C>(stage, a[(kk + 1) & 1], b[(kk + 1) & 1], kk + 1, arow, brow, lane);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < C::FN; ++fn)
        acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[kk & 1][fm], b[kk & 1][fn], acc[fm][fn], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Tile order.  Workgroups are dispatched round-robin over the 8 XCDs
// (workgroup b runs on XCD b % 8), and each XCD fills its own L2 from the
// Infinity Cache / HBM.  The tile grid is cut into an xgm x xgn grid of
// rectangles (xgm * xgn = 8), one per XCD, so an XCD fetches only the A rows
// and B rows of its rectangle; the host picks the cut that minimizes those
// bytes (tm_rows * BM + tn_cols * BN per XCD).  Inside a rectangle tiles go in
// groups of `group` row tiles sweeping the column tiles, so the panels in
// flight are shared by concurrent workgroups.  Rectangles differ by at most
// one row / column tile; the grid has 8 x (largest rectangle) workgroups and
// the surplus ones of smaller rectangles return at once (valid = false).
// tile_coords_in cuts the grid over nx XCD groups (xgm * xgn = nx) and
// returns tile i of group x's rectangle.
__device__ __forceinline__ bool tile_coords_in(int x, int i, int nx, int tiles_m, int tiles_n, int xgn, int group,
                                               int& tm, int& tn) {
  const int xgm = nx / xgn;
  const int gx = x / xgn, gy = x % xgn;
  const int tm0 = gx * tiles_m / xgm, tm1 = (gx + 1) * tiles_m / xgm;
  const int tn0 = gy * tiles_n / xgn, tn1 = (gy + 1) * tiles_n / xgn;
  const int rm = tm1 - tm0, rn = tn1 - tn0;
  if (i >= rm * rn) return false;
  const int per_group = group * rn;
  const int g = i / per_group, first = g * group;
  const int gsz = (rm - first) < group ? (rm - first) : group;
  const int r = i % per_group;
  tm = tm0 + first + r % gsz;
  tn = tn0 + r / gsz;
  return true;
}

__device__ __forceinline__ bool tile_coords(int bid, int tiles_m, int tiles_n, int xgn, int group, int& tm,
                                            int& tn) {
  return tile_coords_in(bid % 8, bid / 8, 8, tiles_m, tiles_n, xgn, group, tm, tn);
}

// Statically unrolled K loop: with no loop-carried merge point the compiler
// knows exactly which stage each LDS-DMA wrote, so the only waits are the
// explicit per-tile vmcnt counts.
template <class C, int KT, int STAGES>
struct PipeSteps {
  template <int kt>
  static __device__ __forceinline__ void run(uint16_t* const (&st)[8], const PipeState<C>& ps,
                                             f32x16 (&acc)[C::FM][C::FN], int wm, int wn, int lane) {
    if constexpr (kt < KT) {
      constexpr int later = (KT - 1 - kt) < (STAGES - 2) ? (KT - 1 - kt) : (STAGES - 2);
      QV_WAIT_VM(later * C::LOADS);
      QV_BARRIER();
      if constexpr (kt + STAGES - 1 < KT) pipe_issue<C>(ps, st[(kt + STAGES - 1) % STAGES], kt + STAGES - 1);
      pipe_compute<C>(st[kt % STAGES], acc, wm, wn, lane);
      run<kt + 1>(st, ps, acc, wm, wn, lane);
    }
  }
};

// KT = K / 64 pipeline steps is a compile-time constant (the tower's K is
// 1280 or 5120).
template <int BM, int BN, int WM, int WN, int STAGES, int KT, class Epi, class RowMap>
__global__ __launch_bounds__(WM * WN * 64) void k_gemm_pipe(const uint16_t* __restrict__ A, int lda,
                                                            const uint16_t* __restrict__ B, int ldb, int M, int N,
                                                            int xgn, int group, Epi epi, RowMap rmap) {
  using C = PipeCfg<BM, BN, WM, WN, STAGES>;
  constexpr int SE = C::STAGE_ELEMS;
  __shared__ __attribute__((aligned(1024))) uint16_t st0[SE];
  __shared__ __attribute__((aligned(1024))) uint16_t st1[SE];
  __shared__ __attribute__((aligned(1024))) uint16_t st2[STAGES > 2 ? SE : 8];
  __shared__ __attribute__((aligned(1024))) uint16_t st3[STAGES > 3 ? SE : 8];
  __shared__ __attribute__((aligned(1024))) uint16_t st4[STAGES > 4 ? SE : 8];
  __shared__ __attribute__((aligned(1024))) uint16_t st5[STAGES > 5 ? SE : 8];
  __shared__ __attribute__((aligned(1024))) uint16_t st6[STAGES > 6 ? SE : 8];
  __shared__ __attribute__((aligned(1024))) uint16_t st7[STAGES > 7 ? SE : 8];
  uint16_t* const st[8] = {st0, st1, st2, st3, st4, st5, st6, st7};

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int tiles_n = (N + BN - 1) / BN, tiles_m = (M + BM - 1) / BM;
  int tm, tn;
  if (!tile_coords(blockIdx.x, tiles_m, tiles_n, xgn, group, tm, tn)) return;  // uniform over the workgroup
  const int m0 = tm * BM, n0 = tn * BN;

  PipeState<C> ps;
  pipe_setup<C>(ps, A, lda, B, ldb, M, N, m0, n0, rmap, wave, lane);

  f32x16 acc[C::FM][C::FN];
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // epilogue values (issued before the ring, so waiting for them never
  // waits for a ring load)
  const auto pre = epi.template prefetch<C::FM, C::FN, false>(m0 + wm * C::TM, n0 + wn * C::TN, lane, M, N, true);

  // prologue: STAGES - 1 steps in flight
#pragma unroll
  for (int s = 0; s < STAGES - 1; ++s)
    if (s < KT) pipe_issue<C>(ps, st[s], s);
  PipeSteps<C, KT, STAGES>::template run<0>(st, ps, acc, wm, wn, lane);

  constexpr int SLOT = Epi::kPatchFloats;
  // every wave is done reading the ring: reuse it as one staged-epilogue
  // patch per wave
  constexpr int PER = (SE * 2) / (SLOT * 4);
  static_assert(PER >= 1 && PER * STAGES >= C::NW, "per-wave slots fit in the ring");
  QV_BARRIER();
  const int sb = wave / PER;
  uint16_t* sbuf = sb == 0 ? st0 : sb == 1 ? st1 : sb == 2 ? st2 : sb == 3 ? st3 : sb == 4 ? st4 : sb == 5 ? st5
                 : sb == 6 ? st6 : st7;
  float* slot = reinterpret_cast<float*>(sbuf) + (wave % PER) * SLOT;
  if constexpr (Epi::kStaged) {
    epi.apply_staged(acc, slot, m0 + wm * C::TM, n0 + wn * C::TN, lane, M, N, pre);
  } else {
    epi.apply(acc, m0 + wm * C::TM, n0 + wn * C::TN, lane, M, N);
  }
}

// ------------------------------------------------------- warp-specialized
// The address unit of a CU moves 64 bytes per clock, so one 1 KB LDS-DMA
// instruction occupies it for 16 clocks; a wave that issues its share of a
// stage while the unit is saturated stalls at issue, and its matrix pipe
// idles.  Here NP producer waves issue every load of the ring and never
// touch the MFMA pipe, while WM x WN consumer waves only read LDS and
// multiply.  Both roles meet at one workgroup barrier per k-step: barrier kt
// publishes stage kt (its producer-side vmcnt wait came first) and tells
// the producers that stage kt - 1 (its buffer is refilled next) is free.
// Producers also take part in the barrier that ends the main loop, so both
// roles execute the same number of barriers.
template <int BM, int BN, int NP, int LP, class RowMap>
__device__ __forceinline__ void ws_setup(const char* (&gsrc)[LP], uint32_t (&ldst)[LP], const uint16_t* A, int lda,
                                         const uint16_t* B, int ldb, int M, int N, int m0, int n0, int pw,
                                         int lane, RowMap rmap) {
#pragma unroll
  for (int i = 0; i < LP; ++i) {
    const int blk = i * NP + pw;                // 1 KB block of the stage
    const int q = blk * 64 + lane;              // 16-byte slot
    const bool isA = q < BM * 8;
    const int qq = isA ? q : q - BM * 8;
    const int r = qq >> 3;
    const int c = swz_chunk(r, qq & 7);
    if (isA) {
      int g = m0 + r;
      g = g < M ? g : M - 1;
      gsrc[i] = reinterpret_cast<const char*>(A + (size_t)g * lda + c * 8);
    } else {
      int g = n0 + r;
      g = g < N ? g : N - 1;
      gsrc[i] = reinterpret_cast<const char*>(B + (size_t)rmap(g) * ldb + c * 8);
    }
    ldst[i] = (uint32_t)(blk * 1024);
  }
}

template <int LP>
__device__ __forceinline__ void ws_issue(const char* const (&gsrc)[LP], const uint32_t (&ldst)[LP], uint16_t* stage,
                                         int kt) {
#pragma unroll
  for (int i = 0; i < LP; ++i)
    __builtin_amdgcn_global_load_lds((gas_ptr)(gsrc[i] + (size_t)kt * 128),
                                     (las_ptr)(reinterpret_cast<char*>(stage) + ldst[i]), 16, 0, 0);
}

template <int KT, int STAGES, int LP>
struct WsProducer {
  template <int kt>
  static __device__ __forceinline__ void run(uint16_t* const (&st)[8], const char* const (&gsrc)[LP],
                                             const uint32_t (&ldst)[LP]) {
    if constexpr (kt < KT) {
      constexpr int later = (KT - 1 - kt) < (STAGES - 2) ? (KT - 1 - kt) : (STAGES - 2);
      QV_WAIT_VM(later * LP);
      QV_BARRIER();
      if constexpr (kt + STAGES - 1 < KT) ws_issue<LP>(gsrc, ldst, st[(kt + STAGES - 1) % STAGES], kt + STAGES - 1);
      run<kt + 1>(st, gsrc, ldst);
    }
  }
};

template <class C, int KT, int STAGES>
struct WsConsumer {
  template <int kt>
  static __device__ __forceinline__ void run(uint16_t* const (&st)[8], f32x16 (&acc)[C::FM][C::FN], int wm, int wn,
                                             int lane) {
    if constexpr (kt < KT) {
      QV_BARRIER();
      pipe_compute<C>(st[kt % STAGES], acc, wm, wn, lane);
      run<kt + 1>(st, acc, wm, wn, lane);
    }
  }
};

// Split-K: a workgroup multiplies the r-th run of KT * 64 columns of A and B,
// and its epilogue is the one epi_at_split() derives for that run (a
// partial-sum epilogue writes its own slice; every other epilogue is used as
// is, with one run).  With xruns = 1 the run is blockIdx.y and every XCD
// takes a rectangle of every run's tiles.  With xruns in {2, 4, 8} the grid
// is one row and the runs are spread over the XCDs instead: XCD x works on
// run x / (8 / xruns) only, and the 8 / xruns XCDs of a run cut its tile
// grid into rectangles, so an XCD fetches the A and B panels of one K range
// (fewer, larger rectangles share more of each panel).
template <class E>
__device__ __forceinline__ E epi_at_split(const E& e, int) {
  return e;
}

__device__ __forceinline__ bool run_tile_coords(int xruns, int tiles_m, int tiles_n, int xgn, int group, int& tm,
                                                int& tn, int& run) {
  if (xruns > 1) {
    const int x = blockIdx.x % 8, nx = 8 / xruns;
    run = x / nx;
    return tile_coords_in(x % nx, blockIdx.x / 8, nx, tiles_m, tiles_n, xgn, group, tm, tn);
  }
  run = blockIdx.y;
  return tile_coords(blockIdx.x, tiles_m, tiles_n, xgn, group, tm, tn);
}

template <int BM, int BN, int WM, int WN, int STAGES, int KT, int NP, class Epi, class RowMap>
__global__ __launch_bounds__((WM * WN + NP) * 64) void k_gemm_ws(const uint16_t* __restrict__ A, int lda,
                                                                const uint16_t* __restrict__ B, int ldb, int M,
                                                                int N, int xgn, int group, int xruns, Epi epi_all,
                                                                RowMap rmap) {
  using C = PipeCfg<BM, BN, WM, WN, STAGES>;
  constexpr int NC = WM * WN;
  constexpr int BLOCKS = (BM + BN) * 8 / 64;  // 1 KB blocks per stage
  constexpr int LP = BLOCKS / NP;
  static_assert(BLOCKS % NP == 0, "stage blocks split evenly over the producers");
  static_assert(LP * (STAGES - 1) <= 63, "producer loads in flight fit the 6-bit vmcnt");
  constexpr int SE = C::STAGE_ELEMS;
  __shared__ __attribute__((aligned(1024))) uint16_t st0[SE];
  __shared__ __attribute__((aligned(1024))) uint16_t st1[SE];
  __shared__ __attribute__((aligned(1024))) uint16_t st2[STAGES > 2 ? SE : 8];
  __shared__ __attribute__((aligned(1024))) uint16_t st3[STAGES > 3 ? SE : 8];
  __shared__ __attribute__((aligned(1024))) uint16_t st4[STAGES > 4 ? SE : 8];
  __shared__ __attribute__((aligned(1024))) uint16_t st5[STAGES > 5 ? SE : 8];
  __shared__ __attribute__((aligned(1024))) uint16_t st6[STAGES > 6 ? SE : 8];
  __shared__ __attribute__((aligned(1024))) uint16_t st7[STAGES > 7 ? SE : 8];
  uint16_t* const st[8] = {st0, st1, st2, st3, st4, st5, st6, st7};

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tiles_n = (N + BN - 1) / BN, tiles_m = (M + BM - 1) / BM;
  int tm, tn, run;
  if (!run_tile_coords(xruns, tiles_m, tiles_n, xgn, group, tm, tn, run)) return;  // uniform over the workgroup
  const int m0 = tm * BM, n0 = tn * BN;
  A += (size_t)run * KT * 64;
  B += (size_t)run * KT * 64;
  const Epi epi = epi_at_split(epi_all, run);

  if (wave >= NC) {
    const char* gsrc[LP];
    uint32_t ldst[LP];
    ws_setup<BM, BN, NP, LP>(gsrc, ldst, A, lda, B, ldb, M, N, m0, n0, wave - NC, lane, rmap);
#pragma unroll
    for (int s = 0; s < STAGES - 1; ++s)
      if (s < KT) ws_issue<LP>(gsrc, ldst, st[s], s);
    WsProducer<KT, STAGES, LP>::template run<0>(st, gsrc, ldst);
    QV_BARRIER();  // pairs with the consumers' end-of-loop barrier
    return;
  }

  const int wm = wave / WN, wn = wave % WN;
  // epilogue values: a consumer issues no ring loads, so its dependent loads
  // (rotary entries after token info) cost the K loop nothing
  const auto pre = epi.template prefetch<C::FM, C::FN, true>(m0 + wm * C::TM, n0 + wn * C::TN, lane, M, N, true);
  f32x16 acc[C::FM][C::FN];
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  WsConsumer<C, KT, STAGES>::template run<0>(st, acc, wm, wn, lane);

  // every consumer is done reading the ring and every load has landed
  constexpr int SLOT = Epi::kPatchFloats;
  constexpr int PER = (SE * 2) / (SLOT * 4);
  static_assert(PER >= 1 && PER * STAGES >= NC, "per-wave slots fit in the ring");
  QV_BARRIER();
  const int sb = wave / PER;
  uint16_t* sbuf = sb == 0 ? st0 : sb == 1 ? st1 : sb == 2 ? st2 : sb == 3 ? st3 : sb == 4 ? st4 : sb == 5 ? st5
                 : sb == 6 ? st6 : st7;
  float* slot = reinterpret_cast<float*>(sbuf) + (wave % PER) * SLOT;
  epi.apply_staged(acc, slot, m0 + wm * C::TM, n0 + wn * C::TN, lane, M, N, pre);
}

// ------------------------------------------- int8 weights (warp-specialized)
// Same ring and consumers as k_gemm_ws; B is int8 codes q [N][ldb] with one
// float32 scale s per row.  Because s belongs to an output column,
// C[m][n] = s[n] * sum_k A[m][k] q[n][k]: the ring holds the codes themselves
// as bf16 (exact, |q| <= 127) and the consumers multiply their accumulators
// by s before the epilogue, which is unchanged.
//
// Two kinds of producer waves.  NPA waves move A by LDS-DMA exactly as in
// k_gemm_ws.  NPB waves fetch B with 16-byte global loads (16 codes of one
// row) into registers, STAGES stages ahead, and at step kt convert B(kt + 1)
// (one sign-extending byte convert per code, one pack per pair) and write it
// to its ring buffer, so the conversion overlaps the wait for A(kt).  The
// roles stay in separate waves because a wave that writes LDS while its own
// LDS-DMA loads are in flight gets a wait for all of them from the compiler.

// Two floats to one dword of bf16, round to nearest even.
__device__ __forceinline__ uint32_t pack_bf16_pair(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// A-only producer wave: its 1 KB blocks of the A tile (same swizzle as ws_setup).
template <int BM, int NPA, int LPA>
__device__ __forceinline__ void i8_a_setup(const char* (&gsrc)[LPA], uint32_t (&ldst)[LPA], const uint16_t* A,
                                           int lda, int M, int m0, int pw, int lane) {
#pragma unroll
  for (int i = 0; i < LPA; ++i) {
    const int blk = i * NPA + pw;
    const int q = blk * 64 + lane;
    const int r = q >> 3;
    int g = m0 + r;
    g = g < M ? g : M - 1;
    gsrc[i] = reinterpret_cast<const char*>(A + (size_t)g * lda + swz_chunk(r, q & 7) * 8);
    ldst[i] = (uint32_t)(blk * 1024);
  }
}

// B producer wave.  Items are (row r, group j of 16 codes = two 16-byte bf16
// chunks in LDS); a stage has BN * 4 of them, split evenly over the NPB * 64
// lanes (four lanes read one row's 64 bytes).  The waits for the B
// registers are the compiler's (plain loads into registers).
template <int BM, int BN, int NPB, int STAGES, int KT, class RowMap>
struct I8BProd {
  static constexpr int ITEMS = BN * 4;
  static constexpr int LB = ITEMS / (NPB * 64);
  static_assert(ITEMS % (NPB * 64) == 0, "whole items per producer lane");
  static_assert(STAGES >= 3, "B(kt + 1) is written while the consumers read stage kt - 1");
  uint16_t* const* st;
  const int8_t* bsrc[LB];
  uint32_t bdst0[LB], bdst1[LB];
  uint4 breg[STAGES][LB];

  __device__ __forceinline__ void setup(uint16_t* const* st_, const int8_t* B, int ldb, int N, int n0, int pw,
                                        int lane, RowMap rmap) {
    st = st_;
#pragma unroll
    for (int i = 0; i < LB; ++i) {
      const int item = (i * NPB + pw) * 64 + lane;
      const int r = item >> 2, j = item & 3;
      int g = n0 + r;
      g = g < N ? g : N - 1;
      bsrc[i] = B + (size_t)rmap(g) * ldb + 16 * j;
      const uint32_t rowb = (uint32_t)(BM * 64 * 2 + r * 128);
      bdst0[i] = rowb + ((uint32_t)swz_chunk(r, 2 * j) << 4);
      bdst1[i] = rowb + ((uint32_t)swz_chunk(r, 2 * j + 1) << 4);
    }
  }
  template <int j>
  __device__ __forceinline__ void issue() {
    if constexpr (j < KT) {
#pragma unroll
      for (int i = 0; i < LB; ++i) breg[j % STAGES][i] = *reinterpret_cast<const uint4*>(bsrc[i] + (size_t)j * 64);
    }
  }
  // codes of stage j -> bf16 in its ring buffer, in the layout the DMA gives A
  template <int j>
  __device__ __forceinline__ void convert() {
    char* base = reinterpret_cast<char*>(st[j % STAGES]);
#pragma unroll
    for (int i = 0; i < LB; ++i) {
      const uint4 w = breg[j % STAGES][i];
      const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
      uint32_t pk[8];
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const float f0 = (float)(int8_t)wd[d];
        const float f1 = (float)(int8_t)(wd[d] >> 8);
        const float f2 = (float)(int8_t)(wd[d] >> 16);
        const float f3 = (float)((int32_t)wd[d] >> 24);
        pk[2 * d] = pack_bf16_pair(f0, f1);
        pk[2 * d + 1] = pack_bf16_pair(f2, f3);
      }
      *reinterpret_cast<uint4*>(base + bdst0[i]) = make_uint4(pk[0], pk[1], pk[2], pk[3]);
      *reinterpret_cast<uint4*>(base + bdst1[i]) = make_uint4(pk[4], pk[5], pk[6], pk[7]);
    }
  }
  // step kt: B(kt + 1) into its buffer (free: the consumers finished stage
  // kt + 1 - STAGES before barrier kt - 1), its registers refilled with
  // B(kt + 1 + STAGES); then barrier kt, which publishes B(kt) (written a
  // step earlier) together with the A producers' stage kt
  template <int kt>
  __device__ __forceinline__ void step() {
    if constexpr (kt < KT) {
      if constexpr (kt + 1 < KT) {
        convert<kt + 1>();
        issue<kt + 1 + STAGES>();
      }
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS writes are done
      QV_BARRIER();
      step<kt + 1>();
    }
  }
  __device__ __forceinline__ void run() {
    issue<0>();
    issue<1>();
    issue<2>();
    if constexpr (STAGES > 3) issue<3>();
    convert<0>();
    issue<STAGES>();
    step<0>();
  }
};

template <int BM, int BN, int WM, int WN, int STAGES, int KT, int NPA, int NPB, class Epi, class RowMap>
__global__ __launch_bounds__((WM * WN + NPA + NPB) * 64) void k_gemm_ws_i8(
    const uint16_t* __restrict__ A, int lda, const int8_t* __restrict__ B, int ldb, const float* __restrict__ bscale,
    int M, int N, int xgn, int group, int xruns, Epi epi_all, RowMap rmap) {
  using C = PipeCfg<BM, BN, WM, WN, STAGES>;
  constexpr int NC = WM * WN;
  constexpr int ABLK = BM * 8 / 64;
  constexpr int LPA = ABLK / NPA;
  static_assert(ABLK % NPA == 0, "A blocks split evenly over the A producers");
  static_assert(LPA * (STAGES - 1) <= 63, "A loads in flight fit the 6-bit vmcnt");
  static_assert(STAGES == 3 || STAGES == 4, "3 or 4 stages");
  constexpr int SE = C::STAGE_ELEMS;
  __shared__ __attribute__((aligned(1024))) uint16_t st0[SE];
  __shared__ __attribute__((aligned(1024))) uint16_t st1[SE];
  __shared__ __attribute__((aligned(1024))) uint16_t st2[SE];
  __shared__ __attribute__((aligned(1024))) uint16_t st3[STAGES > 3 ? SE : 8];
  uint16_t* const st[8] = {st0, st1, st2, st3, st0, st0, st0, st0};

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tiles_n = (N + BN - 1) / BN, tiles_m = (M + BM - 1) / BM;
  int tm, tn, run;
  if (!run_tile_coords(xruns, tiles_m, tiles_n, xgn, group, tm, tn, run)) return;  // uniform over the workgroup
  const int m0 = tm * BM, n0 = tn * BN;
  A += (size_t)run * KT * 64;
  B += (size_t)run * KT * 64;
  const Epi epi = epi_at_split(epi_all, run);

  if (wave >= NC + NPA) {
    I8BProd<BM, BN, NPB, STAGES, KT, RowMap> p;
    p.setup(st, B, ldb, N, n0, wave - NC - NPA, lane, rmap);
    p.run();
    QV_BARRIER();  // pairs with the consumers' end-of-loop barrier
    return;
  }
  if (wave >= NC) {
    const char* gsrc[LPA];
    uint32_t ldst[LPA];
    i8_a_setup<BM, NPA, LPA>(gsrc, ldst, A, lda, M, m0, wave - NC, lane);
#pragma unroll
    for (int s = 0; s < STAGES - 1; ++s)
      if (s < KT) ws_issue<LPA>(gsrc, ldst, st[s], s);
    WsProducer<KT, STAGES, LPA>::template run<0>(st, gsrc, ldst);
    QV_BARRIER();
    return;
  }

  const int wm = wave / WN, wn = wave % WN;
  const auto pre = epi.template prefetch<C::FM, C::FN, true>(m0 + wm * C::TM, n0 + wn * C::TN, lane, M, N, true);
  // this lane's output columns' weight-row scales, fetched before the loop
  float sc[C::FN];
#pragma unroll
  for (int fn = 0; fn < C::FN; ++fn) {
    const int col = n0 + wn * C::TN + fn * 32 + (lane & 31);
    sc[fn] = col < N ? bscale[rmap(col)] : 0.f;
  }
  f32x16 acc[C::FM][C::FN];
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  WsConsumer<C, KT, STAGES>::template run<0>(st, acc, wm, wn, lane);
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] *= sc[j];

  constexpr int SLOT = Epi::kPatchFloats;
  constexpr int PER = (SE * 2) / (SLOT * 4);
  static_assert(PER >= 1 && PER * STAGES >= NC, "per-wave slots fit in the ring");
  QV_BARRIER();
  const int sb = wave / PER;
  uint16_t* sbuf = sb == 0 ? st0 : sb == 1 ? st1 : sb == 2 ? st2 : st3;
  float* slot = reinterpret_cast<float*>(sbuf) + (wave % PER) * SLOT;
  epi.apply_staged(acc, slot, m0 + wm * C::TM, n0 + wn * C::TN, lane, M, N, pre);
}

}  // namespace qv
