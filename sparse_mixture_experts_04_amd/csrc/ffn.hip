// Expert MLPs as grouped GEMMs: gate/up with a fused SwiGLU, then down.
//
// "Under The Hood: Inkling", "MoE: the expert configuration": routed
// experts are SwiGLU MLPs, and the shared experts use the same width;
// "Inkling, Dissected", 02: the shared experts (2 in the pages' layer)
// process every token.
//
// Work is a list of groups g = 0..E+S-1: routed expert g owns the rows
// offsets[g]..offsets[g+1] of the expert-sorted pair order; shared expert
// g-E owns all T tokens.  A group's rows are cut into tiles of MT rows
// (tile_plan), and each (group, row tile, column tile) is one work item.
// The GEMM kernels are persistent: every workgroup walks its share of the
// item list, read from device memory, so no count ever returns to the host.
//
// XCD-aware order: workgroup w runs on XCD w % 8.  The item list is cut into
// 8 contiguous chunks, one per XCD, and the 32 workgroups of an XCD take
// consecutive items of their chunk from a counter; a workgroup whose chunk
// is used up takes what the other chunks have left (claim_item).  Items of
// one group are ordered column tile outer, row tile inner, so the
// workgroups running together on an XCD share a weight tile (read from HBM
// once) and the group's activation rows stay in that XCD's L2.  (The FP4
// kernel keeps a static slot order: its items are short and HBM-bound, and
// a counter per item made it 15% slower.)
#include "ffn_common.h"

namespace moe {

// ------------------------------------------------------------- tile plan

// tile_start[g] = first row tile of group g; tile_start[E+S] = total.  The
// kCtrSets * kXcds work counters that follow (one set for the gate/up GEMM,
// one for the down GEMM that reuses this plan) are zeroed.
__global__ __launch_bounds__(512) void tile_plan_kernel(const int32_t* __restrict__ offsets,
                                                        int E, int S, int T, int MT,
                                                        int32_t* __restrict__ tile_start) {
  __shared__ int sc[512];
  const int g = threadIdx.x;
  const int G = E + S;
  int rows = 0;
  if (g < E) rows = offsets[g + 1] - offsets[g];
  else if (g < G) rows = T;
  const int nt = (rows + MT - 1) / MT;
  sc[g] = nt;
  __syncthreads();
  for (int off = 1; off < 512; off <<= 1) {
    const int v = g >= off ? sc[g - off] : 0;
    __syncthreads();
    sc[g] += v;
    __syncthreads();
  }
  if (g < G) tile_start[g] = sc[g] - nt;
  if (g == G - 1) tile_start[G] = sc[g];
  if (g < kCtrSets * kXcds) tile_start[G + 1 + g] = 0;
}

hipError_t launch_tile_plan(const Shape& s, const int32_t* offsets, int row_tile,
                            int32_t* tile_start, hipStream_t st) {
  if (row_tile == BigCfgRows || row_tile == MidCfgRows)
    return launch_tile_plan_big(s, offsets, row_tile, tile_start, st);
  tile_plan_kernel<<<1, 512, 0, st>>>(offsets, s.E, s.S, s.T, row_tile, tile_start);
  return hipGetLastError();
}

// Row tile by the mean rows per routed expert (measured crossovers: the
// 128-row tiles are 7-12% faster than the 256-row ones at 64-96 rows per
// expert, even at ~192 and 6% slower at 384).
int ffn_row_tile(const Shape& s) {
  if (!s.bf16) return 32;
  const long long per_expert = static_cast<long long>(s.T) * s.k / s.E;
  return per_expert < 48 ? 32 : per_expert < 160 ? MidCfgRows : BigCfgRows;
}

// -------------------------------------------------------- bf16 MFMA GEMM

// Tile: MT rows x 256 weight rows, K step 64, 256 threads (4 waves).
// GATED: the 256 weight rows are 128 output columns of W_gate interleaved
// with the same 128 columns of W_up in blocks of 32, so each wave holds the
// gate and up accumulators of the same outputs and applies SwiGLU in
// registers.  Otherwise the 256 weight rows are 256 output columns.
//
// Data path: global -> LDS with the gfx950 direct loads (global_load_lds,
// 16 bytes per lane, one contiguous KiB per wave instruction) into an
// NS-stage ring; no staging registers.  LDS rows are 128 bytes (64 bf16)
// and the 16-byte chunk c of row r sits in slot c ^ swz(r), with
// swz(r) = (r & 7) ^ ((r >> 3) & 1): the MFMA fragment reads (one chunk of
// 32 consecutive rows) then hit distinct 16-byte bank groups both within
// every 8 lanes (128-byte window) and within every 16 lanes (256-byte
// window).  An A load covers 8 rows and is skipped when none of them holds
// a row of the tile (a decode tile holds a row or two): those LDS rows only
// feed accumulator rows that are never stored, and the wave's wait counts
// follow its number of loads.
// Matrix cores: v_mfma_f32_32x32x16_bf16, fp32 accumulation.
template <int MT, bool GATED>
struct Bf16Cfg {
  static constexpr int BK = 64;
  static constexpr int NB = 256;
  static constexpr int WAVES_M = MT >= 64 ? 2 : 1;
  static constexpr int WAVES_N = 4 / WAVES_M;
  static constexpr int WM = MT / WAVES_M;
  static constexpr int WN = NB / WAVES_N;
  static constexpr int BM = WM / 32;
  static constexpr int BN = WN / 32;
  static constexpr int NOUT = GATED ? NB / 2 : NB;
  static constexpr int NS = MT >= 64 ? 3 : 4;           // LDS ring stages
  static constexpr int A_LOADS = MT * 128 / 1024 / 4;   // KiB loads per wave per stage
  static constexpr int B_LOADS = NB * 128 / 1024 / 4;
  static constexpr int LPW = A_LOADS + B_LOADS;
  static_assert((NS - 2) * LPW < 64, "vmcnt range");
};

template <int MT, bool GATED>
struct TileCtx {
  using C = Bf16Cfg<MT, GATED>;
  const bf16_t* a_src[C::A_LOADS];  // per-lane source of each A load (chunk applied)
  const bf16_t* b_src0;             // first B load of this lane (row only)
  const bf16_t* b_src1;             // GATED: first W_up load
  size_t b_step;                    // elements between consecutive B loads (8 rows)
  int bch[2];                       // this lane's chunk offset for even / odd loads
  int na;                           // A loads this wave issues per stage (wave-uniform)

  // Loads of one stage (K columns k0..k0+63) into the LDS tiles sA, sB.
  __device__ __forceinline__ void issue(int k0, bf16_t* sA, bf16_t* sB, int wave) const {
#pragma unroll
    for (int q = 0; q < C::A_LOADS; ++q)
      if (q < na) dma16(a_src[q] + k0, sA + (wave * C::A_LOADS + q) * 512);
#pragma unroll
    for (int q = 0; q < C::B_LOADS; ++q) {
      const bf16_t* src;
      if (GATED) src = (q < C::B_LOADS / 2 ? b_src0 + q * b_step
                                           : b_src1 + (q - C::B_LOADS / 2) * b_step);
      else src = b_src0 + q * b_step;
      dma16(src + bch[q & 1] + k0, sB + (wave * C::B_LOADS + q) * 512);
    }
  }
};

template <int MT, bool GATED>
__device__ __forceinline__ void load_frags(const bf16_t* sA, const bf16_t* sB, int kk, int wm,
                                           int wn, int lane,
                                           bf16x8_t (&af)[Bf16Cfg<MT, GATED>::BM],
                                           bf16x8_t (&bfr)[Bf16Cfg<MT, GATED>::BN]) {
  using C = Bf16Cfg<MT, GATED>;
  const int r32 = lane & 31;
  const int c = kk * 2 + (lane >> 5);
#pragma unroll
  for (int i = 0; i < C::BM; ++i) {
    const int row = wm * C::WM + i * 32 + r32;
    af[i] = *reinterpret_cast<const bf16x8_t*>(sA + row * 64 + ((c ^ swz(row)) << 3));
  }
#pragma unroll
  for (int j = 0; j < C::BN; ++j) {
    const int row = wn * C::WN + j * 32 + r32;
    bfr[j] = *reinterpret_cast<const bf16x8_t*>(sB + row * 64 + ((c ^ swz(row)) << 3));
  }
}

template <int MT, bool GATED>
__device__ __forceinline__ void mfma_frags(const bf16x8_t (&af)[Bf16Cfg<MT, GATED>::BM],
                                           const bf16x8_t (&bfr)[Bf16Cfg<MT, GATED>::BN],
                                           f32x16_t (&acc)[Bf16Cfg<MT, GATED>::BM]
                                                          [Bf16Cfg<MT, GATED>::BN]) {
  using C = Bf16Cfg<MT, GATED>;
#pragma unroll
  for (int i = 0; i < C::BM; ++i)
#pragma unroll
    for (int j = 0; j < C::BN; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
}

// The 4 MFMA K-substeps of one stage; the fragments of substep kk+1 are
// read from LDS before the MFMAs of substep kk are issued.
template <int MT, bool GATED>
__device__ __forceinline__ void compute_stage(const bf16_t* sA, const bf16_t* sB, int wm,
                                              int wn, int lane,
                                              f32x16_t (&acc)[Bf16Cfg<MT, GATED>::BM]
                                                             [Bf16Cfg<MT, GATED>::BN]) {
  using C = Bf16Cfg<MT, GATED>;
  bf16x8_t a0[C::BM], b0[C::BN], a1[C::BM], b1[C::BN];
  load_frags<MT, GATED>(sA, sB, 0, wm, wn, lane, a0, b0);
  load_frags<MT, GATED>(sA, sB, 1, wm, wn, lane, a1, b1);
  mfma_frags<MT, GATED>(a0, b0, acc);
  load_frags<MT, GATED>(sA, sB, 2, wm, wn, lane, a0, b0);
  mfma_frags<MT, GATED>(a1, b1, acc);
  load_frags<MT, GATED>(sA, sB, 3, wm, wn, lane, a1, b1);
  mfma_frags<MT, GATED>(a0, b0, acc);
  mfma_frags<MT, GATED>(a1, b1, acc);
  // Schedule: substep 0's reads, then each substep's MFMAs interleaved one
  // by one with the next substep's reads, so LDS latency hides behind MFMAs.
  constexpr int NR = C::BM + C::BN;       // fragment reads per substep
  constexpr int NM = C::BM * C::BN;       // MFMAs per substep
  __builtin_amdgcn_sched_group_barrier(0x100, NR, 0);
#pragma unroll
  for (int kk = 0; kk < 3; ++kk) {
#pragma unroll
    for (int q = 0; q < NM; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (q < NR) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
  }
  __builtin_amdgcn_sched_group_barrier(0x008, NM, 0);
}

// One k-step of the ring: wait for this stage, barrier, refill the slot read
// one step ago, compute.  U is the ring slot (compile-time).  The refill is
// unconditional so that the compiler can tell the LDS buffers apart when it
// places its own waits: past the last K step it reloads the last step (an
// L2 hit whose slot is never read).  Exactly NS-2 stages are then always in
// flight behind the one being consumed.
template <int MT, bool GATED, int U>
__device__ __forceinline__ void ring_step(const TileCtx<MT, GATED>& t, int kt, int nk,
                                          bf16_t* const (&sA)[4], bf16_t* const (&sB)[4], int wave,
                                          int wm, int wn, int lane,
                                          f32x16_t (&acc)[Bf16Cfg<MT, GATED>::BM]
                                                         [Bf16Cfg<MT, GATED>::BN]) {
  using C = Bf16Cfg<MT, GATED>;
  constexpr int NXT = (U + C::NS - 1) % C::NS;
  static_assert(C::A_LOADS <= 2, "wait cases");
  if (t.na == C::A_LOADS) wait_vm<(C::NS - 2) * C::LPW>();
  else if (t.na == C::A_LOADS - 1) wait_vm<(C::NS - 2) * (C::LPW - 1)>();
  else wait_vm<(C::NS - 2) * (C::LPW - 2)>();
  lds_barrier();
  const int kn = kt + C::NS - 1 < nk ? kt + C::NS - 1 : nk - 1;
  t.issue(kn * C::BK, sA[NXT], sB[NXT], wave);
  compute_stage<MT, GATED>(sA[U], sB[U], wm, wn, lane, acc);
}

template <int MT, bool GATED>
__global__ __launch_bounds__(256, 1) void ffn_bf16_kernel(FfnArgs p) {
  using C = Bf16Cfg<MT, GATED>;
  __shared__ __attribute__((aligned(1024))) bf16_t sA0[MT * 64];
  __shared__ __attribute__((aligned(1024))) bf16_t sA1[MT * 64];
  __shared__ __attribute__((aligned(1024))) bf16_t sA2[MT * 64];
  __shared__ __attribute__((aligned(1024))) bf16_t sA3[C::NS > 3 ? MT * 64 : 1];
  __shared__ __attribute__((aligned(1024))) bf16_t sB0[C::NB * 64];
  __shared__ __attribute__((aligned(1024))) bf16_t sB1[C::NB * 64];
  __shared__ __attribute__((aligned(1024))) bf16_t sB2[C::NB * 64];
  __shared__ __attribute__((aligned(1024))) bf16_t sB3[C::NS > 3 ? C::NB * 64 : 1];
  __shared__ int ts[512];
  bf16_t* const sA[4] = {sA0, sA1, sA2, sA3};
  bf16_t* const sB[4] = {sB0, sB1, sB2, sB3};

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave % C::WAVES_M;
  const int wn = wave / C::WAVES_M;
  const int G = p.E + p.S;

  for (int g = tid; g <= G; g += 256) ts[g] = p.tile_start[g];
  __syncthreads();

  const long long total = static_cast<long long>(ts[G]) * p.n_tiles;
  const int xcd = blockIdx.x & 7;
  __shared__ long long s_item;

  const bf16_t* A = static_cast<const bf16_t*>(p.a);
  const size_t kT = static_cast<size_t>(p.k) * p.T;
  // Load j of a stage fills LDS rows 8j..8j+7; its lane l lands in slot l%8
  // of row 8j + l/8 and so must fetch global chunk (l%8) ^ swz(8j + l/8),
  // i.e. (l%8) ^ (l/8) ^ (j & 1).
  const int lrow = lane >> 3;
  const int lchunk[2] = {((lane & 7) ^ lrow) * 8, ((lane & 7) ^ lrow ^ 1) * 8};
  static_assert(C::B_LOADS % 2 == 0, "B load parity follows q");
  const int nk = p.K / C::BK;

  for (;;) {
    // persistent: the next item of this XCD's chunk, then of the others'
    if (tid == 0) s_item = claim_item(p.counters, xcd, total);
    __syncthreads();
    const long long it = s_item;
    if (it < 0) break;
    const Item item = decode_item(it, ts, G, p.n_tiles, MT, p.offsets, p.T, p.E);
    const int g = item.g;
    const bool routed = g < p.E;
    const size_t row_base = routed ? static_cast<size_t>(p.offsets[g])
                                   : kT + static_cast<size_t>(g - p.E) * p.T;
    TileCtx<MT, GATED> t;
    {
      const int left = item.rows - 8 * wave * C::A_LOADS;   // rows from this wave's first group
      const int groups = left <= 0 ? 0 : (left + 7) / 8;
      t.na = groups < C::A_LOADS ? groups : C::A_LOADS;
    }
#pragma unroll
    for (int q = 0; q < C::A_LOADS; ++q) {
      int r = (wave * C::A_LOADS + q) * 8 + lrow;
      r = r < item.rows ? r : item.rows - 1;
      const int rr = item.m0 + r;
      size_t src_row;
      if (GATED) src_row = routed ? static_cast<size_t>(p.sorted_pair[row_base + rr] / p.k)
                                  : static_cast<size_t>(rr);
      else src_row = row_base + rr;
      t.a_src[q] = A + src_row * p.K + lchunk[(wave * C::A_LOADS + q) & 1];
    }
    const size_t wstride = static_cast<size_t>(p.N) * p.K;
    const int ge = routed ? g : g - p.E;
    t.b_step = static_cast<size_t>(8) * p.K;
    t.bch[0] = lchunk[0];
    t.bch[1] = lchunk[1];
    if (GATED) {
      // wave w loads rows 64w..64w+63: W_gate columns n*128 + 32w + (0..31),
      // then the same W_up columns
      const int col = item.n * C::NOUT + wave * 32 + lrow;
      const bf16_t* wg = static_cast<const bf16_t*>(routed ? p.w0 : p.ws0) + ge * wstride;
      const bf16_t* wu = static_cast<const bf16_t*>(routed ? p.w1 : p.ws1) + ge * wstride;
      t.b_src0 = wg + static_cast<size_t>(col) * p.K;
      t.b_src1 = wu + static_cast<size_t>(col) * p.K;
    } else {
      const int col = item.n * C::NOUT + wave * C::B_LOADS * 8 + lrow;
      const bf16_t* wd = static_cast<const bf16_t*>(routed ? p.w0 : p.ws0) + ge * wstride;
      t.b_src0 = wd + static_cast<size_t>(col) * p.K;
      t.b_src1 = t.b_src0;
    }

    f32x16_t acc[C::BM][C::BN];
#pragma unroll
    for (int i = 0; i < C::BM; ++i)
#pragma unroll
      for (int j = 0; j < C::BN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    // every wave is done with the previous item's LDS before refilling it
    wait_vm<0>();
    lds_barrier();
#pragma unroll
    for (int s = 0; s < C::NS - 1; ++s) t.issue((s < nk ? s : nk - 1) * C::BK, sA[s], sB[s], wave);

    for (int kt = 0; kt < nk; kt += C::NS) {
      ring_step<MT, GATED, 0>(t, kt, nk, sA, sB, wave, wm, wn, lane, acc);
      if (kt + 1 < nk) ring_step<MT, GATED, 1>(t, kt + 1, nk, sA, sB, wave, wm, wn, lane, acc);
      if (kt + 2 < nk) ring_step<MT, GATED, 2>(t, kt + 2, nk, sA, sB, wave, wm, wn, lane, acc);
      if constexpr (C::NS > 3)
        if (kt + 3 < nk) ring_step<MT, GATED, 3>(t, kt + 3, nk, sA, sB, wave, wm, wn, lane, acc);
    }

    // ---- epilogue.  32x32 accumulator layout: lane l holds column l%32 and
    // rows 8*(r/4) + 4*(l/32) + r%4 for r = 0..15.
    bf16_t* out = static_cast<bf16_t*>(routed ? p.out_routed : p.out_shared);
    const size_t orow0 = routed ? static_cast<size_t>(p.offsets[g]) + item.m0
                                : static_cast<size_t>(g - p.E) * p.T + item.m0;
#pragma unroll
    for (int i = 0; i < C::BM; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = wm * C::WM + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (row >= item.rows) continue;
        bf16_t* orow = out + (orow0 + row) * p.ldo;
        if (GATED) {
#pragma unroll
          for (int j = 0; j < C::BN; j += 2) {
            const float gt = acc[i][j][r];
            const float up = acc[i][j + 1][r];
            const float hv = gt / (1.0f + __expf(-gt)) * up;
            const int col = item.n * C::NOUT + wn * (C::WN / 2) + (j >> 1) * 32 + (lane & 31);
            orow[col] = f32_to_bf16(hv);
          }
        } else {
#pragma unroll
          for (int j = 0; j < C::BN; ++j) {
            const int col = item.n * C::NOUT + wn * C::WN + j * 32 + (lane & 31);
            orow[col] = f32_to_bf16(acc[i][j][r]);
          }
        }
      }
    }
  }
}

// --------------------------------------------------- fp32 GEMM (fp32 act)

// Plain fp32 path for fp32 layers: tile 32 rows x 64 weight rows, K step
// 16.  GATED: weight rows 0..31 are W_gate columns, 32..63 the same W_up
// columns; thread (row, c) owns 4 outputs.  Otherwise 64 output columns,
// 8 per thread.
template <bool GATED>
__global__ __launch_bounds__(256) void ffn_f32_kernel(FfnArgs p) {
  constexpr int MT = 32, NB = 64, BK = 16;
  constexpr int NOUT = GATED ? 32 : 64;
  __shared__ float sA[MT][BK + 1];
  __shared__ float sB[NB][BK + 1];
  __shared__ int ts[512];
  const int tid = threadIdx.x;
  const int G = p.E + p.S;
  for (int g = tid; g <= G; g += 256) ts[g] = p.tile_start[g];
  __syncthreads();
  const long long total = static_cast<long long>(ts[G]) * p.n_tiles;
  const float* A = static_cast<const float*>(p.a);
  const size_t kT = static_cast<size_t>(p.k) * p.T;
  const int row = tid >> 3, cg = tid & 7;

  for (long long it = blockIdx.x; it < total; it += gridDim.x) {
    const Item item = decode_item(it, ts, G, p.n_tiles, MT, p.offsets, p.T, p.E);
    const int g = item.g;
    const bool routed = g < p.E;
    const size_t row_base = routed ? static_cast<size_t>(p.offsets[g])
                                   : kT + static_cast<size_t>(g - p.E) * p.T;
    const size_t wstride = static_cast<size_t>(p.N) * p.K;
    const int ge = routed ? g : g - p.E;
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int k0 = 0; k0 < p.K; k0 += BK) {
      for (int i = tid; i < MT * BK; i += 256) {
        const int r = i / BK, kk = i % BK;
        int rr = r < item.rows ? r : item.rows - 1;
        rr += item.m0;
        size_t src;
        if (GATED) src = routed ? static_cast<size_t>(p.sorted_pair[row_base + rr] / p.k) : rr;
        else src = row_base + rr;
        sA[r][kk] = A[src * p.K + k0 + kk];
      }
      for (int i = tid; i < NB * BK; i += 256) {
        const int r = i / BK, kk = i % BK;
        const float* w;
        int wrow;
        if (GATED) {
          w = static_cast<const float*>(r < 32 ? (routed ? p.w0 : p.ws0) : (routed ? p.w1 : p.ws1));
          wrow = item.n * NOUT + (r & 31);
        } else {
          w = static_cast<const float*>(routed ? p.w0 : p.ws0);
          wrow = item.n * NOUT + r;
        }
        sB[r][kk] = w[ge * wstride + static_cast<size_t>(wrow) * p.K + k0 + kk];
      }
      __syncthreads();
#pragma unroll
      for (int kk = 0; kk < BK; ++kk) {
        const float a = sA[row][kk];
        if (GATED) {
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            acc[c] = fmaf(a, sB[cg * 4 + c][kk], acc[c]);
            acc[4 + c] = fmaf(a, sB[32 + cg * 4 + c][kk], acc[4 + c]);
          }
        } else {
#pragma unroll
          for (int c = 0; c < 8; ++c) acc[c] = fmaf(a, sB[cg * 8 + c][kk], acc[c]);
        }
      }
      __syncthreads();
    }
    if (row < item.rows) {
      float* out = static_cast<float*>(routed ? p.out_routed : p.out_shared);
      const size_t orow = routed ? static_cast<size_t>(p.offsets[g]) + item.m0 + row
                                 : static_cast<size_t>(g - p.E) * p.T + item.m0 + row;
      if (GATED) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const float gt = acc[c], up = acc[4 + c];
          out[orow * p.ldo + item.n * NOUT + cg * 4 + c] = gt / (1.0f + expf(-gt)) * up;
        }
      } else {
#pragma unroll
        for (int c = 0; c < 8; ++c) out[orow * p.ldo + item.n * NOUT + cg * 8 + c] = acc[c];
      }
    }
  }
}

// ------------------------------------------------------------------ host

static int device_cus() {
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 256;
  return cus > 0 ? cus : 256;
}

// Sum of the K-slice partials of the shared experts' tiles, in slice
// order, then what the kernel's epilogue does: SwiGLU of each gate/up
// column pair (GATED; a tile's 256 weight rows hold, for each 32-column
// group w of the 128 outputs, the W_gate rows then the W_up rows) or the
// bf16 rounding of the down output.  One thread per output element.
template <bool GATED>
__global__ __launch_bounds__(256) void shared_reduce_kernel(const float* __restrict__ part,
                                                            int ksplit, int rows, int ldp,
                                                            int nout, bf16_t* __restrict__ out) {
  const long long n = static_cast<long long>(rows) * nout;
  const long long stride = static_cast<long long>(gridDim.x) * blockDim.x;
  const size_t slice = static_cast<size_t>(rows) * ldp;
  for (long long i = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += stride) {
    const int row = static_cast<int>(i / nout);
    const int c = static_cast<int>(i % nout);
    const float* pr = part + static_cast<size_t>(row) * ldp;
    if (GATED) {
      const int col = (c >> 7) * 256 + ((c >> 5) & 3) * 64 + (c & 31);
      float gt = 0.0f, up = 0.0f;
      for (int ks = 0; ks < ksplit; ++ks) {
        gt += pr[ks * slice + col];
        up += pr[ks * slice + col + 32];
      }
      out[i] = f32_to_bf16(gt / (1.0f + __expf(-gt)) * up);
    } else {
      float v = 0.0f;
      for (int ks = 0; ks < ksplit; ++ks) v += pr[ks * slice + c];
      out[i] = f32_to_bf16(v);
    }
  }
}

int fp4_shared_slices(int K) { return K / 32 < kFp4SharedSlices ? K / 32 : kFp4SharedSlices; }

size_t shared_partial_floats(const Shape& s) {
  if (!s.w_fp4 || !s.bf16 || s.S == 0) return 0;
  const size_t rows = static_cast<size_t>(s.S) * s.T;
  const size_t g = kFp4SharedSlices * rows * 2 * s.F;
  const size_t d = kFp4SharedSlices * rows * s.d;
  return g > d ? g : d;
}

// The shared experts' slices of the FP4 launch summed (shared_reduce_kernel)
// into h's shared rows (GATED, with SwiGLU) or y_shared.
template <bool GATED>
static hipError_t reduce_fp4_shared(const FfnArgs& a, const Shape& s, hipStream_t st) {
  const int rows = s.S * s.T;
  const int nout = GATED ? s.F : s.d;
  const long long n = static_cast<long long>(rows) * nout;
  const long long blocks = (n + 255) / 256;
  shared_reduce_kernel<GATED><<<static_cast<unsigned>(blocks < 4096 ? blocks : 4096), 256, 0,
                                st>>>(a.part, a.ksplit, rows, a.n_tiles * 256, nout,
                                      static_cast<bf16_t*>(a.out_shared));
  return hipGetLastError();
}

template <int MT, bool GATED>
static hipError_t run_bf16(const FfnArgs& a, hipStream_t st) {
  int grid = device_cus();
  grid = (grid + 7) / 8 * 8;
  ffn_bf16_kernel<MT, GATED><<<grid, 256, 0, st>>>(a);
  return hipGetLastError();
}

static hipError_t record_marks(hipEvent_t* marks, hipStream_t st) {
  if (marks && hipEventRecord(marks[0], st) != hipSuccess) return hipErrorInvalidValue;
  return hipSuccess;
}

template <bool GATED>
static hipError_t run_f32(const FfnArgs& a, hipStream_t st) {
  ffn_f32_kernel<GATED><<<device_cus() * 4, 256, 0, st>>>(a);
  return hipGetLastError();
}

hipError_t launch_gate_up(const Shape& s, const void* x, const void* wg, const void* wu,
                          const void* wsg, const void* wsu, const uint8_t* scg,
                          const uint8_t* scu, const int32_t* offsets,
                          const int32_t* sorted_pair, const int32_t* tile_start, int row_tile,
                          void* h, float* part, hipEvent_t* marks, hipStream_t st,
                          const float* fold_gates) {
  if (s.T == 0) return record_marks(marks, st);
  FfnArgs a{};
  a.gates = fold_gates;
  a.sc0 = scg;
  a.sc1 = scu;
  a.a = x;
  a.w0 = wg;
  a.w1 = wu;
  a.ws0 = wsg;
  a.ws1 = wsu;
  a.offsets = offsets;
  a.sorted_pair = sorted_pair;
  a.tile_start = tile_start;
  const size_t esz = s.bf16 ? 2 : 4;
  a.out_routed = h;
  a.out_shared = static_cast<char*>(h) + static_cast<size_t>(s.k) * s.T * s.F * esz;
  a.T = s.T;
  a.K = s.d;
  a.N = s.F;
  a.E = s.E;
  a.S = s.S;
  a.k = s.k;
  a.ldo = s.F;
  if (s.bf16) {
    a.n_tiles = s.F / 128;
    if (row_tile != 32) return launch_big(a, true, row_tile, tile_start, kCtrGateUp, marks, st);
    if (fold_gates) return hipErrorInvalidValue;  // the fused combine is large-batch only
    int32_t* ctr = const_cast<int32_t*>(tile_start) + s.E + s.S + 1;
    a.counters = ctr + kCtrGateUp * kXcds;  // FP4 kernel: static order, no counters
    if (s.w_fp4) {  // routed experts in FP4 and the bf16 shared experts, one launch
      if (s.S > 0 && !part) return hipErrorInvalidValue;
      a.ksplit = s.S > 0 ? fp4_shared_slices(s.d) : 0;
      a.part = part;
      hipError_t e = launch_fp4(a, true, st);
      if (e == hipSuccess && s.S > 0) e = reduce_fp4_shared<true>(a, s, st);
      return e == hipSuccess ? record_marks(marks, st) : e;
    }
    hipError_t e = run_bf16<32, true>(a, st);
    return e == hipSuccess ? record_marks(marks, st) : e;
  }
  a.n_tiles = s.F / 32;
  hipError_t e = run_f32<true>(a, st);
  return e == hipSuccess ? record_marks(marks, st) : e;
}

hipError_t launch_down(const Shape& s, const void* wd, const void* wsd, const uint8_t* scd,
                       const int32_t* offsets, const int32_t* tile_start, int row_tile,
                       const void* h, void* y_routed, void* y_shared, float* part,
                       hipEvent_t* marks, hipStream_t st, bool routed_only,
                       bool shared_partials) {
  if (s.T == 0) return record_marks(marks, st);
  if (shared_partials && (!s.w_fp4 || !s.bf16 || s.S == 0)) return hipErrorInvalidValue;
  FfnArgs a{};
  a.sc0 = scd;
  a.a = h;
  a.w0 = wd;
  a.ws0 = wsd;
  a.offsets = offsets;
  a.tile_start = tile_start;
  a.out_routed = y_routed;
  a.out_shared = y_shared;
  a.T = s.T;
  a.K = s.F;
  a.N = s.d;
  a.E = s.E;
  a.S = s.S;
  a.k = s.k;
  a.ldo = s.d;
  if (s.bf16) {
    a.n_tiles = s.d / 256;
    a.g_hi = routed_only ? s.E : 0;
    if (row_tile != 32) return launch_big(a, false, row_tile, tile_start, kCtrDown, marks, st);
    if (routed_only) return hipErrorInvalidValue;  // the fused combine is large-batch only
    int32_t* ctr = const_cast<int32_t*>(tile_start) + s.E + s.S + 1;
    a.counters = ctr + kCtrDown * kXcds;  // FP4 kernel: static order, no counters
    if (s.w_fp4) {
      if (s.S > 0 && !part) return hipErrorInvalidValue;
      a.ksplit = s.S > 0 ? fp4_shared_slices(s.F) : 0;
      a.part = part;
      hipError_t e = launch_fp4(a, false, st);
      if (e == hipSuccess && s.S > 0 && !shared_partials) e = reduce_fp4_shared<false>(a, s, st);
      return e == hipSuccess ? record_marks(marks, st) : e;
    }
    hipError_t e = run_bf16<32, false>(a, st);
    return e == hipSuccess ? record_marks(marks, st) : e;
  }
  a.n_tiles = s.d / 64;
  hipError_t e = run_f32<false>(a, st);
  return e == hipSuccess ? record_marks(marks, st) : e;
}

hipError_t launch_shared_combine(const Shape& s, const void* wsd, const int32_t* tile_start,
                                 int row_tile, const void* h, const void* y_routed,
                                 const float* gates, const int32_t* pair_pos, void* y,
                                 hipStream_t st) {
  if (s.T == 0) return hipSuccess;
  if (!s.bf16 || s.S == 0 || (row_tile != BigCfgRows && row_tile != MidCfgRows))
    return hipErrorInvalidValue;
  FfnArgs a{};
  a.a = h;
  a.ws0 = wsd;
  a.T = s.T;
  a.E = 0;          // one group: the T token rows of the shared experts
  a.S = 1;
  a.k = s.k;
  a.K = s.S * s.F;  // the shared experts one after the other
  a.kcat = s.F;
  a.N = s.d;
  a.ldo = s.d;
  a.n_tiles = s.d / 256;
  a.gates = gates;
  a.pair_pos = pair_pos;
  a.y_routed = y_routed;
  a.y = y;
  int32_t* ctr = const_cast<int32_t*>(tile_start) + s.E + s.S + 1 + kCtrCombine * kXcds;
  return launch_big_combine(a, row_tile, ctr, st);
}

}  // namespace moe
