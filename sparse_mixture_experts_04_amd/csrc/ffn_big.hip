// Expert GEMMs for large batches: row tiles of up to 256 rows (K step 32),
// or of up to 128 rows (K step 64) when the experts hold fewer than ~160
// rows each.
//
// Same computation as the 32-row kernel in ffn.hip ("Under The Hood:
// Inkling", expert configuration: SwiGLU experts; "Inkling, Dissected", 02:
// routed and shared experts), with a tile shaped for the matrix cores when
// the routed experts hold hundreds of rows each:
//
// * Tile: up to MT rows x 256 weight rows, 512 threads (BigShape: MT = 256
//   with K step 32, or MT = 128 with K step 64).  Wave (wm, wn) =
//   (wave / 4, wave % 4) owns weight rows 64wn..64wn+63 (two 32-wide MFMA
//   column blocks) and the 32-row blocks 2i + wm, i < MT / 64.
//   A tile that is only partly filled skips the MFMAs (and fragment reads)
//   of its empty row blocks, so its cost follows its row count in steps of
//   32 rows.
// * Row tiles: a group of L rows is cut into t = ceil(L / MT) tiles of
//   nearly equal size (multiples of 32 rows but the last), all in one
//   launch, so every weight tile of an expert is streamed while all of its
//   rows use it.
// * GATED: the 64 weight rows of column group wn are the W_gate columns
//   32wn..32wn+31 of the 128-column output tile followed by the same W_up
//   columns; SwiGLU is applied to the accumulators in registers.
// * Data path: direct global -> LDS loads into separate rings for the two
//   operands, LDS rows of one K step (64 or 128 bytes) with chunk c of row
//   r in slot c ^ row_swz(r), which keeps the fragment reads free of bank
//   conflicts (see row_swz).  The 128-row shape moves twice the bytes per
//   K step, so its barriers and waits are spread over twice the loads:
//   tiles with few rows carry few MFMAs per step, and the per-step cost
//   dominates them.
// * Scheduling: persistent workgroups; the item list is cut into one
//   contiguous chunk per XCD and the workgroups of an XCD take the next item
//   of their chunk from a counter, so consecutive items (sharing weight and
//   activation tiles) run together on one XCD and uneven items balance.  A
//   workgroup whose chunk is used up takes the remaining items of the other
//   XCDs' chunks from their counters (7% faster at T=16384: the chunks hold
//   equal item counts but unequal work).
#include "ffn_common.h"

namespace moe {

// Tile shape: MT rows x 256 weight rows, K step BK (64-byte LDS rows for
// BK = 32, 128-byte rows for BK = 64), NSA / NSB ring slots for the two
// operands.
template <int MT_, int BK_, int NSA_, int NSB_>
struct BigShape {
  static constexpr int THREADS = 512;
  static constexpr int WAVES = THREADS / 64;
  static constexpr int MT = MT_;
  static constexpr int NB = 256;
  static constexpr int BK = BK_;
  static constexpr int NSA = NSA_;                    // A (activation) ring slots
  static constexpr int NSB = NSB_;                    // B (weight) ring slots
  static constexpr int BM = MT / 32 / 2;              // row blocks per wave
  static constexpr int BN = 2;                        // column blocks per wave
  static constexpr int KK = BK / 16;                  // MFMA substeps per stage
  static constexpr int CPR = BK / 8;                  // 16-byte chunks per LDS row
  static constexpr int RPL = 64 / CPR;                // LDS rows per 1 KiB load
  static constexpr int A_STAGE = MT * BK;             // bf16 elements of one A stage
  static constexpr int B_STAGE = NB * BK;             // ... and of one B stage
  static constexpr int LPW_A = A_STAGE * 2 / 1024 / (WAVES / 2);  // 1 KiB loads per loading wave
  static constexpr int LPW_B = B_STAGE * 2 / 1024 / (WAVES / 2);
  static constexpr int LPW_MAX = LPW_A > LPW_B ? LPW_A : LPW_B;
  static constexpr int LDS_ELEMS = NSA * A_STAGE + NSB * B_STAGE;
  static_assert((NSB - 2) * LPW_B < 64 && (NSA - 2) * LPW_A < 64, "vmcnt range");
  static_assert(BK == 32 || BK == 64, "LDS row layouts");
  static_assert(6 % NSA == 0 && 6 % NSB == 0, "the K loop is unrolled by 6");
};
// 256-row tiles with K step 32 (the most MFMA work per loaded byte), and
// 128-row tiles with K step 64 for experts of up to ~200 rows: twice the
// bytes per barrier, for groups whose K steps carry few MFMAs.
using BigCfg = BigShape<256, 32, 3, 6>;
using MidCfg = BigShape<128, 64, 3, 3>;
static_assert(BigCfg::MT == BigCfgRows && MidCfg::MT == MidCfgRows, "row tiles");
static_assert(BigCfg::LDS_ELEMS * 2 <= 147456 && MidCfg::LDS_ELEMS * 2 <= 147456, "LDS");

// Slot of chunk c in LDS row r is c ^ row_swz(r).  gfx950 serves a ds_read_b128
// 16 lanes per cycle over 64 banks of 4 bytes (one 256-byte bank row); the
// 16 lanes of a cycle are 4 lane quads whose quad indices within the half
// wave have equal parity (lanes 0-3, 12-15, 20-27 together).  A fragment
// read (lane l: row l % 32, chunk 2kk + l / 32) then touches the 16 slots of
// a bank row exactly once per cycle when row_swz(r) = (r >> 2) & 3 for
// 64-byte rows (measured: no bank-conflict cycles), and with
// row_swz(r) = (r & 7) ^ ((r >> 3) & 1) for 128-byte rows (the layout of
// the 32-row kernel, also measured conflict-free).  Rows of a 32-row block
// differ only above bit 4, so the slot depends on the row inside its block.
template <class C>
__device__ __forceinline__ int row_swz(int row) {
  if constexpr (C::BK == 32) return (row >> 2) & 3;
  else return (row & 7) ^ ((row >> 3) & 1);
}

// Source chunk (in elements) that lane l fetches for load j of a stage: the
// load fills LDS rows RPL*j.. and the lane lands in slot l % CPR of row
// RPL*j + l / CPR, so it fetches chunk (l % CPR) ^ row_swz(that row).
template <class C>
__device__ __forceinline__ int src_chunk(int lane, int j) {
  if constexpr (C::BK == 32) return ((lane & 3) ^ ((lane >> 4) & 3)) * 8;
  else return ((lane & 7) ^ (lane >> 3) ^ (j & 1)) * 8;
}

// Wave group 0 loads the weight (B) tiles, group 1 the activation (A)
// tiles; each wave issues L 1 KiB loads per stage (LPW_B or LPW_A), load
// j = L * (wave % 4) + q filling LDS rows RPL*j.. of its operand's slot.
// KCAT (the fused shared-expert down + combine): K runs over the S shared
// experts one after the other, and from K offset kcat on a load's source
// moves on by `jump` elements (to the next expert's h rows or W_down rows).
template <class C, bool KCAT = false>
struct BigCtx {
  const bf16_t* src[C::LPW_MAX];  // per-lane source of each load (chunk applied)
  long long jump = 0;             // wave-uniform (KCAT only)
  int kcat = 0x7fffffff;

  template <int L>
  __device__ __forceinline__ void issue(int k0, bf16_t* slot, int wig) const {
    long long off = k0;
    if constexpr (KCAT) off += k0 >= kcat ? jump : 0;
#pragma unroll
    for (int q = 0; q < L; ++q) dma16(src[q] + off, slot + (wig * L + q) * 512);
  }
};

// Fragments of one stage for one wave: KK MFMA substeps x (BM row blocks of
// A, 2 column blocks of B).  Row block i of group grp is tile row block
// 2i + grp (groups interleave so a partly filled tile stays balanced).
template <class C>
struct BigFrags {
  bf16x8_t a[C::KK][C::BM];
  bf16x8_t b[C::KK][C::BN];
};

// Fragment reads.  Rows of a 32-row block differ only above bit 4, so the
// swizzle depends only on the lane's row inside the block: one per-lane
// offset per substep (`off[kk]`, in elements) plus a compile-time block
// offset addresses every fragment.  NV is the number of this wave's row
// blocks that hold rows of the tile (a compile-time count, so that the
// reads and MFMAs of a step are straight-line code).
template <class C, int GRP, int NV>
__device__ __forceinline__ void big_read_frags(const bf16_t* sA, const bf16_t* sB, int wn,
                                               const int (&off)[C::KK], BigFrags<C>& f) {
  constexpr int BLK = 32 * C::BK;  // elements of a 32-row block
#pragma unroll
  for (int kk = 0; kk < C::KK; ++kk) {
#pragma unroll
    for (int j = 0; j < C::BN; ++j)
      f.b[kk][j] =
          *reinterpret_cast<const bf16x8_t*>(sB + (wn * 2 + j) * BLK + off[kk]);
#pragma unroll
    for (int i = 0; i < NV; ++i)
      f.a[kk][i] = *reinterpret_cast<const bf16x8_t*>(sA + (2 * i + GRP) * BLK + off[kk]);
  }
}

// The weight fragment is the MFMA's first operand, so each accumulator block
// is the transposed product (output columns down the lane's registers, tile
// rows across lanes): a lane then holds 4 consecutive output columns of one
// row, which the epilogue writes as one 8-byte word.
template <class C, int NV>
__device__ __forceinline__ void big_mfma(const BigFrags<C>& f, f32x16_t (&acc)[C::BM][C::BN]) {
#pragma unroll
  for (int kk = 0; kk < C::KK; ++kk)
#pragma unroll
    for (int i = 0; i < NV; ++i)
#pragma unroll
        for (int j = 0; j < C::BN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.b[kk][j], f.a[kk][i], acc[i][j],
                                                              0, 0, 0);
}

// The K loop with the two wave groups in ping-pong.  Barrier points are
// numbered 0, 1, 2, ...; group 0 runs memory(j) between points 2j and 2j+1
// and compute(j) between 2j+1 and 2j+2, group 1 the same one point later.
// So on every SIMD one wave issues MFMAs while its partner reads fragments
// and issues loads.
//   memory(j): read stage j's fragments into registers; group 0 issues its
//              share of the B loads of stage j+5 into the B slot of stage
//              j-1, group 1 its share of the A loads of stage j+2 into the
//              A slot of stage j-1 (both groups finished reading those one
//              point earlier); wait for the fragment reads;
//   compute(j): the MFMAs of stage j from registers.
// Before every even point 2j, every wave has waited for its loads of stage
// j (the loads of later stages stay in flight: four for B, one for A), so
// stage j is complete in LDS when group 0 starts reading it.  Weights come
// from HBM with a long latency and get the deep ring; activation rows are
// mostly L2 hits.  A wave's loads complete in issue order, so keeping each
// operand on its own waves lets the B loads run far ahead without the A
// waits depending on them.  Past the last K step the loads repeat the last
// step (L2 hits into slots never read), which keeps the counts uniform.
// GRP (the wave's group) and NV are compile-time, so a step has no
// branches: the MFMAs and fragment reads of a step are straight-line code.
template <class C, int U, bool GATED, int GRP, int NV, class Ctx>
__device__ __forceinline__ void big_pp_step(const Ctx& t, int kt, int nk,
                                            bf16_t* const (&sA)[C::NSA],
                                            bf16_t* const (&sB)[C::NSB], int wig,
                                            const int (&off)[C::KK],
                                            f32x16_t (&acc)[C::BM][C::BN]) {
  BigFrags<C> f;
  big_read_frags<C, GRP, NV>(sA[U % C::NSA], sB[U % C::NSB], wig, off, f);
  if constexpr (GRP == 0) {
    const int ks = kt + C::NSB - 1 < nk ? kt + C::NSB - 1 : nk - 1;
    t.template issue<C::LPW_B>(ks * C::BK, sB[(U + C::NSB - 1) % C::NSB], wig);
  } else {
    const int ks = kt + C::NSA - 1 < nk ? kt + C::NSA - 1 : nk - 1;
    t.template issue<C::LPW_A>(ks * C::BK, sA[(U + C::NSA - 1) % C::NSA], wig);
  }
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): fragments in registers
  if constexpr (GRP == 1) wait_vm<(C::NSA - 2) * C::LPW_A>();
  lds_barrier();
  big_mfma<C, NV>(f, acc);
  if constexpr (GRP == 0) wait_vm<(C::NSB - 2) * C::LPW_B>();
  lds_barrier();
}

template <class C, bool GATED, int GRP, int NV, class Ctx>
__device__ __forceinline__ void big_kloop(const Ctx& t, int nk,
                                          bf16_t* const (&sA)[C::NSA],
                                          bf16_t* const (&sB)[C::NSB], int wave, int lane,
                                          f32x16_t (&acc)[C::BM][C::BN]) {
  constexpr int grp = GRP;
  const int wig = wave & 3;
  const int r32 = lane & 31;
  int off[C::KK];
#pragma unroll
  for (int kk = 0; kk < C::KK; ++kk)
    off[kk] = r32 * C::BK + (((2 * kk + (lane >> 5)) ^ row_swz<C>(r32)) << 3);
  if (grp == 0) {
#pragma unroll
    for (int s = 0; s < C::NSB - 1; ++s)
      t.template issue<C::LPW_B>((s < nk ? s : nk - 1) * C::BK, sB[s], wig);
    wait_vm<(C::NSB - 2) * C::LPW_B>();
  } else {
#pragma unroll
    for (int s = 0; s < C::NSA - 1; ++s)
      t.template issue<C::LPW_A>((s < nk ? s : nk - 1) * C::BK, sA[s], wig);
    wait_vm<(C::NSA - 2) * C::LPW_A>();
  }
  lds_barrier();                  // point 0: stage 0 complete
  if (grp == 1) lds_barrier();    // point 1 for group 1 (its phase 0 is idle)
  for (int kt = 0; kt < nk; kt += 6) {
    big_pp_step<C, 0, GATED, GRP, NV>(t, kt, nk, sA, sB, wig, off, acc);
    if (kt + 1 < nk) big_pp_step<C, 1, GATED, GRP, NV>(t, kt + 1, nk, sA, sB, wig, off, acc);
    if (kt + 2 < nk) big_pp_step<C, 2, GATED, GRP, NV>(t, kt + 2, nk, sA, sB, wig, off, acc);
    if (kt + 3 < nk) big_pp_step<C, 3, GATED, GRP, NV>(t, kt + 3, nk, sA, sB, wig, off, acc);
    if (kt + 4 < nk) big_pp_step<C, 4, GATED, GRP, NV>(t, kt + 4, nk, sA, sB, wig, off, acc);
    if (kt + 5 < nk) big_pp_step<C, 5, GATED, GRP, NV>(t, kt + 5, nk, sA, sB, wig, off, acc);
  }
  if (grp == 0) lds_barrier();    // both groups pass the same number of points
}

// The K loop instantiated for the wave's group and its count of row blocks
// holding rows (nv, 0..BM; chosen once per item).
template <class C, bool GATED, int GRP, int NV, class Ctx>
__device__ __forceinline__ void big_kloop_nv(const Ctx& t, int nk, bf16_t* const (&sA)[C::NSA],
                                             bf16_t* const (&sB)[C::NSB], int wave, int lane,
                                             int nv, f32x16_t (&acc)[C::BM][C::BN]) {
  if constexpr (NV == 0) {
    big_kloop<C, GATED, GRP, 0>(t, nk, sA, sB, wave, lane, acc);
  } else {
    if (nv == NV) big_kloop<C, GATED, GRP, NV>(t, nk, sA, sB, wave, lane, acc);
    else big_kloop_nv<C, GATED, GRP, NV - 1>(t, nk, sA, sB, wave, lane, nv, acc);
  }
}

// Epilogue of the fused shared-expert down + combine ("Inkling, Dissected",
// 02b: the layer output is the gate-weighted sum of the token's 6 routed
// and the shared experts' outputs).  The LDS tile holds, for the tile's
// tokens and 256 output columns, the shared experts' down products of their
// gate-scaled h rows (their gate-weighted sum, rounded to bf16).  Each thread
// takes 16-byte chunks (8 columns of one token) and sums in fp32, in a fixed
// order: the routed slots in rank order by fma of gate and y_routed row (a
// pair dropped at its expert's capacity, pair_pos < 0, left out), then the
// shared value; one rounding to bf16 into y.  The loads of kCombineBatch
// chunks are issued before any sum, so they are in flight together.
constexpr int kTopK = 6;          // routed experts per token (the descriptor enforces it)
constexpr int kCombineBatch = 4;  // chunks per thread in flight
template <class C, int CPR>
__device__ __forceinline__ void combine_epilogue(const FfnArgs& p, const Item& item,
                                                 const bf16_t* tile, int col0, int tid) {
  const bf16_t* yr = static_cast<const bf16_t*>(p.y_routed);
  bf16_t* yo = static_cast<bf16_t*>(p.y);
  const int ns = p.K / p.kcat;       // shared experts
  const int gstride = kTopK + ns;    // gates per token
  const int n = item.rows * CPR;
  for (int c0 = tid; c0 < n; c0 += kCombineBatch * C::THREADS) {
    int pos[kCombineBatch][kTopK];
    float gw[kCombineBatch][kTopK];
    uint4 v[kCombineBatch][kTopK];
#pragma unroll
    for (int b = 0; b < kCombineBatch; ++b) {
      const int c = c0 + b * C::THREADS;
      const int t = item.m0 + (c < n ? c / CPR : 0);
#pragma unroll
      for (int j = 0; j < kTopK; ++j) {
        pos[b][j] = c < n ? p.pair_pos[static_cast<size_t>(t) * kTopK + j] : -1;
        gw[b][j] = p.gates[static_cast<size_t>(t) * gstride + j];
      }
    }
#pragma unroll
    for (int b = 0; b < kCombineBatch; ++b) {
      const int ch = (c0 + b * C::THREADS) % CPR;
#pragma unroll
      for (int j = 0; j < kTopK; ++j)
        v[b][j] = pos[b][j] >= 0
                      ? *reinterpret_cast<const uint4*>(
                            yr + static_cast<size_t>(pos[b][j]) * p.ldo + col0 + ch * 8)
                      : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int b = 0; b < kCombineBatch; ++b) {
      const int c = c0 + b * C::THREADS;
      if (c >= n) continue;
      const int row = c / CPR, ch = c % CPR;
      float acc[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
#pragma unroll
      for (int j = 0; j < kTopK; ++j) {
        if (pos[b][j] < 0) continue;
        const uint32_t w[4] = {v[b][j].x, v[b][j].y, v[b][j].z, v[b][j].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[2 * e] = fmaf(gw[b][j], __uint_as_float(w[e] << 16), acc[2 * e]);
          acc[2 * e + 1] = fmaf(gw[b][j], __uint_as_float(w[e] & 0xffff0000u), acc[2 * e + 1]);
        }
      }
      const uint4 sv = *reinterpret_cast<const uint4*>(
          tile + row * (CPR * 8) + ((ch ^ (row & (CPR - 1))) << 3));
      const uint32_t sw[4] = {sv.x, sv.y, sv.z, sv.w};
      uint32_t o[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float lo = acc[2 * e] + __uint_as_float(sw[e] << 16);
        const float hi = acc[2 * e + 1] + __uint_as_float(sw[e] & 0xffff0000u);
        o[e] = static_cast<uint32_t>(f32_to_bf16(lo)) |
               (static_cast<uint32_t>(f32_to_bf16(hi)) << 16);
      }
      *reinterpret_cast<uint4*>(yo + static_cast<size_t>(item.m0 + row) * p.ldo + col0 +
                                ch * 8) = make_uint4(o[0], o[1], o[2], o[3]);
    }
  }
}

// One launch covers every row tile of every group (of groups 0..g_hi-1).
// `plan` holds the row tiles per group as an exclusive prefix (G+1
// entries); `counters` the per-XCD work counters, zero at launch.
// COMBINE: the fused shared-expert down + combine.  One group of T token
// rows (p.E = 0, p.S = 1, its tiles computed here, not read from the
// plan); the K loop covers the shared experts' gate-scaled h rows against
// their W_down one expert after the other (p.K = S * F, rows p.kcat = F
// long), and the epilogue adds the routed outputs of each token's pairs
// (see combine_epilogue) and writes y.
template <class C, bool GATED, bool COMBINE = false>
__global__ __launch_bounds__(512, 1) void ffn_big_kernel(FfnArgs p, const int32_t* plan,
                                                         int32_t* counters) {
  // ring slots of the A and B tiles; after the K loop the same memory
  // stages the output tile for coalesced stores
  __shared__ __attribute__((aligned(1024))) bf16_t lds[C::LDS_ELEMS];
  __shared__ int ts[512];
  __shared__ long long s_item;
  bf16_t* sA[C::NSA];
  bf16_t* sB[C::NSB];
#pragma unroll
  for (int i = 0; i < C::NSA; ++i) sA[i] = lds + i * C::A_STAGE;
#pragma unroll
  for (int i = 0; i < C::NSB; ++i) sB[i] = lds + C::NSA * C::A_STAGE + i * C::B_STAGE;
  static_assert(C::MT * (GATED ? C::NB / 2 : C::NB) <= C::LDS_ELEMS, "output tile");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int wm = wave >> 2, wn = wave & 3;
  const int G = p.E + p.S;
  if constexpr (COMBINE) {
    if (tid == 0) {
      ts[0] = 0;
      ts[1] = (p.T + C::MT - 1) / C::MT;
    }
  } else {
    for (int g = tid; g <= G; g += C::THREADS) ts[g] = plan[g];
  }
  __syncthreads();

  const int g_hi = p.g_hi > 0 ? p.g_hi : G;
  const long long total = static_cast<long long>(ts[g_hi]) * p.n_tiles;
  const int xcd = blockIdx.x % kXcds;

  const bf16_t* A = static_cast<const bf16_t*>(p.a);
  const size_t kT = static_cast<size_t>(p.k) * p.T;
  const int nk = p.K / C::BK;
  const int kld = COMBINE ? p.kcat : p.K;  // row length of h and W
  const size_t wstride = static_cast<size_t>(p.N) * kld;
  // load j of a stage fills LDS rows RPL*j..; lane l lands in row
  // RPL*j + l / CPR (src_chunk gives the chunk it fetches)
  const int lrow = lane / C::CPR;

  for (;;) {
    // the next item of this XCD's chunk, then of the others' (claim_item)
    if (tid == 0) s_item = claim_item(counters, xcd, total);
    __syncthreads();  // also: every wave is done with the previous item's LDS
    const long long gitem = s_item;
    if (gitem < 0) break;
    const Item item = decode_item(gitem, ts, G, p.n_tiles, C::MT, p.offsets, p.T, p.E, true);
    const int g = item.g;
    const bool routed = g < p.E;
    const size_t row_base = routed ? static_cast<size_t>(p.offsets[g])
                                   : kT + static_cast<size_t>(g - p.E) * p.T;
    BigCtx<C, COMBINE> t;
    if (wm == 1) {
#pragma unroll
      for (int q = 0; q < C::LPW_A; ++q) {
        const int j = wn * C::LPW_A + q;
        int r = j * C::RPL + lrow;
        r = r < item.rows ? r : item.rows - 1;
        const int rr = item.m0 + r;
        size_t src_row;
        if (GATED) src_row = routed ? static_cast<size_t>(p.sorted_pair[row_base + rr] / p.k)
                                    : static_cast<size_t>(rr);
        else src_row = row_base + rr;
        t.src[q] = A + src_row * kld + src_chunk<C>(lane, j);
      }
      if (COMBINE) {  // the next shared expert's rows of h
        t.jump = static_cast<long long>(p.T) * kld - kld;
        t.kcat = p.kcat;
      }
    } else {
      const int ge = routed ? g : g - p.E;
#pragma unroll
      for (int q = 0; q < C::LPW_B; ++q) {
        const int j = wn * C::LPW_B + q;
        const int R = j * C::RPL + lrow;  // LDS B row
        const int cg = R >> 6, rl = R & 63;
        const bf16_t* base;
        int col;
        if (GATED) {
          const bool up = rl >= 32;
          base = static_cast<const bf16_t*>(up ? (routed ? p.w1 : p.ws1)
                                               : (routed ? p.w0 : p.ws0));
          col = item.n * (C::NB / 2) + cg * 32 + (rl & 31);
        } else {
          base = static_cast<const bf16_t*>(routed ? p.w0 : p.ws0);
          col = item.n * C::NB + R;
        }
        t.src[q] = base + ge * wstride + static_cast<size_t>(col) * kld + src_chunk<C>(lane, j);
      }
      if (COMBINE) {  // the next shared expert's W_down
        t.jump = static_cast<long long>(wstride) - kld;
        t.kcat = p.kcat;
      }
    }

    f32x16_t acc[C::BM][C::BN];
#pragma unroll
    for (int i = 0; i < C::BM; ++i)
#pragma unroll
      for (int j = 0; j < C::BN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    // row blocks of this wave's group (2i + wm) that hold rows of the tile
    const int nblk = (item.rows + 31) >> 5;
    const int nv = min((nblk - wm + 1) >> 1, C::BM);
    if (wm == 0) big_kloop_nv<C, GATED, 0, C::BM>(t, nk, sA, sB, wave, lane, nv, acc);
    else big_kloop_nv<C, GATED, 1, C::BM>(t, nk, sA, sB, wave, lane, nv, acc);
    // the last steps refill ring slots with copies of the final stage, and
    // those copies may still be landing: drain every wave's loads before the
    // ring memory is reused for the output tile
    wait_vm<0>();
    __syncthreads();

    // ---- epilogue: block (i, j) holds the transposed product: lane l ->
    // tile row (2i + wm) * 32 + l % 32, registers 4q..4q+3 -> output
    // columns 8q + 4 (l / 32) + 0..3 of column block j.  Each lane writes
    // 8 bytes at a time into the LDS tile, whose 16-byte chunk c of row r
    // sits in slot c ^ (r % CPR); then 16-byte coalesced global stores.
    constexpr int NOUT = GATED ? C::NB / 2 : C::NB;
    constexpr int CPR = NOUT / 8;  // 16-byte chunks per row
    bf16_t* tile = lds;  // [MT][NOUT]
#pragma unroll
    for (int i = 0; i < C::BM; ++i) {
      const int row = (2 * i + wm) * 32 + (lane & 31);
      bf16_t* trow = tile + row * NOUT + 4 * (lane >> 5);
      const int sw = row & (CPR - 1);
      if (GATED) {
        // with p.gates, a shared expert's row of h (token m0 + row) carries
        // that token's gate for the expert, for the fused down + combine
        float gsc = 1.0f;
        if (p.gates && !routed)
          gsc = row < item.rows ? p.gates[static_cast<size_t>(item.m0 + row) * (p.k + p.S) +
                                          p.k + (g - p.E)]
                                : 0.0f;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          uint32_t w[2];
#pragma unroll
          for (int t2 = 0; t2 < 2; ++t2) {
            float v[2];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
              const float gt = acc[i][0][4 * q + 2 * t2 + e];
              const float up = acc[i][1][4 * q + 2 * t2 + e];
              v[e] = gt * __builtin_amdgcn_rcpf(1.0f + __expf(-gt)) * up * gsc;
            }
            w[t2] = static_cast<uint32_t>(f32_to_bf16(v[0])) |
                    (static_cast<uint32_t>(f32_to_bf16(v[1])) << 16);
          }
          const int ch = wn * 4 + q;
          *reinterpret_cast<uint2*>(trow + ((ch ^ sw) << 3)) = make_uint2(w[0], w[1]);
        }
      } else {
#pragma unroll
        for (int j = 0; j < C::BN; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const f32x16_t& a = acc[i][j];
            const uint32_t w0 = static_cast<uint32_t>(f32_to_bf16(a[4 * q])) |
                                (static_cast<uint32_t>(f32_to_bf16(a[4 * q + 1])) << 16);
            const uint32_t w1 = static_cast<uint32_t>(f32_to_bf16(a[4 * q + 2])) |
                                (static_cast<uint32_t>(f32_to_bf16(a[4 * q + 3])) << 16);
            const int ch = wn * 8 + j * 4 + q;
            *reinterpret_cast<uint2*>(trow + ((ch ^ sw) << 3)) = make_uint2(w0, w1);
          }
      }
    }
    __syncthreads();
    const int col0 = item.n * NOUT;
    if constexpr (COMBINE) {
      combine_epilogue<C, CPR>(p, item, tile, col0, tid);
    } else {
      bf16_t* out = static_cast<bf16_t*>(routed ? p.out_routed : p.out_shared);
      const size_t orow0 = routed ? static_cast<size_t>(p.offsets[g]) + item.m0
                                  : static_cast<size_t>(g - p.E) * p.T + item.m0;
      for (int c = tid; c < item.rows * CPR; c += C::THREADS) {
        const int row = c / CPR, ch = c % CPR;
        *reinterpret_cast<uint4*>(out + (orow0 + row) * p.ldo + col0 + ch * 8) =
            *reinterpret_cast<const uint4*>(tile + row * NOUT + ((ch ^ (row & (CPR - 1))) << 3));
      }
    }
  }
}

static int device_cus_big() {
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 256;
  return cus > 0 ? cus : 256;
}

// Tile plan of the large-batch GEMMs: group g (routed expert g, then the
// shared experts) with L rows gets ceil(L / mt) row tiles.  Writes the
// exclusive prefix over groups and zeroes both GEMMs' work counters.
__global__ __launch_bounds__(512) void tile_plan_big_kernel(const int32_t* __restrict__ offsets,
                                                            int E, int S, int T, int mt,
                                                            int32_t* __restrict__ plan) {
  __shared__ int sf[512];
  const int g = threadIdx.x;
  const int G = E + S;
  int rows = 0;
  if (g < E) rows = offsets[g + 1] - offsets[g];
  else if (g < G) rows = T;
  const int nt = (rows + mt - 1) / mt;
  sf[g] = nt;
  __syncthreads();
  for (int off = 1; off < 512; off <<= 1) {
    const int v = g >= off ? sf[g - off] : 0;
    __syncthreads();
    sf[g] += v;
    __syncthreads();
  }
  if (g < G) plan[g] = sf[g] - nt;
  if (g == G - 1) plan[G] = sf[g];
  if (g < kCtrSets * kXcds) plan[G + 1 + g] = 0;
}

hipError_t launch_tile_plan_big(const Shape& s, const int32_t* offsets, int mt, int32_t* plan,
                                hipStream_t st) {
  tile_plan_big_kernel<<<1, 512, 0, st>>>(offsets, s.E, s.S, s.T, mt, plan);
  return hipGetLastError();
}

hipError_t launch_big(const FfnArgs& a, bool gated, int mt, const int32_t* plan, int which,
                      hipEvent_t* marks, hipStream_t st) {
  const int G = a.E + a.S;
  int32_t* ctr = const_cast<int32_t*>(plan) + (G + 1) + which * kXcds;
  const int grid = (device_cus_big() + kXcds - 1) / kXcds * kXcds;
  if (mt == MidCfg::MT) {
    if (gated) ffn_big_kernel<MidCfg, true><<<grid, MidCfg::THREADS, 0, st>>>(a, plan, ctr);
    else ffn_big_kernel<MidCfg, false><<<grid, MidCfg::THREADS, 0, st>>>(a, plan, ctr);
  } else {
    if (gated) ffn_big_kernel<BigCfg, true><<<grid, BigCfg::THREADS, 0, st>>>(a, plan, ctr);
    else ffn_big_kernel<BigCfg, false><<<grid, BigCfg::THREADS, 0, st>>>(a, plan, ctr);
  }
  if (marks && hipEventRecord(marks[0], st) != hipSuccess) return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_big_combine(const FfnArgs& a, int mt, int32_t* counters, hipStream_t st) {
  if (a.T == 0) return hipSuccess;
  if (a.E != 0 || a.S != 1 || a.k != kTopK || a.kcat <= 0 || a.K % a.kcat != 0 ||
      a.K / a.kcat > 2 || a.n_tiles * 256 != a.N || !a.y || !a.y_routed || !a.gates ||
      !a.pair_pos || !counters)
    return hipErrorInvalidValue;
  const int grid = (device_cus_big() + kXcds - 1) / kXcds * kXcds;
  if (mt == MidCfg::MT)
    ffn_big_kernel<MidCfg, false, true><<<grid, MidCfg::THREADS, 0, st>>>(a, nullptr, counters);
  else
    ffn_big_kernel<BigCfg, false, true><<<grid, BigCfg::THREADS, 0, st>>>(a, nullptr, counters);
  return hipGetLastError();
}

}  // namespace moe
