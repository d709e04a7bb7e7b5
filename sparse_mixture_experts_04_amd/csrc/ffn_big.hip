// Expert GEMMs for large batches: row tiles of up to 256 rows.
//
// Same computation as the 32-row kernel in ffn.hip ("Under The Hood:
// Inkling", expert configuration: SwiGLU experts; "Inkling, Dissected", 02:
// routed and shared experts), with a tile shaped for the matrix cores when
// the routed experts hold hundreds of rows each:
//
// * Tile: up to 256 rows x 256 weight rows, K step 32, 512 threads.  Wave
//   (wm, wn) = (wave / 4, wave % 4) owns weight rows 64wn..64wn+63 (two
//   32-wide MFMA column blocks) and the 32-row blocks 2i + wm, i = 0..3.
//   A tile that is only partly filled skips the MFMAs (and fragment reads)
//   of its empty row blocks, so its cost follows its row count in steps of
//   32 rows.
// * Row tiles: a group of L rows is cut into t = ceil(L / 256) tiles of
//   nearly equal size (multiples of 32 rows but the last), all in one
//   launch, so every weight tile of an expert is streamed while all of its
//   rows use it.
// * GATED: the 64 weight rows of column group wn are the W_gate columns
//   32wn..32wn+31 of the 128-column output tile followed by the same W_up
//   columns; SwiGLU is applied to the accumulators in registers.
// * Data path: direct global -> LDS loads into separate rings for the two
//   operands (16 KiB per operand stage), 64-byte LDS rows with chunk c of
//   row r in slot c ^ swz4(r), which keeps the fragment reads free of bank
//   conflicts (see swz4).
// * Scheduling: persistent workgroups; the item list is cut into one
//   contiguous chunk per XCD and the workgroups of an XCD take the next item
//   of their chunk from a counter, so consecutive items (sharing weight and
//   activation tiles) run together on one XCD and uneven items balance.  A
//   workgroup whose chunk is used up takes the remaining items of the other
//   XCDs' chunks from their counters (7% faster at T=16384: the chunks hold
//   equal item counts but unequal work).
#include "ffn_common.h"

namespace moe {

struct BigCfg {
  static constexpr int THREADS = 512;
  static constexpr int WAVES = THREADS / 64;
  static constexpr int BK = 32;
  static constexpr int MT = 256;
  static constexpr int NB = 256;
  static constexpr int NSA = 3;                       // A (activation) ring slots
  static constexpr int NSB = 6;                       // B (weight) ring slots
  static constexpr int BM = MT / 32 / 2;              // row blocks per wave
  static constexpr int BN = 2;                        // column blocks per wave
  static constexpr int LPW = MT * 64 / 1024 / (WAVES / 2);  // KiB loads per loading wave
  static constexpr int STAGE_ELEMS = MT * BK;         // bf16 elements of one operand stage
  static_assert(MT == NB, "both operands use the same load shape");
  static_assert((NSB - 2) * LPW < 64, "vmcnt range");
};

// Slot of chunk c in LDS row r is c ^ swz4(r).  gfx950 serves a ds_read_b128
// 16 lanes per cycle over 64 banks of 4 bytes (one 256-byte bank row); the
// 16 lanes of a cycle are 4 lane quads whose quad indices within the half
// wave have equal parity (lanes 0-3, 12-15, 20-27 together).  A fragment
// read (lane l: row l % 32, chunk 2kk + l / 32) then touches the 16 slots of
// a bank row exactly once per cycle when swz4(r) = (r >> 2) & 3 (measured:
// no bank-conflict cycles).
__device__ __forceinline__ int swz4(int row) { return (row >> 2) & 3; }

// Wave group 0 loads the weight (B) tiles, group 1 the activation (A)
// tiles; each wave issues LPW 1 KiB loads per stage, load j = 4 * (wave % 4)
// + q filling LDS rows 16j..16j+15 of its operand's slot.
struct BigCtx {
  using C = BigCfg;
  const bf16_t* src[C::LPW];  // per-lane source of each load (chunk applied)

  __device__ __forceinline__ void issue(int k0, bf16_t* slot, int wig) const {
#pragma unroll
    for (int q = 0; q < C::LPW; ++q) dma16(src[q] + k0, slot + (wig * C::LPW + q) * 512);
  }
};

// Fragments of one stage for one wave: 2 MFMA substeps x (4 row blocks of
// A, 2 column blocks of B).  Row block i of group grp is tile row block
// 2i + grp (groups interleave so a partly filled tile stays balanced).
struct BigFrags {
  bf16x8_t a[2][BigCfg::BM];
  bf16x8_t b[2][BigCfg::BN];
};

// Fragment reads.  Rows of a 32-row block differ only above bit 4, so the
// swizzle depends only on the lane's row inside the block: one per-lane
// offset per substep (`off[kk]`, in elements) plus a compile-time block
// offset addresses every fragment.  `nv` (wave-uniform) is the number of
// this wave's row blocks that hold rows of the tile.
__device__ __forceinline__ void big_read_frags(const bf16_t* sA, const bf16_t* sB, int grp,
                                               int wn, int nv, const int (&off)[2],
                                               BigFrags& f) {
  using C = BigCfg;
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
    for (int j = 0; j < C::BN; ++j)
      f.b[kk][j] =
          *reinterpret_cast<const bf16x8_t*>(sB + (wn * 2 + j) * 1024 + off[kk]);
#pragma unroll
    for (int i = 0; i < C::BM; ++i)
      if (i < nv)
        f.a[kk][i] = *reinterpret_cast<const bf16x8_t*>(sA + (2 * i + grp) * 1024 + off[kk]);
  }
}

// The weight fragment is the MFMA's first operand, so each accumulator block
// is the transposed product (output columns down the lane's registers, tile
// rows across lanes): a lane then holds 4 consecutive output columns of one
// row, which the epilogue writes as one 8-byte word.
__device__ __forceinline__ void big_mfma(const BigFrags& f, int nv,
                                         f32x16_t (&acc)[BigCfg::BM][BigCfg::BN]) {
  using C = BigCfg;
#pragma unroll
  for (int kk = 0; kk < 2; ++kk)
#pragma unroll
    for (int i = 0; i < C::BM; ++i)
      if (i < nv)
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
template <int U, bool GATED>
__device__ __forceinline__ void big_pp_step(const BigCtx& t, int kt, int nk,
                                            bf16_t* const (&sA)[BigCfg::NSA],
                                            bf16_t* const (&sB)[BigCfg::NSB], int grp, int wig,
                                            int nv, const int (&off)[2],
                                            f32x16_t (&acc)[BigCfg::BM][BigCfg::BN]) {
  using C = BigCfg;
  BigFrags f;
  big_read_frags(sA[U % C::NSA], sB[U % C::NSB], grp, wig, nv, off, f);
  {
    const int ahead = grp == 0 ? C::NSB - 1 : C::NSA - 1;
    const int ks = kt + ahead < nk ? kt + ahead : nk - 1;
    bf16_t* slot = grp == 0 ? sB[(U + C::NSB - 1) % C::NSB] : sA[(U + C::NSA - 1) % C::NSA];
    t.issue(ks * C::BK, slot, wig);
  }
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): fragments in registers
  if (grp == 1) wait_vm<(C::NSA - 2) * C::LPW>();
  lds_barrier();
  big_mfma(f, nv, acc);
  if (grp == 0) wait_vm<(C::NSB - 2) * C::LPW>();
  lds_barrier();
}

template <bool GATED>
__device__ __forceinline__ void big_kloop(const BigCtx& t, int nk,
                                          bf16_t* const (&sA)[BigCfg::NSA],
                                          bf16_t* const (&sB)[BigCfg::NSB], int wave, int lane,
                                          int nv, f32x16_t (&acc)[BigCfg::BM][BigCfg::BN]) {
  using C = BigCfg;
  const int grp = wave >> 2, wig = wave & 3;
  const int r32 = lane & 31;
  const int off[2] = {r32 * 32 + (((lane >> 5) ^ swz4(r32)) << 3),
                      r32 * 32 + (((2 + (lane >> 5)) ^ swz4(r32)) << 3)};
  if (grp == 0) {
#pragma unroll
    for (int s = 0; s < C::NSB - 1; ++s) t.issue((s < nk ? s : nk - 1) * C::BK, sB[s], wig);
    wait_vm<(C::NSB - 2) * C::LPW>();
  } else {
#pragma unroll
    for (int s = 0; s < C::NSA - 1; ++s) t.issue((s < nk ? s : nk - 1) * C::BK, sA[s], wig);
    wait_vm<(C::NSA - 2) * C::LPW>();
  }
  lds_barrier();                  // point 0: stage 0 complete
  if (grp == 1) lds_barrier();    // point 1 for group 1 (its phase 0 is idle)
  for (int kt = 0; kt < nk; kt += 6) {
    big_pp_step<0, GATED>(t, kt, nk, sA, sB, grp, wig, nv, off, acc);
    if (kt + 1 < nk) big_pp_step<1, GATED>(t, kt + 1, nk, sA, sB, grp, wig, nv, off, acc);
    if (kt + 2 < nk) big_pp_step<2, GATED>(t, kt + 2, nk, sA, sB, grp, wig, nv, off, acc);
    if (kt + 3 < nk) big_pp_step<3, GATED>(t, kt + 3, nk, sA, sB, grp, wig, nv, off, acc);
    if (kt + 4 < nk) big_pp_step<4, GATED>(t, kt + 4, nk, sA, sB, grp, wig, nv, off, acc);
    if (kt + 5 < nk) big_pp_step<5, GATED>(t, kt + 5, nk, sA, sB, grp, wig, nv, off, acc);
  }
  if (grp == 0) lds_barrier();    // both groups pass the same number of points
}

// One launch covers every row tile of every group.  `plan` holds the row
// tiles per group as an exclusive prefix (G+1 entries); `counters` the
// per-XCD work counters, zero at launch.
template <bool GATED>
__global__ __launch_bounds__(512, 1) void ffn_big_kernel(FfnArgs p, const int32_t* plan,
                                                         int32_t* counters) {
  using C = BigCfg;
  // ring slots of the A and B tiles; after the K loop the same memory
  // stages the output tile for coalesced stores
  __shared__ __attribute__((aligned(1024))) bf16_t lds[(C::NSA + C::NSB) * C::STAGE_ELEMS];
  __shared__ int ts[512];
  __shared__ long long s_item;
  bf16_t* const sA[C::NSA] = {lds, lds + C::STAGE_ELEMS, lds + 2 * C::STAGE_ELEMS};
  bf16_t* sB[C::NSB];
#pragma unroll
  for (int i = 0; i < C::NSB; ++i) sB[i] = lds + (C::NSA + i) * C::STAGE_ELEMS;
  static_assert(C::NSA == 3, "slot list");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int wm = wave >> 2, wn = wave & 3;
  const int G = p.E + p.S;
  for (int g = tid; g <= G; g += C::THREADS) ts[g] = plan[g];
  __syncthreads();

  const long long total = static_cast<long long>(ts[G]) * p.n_tiles;
  const int xcd = blockIdx.x % kXcds;

  const bf16_t* A = static_cast<const bf16_t*>(p.a);
  const size_t kT = static_cast<size_t>(p.k) * p.T;
  const int nk = p.K / C::BK;
  const size_t wstride = static_cast<size_t>(p.N) * p.K;
  // load j of a stage fills LDS rows 16j..16j+15; lane l lands in slot l%4
  // of row 16j + l/4 and fetches chunk (l%4) ^ swz4(16j + l/4), which is
  // (l%4) ^ ((l >> 4) & 3) for every j
  const int lrow = lane >> 2;
  const int lchunk = ((lane & 3) ^ ((lane >> 4) & 3)) * 8;

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
    BigCtx t;
    if (wm == 1) {
#pragma unroll
      for (int q = 0; q < C::LPW; ++q) {
        const int j = wn * C::LPW + q;
        int r = j * 16 + lrow;
        r = r < item.rows ? r : item.rows - 1;
        const int rr = item.m0 + r;
        size_t src_row;
        if (GATED) src_row = routed ? static_cast<size_t>(p.sorted_pair[row_base + rr] / p.k)
                                    : static_cast<size_t>(rr);
        else src_row = row_base + rr;
        t.src[q] = A + src_row * p.K + lchunk;
      }
    } else {
      const int ge = routed ? g : g - p.E;
#pragma unroll
      for (int q = 0; q < C::LPW; ++q) {
        const int j = wn * C::LPW + q;
        const int R = j * 16 + lrow;  // LDS B row
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
        t.src[q] = base + ge * wstride + static_cast<size_t>(col) * p.K + lchunk;
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
    big_kloop<GATED>(t, nk, sA, sB, wave, lane, nv, acc);
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
              v[e] = gt * __builtin_amdgcn_rcpf(1.0f + __expf(-gt)) * up;
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
    bf16_t* out = static_cast<bf16_t*>(routed ? p.out_routed : p.out_shared);
    const size_t orow0 = routed ? static_cast<size_t>(p.offsets[g]) + item.m0
                                : static_cast<size_t>(g - p.E) * p.T + item.m0;
    const int col0 = item.n * NOUT;
    for (int c = tid; c < item.rows * CPR; c += C::THREADS) {
      const int row = c / CPR, ch = c % CPR;
      *reinterpret_cast<uint4*>(out + (orow0 + row) * p.ldo + col0 + ch * 8) =
          *reinterpret_cast<const uint4*>(tile + row * NOUT + ((ch ^ (row & (CPR - 1))) << 3));
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
// shared experts) with L rows gets ceil(L / 256) row tiles.  Writes the
// exclusive prefix over groups and zeroes both GEMMs' work counters.
__global__ __launch_bounds__(512) void tile_plan_big_kernel(const int32_t* __restrict__ offsets,
                                                            int E, int S, int T,
                                                            int32_t* __restrict__ plan) {
  __shared__ int sf[512];
  const int g = threadIdx.x;
  const int G = E + S;
  int rows = 0;
  if (g < E) rows = offsets[g + 1] - offsets[g];
  else if (g < G) rows = T;
  const int nt = (rows + BigCfg::MT - 1) / BigCfg::MT;
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

hipError_t launch_tile_plan_big(const Shape& s, const int32_t* offsets, int32_t* plan,
                                hipStream_t st) {
  tile_plan_big_kernel<<<1, 512, 0, st>>>(offsets, s.E, s.S, s.T, plan);
  return hipGetLastError();
}

hipError_t launch_big(const FfnArgs& a, bool gated, const int32_t* plan, int which,
                      hipEvent_t* marks, hipStream_t st) {
  const int G = a.E + a.S;
  int32_t* ctr = const_cast<int32_t*>(plan) + (G + 1) + which * kXcds;
  const int grid = (device_cus_big() + kXcds - 1) / kXcds * kXcds;
  if (gated) ffn_big_kernel<true><<<grid, BigCfg::THREADS, 0, st>>>(a, plan, ctr);
  else ffn_big_kernel<false><<<grid, BigCfg::THREADS, 0, st>>>(a, plan, ctr);
  if (marks && hipEventRecord(marks[0], st) != hipSuccess) return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace moe
