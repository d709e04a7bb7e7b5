// Internal declarations shared by the expert GEMM kernels.
#pragma once

#include "common.h"

namespace moe {

// ------------------------------------------------------------ item walk

// Number of XCDs, and of the per-XCD work counters stored after
// tile_start[E+S].
constexpr int kXcds = 8;

struct Item {
  int g;      // group
  int m0;     // first row of the tile inside the group
  int rows;   // valid rows in the tile
  int n;      // column tile
  int grows;  // rows of the group
};

// A wave-uniform read of device memory through the scalar data cache: its
// completion is counted by lgkmcnt, not vmcnt, so using the value does not
// wait for the wave's vector loads in flight (e.g. direct-to-LDS loads of
// later K steps).  Reads only.
typedef const int32_t __attribute__((address_space(4)))* const_scalar_i32;
__device__ __forceinline__ int32_t sload(const int32_t* base, int idx) {
  return ((const_scalar_i32)base)[__builtin_amdgcn_readfirstlane(idx)];
}

// Binary search over tile_start (in LDS), then the item's place in its
// group.  A group's row tiles are taken in bands of up to kBand tiles; a
// band's items run column tile outer, row tile inner.  Routed experts at
// large batch have a few row tiles (one band: each weight tile is read from
// HBM once while all of the expert's rows use it); the shared experts'
// many row tiles go band by band, so the workgroups running together on an
// XCD share both activation and weight tiles.
constexpr int kBand = 8;

// balanced: a group of L rows in t row tiles gets tiles of
// base = 32 * ceil(L / (32 t)) rows (the last one the rest, at least one
// row); otherwise row tile m starts at m * MT.
__device__ __forceinline__ Item decode_item(long long it, const int* ts, int G, int n_tiles,
                                            int MT, const int32_t* __restrict__ offsets, int T,
                                            int E, bool balanced = false) {
  int lo = 0, hi = G;  // find last g with ts[g] * n_tiles <= it
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (static_cast<long long>(ts[mid]) * n_tiles <= it) lo = mid;
    else hi = mid;
  }
  Item r;
  r.g = lo;
  const int mt = ts[lo + 1] - ts[lo];
  const int local = static_cast<int>(it - static_cast<long long>(ts[lo]) * n_tiles);
  const int band = mt < kBand ? mt : kBand;
  const int full = mt / band;
  const int in_full = full * band * n_tiles;
  int m;
  if (local < in_full) {
    const int b = local / (band * n_tiles);
    const int rem = local - b * band * n_tiles;
    r.n = rem / band;
    m = b * band + rem % band;
  } else {
    const int last = mt - full * band;
    const int rem = local - in_full;
    r.n = rem / last;
    m = full * band + rem % last;
  }
  r.grows = lo < E ? offsets[lo + 1] - offsets[lo] : T;
  const int base = balanced ? (r.grows + 32 * mt - 1) / (32 * mt) * 32 : MT;
  r.m0 = m * base;
  const int left = r.grows - r.m0;
  r.rows = left < base ? left : base;
  return r;
}

struct FfnArgs {
  const void* a;          // gate/up: x [T, K]; down: h [(k+S)T, K]
  const void* w0;         // routed weights: gate (gate/up) or down  [E, N, K]
  const void* w1;         // routed up weights (gate/up only)
  const void* ws0;        // shared weights                          [S, N, K]
  const void* ws1;
  const int32_t* offsets;
  const int32_t* sorted_pair;
  const int32_t* tile_start;
  void* out_routed;       // row offsets[g] + r
  void* out_shared;       // row (g-E)*T + r
  int T, K, N, E, S, k;   // N = weight rows per expert (F for gate/up, d for down)
  int ldo;                // row length of the output
  int n_tiles;            // column tiles
  const uint8_t* sc0;     // FP4 routed weights: scales of w0 / w1 [E, K/128, N, 4]
  const uint8_t* sc1;
  int ksplit;             // FP4 kernel: K slices of a shared-expert tile (0: none)
  float* part;            // FP4 kernel: fp32 partial tiles [ksplit][S*T][n_tiles*256]
  int32_t* counters;      // ffn_bf16_kernel: kXcds work counters, zero at launch
  int g_hi;               // large-batch kernel: groups 0..g_hi-1 only (0: all E + S)
  // Fused shared experts + combine (large-batch forward, S > 0):
  const float* gates;     // gate/up: [T, k+S]; each shared row of h is scaled by its
                          // token's shared gate (null: no scaling)
  const int32_t* pair_pos;  // combine launch: [T*k] row of each pair in y_routed, or -1
  const void* y_routed;   // combine launch: routed expert outputs [T*k, d]
  void* y;                // combine launch: the layer output [T, d]
  int kcat;               // combine launch: K of one shared expert (F); the K loop runs
                          // over the S shared experts' h and W_down one after the other
};

// Work counters after the last entry of a tile plan (zeroed by the kernel
// that writes the plan): one set of kXcds for the gate/up GEMM, one for the
// down GEMM that reuses the plan and one for the fused shared-expert down +
// combine launch.
enum { kCtrGateUp = 0, kCtrDown = 1, kCtrCombine = 2, kCtrSets = 3 };

// Next work item of a persistent workgroup on XCD `xcd`: the next index of
// that XCD's contiguous chunk of [0, total), or once it is used up the next
// unclaimed index of another XCD's chunk, or -1 when all are taken.  Each
// counter hands out every index once.
__device__ __forceinline__ long long claim_item(int32_t* counters, int xcd, long long total) {
  const long long chunk = (total + kXcds - 1) / kXcds;
  for (int h = 0; h < kXcds; ++h) {
    const int x = (xcd + h) % kXcds;
    const long long bx = x * chunk;
    const long long lx = (bx + chunk < total ? bx + chunk : total) - bx;
    if (lx <= 0) continue;
    const int v = atomicAdd(&counters[x], 1);
    if (v < lx) return bx + v;
  }
  return -1;
}

// ---------------------------------------------------------- LDS helpers


__device__ __forceinline__ int swz(int row) { return (row & 7) ^ ((row >> 3) & 1); }

__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
}

// s_waitcnt vmcnt(n), leaving the other counters alone (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

// One direct global -> LDS load: 16 bytes per lane from `src`, the wave's 64
// lanes filling the KiB at `dst` (wave-uniform) in lane order.  Written as
// inline asm so that the compiler does not track these LDS writes (it would
// otherwise fall back to waiting for every outstanding load before each LDS
// read); the ring synchronises them explicitly with vmcnt waits and
// barriers.  The asm has no output registers.  It names m0 as clobbered;
// the compiler reserves m0 and warns that it does not save it around asm,
// which is harmless here: in the generated gfx950 code of these kernels
// every write and read of m0 is one of these asm blocks (no register-array
// indexing through m0, no messages, no compiler-issued LDS DMA).
__device__ __forceinline__ void dma16(const bf16_t* src, bf16_t* dst) {
  const uint32_t lds = __builtin_amdgcn_readfirstlane(
      static_cast<uint32_t>(reinterpret_cast<uintptr_t>(LDS_PTR(dst))));
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(src), "s"(lds)
               : "m0");
}


// Row tiles of the large-batch GEMMs (256 rows with K step 32; 128 rows
// with K step 64 for experts of a few hundred rows or fewer) and their plan.
constexpr int BigCfgRows = 256;
constexpr int MidCfgRows = 128;
hipError_t launch_tile_plan_big(const Shape& s, const int32_t* offsets, int mt, int32_t* plan,
                                hipStream_t st);
// Large-batch GEMMs with row tiles of mt (BigCfgRows or MidCfgRows) rows:
// `plan` is the layout written by tile_plan_big_kernel for that mt;
// `which` (0 = gate/up, 1 = down) picks the work counters; marks[0]
// (optional) is recorded after the GEMM launch.
hipError_t launch_big(const FfnArgs& a, bool gated, int mt, const int32_t* plan, int which,
                      hipEvent_t* marks, hipStream_t st);
// The shared experts' down GEMM fused with the combine: one launch over
// ceil(T / mt) token tiles x d / 256 column tiles, after the routed down
// GEMM has written y_routed.  a: E = 0 and S = 1 (one group of T token
// rows), K = S_shared * F, kcat = F, N = ldo = d, a = h (its shared rows
// scaled by their gates), ws0 = the shared experts' W_down, y, y_routed,
// gates, pair_pos.  counters: kXcds work counters, zero at launch.
hipError_t launch_big_combine(const FfnArgs& a, int mt, int32_t* counters, hipStream_t st);
// Tile plan of the large-batch GEMM: [row tiles per group, exclusive
// prefix (G+1) | work counters kCtrSets GEMMs x kXcds].
inline int big_plan_ints(int G) { return (G + 1) + kCtrSets * kXcds; }

// Decode-batch GEMMs over the routed groups with FP4 weights (ffn_fp4.hip);
// with a.ksplit > 0 the same launch also runs the shared experts' bf16
// tiles in a.ksplit K slices, writing fp32 partials to a.part
// ([ksplit][S*T][n_tiles*256]) for shared_reduce.
hipError_t launch_fp4(const FfnArgs& a, bool gated, hipStream_t st);
// K slices of a shared-expert tile in the FP4 launch (fp4_shared_slices
// gives fewer when K has fewer than 4 steps of 32).
constexpr int kFp4SharedSlices = kFp4SharedSlicesMax;

}  // namespace moe
