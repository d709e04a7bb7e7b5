// Dispatch: group the (token, slot) pairs by expert, and the bias update.
//
// "Inkling, Dissected", 02: each token visits the 6 routed experts it chose;
// 02e: the load L_e is the number of tokens that selected expert e, the
// ideal load is the total selections divided by the number of experts, and
// once a batch is done b_e moves by gamma * sign(ideal - L_e).
//
// The grouping is histogram -> exclusive scan -> stable scatter, with no
// atomic deciding any output position:
//   1. dispatch_count   one block per segment of kDispatchSeg pairs counts
//                       its pairs per expert in LDS;
//   2. dispatch_scan    one block turns the segment counts into the loads,
//                       the offsets of the kept rows and each segment's
//                       running count per expert;
//   3. dispatch_scatter one wave per segment walks its pairs in order, 64 at a
//                       time; lanes holding the same expert find each other
//                       with 8 ballots (one per id bit), so a pair's rank is
//                       its segment's running count + earlier pairs of that
//                       expert.
// Within an expert the pairs therefore come out in ascending pair number,
// i.e. ascending token.  Capacity ("Inkling, Dissected" 02d): a pair whose
// rank reaches the expert's capacity is dropped (pair_pos = -1).  A pair
// whose expert id lies outside [0, E) is counted nowhere and also gets
// pair_pos = -1.
#include "ffn_common.h"  // the tile plan's layout (work counters after it)

namespace moe {

__global__ __launch_bounds__(256) void dispatch_count(const int32_t* __restrict__ topk,
                                                      long long npairs, int E,
                                                      int32_t* __restrict__ seg_counts) {
  __shared__ int hist[256];
  for (int e = threadIdx.x; e < E; e += 256) hist[e] = 0;
  __syncthreads();
  const long long base = static_cast<long long>(blockIdx.x) * kDispatchSeg;
  for (int i = threadIdx.x; i < kDispatchSeg; i += 256) {
    const long long p = base + i;
    if (p < npairs) {
      const int e = topk[p];
      if (static_cast<unsigned>(e) < static_cast<unsigned>(E)) atomicAdd(&hist[e], 1);
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256)
    seg_counts[static_cast<size_t>(blockIdx.x) * E + e] = hist[e];
}

// One block of 256 threads, thread e owns expert e (E <= 256).  Turns the
// segment counts into each segment's running count of expert e's earlier
// pairs, writes the demand counts and the offsets of the kept rows
// (min(count, capacity) per expert).
__global__ __launch_bounds__(256) void dispatch_scan(int32_t* __restrict__ seg_counts, int nseg,
                                                     int E, int capacity,
                                                     int32_t* __restrict__ counts,
                                                     int32_t* __restrict__ offsets) {
  __shared__ int sc[256];
  const int e = threadIdx.x;
  int tot = 0;
  if (e < E) {
    // 8 segments at a time: their loads go out together (at T=16384 there
    // are 192 segments, and one load at a time would cost a round trip each)
    int s = 0;
    for (; s + 8 <= nseg; s += 8) {
      int c[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) c[j] = seg_counts[static_cast<size_t>(s + j) * E + e];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        seg_counts[static_cast<size_t>(s + j) * E + e] = tot;
        tot += c[j];
      }
    }
    for (; s < nseg; ++s) {
      const size_t i = static_cast<size_t>(s) * E + e;
      const int c = seg_counts[i];
      seg_counts[i] = tot;
      tot += c;
    }
  }
  const int kept = tot < capacity ? tot : capacity;
  sc[e] = kept;
  __syncthreads();
  for (int off = 1; off < 256; off <<= 1) {
    const int v = e >= off ? sc[e - off] : 0;
    __syncthreads();
    sc[e] += v;
    __syncthreads();
  }
  if (e < E) {
    counts[e] = tot;
    offsets[e] = sc[e] - kept;
  }
  if (e == E - 1) offsets[E] = sc[e];
}

__global__ __launch_bounds__(64) void dispatch_scatter(const int32_t* __restrict__ topk,
                                                       long long npairs, int E, int capacity,
                                                       const int32_t* __restrict__ seg_base,
                                                       const int32_t* __restrict__ offsets,
                                                       int32_t* __restrict__ sorted_pair,
                                                       int32_t* __restrict__ pair_pos) {
  __shared__ int run[256];
  __shared__ int off[256];
  const int lane = threadIdx.x;
  for (int e = lane; e < E; e += 64) {
    run[e] = seg_base[static_cast<size_t>(blockIdx.x) * E + e];
    off[e] = offsets[e];
  }
  __syncthreads();
  const long long base = static_cast<long long>(blockIdx.x) * kDispatchSeg;
  for (int c = 0; c < kDispatchSeg; c += 64) {
    const long long p = base + c + lane;
    const bool in_range = p < npairs;
    const int e = in_range ? topk[p] : 0;
    const bool valid = in_range && static_cast<unsigned>(e) < static_cast<unsigned>(E);
    // a pair whose id is outside [0, E) joins no expert: it is marked
    // dropped, so that combine leaves it out like a pair over capacity
    if (in_range && !valid) pair_pos[p] = -1;
    unsigned long long peers = __ballot(valid);
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const bool bit = (e >> b) & 1;
      const unsigned long long m = __ballot(valid && bit);
      peers &= bit ? m : ~m;
    }
    int cnt = 0;
    if (valid) {
      // rank of this pair among expert e's pairs (ascending p)
      const int r = run[e] + __popcll(peers & ((1ull << lane) - 1ull));
      if (r < capacity) {
        const int pos = off[e] + r;
        sorted_pair[pos] = static_cast<int32_t>(p);
        pair_pos[p] = pos;
      } else {
        pair_pos[p] = -1;
      }
      cnt = __popcll(peers);
    }
    __syncthreads();
    // the highest lane of each group of equal experts advances the counter
    if (valid && (peers >> lane) == 1ull) run[e] += cnt;
    __syncthreads();
  }
}

// Small batches (at most kDispatchSmallPairs pairs, e.g. decode steps): the
// three passes in one workgroup of 512 threads, where each launch would
// otherwise cost more than its work.  Wave w plays the part of a segment: it
// owns the contiguous pairs w*seg .. w*seg+seg-1 (seg a multiple of 64), so
// counts, offsets and ranks are those of the multi-block passes.  With
// tile_start set it then writes the row-tile plan of the decode GEMMs
// (tile_start[g] = first tile of group g, tile_start[E+S] = total, the work
// counters after it zeroed: what tile_plan_kernel writes), and with
// gamma != 0 applies the bias update (the router has read the bias by then).
__global__ __launch_bounds__(512) void dispatch_small(
    const int32_t* __restrict__ topk, int npairs, int E, int capacity,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ sorted_pair, int32_t* __restrict__ pair_pos, int S, int T, int MT,
    int32_t* __restrict__ tile_start, long long kT, float gamma, float* __restrict__ bias) {
  constexpr int W = 8;
  __shared__ int run[W][256];  // per wave: its count of expert e, then its running rank
  __shared__ int off[256];
  __shared__ int sc[512];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int seg = (npairs + W * 64 - 1) / (W * 64) * 64;
  const int pb = w * seg;
  const int pe = pb + seg < npairs ? pb + seg : npairs;
  for (int i = tid; i < W * 256; i += 512) (&run[0][0])[i] = 0;
  __syncthreads();
  for (int p = pb + lane; p < pe; p += 64) {
    const int e = topk[p];
    if (static_cast<unsigned>(e) < static_cast<unsigned>(E)) atomicAdd(&run[w][e], 1);
  }
  __syncthreads();
  // thread e: the waves' counts become their running bases; demand and kept
  int tot = 0;
  if (tid < E) {
#pragma unroll
    for (int ww = 0; ww < W; ++ww) {
      const int c = run[ww][tid];
      run[ww][tid] = tot;
      tot += c;
    }
  }
  const int kept = tid < E ? (tot < capacity ? tot : capacity) : 0;
  sc[tid] = kept;
  __syncthreads();
  for (int o = 1; o < 512; o <<= 1) {
    const int v = tid >= o ? sc[tid - o] : 0;
    __syncthreads();
    sc[tid] += v;
    __syncthreads();
  }
  if (tid < E) {
    counts[tid] = tot;
    offsets[tid] = sc[tid] - kept;
    off[tid] = sc[tid] - kept;
  }
  if (tid == E - 1) offsets[E] = sc[tid];
  __syncthreads();
  // stable scatter, 64 pairs at a time per wave (every wave runs seg / 64
  // rounds, so the block barriers below are reached by all)
  for (int c = 0; c < seg; c += 64) {
    const int p = pb + c + lane;
    const bool in_range = p < pe;
    const int e = in_range ? topk[p] : 0;
    const bool valid = in_range && static_cast<unsigned>(e) < static_cast<unsigned>(E);
    if (in_range && !valid) pair_pos[p] = -1;
    unsigned long long peers = __ballot(valid);
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const bool bit = (e >> b) & 1;
      const unsigned long long m = __ballot(valid && bit);
      peers &= bit ? m : ~m;
    }
    int cnt = 0;
    if (valid) {
      const int r = run[w][e] + __popcll(peers & ((1ull << lane) - 1ull));
      if (r < capacity) {
        const int pos = off[e] + r;
        sorted_pair[pos] = p;
        pair_pos[p] = pos;
      } else {
        pair_pos[p] = -1;
      }
      cnt = __popcll(peers);
    }
    __syncthreads();
    if (valid && (peers >> lane) == 1ull) run[w][e] += cnt;
    __syncthreads();
  }
  if (tile_start) {
    // thread g: row tiles of group g (routed: its kept rows; shared: T)
    const int G = E + S;
    int rows = 0;
    if (tid < E) rows = kept;
    else if (tid < G) rows = T;
    const int nt = (rows + MT - 1) / MT;
    __syncthreads();  // every thread is past its last read of sc
    sc[tid] = nt;
    __syncthreads();
    for (int o = 1; o < 512; o <<= 1) {
      const int v = tid >= o ? sc[tid - o] : 0;
      __syncthreads();
      sc[tid] += v;
      __syncthreads();
    }
    if (tid < G) tile_start[tid] = sc[tid] - nt;
    if (tid == G - 1) tile_start[G] = sc[tid];
    if (tid < kCtrSets * kXcds) tile_start[G + 1 + tid] = 0;
  }
  if (gamma != 0.0f && tid < E) {
    const long long diff = kT - static_cast<long long>(E) * tot;
    const float sgn = diff > 0 ? 1.0f : (diff < 0 ? -1.0f : 0.0f);
    bias[tid] = bias[tid] + gamma * sgn;
  }
}

bool dispatch_is_small(const Shape& s) {
  return static_cast<long long>(s.T) * s.k <= kDispatchSmallPairs && s.E <= 256 &&
         s.E + s.S <= 512;
}

hipError_t launch_dispatch_small(const Shape& s, const int32_t* topk_idx, int32_t* counts,
                                 int32_t* offsets, int32_t* sorted_pair, int32_t* pair_pos,
                                 int row_tile, int32_t* tile_start, float gamma, float* bias,
                                 hipStream_t st) {
  if (!dispatch_is_small(s)) return hipErrorInvalidValue;
  dispatch_small<<<1, 512, 0, st>>>(topk_idx, s.T * s.k, s.E, s.capacity, counts, offsets,
                                    sorted_pair, pair_pos, s.S, s.T, row_tile, tile_start,
                                    static_cast<long long>(s.k) * s.T, gamma, bias);
  return hipGetLastError();
}

hipError_t launch_dispatch(const Shape& s, const int32_t* topk_idx, int32_t* counts,
                           int32_t* offsets, int32_t* sorted_pair, int32_t* pair_pos,
                           int32_t* seg_counts, hipStream_t st) {
  if (dispatch_is_small(s))
    return launch_dispatch_small(s, topk_idx, counts, offsets, sorted_pair, pair_pos, 32,
                                 nullptr, 0.0f, nullptr, st);
  const long long npairs = static_cast<long long>(s.T) * s.k;
  const int nseg = dispatch_segments(s);
  if (nseg > 0) dispatch_count<<<nseg, 256, 0, st>>>(topk_idx, npairs, s.E, seg_counts);
  dispatch_scan<<<1, 256, 0, st>>>(seg_counts, nseg, s.E, s.capacity, counts, offsets);
  if (nseg > 0)
    dispatch_scatter<<<nseg, 64, 0, st>>>(topk_idx, npairs, s.E, s.capacity, seg_counts,
                                          offsets, sorted_pair, pair_pos);
  return hipGetLastError();
}

// ------------------------------------------------------------ bias update

// b[e] += gamma * sign(k*T - E*L_e): the sign is exact integer arithmetic
// and gamma * sign is exact, so the fp32 result is one rounded addition.
__global__ __launch_bounds__(256) void bias_update_kernel(const int32_t* __restrict__ counts,
                                                          int E, long long kT, float gamma,
                                                          float* __restrict__ bias) {
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= E) return;
  const long long diff = kT - static_cast<long long>(E) * counts[e];
  const float sgn = diff > 0 ? 1.0f : (diff < 0 ? -1.0f : 0.0f);
  bias[e] = bias[e] + gamma * sgn;
}

hipError_t launch_bias_update(const Shape& s, const int32_t* counts, float gamma, float* bias,
                              hipStream_t st) {
  bias_update_kernel<<<(s.E + 255) / 256, 256, 0, st>>>(
      counts, s.E, static_cast<long long>(s.k) * s.T, gamma, bias);
  return hipGetLastError();
}

}  // namespace moe
