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
#include "common.h"

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

hipError_t launch_dispatch(const Shape& s, const int32_t* topk_idx, int32_t* counts,
                           int32_t* offsets, int32_t* sorted_pair, int32_t* pair_pos,
                           int32_t* seg_counts, hipStream_t st) {
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
