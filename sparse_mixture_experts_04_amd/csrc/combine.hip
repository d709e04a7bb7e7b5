// Combine: y_t = sum over the k + S contributors of g * expert output.
//
// "Inkling, Dissected", 02 and 02b: the layer output is the gate-weighted
// sum of the chosen routed experts' outputs (6 of them) and the shared
// experts' outputs (2 in the layer of the pages; 0 to 2 here); a pair
// dropped at its expert's capacity (pair_pos < 0, 02d) contributes
// nothing.  Each output element is summed in fp32 in a fixed order
// (routed slots in rank order, then the shared experts), from rows found
// through pair_pos, with no atomics: the result is deterministic.
#include "common.h"

namespace moe {

template <typename T> struct Vec;
template <> struct Vec<bf16_t> {
  static constexpr int N = 8;  // 16-byte loads
  __device__ static void load(const bf16_t* p, float (&v)[8]) {
    const uint4 u = *reinterpret_cast<const uint4*>(p);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  __device__ static void store(bf16_t* p, const float (&v)[8]) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = static_cast<uint32_t>(f32_to_bf16(v[2 * i])) |
             (static_cast<uint32_t>(f32_to_bf16(v[2 * i + 1])) << 16);
    *reinterpret_cast<uint4*>(p) = make_uint4(w[0], w[1], w[2], w[3]);
  }
};
template <> struct Vec<float> {
  static constexpr int N = 4;
  __device__ static void load(const float* p, float (&v)[4]) {
    const float4 u = *reinterpret_cast<const float4*>(p);
    v[0] = u.x; v[1] = u.y; v[2] = u.z; v[3] = u.w;
  }
  __device__ static void store(float* p, const float (&v)[4]) {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  }
};

// Block b handles token b / nchunk, columns (b % nchunk) * CB * VEC + ...
// Every contributor row is loaded before the sums start, so the loads of a
// thread are in flight together; a dropped pair loads row 0 (a valid
// address) and is left out of the sum, which keeps the fixed order.
constexpr int CB = 128;  // threads per block
template <typename T, int K, int S>
__global__ __launch_bounds__(CB) void combine_kernel(const T* __restrict__ yr,
                                                     const T* __restrict__ ys,
                                                     const float* __restrict__ gates,
                                                     const int32_t* __restrict__ pair_pos,
                                                     int Tn, int d, int nchunk,
                                                     T* __restrict__ y) {
  constexpr int V = Vec<T>::N;
  const int t = blockIdx.x / nchunk;
  const int c0 = ((blockIdx.x % nchunk) * CB + threadIdx.x) * V;
  if (c0 >= d) return;
  int pos[K];
  float g[K + S];
#pragma unroll
  for (int j = 0; j < K; ++j) pos[j] = pair_pos[static_cast<size_t>(t) * K + j];
#pragma unroll
  for (int j = 0; j < K + S; ++j) g[j] = gates[static_cast<size_t>(t) * (K + S) + j];
  float v[K + S][V];
#pragma unroll
  for (int j = 0; j < K; ++j)
    Vec<T>::load(yr + static_cast<size_t>(pos[j] < 0 ? 0 : pos[j]) * d + c0, v[j]);
#pragma unroll
  for (int s = 0; s < S; ++s)
    Vec<T>::load(ys + (static_cast<size_t>(s) * Tn + t) * d + c0, v[K + s]);
  float acc[V];
#pragma unroll
  for (int i = 0; i < V; ++i) acc[i] = 0.0f;
#pragma unroll
  for (int j = 0; j < K; ++j) {
    if (pos[j] < 0) continue;  // dropped at the expert's capacity
#pragma unroll
    for (int i = 0; i < V; ++i) acc[i] = fmaf(g[j], v[j][i], acc[i]);
  }
#pragma unroll
  for (int s = 0; s < S; ++s)
#pragma unroll
    for (int i = 0; i < V; ++i) acc[i] = fmaf(g[K + s], v[K + s][i], acc[i]);
  Vec<T>::store(y + static_cast<size_t>(t) * d + c0, acc);
}

// Layers with FP4 routed weights: the shared experts' down outputs arrive
// as ksplit fp32 K-slice partials (part[ks][s*Tn + t][c], ldp columns per
// row).  Each output is summed in slice order and rounded to bf16, the
// value the reduction pass would have stored as y_shared, then combined as
// in combine_kernel.
template <int K, int S>
__global__ __launch_bounds__(CB) void combine_part_kernel(const bf16_t* __restrict__ yr,
                                                          const float* __restrict__ part,
                                                          int ksplit, int ldp,
                                                          const float* __restrict__ gates,
                                                          const int32_t* __restrict__ pair_pos,
                                                          int Tn, int d, int nchunk,
                                                          bf16_t* __restrict__ y) {
  constexpr int V = 8;
  const int t = blockIdx.x / nchunk;
  const int c0 = ((blockIdx.x % nchunk) * CB + threadIdx.x) * V;
  if (c0 >= d) return;
  int pos[K];
  float g[K + S];
#pragma unroll
  for (int j = 0; j < K; ++j) pos[j] = pair_pos[static_cast<size_t>(t) * K + j];
#pragma unroll
  for (int j = 0; j < K + S; ++j) g[j] = gates[static_cast<size_t>(t) * (K + S) + j];
  float v[K + S][V];
#pragma unroll
  for (int j = 0; j < K; ++j)
    Vec<bf16_t>::load(yr + static_cast<size_t>(pos[j] < 0 ? 0 : pos[j]) * d + c0, v[j]);
  const size_t slice = static_cast<size_t>(S) * Tn * ldp;
  float ps[S][kFp4SharedSlicesMax][V];
#pragma unroll
  for (int s = 0; s < S; ++s)
#pragma unroll
    for (int ks = 0; ks < kFp4SharedSlicesMax; ++ks)
      if (ks < ksplit) {
        const float* src = part + ks * slice + (static_cast<size_t>(s) * Tn + t) * ldp + c0;
        float lo[4], hi[4];
        Vec<float>::load(src, lo);
        Vec<float>::load(src + 4, hi);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          ps[s][ks][i] = lo[i];
          ps[s][ks][4 + i] = hi[i];
        }
      }
#pragma unroll
  for (int s = 0; s < S; ++s)
#pragma unroll
    for (int i = 0; i < V; ++i) {
      float sum = 0.0f;
#pragma unroll
      for (int ks = 0; ks < kFp4SharedSlicesMax; ++ks)
        if (ks < ksplit) sum += ps[s][ks][i];
      v[K + s][i] = bf16_to_f32(f32_to_bf16(sum));
    }
  float acc[V];
#pragma unroll
  for (int i = 0; i < V; ++i) acc[i] = 0.0f;
#pragma unroll
  for (int j = 0; j < K; ++j) {
    if (pos[j] < 0) continue;  // dropped at the expert's capacity
#pragma unroll
    for (int i = 0; i < V; ++i) acc[i] = fmaf(g[j], v[j][i], acc[i]);
  }
#pragma unroll
  for (int s = 0; s < S; ++s)
#pragma unroll
    for (int i = 0; i < V; ++i) acc[i] = fmaf(g[K + s], v[K + s][i], acc[i]);
  Vec<bf16_t>::store(y + static_cast<size_t>(t) * d + c0, acc);
}

hipError_t launch_combine_part(const Shape& s, const void* y_routed, const float* part,
                               int ksplit, const float* gates, const int32_t* pair_pos, void* y,
                               hipStream_t st) {
  if (s.T == 0) return hipSuccess;
  if (!s.bf16 || s.S < 1 || s.S > 2 || ksplit < 1 || ksplit > kFp4SharedSlicesMax ||
      s.d % 256 != 0)
    return hipErrorInvalidValue;
  const int nchunk = (s.d + CB * 8 - 1) / (CB * 8);
  const long long blocks = static_cast<long long>(s.T) * nchunk;
  const bf16_t* yr = static_cast<const bf16_t*>(y_routed);
  bf16_t* out = static_cast<bf16_t*>(y);
  if (s.S == 1)
    combine_part_kernel<6, 1><<<static_cast<unsigned>(blocks), CB, 0, st>>>(
        yr, part, ksplit, s.d, gates, pair_pos, s.T, s.d, nchunk, out);
  else
    combine_part_kernel<6, 2><<<static_cast<unsigned>(blocks), CB, 0, st>>>(
        yr, part, ksplit, s.d, gates, pair_pos, s.T, s.d, nchunk, out);
  return hipGetLastError();
}

template <typename T, int S>
static void run_combine(const Shape& s, const void* y_routed, const void* y_shared,
                        const float* gates, const int32_t* pair_pos, void* y, hipStream_t st) {
  constexpr int V = Vec<T>::N;
  const int nchunk = (s.d + CB * V - 1) / (CB * V);
  const long long blocks = static_cast<long long>(s.T) * nchunk;
  combine_kernel<T, 6, S><<<static_cast<unsigned>(blocks), CB, 0, st>>>(
      static_cast<const T*>(y_routed), static_cast<const T*>(y_shared), gates, pair_pos, s.T,
      s.d, nchunk, static_cast<T*>(y));
}

template <typename T>
static void run_combine_s(const Shape& s, const void* y_routed, const void* y_shared,
                          const float* gates, const int32_t* pair_pos, void* y, hipStream_t st) {
  if (s.S == 0) run_combine<T, 0>(s, y_routed, y_shared, gates, pair_pos, y, st);
  else if (s.S == 1) run_combine<T, 1>(s, y_routed, y_shared, gates, pair_pos, y, st);
  else run_combine<T, 2>(s, y_routed, y_shared, gates, pair_pos, y, st);
}

hipError_t launch_combine(const Shape& s, const void* y_routed, const void* y_shared,
                          const float* gates, const int32_t* pair_pos, void* y,
                          hipStream_t st) {
  if (s.T == 0) return hipSuccess;
  if (s.bf16) run_combine_s<bf16_t>(s, y_routed, y_shared, gates, pair_pos, y, st);
  else run_combine_s<float>(s, y_routed, y_shared, gates, pair_pos, y, st);
  return hipGetLastError();
}

}  // namespace moe
