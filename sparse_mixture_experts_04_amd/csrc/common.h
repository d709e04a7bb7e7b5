// Internal declarations shared by the HIP sources of libmoe.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

typedef uint16_t bf16_t;  // raw bfloat16 bits

// Generic -> LDS address-space cast of a pointer into a __shared__ array.
#define LDS_PTR(p) ((__attribute__((address_space(3))) void*)(p))

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

__device__ __forceinline__ float bf16_to_f32(bf16_t v) {
  return __uint_as_float(static_cast<uint32_t>(v) << 16);
}

// Round to nearest even; NaN stays NaN (gfx950 converts in hardware,
// v_cvt_pk_bf16_f32).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(bf16_t, static_cast<__bf16>(f));
}

template <typename T> struct ActTraits;
template <> struct ActTraits<float> {
  __device__ static float load(const float* p) { return *p; }
  __device__ static void store(float* p, float v) { *p = v; }
};
template <> struct ActTraits<bf16_t> {
  __device__ static float load(const bf16_t* p) { return bf16_to_f32(*p); }
  __device__ static void store(bf16_t* p, float v) { *p = f32_to_bf16(v); }
};

// Shape handed to the launchers (validated on the host beforehand).
struct Shape {
  int T, d, F, E, S, k;
  bool bf16;
  bool gate_logsumexp = false;  // gate normalisation (router only)
  float gate_scale = 1.0f;
  int capacity = 0x7fffffff;     // pairs kept per routed expert
  bool w_fp4 = false;            // routed expert weights in MXFP4
};

// Router columns are padded to a multiple of the router's column tile.
constexpr int kRouterColTile = 64;
constexpr int kRouterChunk = 256;  // K granularity of the split across workgroups
inline int router_cols_padded(const Shape& s) {
  int n = s.E + s.S;
  return (n + kRouterColTile - 1) / kRouterColTile * kRouterColTile;
}
int router_ksplits(const Shape& s);
size_t router_refine_ints(const Shape& s);

// Dispatch segments: pairs handled by one stable-scatter wave.
constexpr int kDispatchSeg = 512;
inline int dispatch_segments(const Shape& s) {
  long long p = static_cast<long long>(s.T) * s.k;
  return static_cast<int>((p + kDispatchSeg - 1) / kDispatchSeg);
}

// Expert GEMM row tile chosen for a shape (routed rows per expert decide).
int ffn_row_tile(const Shape& s);

// ---- launchers (return hipSuccess or the launch error) -------------------
// The three bf16 planes of w_router ([3, router_cols_padded(s), d]).
hipError_t launch_router_planes(const Shape& s, const float* w_router, bf16_t* planes,
                                hipStream_t st);

// prepared: planes from launch_router_planes, or null to split w_router
// into wplanes (workspace) first.  refine: router_refine_ints(s) ints of
// workspace (the tokens the exact pass redoes, with their candidates).
hipError_t launch_router(const Shape& s, const void* x, const float* w_router,
                         const bf16_t* prepared, const float* bias, int32_t* topk_idx,
                         float* gates, float* margin, bf16_t* wplanes, double* partial,
                         int32_t* refine, hipStream_t st);

hipError_t launch_dispatch(const Shape& s, const int32_t* topk_idx, int32_t* counts,
                           int32_t* offsets, int32_t* sorted_pair, int32_t* pair_pos,
                           int32_t* seg_counts, hipStream_t st);

// Small batches (T * k <= kDispatchSmallPairs, E <= 256): the dispatch in
// one launch, optionally followed by the row-tile plan (tile_start set; the
// plan launch_tile_plan writes for row_tile 32) and the bias update
// (gamma != 0; bias as launch_bias_update updates it).  Outputs as
// launch_dispatch's.
constexpr int kDispatchSmallPairs = 4096;
bool dispatch_is_small(const Shape& s);
hipError_t launch_dispatch_small(const Shape& s, const int32_t* topk_idx, int32_t* counts,
                                 int32_t* offsets, int32_t* sorted_pair, int32_t* pair_pos,
                                 int row_tile, int32_t* tile_start, float gamma, float* bias,
                                 hipStream_t st);

hipError_t launch_tile_plan(const Shape& s, const int32_t* offsets, int row_tile,
                            int32_t* tile_start, hipStream_t st);

// marks (optional, may be null): see launch_big; the 32-row path records
// marks[0] and marks[1] together after its single launch.
// scg, scu, scd: scales of the routed weights when they are FP4 (s.w_fp4),
// else unused.
// part: shared_partial_floats(s) floats of workspace (null when 0).
// fold_gates (large-batch tiles only, else null): gates [T, k+S]; each
// shared expert's row of h is scaled by its token's gate for that expert,
// for launch_shared_combine.
hipError_t launch_gate_up(const Shape& s, const void* x, const void* wg, const void* wu,
                          const void* wsg, const void* wsu, const uint8_t* scg,
                          const uint8_t* scu, const int32_t* offsets,
                          const int32_t* sorted_pair, const int32_t* tile_start,
                          int row_tile, void* h, float* part, hipEvent_t* marks,
                          hipStream_t st, const float* fold_gates = nullptr);

// routed_only (large-batch tiles only): the routed experts' tiles alone; the
// shared experts' down GEMM is left to launch_shared_combine.
// shared_partials (FP4 routed weights, S > 0): the shared experts' K-slice
// partials are left in part for launch_combine_part instead of being
// reduced into y_shared.
hipError_t launch_down(const Shape& s, const void* wd, const void* wsd, const uint8_t* scd,
                       const int32_t* offsets, const int32_t* tile_start, int row_tile,
                       const void* h, void* y_routed, void* y_shared, float* part,
                       hipEvent_t* marks, hipStream_t st, bool routed_only = false,
                       bool shared_partials = false);

// The shared experts' down GEMM over their gate-scaled rows of h (from
// launch_gate_up with fold_gates), fused with the combine: writes
// y = sum of the routed contributions (y_routed through pair_pos, in slot
// order) plus the shared experts' gate-weighted outputs.  Large-batch tiles
// (row_tile 128 or 256) and S > 0 only; tile_start is the tile plan whose
// fused-combine work counters it uses.
hipError_t launch_shared_combine(const Shape& s, const void* wsd, const int32_t* tile_start,
                                 int row_tile, const void* h, const void* y_routed,
                                 const float* gates, const int32_t* pair_pos, void* y,
                                 hipStream_t st);

// fp32 floats of the K-slice partials the shared experts need with FP4
// routed weights (0 otherwise); the gate/up and down launches share them.
size_t shared_partial_floats(const Shape& s);

hipError_t launch_quantize_mxfp4(long long E, int N, int K, const void* w, uint8_t* codes,
                                 uint8_t* scales, hipStream_t st);

hipError_t launch_combine(const Shape& s, const void* y_routed, const void* y_shared,
                          const float* gates, const int32_t* pair_pos, void* y,
                          hipStream_t st);

// Combine for layers with FP4 routed weights and S > 0: the shared
// experts' down outputs are read as the ksplit fp32 K-slice partials the FP4
// down launch leaves in part (launch_down with shared_partials), summed and
// rounded as the reduction pass would have stored them.  bf16, d % 256 == 0.
constexpr int kFp4SharedSlicesMax = 4;
hipError_t launch_combine_part(const Shape& s, const void* y_routed, const float* part,
                               int ksplit, const float* gates, const int32_t* pair_pos, void* y,
                               hipStream_t st);
// K slices of a shared-expert tile in the FP4 launch for a GEMM over K.
int fp4_shared_slices(int K);

hipError_t launch_bias_update(const Shape& s, const int32_t* counts, float gamma,
                              float* bias, hipStream_t st);

}  // namespace moe
