// Expert MLPs as grouped GEMMs: gate/up with a fused SwiGLU, then down.
//
// "Under The Hood: Inkling", "MoE: the expert configuration": each routed
// expert is a SwiGLU FFN and the shared experts have the same width;
// "Inkling, Dissected", 02: the 2 shared experts process every token.
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
// consecutive items of their chunk.  Items of one group are ordered column
// tile outer, row tile inner, so the workgroups running together on an XCD
// share a weight tile (read from HBM once) and the group's activation rows
// stay in that XCD's L2.
#include "common.h"

namespace moe {

// ------------------------------------------------------------- tile plan

// tile_start[g] = first row tile of group g; tile_start[E+S] = total.
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
}

hipError_t launch_tile_plan(const Shape& s, const int32_t* offsets, int row_tile,
                            int32_t* tile_start, hipStream_t st) {
  tile_plan_kernel<<<1, 512, 0, st>>>(offsets, s.E, s.S, s.T, row_tile, tile_start);
  return hipGetLastError();
}

int ffn_row_tile(const Shape& s) {
  if (!s.bf16) return 32;
  const long long per_expert = static_cast<long long>(s.T) * s.k / s.E;
  return per_expert < 48 ? 32 : 128;
}

// ------------------------------------------------------------ item walk

struct Item {
  int g;      // group
  int m0;     // first row of the tile inside the group
  int rows;   // valid rows in the tile
  int n;      // column tile
  int grows;  // rows of the group
};

// Binary search over tile_start (in LDS) and the group's item order
// (column tile outer, row tile inner).
__device__ __forceinline__ Item decode_item(long long it, const int* ts, int G, int n_tiles,
                                            int MT, const int32_t* __restrict__ offsets, int T,
                                            int E) {
  int lo = 0, hi = G;  // find last g with ts[g] * n_tiles <= it
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (static_cast<long long>(ts[mid]) * n_tiles <= it) lo = mid;
    else hi = mid;
  }
  // skip empty groups that share the same start
  while (lo + 1 < G && ts[lo + 1] == ts[lo]) ++lo;
  Item r;
  r.g = lo;
  const int mt = ts[lo + 1] - ts[lo];
  const long long local = it - static_cast<long long>(ts[lo]) * n_tiles;
  r.n = static_cast<int>(local / mt);
  const int m = static_cast<int>(local % mt);
  r.grows = lo < E ? offsets[lo + 1] - offsets[lo] : T;
  r.m0 = m * MT;
  const int left = r.grows - r.m0;
  r.rows = left < MT ? left : MT;
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
};

// -------------------------------------------------------- bf16 MFMA GEMM

// Tile: MT rows x 256 weight rows, K step 64, 256 threads.
// GATED: the 256 weight rows are 128 output columns of W_gate interleaved
// with the same 128 columns of W_up in blocks of 32, so each wave holds the
// gate and up accumulators of the same outputs and applies SwiGLU in
// registers.  Otherwise the 256 weight rows are 256 output columns.
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
  static constexpr int LDSROW = BK + 8;  // bf16 elements; 144 B rows spread the banks
  static constexpr int NOUT = GATED ? NB / 2 : NB;
  static constexpr int A_CH = MT * BK / 8 / 256;   // 16-byte chunks per thread
  static constexpr int B_CH = NB * BK / 8 / 256;
  static constexpr int NSTAGE = 2;
  static constexpr int STAGE_ELEMS = (MT + NB) * LDSROW;
  static constexpr size_t LDS_BYTES = static_cast<size_t>(NSTAGE) * STAGE_ELEMS * 2;
};

template <int MT, bool GATED>
__global__ __launch_bounds__(256, 1) void ffn_bf16_kernel(FfnArgs p) {
  using C = Bf16Cfg<MT, GATED>;
  extern __shared__ __attribute__((aligned(16))) bf16_t lds[];
  __shared__ int ts[512];

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
  const int per_xcd = gridDim.x >> 3;
  const int slot = blockIdx.x >> 3;
  const long long chunk = (total + 7) / 8;
  const long long beg = xcd * chunk;
  const long long end = beg + chunk < total ? beg + chunk : total;

  const bf16_t* A = static_cast<const bf16_t*>(p.a);
  const size_t kT = static_cast<size_t>(p.k) * p.T;

  for (long long it = beg + slot; it < end; it += per_xcd) {
    const Item item = decode_item(it, ts, G, p.n_tiles, MT, p.offsets, p.T, p.E);
    const int g = item.g;
    const bool routed = g < p.E;
    const size_t row_base = routed ? static_cast<size_t>(p.offsets[g])
                                   : kT + static_cast<size_t>(g - p.E) * p.T;

    // ---- A rows of this thread's load chunks
    const bf16_t* a_src[C::A_CH];
#pragma unroll
    for (int i = 0; i < C::A_CH; ++i) {
      const int c = tid + 256 * i;
      int r = c >> 3;
      r = r < item.rows ? r : item.rows - 1;
      const int rr = item.m0 + r;
      size_t src_row;
      if (GATED) {
        src_row = routed ? static_cast<size_t>(p.sorted_pair[row_base + rr] / p.k)
                         : static_cast<size_t>(rr);
      } else {
        src_row = row_base + rr;
      }
      a_src[i] = A + src_row * p.K + (c & 7) * 8;
    }
    // ---- weight rows of this thread's load chunks
    const bf16_t* b_src[C::B_CH];
    const size_t wstride = static_cast<size_t>(p.N) * p.K;
#pragma unroll
    for (int i = 0; i < C::B_CH; ++i) {
      const int c = tid + 256 * i;
      const int r = c >> 3;
      const bf16_t* base;
      int wrow;
      if (GATED) {
        const int blk = r >> 5;
        wrow = item.n * C::NOUT + (blk >> 1) * 32 + (r & 31);
        const void* w = (blk & 1) ? (routed ? p.w1 : p.ws1) : (routed ? p.w0 : p.ws0);
        base = static_cast<const bf16_t*>(w) + (routed ? g : g - p.E) * wstride;
      } else {
        wrow = item.n * C::NOUT + r;
        base = static_cast<const bf16_t*>(routed ? p.w0 : p.ws0) + (routed ? g : g - p.E) * wstride;
      }
      b_src[i] = base + static_cast<size_t>(wrow) * p.K + (c & 7) * 8;
    }

    f32x16_t acc[C::BM][C::BN];
#pragma unroll
    for (int i = 0; i < C::BM; ++i)
#pragma unroll
      for (int j = 0; j < C::BN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    uint4 areg[C::A_CH], breg[C::B_CH];
    auto gload = [&](int k0) {
#pragma unroll
      for (int i = 0; i < C::A_CH; ++i) areg[i] = *reinterpret_cast<const uint4*>(a_src[i] + k0);
#pragma unroll
      for (int i = 0; i < C::B_CH; ++i) breg[i] = *reinterpret_cast<const uint4*>(b_src[i] + k0);
    };
    auto lstore = [&](int buf) {
      bf16_t* sA = lds + buf * C::STAGE_ELEMS;
      bf16_t* sB = sA + MT * C::LDSROW;
#pragma unroll
      for (int i = 0; i < C::A_CH; ++i) {
        const int c = tid + 256 * i;
        *reinterpret_cast<uint4*>(sA + (c >> 3) * C::LDSROW + (c & 7) * 8) = areg[i];
      }
#pragma unroll
      for (int i = 0; i < C::B_CH; ++i) {
        const int c = tid + 256 * i;
        *reinterpret_cast<uint4*>(sB + (c >> 3) * C::LDSROW + (c & 7) * 8) = breg[i];
      }
    };

    const int nk = p.K / C::BK;
    gload(0);
    lstore(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      const int buf = kt & 1;
      if (kt + 1 < nk) gload((kt + 1) * C::BK);
      const bf16_t* sA = lds + buf * C::STAGE_ELEMS;
      const bf16_t* sB = sA + MT * C::LDSROW;
#pragma unroll
      for (int kk = 0; kk < C::BK / 16; ++kk) {
        const int kof = kk * 16 + (lane >> 5) * 8;
        bf16x8_t af[C::BM], bfr[C::BN];
#pragma unroll
        for (int i = 0; i < C::BM; ++i)
          af[i] = *reinterpret_cast<const bf16x8_t*>(
              sA + (wm * C::WM + i * 32 + (lane & 31)) * C::LDSROW + kof);
#pragma unroll
        for (int j = 0; j < C::BN; ++j)
          bfr[j] = *reinterpret_cast<const bf16x8_t*>(
              sB + (wn * C::WN + j * 32 + (lane & 31)) * C::LDSROW + kof);
#pragma unroll
        for (int i = 0; i < C::BM; ++i)
#pragma unroll
          for (int j = 0; j < C::BN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
      }
      if (kt + 1 < nk) lstore(buf ^ 1);
      __syncthreads();
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

template <int MT, bool GATED>
static hipError_t run_bf16(const FfnArgs& a, hipStream_t st) {
  using C = Bf16Cfg<MT, GATED>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&ffn_bf16_kernel<MT, GATED>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize,
                                     static_cast<int>(C::LDS_BYTES));
  if (e != hipSuccess) return e;
  int grid = device_cus();
  grid = (grid + 7) / 8 * 8;
  ffn_bf16_kernel<MT, GATED><<<grid, 256, C::LDS_BYTES, st>>>(a);
  return hipGetLastError();
}

template <bool GATED>
static hipError_t run_f32(const FfnArgs& a, hipStream_t st) {
  ffn_f32_kernel<GATED><<<device_cus() * 4, 256, 0, st>>>(a);
  return hipGetLastError();
}

hipError_t launch_gate_up(const Shape& s, const void* x, const void* wg, const void* wu,
                          const void* wsg, const void* wsu, const int32_t* offsets,
                          const int32_t* sorted_pair, const int32_t* tile_start, int row_tile,
                          void* h, hipStream_t st) {
  if (s.T == 0) return hipSuccess;
  FfnArgs a{};
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
    a.n_tiles = s.F / Bf16Cfg<128, true>::NOUT;
    return row_tile == 32 ? run_bf16<32, true>(a, st) : run_bf16<128, true>(a, st);
  }
  a.n_tiles = s.F / 32;
  return run_f32<true>(a, st);
}

hipError_t launch_down(const Shape& s, const void* wd, const void* wsd, const int32_t* offsets,
                       const int32_t* tile_start, int row_tile, const void* h, void* y_routed,
                       void* y_shared, hipStream_t st) {
  if (s.T == 0) return hipSuccess;
  FfnArgs a{};
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
    a.n_tiles = s.d / Bf16Cfg<128, false>::NOUT;
    return row_tile == 32 ? run_bf16<32, false>(a, st) : run_bf16<128, false>(a, st);
  }
  a.n_tiles = s.d / 64;
  return run_f32<false>(a, st);
}

}  // namespace moe
