// Router: z = x . W_r^T, sigmoid affinities, biased top-k, joint gates.
//
// "Inkling, Dissected", 02b "Sigmoid, not softmax": s_i = sigmoid(x . w_i);
// keep the top-6 routed experts by s_i + b_i; g_i = s_i over the sum of s_j
// for j in the kept routed experts and the shared experts.  "Under The Hood:
// Inkling", routing strategy: the top-k runs over the routed experts only,
// the shared experts' scores join the normalisation.
//
// Accuracy.  The gates are compared at 1e-6 relative error, so z must be
// close to exact even at d = 7168 and |z| ~ 4, where one fp32 ulp is
// already 4.8e-7.  W_r (fp32) is split into three bf16 planes,
// w = hi + mid + lo up to ~2^-27 |w|, and x (bf16, or fp32 split the same
// way) is multiplied plane by plane on the bf16 matrix cores, whose
// products are exact in fp32.  Each 32-element K step starts from a zero
// accumulator (the 3 or 6 plane products of that step are its only fp32
// additions) and is then added to an fp64 running sum; the partial logits
// are stored in fp64 and, when small batches split K across workgroups,
// added in fixed order by the selection kernel.  Everything after z
// (sigmoid, keys, top-k, gates) is fp64.
#include "common.h"

namespace moe {

// Gap between adjacent keys (s + b) among a token's k + 1 best under which
// its selection is redone from exact logits (router_refine): far above the
// keys' error from the matrix-core logits (those keys are within ~1e-7 of
// exact; see router_select), so every token whose picks or their order
// could differ from exact arithmetic is redone, and few enough tokens that
// the refinement is cheap.
constexpr double kRefineGap = 1e-5;
// The selection's record of a token for the exact pass: token, candidate
// count (or -1 when there are more than kRefineCand), then the candidates'
// expert ids in ascending order.
constexpr int kRefineCand = 14;
constexpr int kRefineRec = 2 + kRefineCand;

// ---------------------------------------------------------------- planes

__global__ __launch_bounds__(256) void router_split_planes(
    const float* __restrict__ w, int rows, int d, int rows_pad, bf16_t* __restrict__ planes) {
  const size_t n = static_cast<size_t>(rows_pad) * d;
  const size_t stride = static_cast<size_t>(gridDim.x) * blockDim.x;
  for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride) {
    const int r = static_cast<int>(i / d);
    const float v = r < rows ? w[i] : 0.0f;
    const bf16_t hi = f32_to_bf16(v);
    const float r1 = v - bf16_to_f32(hi);      // exact (Sterbenz)
    const bf16_t mid = f32_to_bf16(r1);
    const float r2 = r1 - bf16_to_f32(mid);    // exact
    planes[i] = hi;
    planes[n + i] = mid;
    planes[2 * n + i] = f32_to_bf16(r2);
  }
}

// ---------------------------------------------------------------- logits

typedef uint16_t u16x8_t __attribute__((ext_vector_type(8)));

__device__ __forceinline__ void split3(const float (&v)[8], bf16x8_t& p0, bf16x8_t& p1,
                                       bf16x8_t& p2) {
  u16x8_t a, b, c;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const bf16_t hi = f32_to_bf16(v[i]);
    const float r1 = v[i] - bf16_to_f32(hi);
    const bf16_t mid = f32_to_bf16(r1);
    const float r2 = r1 - bf16_to_f32(mid);
    a[i] = hi;
    b[i] = mid;
    c[i] = f32_to_bf16(r2);
  }
  p0 = __builtin_bit_cast(bf16x8_t, a);
  p1 = __builtin_bit_cast(bf16x8_t, b);
  p2 = __builtin_bit_cast(bf16x8_t, c);
}

// x fragments of one K step for the 4 row blocks of a lane, straight from
// global memory (fp32 x is split into its 3 bf16 planes on the fly).
template <int NXP>
__device__ __forceinline__ void router_load_x(const void* __restrict__ xv, const size_t (&xoff)[4],
                                              int k, bf16x8_t (&a)[NXP][4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (NXP == 1) {
      const bf16_t* xp = static_cast<const bf16_t*>(xv) + xoff[i] + k;
      a[0][i] = *reinterpret_cast<const bf16x8_t*>(xp);
    } else {
      const float* xp = static_cast<const float*>(xv) + xoff[i] + k;
      const float4 v0 = *reinterpret_cast<const float4*>(xp);
      const float4 v1 = *reinterpret_cast<const float4*>(xp + 4);
      const float v[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
      split3(v, a[0][i], a[1][i], a[2][i]);
    }
  }
}

// Workgroup tile: 128 tokens x 64 router columns over one K range.
// 4 waves: wave (wm, wn) owns tokens wm*64..+64 and columns wn*32..+32 as
// 4 x 2 blocks of 16x16 (MFMA 16x16x32 bf16).  The W planes are staged in
// LDS (shared by the 4 waves); x fragments are loaded straight from global.
// NXP = number of x planes: 1 for bf16 x, 3 for fp32 x.
template <int NXP>
__global__ __launch_bounds__(256) void router_logits(
    const void* __restrict__ xv, const bf16_t* __restrict__ planes, int T, int d, int npad,
    int nks, int chunk, double* __restrict__ partial, int32_t* __restrict__ refine) {
  if ((blockIdx.x | blockIdx.y | blockIdx.z | threadIdx.x) == 0) refine[0] = 0;
  constexpr int KS = 32;
  constexpr int LDSW = KS + 8;
  const int steps_per_chunk = chunk / KS;
  __shared__ __attribute__((aligned(16))) bf16_t sB[2][3][64][LDSW];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int tok0 = blockIdx.x * 128 + wm * 64;
  const int col0 = blockIdx.y * 64;

  const int nch = d / chunk;
  const int ch_b = static_cast<int>(static_cast<long long>(blockIdx.z) * nch / nks);
  const int ch_e = static_cast<int>(static_cast<long long>(blockIdx.z + 1) * nch / nks);
  const int kbeg = ch_b * chunk;
  const int nsteps = (ch_e - ch_b) * steps_per_chunk;

  // B staging: each thread moves the same 16-byte chunk of the 3 planes.
  const size_t pstride = static_cast<size_t>(npad) * d;
  const int brow = tid >> 2, bkc = (tid & 3) * 8;
  const bf16_t* bsrc = planes + static_cast<size_t>(col0 + brow) * d + bkc;
  uint4 breg[3];

  // x rows of this lane (clamped to a valid row; clamped rows are not stored)
  const int ak = (lane >> 4) * 8;
  size_t xoff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int r = tok0 + i * 16 + (lane & 15);
    r = r < T ? r : T - 1;
    xoff[i] = static_cast<size_t>(r) * d + ak;
  }

  double run[4][2][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) run[i][j][r] = 0.0;

#pragma unroll
  for (int p = 0; p < 3; ++p)
    breg[p] = *reinterpret_cast<const uint4*>(bsrc + p * pstride + kbeg);
#pragma unroll
  for (int p = 0; p < 3; ++p) *reinterpret_cast<uint4*>(&sB[0][p][brow][bkc]) = breg[p];
  __syncthreads();

  bf16x8_t a[NXP][4], an[NXP][4];
  router_load_x<NXP>(xv, xoff, kbeg, an);

  for (int s = 0; s < nsteps; ++s) {
    const int k = kbeg + s * KS;
    const int buf = s & 1;
#pragma unroll
    for (int q = 0; q < NXP; ++q)
#pragma unroll
      for (int i = 0; i < 4; ++i) a[q][i] = an[q][i];
    if (s + 1 < nsteps) {
#pragma unroll
      for (int p = 0; p < 3; ++p)
        breg[p] = *reinterpret_cast<const uint4*>(bsrc + p * pstride + k + KS);
      router_load_x<NXP>(xv, xoff, k + KS, an);
    }
    bf16x8_t b[3][2];
#pragma unroll
    for (int p = 0; p < 3; ++p)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        b[p][j] = *reinterpret_cast<const bf16x8_t*>(&sB[buf][p][wn * 32 + j * 16 + (lane & 15)][ak]);

#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        f32x4_t c = {0.f, 0.f, 0.f, 0.f};
        if constexpr (NXP == 1) {
          c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[0][i], b[2][j], c, 0, 0, 0);
          c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[0][i], b[1][j], c, 0, 0, 0);
          c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[0][i], b[0][j], c, 0, 0, 0);
        } else {
          c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[2][i], b[0][j], c, 0, 0, 0);
          c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[1][i], b[1][j], c, 0, 0, 0);
          c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[0][i], b[2][j], c, 0, 0, 0);
          c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[1][i], b[0][j], c, 0, 0, 0);
          c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[0][i], b[1][j], c, 0, 0, 0);
          c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[0][i], b[0][j], c, 0, 0, 0);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) run[i][j][r] += static_cast<double>(c[r]);
      }

    if (s + 1 < nsteps) {
#pragma unroll
      for (int p = 0; p < 3; ++p)
        *reinterpret_cast<uint4*>(&sB[buf ^ 1][p][brow][bkc]) = breg[p];
    }
    __syncthreads();
  }

  // 16x16 accumulator layout: lane l holds column l%16, rows 4*(l/16)+r.
  double* out = partial + static_cast<size_t>(blockIdx.z) * T * npad;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = tok0 + i * 16 + 4 * (lane >> 4) + r;
        const int c = col0 + wn * 32 + j * 16 + (lane & 15);
        if (t < T) out[static_cast<size_t>(t) * npad + c] = run[i][j][r];
      }
}

// Logits for bf16 x with direct global -> LDS loads.  Same tile and
// arithmetic as router_logits<1> (128 tokens x 64 columns, MFMA 16x16x32,
// a fresh fp32 accumulator per 32-wide K step added into fp64 sums), with
// the x rows and the three W planes of each K step staged through a ring
// of RS stages so that several steps of loads are in flight.  LDS rows are
// 64 bytes with chunk c of row r in slot c ^ f(m), m = (r >> 2) & 3 and
// f(m) = m ^ parity(m).  gfx950 serves a ds_read_b128 16 lanes per cycle
// over 64 banks of 4 bytes, the 16 lanes being the lane quads of a half
// wave whose quad indices have equal parity; a 16x16 fragment read (lane l:
// row l % 16, chunk l / 16) then hits each 16-byte slot of a bank row once
// per cycle.
constexpr int kRouterRing = 4;
constexpr int kRouterStageElems = (128 + 3 * 64) * 32;  // x rows, then 3 planes x 64 rows

__global__ __launch_bounds__(256) void router_logits_bf16(
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ planes, int T, int d, int npad,
    int nks, int chunk, double* __restrict__ partial, int32_t* __restrict__ refine) {
  if ((blockIdx.x | blockIdx.y | blockIdx.z | threadIdx.x) == 0) refine[0] = 0;
  constexpr int KS = 32;
  constexpr int RS = kRouterRing;
  constexpr int SE = kRouterStageElems;
  constexpr int LPW = 5;  // 1 KiB loads per wave per stage: 8 for x, 12 for the planes
  const int steps_per_chunk = chunk / KS;
  __shared__ __attribute__((aligned(1024))) bf16_t ring[RS * SE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;
  const int tok0 = blockIdx.x * 128;
  const int col0 = blockIdx.y * 64;

  const int nch = d / chunk;
  const int ch_b = static_cast<int>(static_cast<long long>(blockIdx.z) * nch / nks);
  const int ch_e = static_cast<int>(static_cast<long long>(blockIdx.z + 1) * nch / nks);
  const int kbeg = ch_b * chunk;
  const int nsteps = (ch_e - ch_b) * steps_per_chunk;

  // load j (16 LDS rows) of a stage: j < 8 x rows 16j.., else plane
  // (j - 8) / 4, rows 16 ((j - 8) % 4)..; lane l fills slot l % 4 of row
  // l / 4 of its load with source chunk (l % 4) ^ f(row)
  const size_t pstride = static_cast<size_t>(npad) * d;
  const int lrow = lane >> 2;
  // the row of lane l in its load is l / 4, so its m is (l >> 4) & 3
  const int lm = (lane >> 4) & 3;
  const int cbase = (lane & 3) ^ lm ^ ((lm ^ (lm >> 1)) & 1);
  const bf16_t* src[LPW];
  uint32_t dst_off[LPW];
#pragma unroll
  for (int q = 0; q < LPW; ++q) {
    const int j = wave * LPW + q;
    if (j < 8) {
      int r = tok0 + j * 16 + lrow;
      r = r < T ? r : T - 1;
      src[q] = x + static_cast<size_t>(r) * d + kbeg + cbase * 8;
    } else {
      const int jb = j - 8;
      src[q] = planes + (jb >> 2) * pstride +
               static_cast<size_t>(col0 + (jb & 3) * 16 + lrow) * d + kbeg + cbase * 8;
    }
    dst_off[q] = static_cast<uint32_t>(j * 512 * sizeof(bf16_t));
  }
  const uint32_t ring_base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(LDS_PTR(ring)));
  auto issue = [&](int s, int slot) {
    const int ko = (s < nsteps ? s : nsteps - 1) * KS;
#pragma unroll
    for (int q = 0; q < LPW; ++q) {
      const uint32_t m0 = __builtin_amdgcn_readfirstlane(ring_base + slot * SE * 2 + dst_off[q]);
      asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
                   :
                   : "v"(src[q] + ko), "s"(m0)
                   : "m0");
    }
  };

  // fragment offset: row r16 = lane % 16 of a 16-row block, chunk lane / 16
  // (the slot does not depend on the block)
  const int r16 = lane & 15;
  const int m16 = (r16 >> 2) & 3;
  const int f0 = m16 ^ ((m16 ^ (m16 >> 1)) & 1);
  const int cq = lane >> 4;
  const int off = r16 * 32 + ((cq ^ f0) << 3);

  double run[4][2][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) run[i][j][r] = 0.0;

#pragma unroll
  for (int s = 0; s < RS - 1; ++s) issue(s, s);
  for (int s = 0; s < nsteps; ++s) {
    __builtin_amdgcn_s_waitcnt((((RS - 2) * LPW) & 0xF) | (0x7 << 4) | (0xF << 8) |
                               ((((RS - 2) * LPW) >> 4) << 14));  // stage s landed
    __builtin_amdgcn_s_barrier();
    issue(s + RS - 1, (s + RS - 1) % RS);
    const bf16_t* st = ring + (s % RS) * SE;
    bf16x8_t a[4], b[3][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      a[i] = *reinterpret_cast<const bf16x8_t*>(st + (wm * 64 + i * 16) * 32 + off);
#pragma unroll
    for (int p = 0; p < 3; ++p)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        b[p][j] = *reinterpret_cast<const bf16x8_t*>(st + (128 + p * 64 + wn * 32 + j * 16) * 32 +
                                                     off);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        f32x4_t c = {0.f, 0.f, 0.f, 0.f};
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[2][j], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[1][j], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[0][j], c, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 4; ++r) run[i][j][r] += static_cast<double>(c[r]);
      }
  }
  __builtin_amdgcn_s_waitcnt(0 | (0x7 << 4) | (0xF << 8));

  // 16x16 accumulator layout: lane l holds column l%16, rows 4*(l/16)+r.
  double* out = partial + static_cast<size_t>(blockIdx.z) * T * npad;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = tok0 + wm * 64 + i * 16 + 4 * (lane >> 4) + r;
        const int c = col0 + wn * 32 + j * 16 + (lane & 15);
        if (t < T) out[static_cast<size_t>(t) * npad + c] = run[i][j][r];
      }
}

// ------------------------------------------------------------- selection

__device__ __forceinline__ bool better(double ka, int ia, double kb, int ib) {
  return ka > kb || (ka == kb && ia < ib);
}

// Lane exchanges of the wave reductions: step STEP returns the value of
// lane l's partner.  Within a row of 16 lanes by DPP (xor 1, xor 2, then
// each 4-lane group against the other half of its 8 lanes, each 8-lane
// group against the other half of its row: lane i <-> 7 - i and 15 - i);
// across rows by the gfx950 permlane swaps (l <-> l ^ 16, l <-> l ^ 32).
// Every pairing is an involution, so after the six steps every lane holds
// the reduction of all 64 (an associative and commutative one, or a sum
// whose order is the same on every lane).  No exchange goes through LDS.
template <int STEP>
__device__ __forceinline__ int lane_xchg(int v, int lane) {
  if constexpr (STEP == 0) {
    return __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false);   // quad_perm 1,0,3,2
  } else if constexpr (STEP == 1) {
    return __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false);   // quad_perm 2,3,0,1
  } else if constexpr (STEP == 2) {
    return __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, false);  // row_half_mirror
  } else if constexpr (STEP == 3) {
    return __builtin_amdgcn_update_dpp(0, v, 0x140, 0xF, 0xF, false);  // row_mirror
  } else if constexpr (STEP == 4) {
    // odd rows of the first result hold the even rows' values, and the
    // even rows of the second the odd rows'
    const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return (lane & 16) ? static_cast<int>(r[0]) : static_cast<int>(r[1]);
  } else {
    const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return (lane & 32) ? static_cast<int>(r[0]) : static_cast<int>(r[1]);
  }
}

template <int STEP>
__device__ __forceinline__ double lane_xchg64(double v, int lane) {
  const long long u = __double_as_longlong(v);
  const int lo = lane_xchg<STEP>(static_cast<int>(u), lane);
  const int hi = lane_xchg<STEP>(static_cast<int>(u >> 32), lane);
  return __longlong_as_double((static_cast<long long>(hi) << 32) |
                              static_cast<unsigned int>(lo));
}

template <int STEP>
__device__ __forceinline__ void argmax_step(double& bk, int& bj, int lane) {
  const double ok = lane_xchg64<STEP>(bk, lane);
  const int oj = lane_xchg<STEP>(bj, lane);
  if (better(ok, oj, bk, bj)) {
    bk = ok;
    bj = oj;
  }
}

// (bk, bj) := the best pair over the wave (descending key, lower number on
// an exact tie: a total order, so the result does not depend on the order
// of the steps), on every lane.
__device__ __forceinline__ void wave_argmax(double& bk, int& bj, int lane) {
  argmax_step<0>(bk, bj, lane);
  argmax_step<1>(bk, bj, lane);
  argmax_step<2>(bk, bj, lane);
  argmax_step<3>(bk, bj, lane);
  argmax_step<4>(bk, bj, lane);
  argmax_step<5>(bk, bj, lane);
}

// Sum over the wave in a fixed order (the same on every lane).
__device__ __forceinline__ double wave_sum(double v, int lane) {
  v += lane_xchg64<0>(v, lane);
  v += lane_xchg64<1>(v, lane);
  v += lane_xchg64<2>(v, lane);
  v += lane_xchg64<3>(v, lane);
  v += lane_xchg64<4>(v, lane);
  v += lane_xchg64<5>(v, lane);
  return v;
}

// Value of a double on a wave-uniform lane.
__device__ __forceinline__ double read_lane64(double v, int src) {
  const long long u = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_readlane(static_cast<int>(u), src);
  const int hi = __builtin_amdgcn_readlane(static_cast<int>(u >> 32), src);
  return __longlong_as_double((static_cast<long long>(hi) << 32) |
                              static_cast<unsigned int>(lo));
}

// K + 1 rounds of a wave-wide argmax over the candidates the lanes hold:
// candidate j = lane + 64q sits on lane j % 64 (valid[q]; keys, affinities
// s and logits z).  The candidates are numbered in ascending expert id, so
// rank order is descending key with exact ties to the lower number.  Fills,
// on every lane, the numbers, s and z of the K picks and the keys of the
// K + 1 best (the last one for the margin).
template <int K, int Q>
__device__ __forceinline__ void rank_rounds(int lane, const bool (&valid)[Q],
                                            const double (&key)[Q], const double (&sv)[Q],
                                            const double (&zv)[Q], int (&j_sel)[K],
                                            double (&s_sel)[K], double (&z_sel)[K],
                                            double (&k_sel)[K + 1]) {
  bool taken[Q];
#pragma unroll
  for (int q = 0; q < Q; ++q) taken[q] = !valid[q];
#pragma unroll
  for (int r = 0; r <= K; ++r) {
    double bk = -INFINITY;
    int bj = 0x7fffffff;
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      const int j = lane + 64 * q;
      if (!taken[q] && better(key[q], j, bk, bj)) {
        bk = key[q];
        bj = j;
      }
    }
    wave_argmax(bk, bj, lane);
    bj = __builtin_amdgcn_readfirstlane(bj);  // the same on every lane
    k_sel[r] = bk;
    if (r < K) {
      const int q = bj >> 6;
      const int owner = bj & 63;
      double my = sv[0], mz = zv[0];
#pragma unroll
      for (int qq = 1; qq < Q; ++qq) {
        my = q == qq ? sv[qq] : my;
        mz = q == qq ? zv[qq] : mz;
      }
      s_sel[r] = read_lane64(my, owner);
      z_sel[r] = read_lane64(mz, owner);
      if (lane == owner) {
#pragma unroll
        for (int qq = 0; qq < Q; ++qq) taken[qq] = taken[qq] || q == qq;
      }
      j_sel[r] = bj;
    }
  }
}

// Gates of the K picks and the S shared experts (s_sh, z_sh: shared expert
// j's affinity and logit on lane j), then the outputs of token t: topk in
// rank order, gates in slot order, margin = key_K - key_(K+1).  Gates:
// s_j / sum s, or exp(logsigmoid(z_j) - logsumexp logsigmoid(z)), over the
// K + S contributors in slot order, times gate_scale.
template <int K, int S>
__device__ __forceinline__ void write_token(int t, int lane, const int (&i_sel)[K],
                                            const double (&s_pick)[K], const double (&z_pick)[K],
                                            double s_sh, double z_sh,
                                            const double (&k_sel)[K + 1],
                                            int32_t* __restrict__ topk, float* __restrict__ gates,
                                            float* __restrict__ margin, bool logsumexp_norm,
                                            double gate_scale) {
  double s_sel[K + S], z_sel[K + S];
#pragma unroll
  for (int j = 0; j < K; ++j) {
    s_sel[j] = s_pick[j];
    z_sel[j] = z_pick[j];
  }
#pragma unroll
  for (int j = 0; j < S; ++j) {
    s_sel[K + j] = read_lane64(s_sh, j);
    z_sel[K + j] = read_lane64(z_sh, j);
  }
  double denom = 0.0;
  if (logsumexp_norm) {
#pragma unroll
    for (int j = 0; j < K + S; ++j) {
      const double z = z_sel[j];  // logsigmoid(z) = min(z, 0) - log1p(exp(-|z|))
      s_sel[j] = fmin(z, 0.0) - log1p(exp(-fabs(z)));
    }
    double m = s_sel[0];
#pragma unroll
    for (int j = 1; j < K + S; ++j) m = fmax(m, s_sel[j]);
#pragma unroll
    for (int j = 0; j < K + S; ++j) denom += exp(s_sel[j] - m);
    const double lse = m + log(denom);
#pragma unroll
    for (int j = 0; j < K + S; ++j) s_sel[j] = exp(s_sel[j] - lse) * gate_scale;
    denom = 1.0;
  } else {
#pragma unroll
    for (int j = 0; j < K + S; ++j) denom += s_sel[j];
    denom /= gate_scale;
  }
  if (lane < K) {
    int id = i_sel[0];
#pragma unroll
    for (int j = 1; j < K; ++j) id = lane == j ? i_sel[j] : id;
    topk[static_cast<size_t>(t) * K + lane] = id;
  }
  if (lane < K + S) {
    double sj = s_sel[0];
#pragma unroll
    for (int j = 1; j < K + S; ++j) sj = lane == j ? s_sel[j] : sj;
    gates[static_cast<size_t>(t) * (K + S) + lane] = static_cast<float>(sj / denom);
  }
  if (margin && lane == 0) margin[t] = static_cast<float>(k_sel[K - 1] - k_sel[K]);
}

__device__ __forceinline__ double sigmoid64(double z) { return 1.0 / (1.0 + exp(-z)); }

// Logits of token t from the matrix-core partials of K splits kb..ke-1,
// added in split order: lane l gets routed experts l + 64q (zv) and, on
// lanes < S, shared expert E + lane (z_sh; 0 elsewhere).  The partials of
// a group of G splits are loaded for all of the lane's experts before any
// is added (at T=64 K is split 28 ways, and a load at a time per expert
// would cost a round trip each).
template <int EPL, int S, int G>
__device__ __forceinline__ void token_logits(const double* __restrict__ partial, int kb, int ke,
                                             int T, int npad, int E, int t, int lane,
                                             double (&zv)[EPL], double& z_sh) {
  const size_t kstride = static_cast<size_t>(T) * npad;
  const double* row = partial + static_cast<size_t>(t) * npad;
#pragma unroll
  for (int q = 0; q < EPL; ++q) zv[q] = 0.0;
  z_sh = 0.0;
  for (int ks = kb; ks < ke; ks += G) {
    double v[G][EPL], vs[G];
#pragma unroll
    for (int j = 0; j < G; ++j) {
      if (ks + j < ke) {
        const double* r = row + static_cast<size_t>(ks + j) * kstride;
#pragma unroll
        for (int q = 0; q < EPL; ++q) v[j][q] = r[lane + 64 * q];
        vs[j] = lane < S ? r[E + lane] : 0.0;
      }
    }
#pragma unroll
    for (int j = 0; j < G; ++j) {
      if (ks + j < ke) {
#pragma unroll
        for (int q = 0; q < EPL; ++q) zv[q] += v[j][q];
        z_sh += vs[j];
      }
    }
  }
}

// Affinities s = sigmoid(z) and selection keys s + b of the lane's experts.
template <int EPL>
__device__ __forceinline__ void token_keys_from(const double (&zv)[EPL], int lane,
                                                const float* __restrict__ bias,
                                                double (&sv)[EPL], double (&key)[EPL]) {
#pragma unroll
  for (int q = 0; q < EPL; ++q) {
    const int e = lane + 64 * q;
    sv[q] = sigmoid64(zv[q]);
    key[q] = sv[q] + static_cast<double>(bias[e]);
  }
}

// Keys of token t from all nks splits, one wave.
template <int EPL, int S>
__device__ __forceinline__ void token_keys(const double* __restrict__ partial, int nks, int T,
                                           int npad, int E, int t, int lane,
                                           const float* __restrict__ bias, double (&zv)[EPL],
                                           double (&sv)[EPL], double (&key)[EPL],
                                           double& z_sh) {
  token_logits<EPL, S, 4>(partial, 0, nks, T, npad, E, t, lane, zv, z_sh);
  token_keys_from<EPL>(zv, lane, bias, sv, key);
}

// One wave per token, from the matrix-core logits.  Their error (the
// matrix cores round each 32-term partial sum, by up to a few 1e-7 measured
// on gfx950) can reorder keys that lie closer than ~1e-6.  A token with
// two adjacent keys among its K + 1 best closer than kRefineGap is
// therefore appended to `refine` (count at refine[0], tokens from refine[1];
// the list's order does not matter), and router_refine redoes it from
// exact logits; the outputs written here stand for every other token.
//
// WPT = 1: four tokens per workgroup, a wave each.  WPT = 4 (many K splits):
// one token per workgroup; wave w adds splits w*nks/4 .. (w+1)*nks/4 - 1 in
// one round of loads, and wave 0 adds the four sums in wave order and
// selects.
template <int K, int S, int EPL, int WPT>
__global__ __launch_bounds__(256) void router_select(
    const double* __restrict__ partial, int nks, int T, int npad, int E,
    const float* __restrict__ bias, int32_t* __restrict__ topk, float* __restrict__ gates,
    float* __restrict__ margin, bool logsumexp_norm, double gate_scale,
    int32_t* __restrict__ refine) {
  static_assert(WPT == 1 || WPT == 4, "waves per token");
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int t = WPT == 1 ? blockIdx.x * 4 + wave : blockIdx.x;
  if (t >= T) return;  // whole wave (WPT 1) or workgroup (WPT 4) leaves together

  double zv[EPL], sv[EPL], key[EPL], z_sh;
  if constexpr (WPT == 1) {
    token_keys<EPL, S>(partial, nks, T, npad, E, t, lane, bias, zv, sv, key, z_sh);
  } else {
    __shared__ double part_sum[WPT - 1][EPL + 1][64];
    token_logits<EPL, S, 8>(partial, wave * nks / WPT, (wave + 1) * nks / WPT, T, npad, E, t,
                            lane, zv, z_sh);
    if (wave > 0) {
#pragma unroll
      for (int q = 0; q < EPL; ++q) part_sum[wave - 1][q][lane] = zv[q];
      part_sum[wave - 1][EPL][lane] = z_sh;
    }
    __syncthreads();
    if (wave > 0) return;
#pragma unroll
    for (int w = 0; w < WPT - 1; ++w) {
#pragma unroll
      for (int q = 0; q < EPL; ++q) zv[q] += part_sum[w][q][lane];
      z_sh += part_sum[w][EPL][lane];
    }
    token_keys_from<EPL>(zv, lane, bias, sv, key);
  }
  bool valid[EPL];
#pragma unroll
  for (int q = 0; q < EPL; ++q) valid[q] = true;
  int i_sel[K];     // candidate j is expert j here
  double s_pick[K], z_pick[K], k_sel[K + 1];
  rank_rounds<K, EPL>(lane, valid, key, sv, zv, i_sel, s_pick, z_pick, k_sel);
  double gap = INFINITY;
#pragma unroll
  for (int r = 0; r < K; ++r) gap = fmin(gap, k_sel[r] - k_sel[r + 1]);
  const bool listed = gap < kRefineGap;  // the same on every lane
  // the candidates of a listed token: every routed expert whose key lies
  // within kRefineGap of the (K + 1)-th best (lane masks per q)
  unsigned long long m[EPL];
  int nc = 0;
#pragma unroll
  for (int q = 0; q < EPL; ++q) {
    m[q] = __ballot(listed && key[q] >= k_sel[K] - kRefineGap);
    nc += __popcll(m[q]);
  }
  write_token<K, S>(t, lane, i_sel, s_pick, z_pick, sigmoid64(z_sh), z_sh, k_sel, topk, gates,
                    margin, logsumexp_norm, gate_scale);
  if (listed) {
    int slot = 0;
    if (lane == 0) slot = atomicAdd(refine, 1);
    slot = __builtin_amdgcn_readfirstlane(slot);
    int32_t* rec = refine + 1 + static_cast<size_t>(slot) * kRefineRec;
    if (lane == 0) {
      rec[0] = t;
      rec[1] = nc <= kRefineCand ? nc : -1;
    }
    if (nc <= kRefineCand) {
      // in ascending id: q outer, lane inner
      int pos = 0;
#pragma unroll
      for (int q = 0; q < EPL; ++q) {
        if ((m[q] >> lane) & 1ull)
          rec[2 + pos + __popcll(m[q] & ((1ull << lane) - 1ull))] = lane + 64 * q;
        pos += __popcll(m[q]);
      }
    }
  }
}

// Exact logits of the tokens router_select listed, for the experts that can
// rank among their K + 1 best: every routed expert whose matrix-core key is
// within kRefineGap of the (K + 1)-th best (a key's error is far below
// kRefineGap / 2, so no other expert can rank there), and the shared
// experts for the gates.  z = sum_c x[t,c] * w[e,c] in fp64: the products of
// bf16 (or fp32) x and fp32 w are exact in fp64, so z is the dot product to
// fp64 rounding and the picks are those of exact arithmetic unless two keys
// agree to ~1e-15.  One workgroup per listed token (a fixed grid walks the
// list): wave 0 lists the candidates; all 512 threads take 4 consecutive
// elements of K per 2048, and the lane, wave and span sums are added in a
// fixed order; wave 0 then ranks the candidates and writes the token's
// outputs.
template <int K, int S, int EPL>
__global__ __launch_bounds__(512) void router_refine(
    const double* __restrict__ partial, int nks, int T, int npad, int E, int d,
    const void* __restrict__ xv, bool x_bf16, const float* __restrict__ w,
    const int32_t* __restrict__ refine, const float* __restrict__ bias,
    int32_t* __restrict__ topk, float* __restrict__ gates, float* __restrict__ margin,
    bool logsumexp_norm, double gate_scale) {
  constexpr int NW = 8;                   // waves of the workgroup
  constexpr int NB = 9;                   // candidates per group of loads (7 + shared, usually)
  constexpr int CH = 2;                   // 2048-element chunks of K per span
  __shared__ int cand[64 * EPL + S];      // routed candidates, then the shared experts
  __shared__ double zc[64 * EPL + S];     // their exact logits
  __shared__ double wsum[NW][NB];
  __shared__ int s_nc;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int n = refine[0];
  for (int i = blockIdx.x; i < n; i += gridDim.x) {
    const int32_t* rec = refine + 1 + static_cast<size_t>(i) * kRefineRec;
    const int t = rec[0];
    const int nrec = rec[1];
    if (nrec >= 0) {
      // the selection listed the candidates
      if (tid < nrec) cand[tid] = rec[2 + tid];
      if (tid < S) cand[nrec + tid] = E + tid;
      if (tid == 0) s_nc = nrec;
    } else if (wave == 0) {
      // more than kRefineCand candidates: list them again from the keys
      double zv[EPL], sv[EPL], key[EPL], z_unused;
      token_keys<EPL, S>(partial, nks, T, npad, E, t, lane, bias, zv, sv, key, z_unused);
      bool valid[EPL];
#pragma unroll
      for (int q = 0; q < EPL; ++q) valid[q] = true;
      int i_sel[K];
      double s_pick[K], z_pick[K], k_sel[K + 1];
      rank_rounds<K, EPL>(lane, valid, key, sv, zv, i_sel, s_pick, z_pick, k_sel);
      const double thresh = k_sel[K] - kRefineGap;
      // candidates listed in ascending expert id (q outer, lane inner)
      int base = 0;
#pragma unroll
      for (int q = 0; q < EPL; ++q) {
        const bool c = key[q] >= thresh;
        const unsigned long long m = __ballot(c);
        if (c) cand[base + __popcll(m & ((1ull << lane) - 1ull))] = lane + 64 * q;
        base += __popcll(m);
      }
      if (lane < S) cand[base + lane] = E + lane;
      if (lane == 0) s_nc = base;
    }
    __syncthreads();
    const int nc = s_nc;
    const int ntot = nc + S;
    // the candidates' biases, loaded while the exact logits are summed
    const double bias_c =
        wave == 0 && lane < nc && lane < 64 ? static_cast<double>(bias[cand[lane]]) : 0.0;
    // K in spans of 512 threads x 4 elements x CH chunks; each group of NB
    // candidates issues all of its loads for the span before any addition,
    // so a token costs about one round trip per span and group
    for (int span = 0; span < d; span += 2048 * CH) {
      double xs[CH][4];
#pragma unroll
      for (int h = 0; h < CH; ++h) {
        const int c = span + h * 2048 + tid * 4;
#pragma unroll
        for (int e = 0; e < 4; ++e) xs[h][e] = 0.0;
        if (c < d) {
          if (x_bf16) {
            const uint2 v = *reinterpret_cast<const uint2*>(static_cast<const bf16_t*>(xv) +
                                                            static_cast<size_t>(t) * d + c);
            xs[h][0] = bf16_to_f32(static_cast<bf16_t>(v.x & 0xffff));
            xs[h][1] = bf16_to_f32(static_cast<bf16_t>(v.x >> 16));
            xs[h][2] = bf16_to_f32(static_cast<bf16_t>(v.y & 0xffff));
            xs[h][3] = bf16_to_f32(static_cast<bf16_t>(v.y >> 16));
          } else {
            const float4 v = *reinterpret_cast<const float4*>(
                static_cast<const float*>(xv) + static_cast<size_t>(t) * d + c);
            xs[h][0] = v.x;
            xs[h][1] = v.y;
            xs[h][2] = v.z;
            xs[h][3] = v.w;
          }
        }
      }
      for (int b0 = 0; b0 < ntot; b0 += NB) {
        float4 wv[NB][CH];
#pragma unroll
        for (int j = 0; j < NB; ++j)
#pragma unroll
          for (int h = 0; h < CH; ++h) {
            const int c = span + h * 2048 + tid * 4;
            wv[j][h] = (b0 + j < ntot && c < d)
                           ? *reinterpret_cast<const float4*>(
                                 w + static_cast<size_t>(cand[b0 + j]) * d + c)
                           : make_float4(0.f, 0.f, 0.f, 0.f);
          }
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          double acc = 0.0;
#pragma unroll
          for (int h = 0; h < CH; ++h) {
            acc = fma(xs[h][0], static_cast<double>(wv[j][h].x), acc);
            acc = fma(xs[h][1], static_cast<double>(wv[j][h].y), acc);
            acc = fma(xs[h][2], static_cast<double>(wv[j][h].z), acc);
            acc = fma(xs[h][3], static_cast<double>(wv[j][h].w), acc);
          }
          acc = wave_sum(acc, lane);
          if (lane == 0) wsum[wave][j] = acc;
        }
        __syncthreads();
        // the group's sums in a fixed order: waves 0..NW-1, then onto the
        // running logit (spans in order)
        if (tid < NB && b0 + tid < ntot) {
          double v = wsum[0][tid];
#pragma unroll
          for (int q = 1; q < NW; ++q) v += wsum[q][tid];
          zc[b0 + tid] = span == 0 ? v : zc[b0 + tid] + v;
        }
        __syncthreads();
      }
    }
    if (wave == 0) {
      // candidate j = lane + 64q is cand[j] (routed ones only, ascending
      // id); up to 64 of them (always, from a record) sit one per lane
      const double z_sh = lane < S ? zc[nc + lane] : 0.0;
      int j_sel[K], i_sel[K];
      double s_pick[K], z_pick[K], k_sel[K + 1];
      if (nc <= 64) {
        const bool valid[1] = {lane < nc};
        const double zv[1] = {valid[0] ? zc[lane] : 0.0};
        const double sv[1] = {sigmoid64(zv[0])};
        const double key[1] = {valid[0] ? sv[0] + bias_c : -INFINITY};
        rank_rounds<K, 1>(lane, valid, key, sv, zv, j_sel, s_pick, z_pick, k_sel);
      } else {
        bool valid[EPL];
        double zv[EPL], sv[EPL], key[EPL];
#pragma unroll
        for (int q = 0; q < EPL; ++q) {
          const int j = lane + 64 * q;
          valid[q] = j < nc;
          zv[q] = valid[q] ? zc[j] : 0.0;
          sv[q] = sigmoid64(zv[q]);
          key[q] = valid[q] ? sv[q] + static_cast<double>(bias[cand[j]]) : -INFINITY;
        }
        rank_rounds<K, EPL>(lane, valid, key, sv, zv, j_sel, s_pick, z_pick, k_sel);
      }
#pragma unroll
      for (int r = 0; r < K; ++r) i_sel[r] = cand[j_sel[r]];
      write_token<K, S>(t, lane, i_sel, s_pick, z_pick, sigmoid64(z_sh), z_sh, k_sel, topk,
                        gates, margin, logsumexp_norm, gate_scale);
    }
    __syncthreads();
  }
}

// ------------------------------------------------------------------ host

int router_chunk(const Shape& s) { return s.d % kRouterChunk == 0 ? kRouterChunk : 32; }

size_t router_refine_ints(const Shape& s) {
  return 1 + static_cast<size_t>(s.T) * kRefineRec;
}

int router_ksplits(const Shape& s) {
  const int tiles = ((s.T + 127) / 128) * (router_cols_padded(s) / kRouterColTile);
  const int nch = s.d / router_chunk(s);
  int want = (1280 + tiles - 1) / (tiles > 0 ? tiles : 1);  // ~2.5 waves of 2 workgroups per CU
  if (want < 1) want = 1;
  return want < nch ? want : nch;
}

struct SelectArgs {
  const void* x;
  const float* w_router;
  const double* partial;
  int nks, npad;
  const float* bias;
  int32_t* topk_idx;
  float* gates;
  float* margin;
  int32_t* refine;
};

// Workgroups of router_refine: the listed tokens are few (an adjacent pair
// of their best keys lies within kRefineGap), so a fixed grid walks the list.
constexpr int kRefineGrid = 256;

template <int S, int EPL>
static void launch_select(const Shape& s, const SelectArgs& a, hipStream_t st) {
  if (a.nks > 8)  // many splits (small batches): one round of loads per wave
    router_select<6, S, EPL, 4><<<s.T, 256, 0, st>>>(
        a.partial, a.nks, s.T, a.npad, s.E, a.bias, a.topk_idx, a.gates, a.margin,
        s.gate_logsumexp, s.gate_scale, a.refine);
  else
    router_select<6, S, EPL, 1><<<(s.T + 3) / 4, 256, 0, st>>>(
        a.partial, a.nks, s.T, a.npad, s.E, a.bias, a.topk_idx, a.gates, a.margin,
        s.gate_logsumexp, s.gate_scale, a.refine);
  router_refine<6, S, EPL><<<s.T < kRefineGrid ? s.T : kRefineGrid, 512, 0, st>>>(
      a.partial, a.nks, s.T, a.npad, s.E, s.d, a.x, s.bf16, a.w_router, a.refine, a.bias,
      a.topk_idx, a.gates, a.margin, s.gate_logsumexp, s.gate_scale);
}

template <int S>
static void launch_select_e(const Shape& s, const SelectArgs& a, hipStream_t st) {
  if (s.E == 64) launch_select<S, 1>(s, a, st);
  else if (s.E == 128) launch_select<S, 2>(s, a, st);
  else launch_select<S, 4>(s, a, st);
}

hipError_t launch_router_planes(const Shape& s, const float* w_router, bf16_t* planes,
                                hipStream_t st) {
  const int npad = router_cols_padded(s);
  const size_t n = static_cast<size_t>(npad) * s.d;
  int blocks = static_cast<int>((n + 255) / 256);
  if (blocks > 4096) blocks = 4096;
  router_split_planes<<<blocks, 256, 0, st>>>(w_router, s.E + s.S, s.d, npad, planes);
  return hipGetLastError();
}

hipError_t launch_router(const Shape& s, const void* x, const float* w_router,
                         const bf16_t* prepared, const float* bias, int32_t* topk_idx,
                         float* gates, float* margin, bf16_t* wplanes, double* partial,
                         int32_t* refine, hipStream_t st) {
  if (s.T == 0) return hipSuccess;
  const int npad = router_cols_padded(s);
  if (prepared) {
    wplanes = const_cast<bf16_t*>(prepared);  // only read from here on
  } else {
    const hipError_t e = launch_router_planes(s, w_router, wplanes, st);
    if (e != hipSuccess) return e;
  }
  const int nks = router_ksplits(s);
  const int chunk = router_chunk(s);
  dim3 grid((s.T + 127) / 128, npad / kRouterColTile, nks);
  if (s.bf16)
    router_logits_bf16<<<grid, 256, 0, st>>>(static_cast<const bf16_t*>(x), wplanes, s.T, s.d,
                                              npad, nks, chunk, partial, refine);
  else
    router_logits<3><<<grid, 256, 0, st>>>(x, wplanes, s.T, s.d, npad, nks, chunk, partial,
                                           refine);
  const SelectArgs a{x, w_router, partial, nks, npad, bias, topk_idx, gates, margin, refine};
  if (s.S == 0) launch_select_e<0>(s, a, st);
  else if (s.S == 1) launch_select_e<1>(s, a, st);
  else launch_select_e<2>(s, a, st);
  return hipGetLastError();
}

}  // namespace moe
