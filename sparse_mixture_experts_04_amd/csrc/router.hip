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
    int nks, int chunk, double* __restrict__ partial) {
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
    int nks, int chunk, double* __restrict__ partial) {
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

// z = sum of the K-split partial logits in split order.  The loads of a
// group of 8 splits are issued together (small batches split K up to 28
// ways); the additions stay in split order.
__device__ __forceinline__ double sum_partials(const double* __restrict__ partial, size_t kstride,
                                               int nks, size_t off) {
  double z = 0.0;
  int ks = 0;
  for (; ks + 8 <= nks; ks += 8) {
    double v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = partial[(ks + j) * kstride + off];
#pragma unroll
    for (int j = 0; j < 8; ++j) z += v[j];
  }
  for (; ks < nks; ++ks) z += partial[ks * kstride + off];
  return z;
}

__device__ __forceinline__ bool better(double ka, int ia, double kb, int ib) {
  return ka > kb || (ka == kb && ia < ib);
}

// One wave per token.  E = 64 * EPL: lane l owns routed experts l, l+64,
// ...; lanes 0..S-1 also own the shared experts E+lane.  K routed picks in
// rank order (descending key, exact ties to the lower id), then one more
// round for the first expert left out (the margin).
template <int K, int S, int EPL>
__global__ __launch_bounds__(256) void router_select(
    const double* __restrict__ partial, int nks, int T, int npad, int E,
    const float* __restrict__ bias, int32_t* __restrict__ topk, float* __restrict__ gates,
    float* __restrict__ margin, bool logsumexp_norm, double gate_scale) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;  // whole wave leaves together; no block barrier below

  double sv[EPL], zv[EPL], key[EPL];
  bool taken[EPL];
  const size_t kstride = static_cast<size_t>(T) * npad;
#pragma unroll
  for (int q = 0; q < EPL; ++q) {
    const int c = lane + 64 * q;
    zv[q] = sum_partials(partial, kstride, nks, static_cast<size_t>(t) * npad + c);
    const double s = 1.0 / (1.0 + exp(-zv[q]));
    sv[q] = s;
    key[q] = s + static_cast<double>(bias[c]);
    taken[q] = false;
  }
  double s_shared = 0.0, z_shared = 0.0;
  if (lane < S) {
    const double z = sum_partials(partial, kstride, nks, static_cast<size_t>(t) * npad + E + lane);
    s_shared = 1.0 / (1.0 + exp(-z));
    z_shared = z;
  }

  double s_sel[K + S], z_sel[K + S];
  int i_sel[K];
  double k_last = 0.0, k_next = 0.0;
#pragma unroll
  for (int r = 0; r <= K; ++r) {
    double bk = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int q = 0; q < EPL; ++q) {
      const int c = lane + 64 * q;
      if (!taken[q] && better(key[q], c, bk, bi)) {
        bk = key[q];
        bi = c;
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const double ok = __shfl_xor(bk, off);
      const int oi = __shfl_xor(bi, off);
      if (better(ok, oi, bk, bi)) {
        bk = ok;
        bi = oi;
      }
    }
    if (r == K) {
      k_next = bk;
    } else {
      const int q = bi >> 6;
      const int owner = bi & 63;
      double my = sv[0], mz = zv[0];
#pragma unroll
      for (int qq = 1; qq < EPL; ++qq) {
        my = q == qq ? sv[qq] : my;
        mz = q == qq ? zv[qq] : mz;
      }
      s_sel[r] = __shfl(my, owner);
      z_sel[r] = __shfl(mz, owner);
      if (lane == owner) {
#pragma unroll
        for (int qq = 0; qq < EPL; ++qq) taken[qq] = taken[qq] || q == qq;
      }
      i_sel[r] = bi;
      k_last = bk;
    }
  }
#pragma unroll
  for (int j = 0; j < S; ++j) {
    s_sel[K + j] = __shfl(s_shared, j);
    z_sel[K + j] = __shfl(z_shared, j);
  }

  // gates: s_j / sum s, or exp(logsigmoid(z_j) - logsumexp logsigmoid(z)),
  // both over the k kept and S shared contributors in slot order, then
  // times gate_scale.  Written as g_j = num_j / denom.
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
  if (margin && lane == 0) margin[t] = static_cast<float>(k_last - k_next);
}

// ------------------------------------------------------------------ host

int router_chunk(const Shape& s) { return s.d % kRouterChunk == 0 ? kRouterChunk : 32; }

int router_ksplits(const Shape& s) {
  const int tiles = ((s.T + 127) / 128) * (router_cols_padded(s) / kRouterColTile);
  const int nch = s.d / router_chunk(s);
  int want = (1280 + tiles - 1) / (tiles > 0 ? tiles : 1);  // ~2.5 waves of 2 workgroups per CU
  if (want < 1) want = 1;
  return want < nch ? want : nch;
}

template <int S, int EPL>
static void launch_select(const Shape& s, const double* partial, int nks, int npad,
                          const float* bias, int32_t* topk_idx, float* gates, float* margin,
                          hipStream_t st) {
  router_select<6, S, EPL><<<(s.T + 3) / 4, 256, 0, st>>>(partial, nks, s.T, npad, s.E, bias,
                                                          topk_idx, gates, margin,
                                                          s.gate_logsumexp, s.gate_scale);
}

template <int S>
static void launch_select_e(const Shape& s, const double* partial, int nks, int npad,
                            const float* bias, int32_t* topk_idx, float* gates, float* margin,
                            hipStream_t st) {
  if (s.E == 64) launch_select<S, 1>(s, partial, nks, npad, bias, topk_idx, gates, margin, st);
  else if (s.E == 128) launch_select<S, 2>(s, partial, nks, npad, bias, topk_idx, gates, margin, st);
  else launch_select<S, 4>(s, partial, nks, npad, bias, topk_idx, gates, margin, st);
}

hipError_t launch_router(const Shape& s, const void* x, const float* w_router,
                         const float* bias, int32_t* topk_idx, float* gates, float* margin,
                         bf16_t* wplanes, double* partial, hipStream_t st) {
  if (s.T == 0) return hipSuccess;
  const int npad = router_cols_padded(s);
  const size_t n = static_cast<size_t>(npad) * s.d;
  int blocks = static_cast<int>((n + 255) / 256);
  if (blocks > 4096) blocks = 4096;
  router_split_planes<<<blocks, 256, 0, st>>>(w_router, s.E + s.S, s.d, npad, wplanes);
  const int nks = router_ksplits(s);
  const int chunk = router_chunk(s);
  dim3 grid((s.T + 127) / 128, npad / kRouterColTile, nks);
  if (s.bf16)
    router_logits_bf16<<<grid, 256, 0, st>>>(static_cast<const bf16_t*>(x), wplanes, s.T, s.d,
                                              npad, nks, chunk, partial);
  else
    router_logits<3><<<grid, 256, 0, st>>>(x, wplanes, s.T, s.d, npad, nks, chunk, partial);
  if (s.S == 0) launch_select_e<0>(s, partial, nks, npad, bias, topk_idx, gates, margin, st);
  else if (s.S == 1) launch_select_e<1>(s, partial, nks, npad, bias, topk_idx, gates, margin, st);
  else launch_select_e<2>(s, partial, nks, npad, bias, topk_idx, gates, margin, st);
  return hipGetLastError();
}

}  // namespace moe
