// FP4 routed-expert weights: quantization and the decode-batch expert GEMMs.
//
// "Under The Hood: Inkling", "Quantization: BF16 vs NVFP4": the routed
// experts' weights are stored in FP4 with small-block scales (the gates,
// the shared experts and the router stay high precision).  The MI355X
// format is OCP MXFP4: E2M1 codes, one power-of-two (E8M0) scale per 32
// consecutive values along K, converted to bf16 in hardware
// (v_cvt_scalef32_pk_bf16_fp4).  Activations stay bf16 (weight-only FP4):
// decode batches are bound by streaming the weights, so the GEMM keeps the
// bf16 matrix cores and the weight bytes drop to 17/32 of a byte per value.
//
// Layouts (one expert stack [E, N, K], K % 128 == 0):
//   codes  [E, K/128, N, 64] bytes: for each 128-value K tile, the 64 code
//                        bytes of every weight row, rows consecutive (value
//                        2i of the tile in the low nibble of byte i), so the
//                        GEMM's K step over 256 weight rows is one
//                        contiguous 16 KiB block (about 9% faster to stream
//                        from HBM than 256 separate 64-byte row pieces)
//   scales [E, K/128, N, 4] bytes X + 127: for each 128-value K tile, the
//                        scales of its 4 K blocks for every row n, rows
//                        consecutive (a K step's 256 rows read 1 KiB in
//                        pieces of 128 bytes or more)
#include "ffn_common.h"

namespace moe {

// ------------------------------------------------------------ quantize

// One thread per 32-value block.  X = floor(log2 amax) - 2 from amax's
// exponent field (a zero or subnormal amax gives X = -127 after the clamp);
// |v| * 2^-X is exact, then rounded to the E2M1 grid
// {0, 0.5, 1, 1.5, 2, 3, 4, 6} with ties to the even code.
__global__ __launch_bounds__(256) void mxfp4_quantize_kernel(const bf16_t* __restrict__ w,
                                                             long long rows, int K, int N,
                                                             uint8_t* __restrict__ codes,
                                                             uint8_t* __restrict__ scales) {
  const int kb_per_row = K / 32;
  const long long nb = rows * kb_per_row;
  const long long stride = static_cast<long long>(gridDim.x) * blockDim.x;
  for (long long i = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x; i < nb;
       i += stride) {
    const long long r = i / kb_per_row;
    const int kb = static_cast<int>(i - r * kb_per_row);
    const uint4* src = reinterpret_cast<const uint4*>(w + r * K + kb * 32);
    uint32_t u[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint4 v = src[q];
      u[4 * q] = v.x; u[4 * q + 1] = v.y; u[4 * q + 2] = v.z; u[4 * q + 3] = v.w;
    }
    float v[32];
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      v[2 * j] = __uint_as_float(u[j] << 16);
      v[2 * j + 1] = __uint_as_float(u[j] & 0xffff0000u);
      amax = fmaxf(amax, fmaxf(fabsf(v[2 * j]), fabsf(v[2 * j + 1])));
    }
    const int ex = static_cast<int>((__float_as_uint(amax) >> 23) & 0xff);
    int X = ex == 0 ? -127 : ex - 127 - 2;
    X = X < -127 ? -127 : (X > 127 ? 127 : X);
    const float inv = __uint_as_float(static_cast<uint32_t>(127 - X) << 23);  // 2^-X
    uint32_t packed[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      const float m = fabsf(v[j]) * inv;
      uint32_t c = m <= 0.25f ? 0u : m < 0.75f ? 1u : m <= 1.25f ? 2u : m < 1.75f ? 3u
                 : m <= 2.5f ? 4u : m < 3.5f ? 5u : m <= 5.0f ? 6u : 7u;
      c |= (__float_as_uint(v[j]) >> 31) << 3;
      packed[j >> 3] |= c << (4 * (j & 7));
    }
    const long long e = r / N;
    const long long n = r - e * N;
    const long long tile = e * (K / 128) + kb / 4;   // 128-value K tile of expert e
    *reinterpret_cast<uint4*>(codes + (tile * N + n) * 64 + (kb & 3) * 16) =
        make_uint4(packed[0], packed[1], packed[2], packed[3]);
    scales[(tile * N + n) * 4 + (kb & 3)] = static_cast<uint8_t>(X + 127);
  }
}

hipError_t launch_quantize_mxfp4(long long E, int N, int K, const void* w, uint8_t* codes,
                                 uint8_t* scales, hipStream_t st) {
  const long long nb = E * N * (K / 32);
  if (nb == 0) return hipSuccess;
  long long blocks = (nb + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  mxfp4_quantize_kernel<<<static_cast<unsigned>(blocks), 256, 0, st>>>(
      static_cast<const bf16_t*>(w), E * N, K, N, codes, scales);
  return hipGetLastError();
}

// ------------------------------------------------- decode-batch GEMMs

// Tile: 32 rows x 256 weight rows, K step 128, 256 threads (4 waves, wave
// wn owns weight rows 64wn..64wn+63 = two 32-wide MFMA column blocks).
// GATED: weight rows 64c..64c+31 are W_gate columns 32c.. of the 128-column
// output tile and rows 64c+32.. the same W_up columns.
// Per stage, LDS holds
//   A      32 rows x 256 B (bf16), 16-byte chunk c of row r in slot c ^ (r & 15);
//   codes  256 rows x 64 B, chunk c of row r in slot c ^ ((r >> 2) & 3);
//   scales 256 rows x 4 K blocks (bytes);
// all filled with direct global -> LDS loads: per wave up to 2 A loads and
// 4 code loads of 1 KiB and one 256-byte scale load (the 4 scales of each
// of rows 64 wave .. 64 wave + 63).  An A load covers 4 rows and is skipped
// when none of them holds a row of the tile (decode tiles hold a row or
// two): the LDS rows it would fill only feed accumulator rows that are
// never stored, and the wave's wait counts follow its number of loads.  A
// B fragment is 4 code bytes per lane and its block's scale byte (a lane
// reads its row's 4 scales as one dword), converted to bf16 in registers.
struct Fp4Cfg {
  static constexpr int MT = 32;
  static constexpr int NB = 256;
  static constexpr int BK = 128;
  static constexpr int NS = 3;                        // ring stages (two workgroups per CU)
  static constexpr int A_BYTES = MT * BK * 2;        // 8 KiB
  static constexpr int C_BYTES = NB * BK / 2;        // 16 KiB
  static constexpr int S_BYTES = NB * BK / 32;       // 1 KiB
  static constexpr int STAGE = A_BYTES + C_BYTES + S_BYTES;
  static constexpr int A_LOADS = A_BYTES / 1024 / 4;
  static constexpr int C_LOADS = C_BYTES / 1024 / 4;
  static constexpr int LPW = A_LOADS + C_LOADS + 1;
  static_assert((NS - 2) * LPW < 64, "vmcnt range");
  static_assert(BK == 128, "the codes layout tiles K by 128 values (64 bytes per row)");
};

__device__ __forceinline__ void dma4(const void* src, uint32_t lds_addr) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_addr);
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off"
               :
               : "v"(src), "s"(m0)
               : "m0");
}

__device__ __forceinline__ void dma16_lds(const void* src, uint32_t lds_addr) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_addr);
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(src), "s"(m0)
               : "m0");
}

struct Fp4Ctx {
  using C = Fp4Cfg;
  const bf16_t* a_src[C::A_LOADS];   // per lane, chunk applied, K offset 0
  const uint8_t* c_src[C::C_LOADS];  // per lane, chunk applied, K offset 0
  const uint8_t* s_src;              // per lane: 4 scale bytes of K block `wave`
  int na;                            // A loads this wave issues per stage (wave-uniform)

  // loads of stage kt into the ring slot at LDS byte address `slot`
  __device__ __forceinline__ void issue(int kt, uint32_t slot, int wave, int sstride) const {
#pragma unroll
    for (int q = 0; q < C::A_LOADS; ++q)
      if (q < na) dma16_lds(a_src[q] + kt * C::BK, slot + (wave * C::A_LOADS + q) * 1024);
#pragma unroll
    for (int q = 0; q < C::C_LOADS; ++q)
      dma16_lds(c_src[q] + static_cast<size_t>(kt) * sstride * (C::BK / 2),
                slot + C::A_BYTES + (wave * C::C_LOADS + q) * 1024);
    dma4(s_src + static_cast<size_t>(kt) * 4 * sstride,
         slot + C::A_BYTES + C::C_BYTES + wave * 256);
  }
};

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// B fragment from 4 code bytes (8 values) and their block's scale byte:
// converted to bf16 with the scale applied (2^(sb-127); sb = 0 is 2^-127,
// a subnormal float).
__device__ __forceinline__ bf16x8_t fp4_frag(uint32_t word, uint32_t sb) {
  const float scale = __uint_as_float(sb == 0 ? 0x00400000u : sb << 23);
  const bf16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, scale, 0);
  const bf16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, scale, 1);
  const bf16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, scale, 2);
  const bf16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, scale, 3);
  bf16x8_t r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

// One K step of a wave: every LDS read of the stage is issued first (8 A
// fragments, and for each of the wave's two column blocks 8 code words and
// 4 scale bytes), so their latencies overlap; then the conversions and
// MFMAs.  B fragment of substep kk for column block j of wave wn: lane l
// holds the 8 values k = 16kk + 8(l/32) .. of weight row 64wn + 32j + l%32.
__device__ __forceinline__ void fp4_stage(const uint8_t* st, int wn, int lane,
                                          f32x16_t (&acc)[2]) {
  using C = Fp4Cfg;
  constexpr int KK = C::BK / 16;
  const int r32 = lane & 31;
  const int half = lane >> 5;
  const bf16_t* sa = reinterpret_cast<const bf16_t*>(st);
  bf16x8_t a[KK];
  uint32_t word[2][KK];
  uint32_t sb[2][KK / 2];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) {
    const int c = 2 * kk + half;  // 16-byte chunk of the A row
    a[kk] = *reinterpret_cast<const bf16x8_t*>(sa + r32 * 128 + ((c ^ (r32 & 15)) << 3));
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int row = wn * 64 + j * 32 + r32;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const int chunk = (kk >> 1) ^ ((row >> 2) & 3);   // 16-byte chunk holding bytes 8kk..
      word[j][kk] = *reinterpret_cast<const uint32_t*>(
          st + C::A_BYTES + row * 64 + chunk * 16 + (kk & 1) * 8 + half * 4);
    }
    {
      const uint32_t s4 =
          *reinterpret_cast<const uint32_t*>(st + C::A_BYTES + C::C_BYTES + row * 4);
#pragma unroll
      for (int m = 0; m < KK / 2; ++m) sb[j][m] = (s4 >> (8 * m)) & 0xffu;
    }
  }
  __builtin_amdgcn_sched_barrier(0);  // keep every read ahead of the first conversion
#pragma unroll
  for (int kk = 0; kk < KK; ++kk)
#pragma unroll
    for (int j = 0; j < 2; ++j)
      acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[kk], fp4_frag(word[j][kk], sb[j][kk >> 1]),
                                                       acc[j], 0, 0, 0);
}

// ------------------------------------------- shared experts in the launch

// The shared experts' weights stay bf16 ("Under The Hood: Inkling",
// "Quantization: BF16 vs NVFP4"); their tiles run in the same persistent
// launch as the FP4 routed tiles, after each XCD's routed items, so they
// fill the last round of the static item order instead of running alone
// afterwards.  A shared tile: 64 token rows x 256 weight rows (the same
// weight-row layout as the FP4 tiles: for GATED, wave w's rows
// 64w..64w+31 are W_gate columns 32w.. of the 128-column output tile and
// rows 64w+32.. the same W_up columns), one of kFp4SharedSlices K slices,
// K step 32 through the FP4 ring's memory (LDS rows of 64 bytes, chunk c
// of row r in slot c ^ ((r >> 2) & 3)): per stage 64 activation rows (4
// KiB) then 256 weight rows (16 KiB), one activation and four weight loads
// of 1 KiB per wave.  A slice writes its fp32 accumulators to
// part[slice][s*T + row][n*256 + weight row]; shared_reduce_kernel sums the
// slices after the launch.  kFp4SharedSlices slices make a shared item
// stream about as many bytes as an FP4 item (bf16 is 32/17 times the FP4
// bytes per weight).
constexpr int kFp4SharedRows = 64;
constexpr int kFp4MaxGroups = 256 + 2;  // E + S (the descriptor allows E <= 256, S <= 2)
constexpr int kFp4SharedBK = 32;
constexpr int kFp4SharedA = kFp4SharedRows * kFp4SharedBK * 2;   // 4 KiB
constexpr int kFp4SharedB = Fp4Cfg::NB * kFp4SharedBK * 2;      // 16 KiB
static_assert(kFp4SharedA + kFp4SharedB <= Fp4Cfg::STAGE, "a shared stage fits an FP4 stage");

template <bool GATED>
__device__ __forceinline__ void fp4_shared_item(const FfnArgs& p, long long si,
                                                const uint8_t* ring, uint32_t ring_base,
                                                int wave, int lane) {
  using C = Fp4Cfg;
  // si -> (shared expert, column tile, row tile, slice), slice innermost
  const int srt = (p.T + kFp4SharedRows - 1) / kFp4SharedRows;
  const int ks = static_cast<int>(si % p.ksplit);
  long long rest = si / p.ksplit;
  const int mt = static_cast<int>(rest % srt);
  rest /= srt;
  const int n = static_cast<int>(rest % p.n_tiles);
  const int se = static_cast<int>(rest / p.n_tiles);
  const int m0 = mt * kFp4SharedRows;
  const int rows = p.T - m0 < kFp4SharedRows ? p.T - m0 : kFp4SharedRows;
  const int nk_all = p.K / kFp4SharedBK;
  const int kb = ks * nk_all / p.ksplit;
  const int nk = (ks + 1) * nk_all / p.ksplit - kb;

  // load sources (16 LDS rows of 64 bytes per load; lane l lands in row
  // 16j + l/4, slot l%4, and fetches chunk (l%4) ^ ((l >> 4) & 3))
  const int lr = lane >> 2;
  const int sch = ((lane & 3) ^ ((lane >> 4) & 3)) * 8;
  const bf16_t* a_src;
  {
    int r = 16 * wave + lr;
    r = r < rows ? r : rows - 1;
    const size_t row = GATED ? static_cast<size_t>(m0 + r)
                             : static_cast<size_t>(p.k) * p.T +
                                   static_cast<size_t>(se) * p.T + m0 + r;  // h's shared rows
    a_src = static_cast<const bf16_t*>(p.a) + row * p.K + sch;
  }
  const bf16_t* b_src[4];
  const size_t wstride = static_cast<size_t>(p.N) * p.K;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int R = 16 * (4 * wave + q) + lr;  // weight row of the tile
    const bf16_t* base;
    int col;
    if (GATED) {
      const int cg = R >> 6, rl = R & 63;
      base = static_cast<const bf16_t*>(rl >= 32 ? p.ws1 : p.ws0);
      col = n * (C::NB / 2) + cg * 32 + (rl & 31);
    } else {
      base = static_cast<const bf16_t*>(p.ws0);
      col = n * C::NB + R;
    }
    b_src[q] = base + se * wstride + static_cast<size_t>(col) * p.K + sch;
  }
  auto issue = [&](int kt, uint32_t slot) {
    const int k0 = (kb + kt) * kFp4SharedBK;
    dma16_lds(a_src + k0, slot + wave * 1024);
#pragma unroll
    for (int q = 0; q < 4; ++q)
      dma16_lds(b_src[q] + k0, slot + kFp4SharedA + (4 * wave + q) * 1024);
  };

  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
  const int nblk = rows > 32 ? 2 : 1;  // 32-row blocks holding rows

  // fragment offset of substep kk: row r32 = l % 32 of a 32-row block,
  // chunk 2kk + l/32
  const int r32 = lane & 31;
  int off[2];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) off[kk] = r32 * 32 + (((2 * kk + (lane >> 5)) ^ ((r32 >> 2) & 3)) << 3);

  // every wave is done with the previous item's LDS before refilling it
  wait_vm<0>();
  lds_barrier();
#pragma unroll
  for (int s_ = 0; s_ < C::NS - 1; ++s_) issue(s_ < nk ? s_ : nk - 1, ring_base + s_ * C::STAGE);
  for (int kt = 0; kt < nk; ++kt) {
    wait_vm<(C::NS - 2) * 5>();  // stage kt landed (5 loads per wave per stage)
    lds_barrier();
    const int kn = kt + C::NS - 1 < nk ? kt + C::NS - 1 : nk - 1;
    issue(kn, ring_base + ((kt + C::NS - 1) % C::NS) * C::STAGE);
    const bf16_t* sA = reinterpret_cast<const bf16_t*>(ring + (kt % C::NS) * C::STAGE);
    const bf16_t* sB = sA + kFp4SharedA / 2;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      bf16x8_t b[2];
#pragma unroll
      for (int j = 0; j < 2; ++j)
        b[j] = *reinterpret_cast<const bf16x8_t*>(sB + (64 * wave + 32 * j) * 32 + off[kk]);
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        if (i >= nblk) continue;
        const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(sA + i * 32 * 32 + off[kk]);
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b[j], acc[i][j], 0, 0, 0);
      }
    }
  }

  // fp32 partials: lane l holds weight row 32j + l%32 of the wave's 64 and
  // token rows 8(r/4) + 4(l/32) + r%4 of block i
  const size_t ldp = static_cast<size_t>(p.n_tiles) * C::NB;
  float* prow0 = p.part + (static_cast<size_t>(ks) * p.S * p.T +
                           static_cast<size_t>(se) * p.T + m0) * ldp +
                 static_cast<size_t>(n) * C::NB + 64 * wave + (lane & 31);
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
      if (row >= rows) continue;
#pragma unroll
      for (int j = 0; j < 2; ++j) prow0[row * ldp + 32 * j] = acc[i][j][r];
    }
}

// ------------------------------------------------------- routed items

// What the issuing side needs of a routed item: the item, its group's first
// row in the expert-sorted order, and the source row of each of the lane's A
// loads (the token for gate/up, the row of h for down).  The tile plan and
// the group offsets are in LDS and the gate/up token rows are read with
// sload, so building it does not wait for the direct loads in flight.
struct Fp4Meta {
  Item item;
  int row_base;
  int src_row[Fp4Cfg::A_LOADS];
};

template <bool GATED>
__device__ __forceinline__ Fp4Meta fp4_meta(const FfnArgs& p, const int* ts, const int* ofs,
                                            long long it, int wave, int lane) {
  using C = Fp4Cfg;
  Fp4Meta m;
  const Item d = decode_item(it, ts, p.E + p.S, p.n_tiles, C::MT, ofs, p.T, p.E);
  m.item.g = __builtin_amdgcn_readfirstlane(d.g);
  m.item.m0 = __builtin_amdgcn_readfirstlane(d.m0);
  m.item.rows = __builtin_amdgcn_readfirstlane(d.rows);
  m.item.n = __builtin_amdgcn_readfirstlane(d.n);
  m.item.grows = __builtin_amdgcn_readfirstlane(d.grows);
  m.row_base = __builtin_amdgcn_readfirstlane(ofs[m.item.g]);
  // A load j fills rows 4j..4j+3 (lane l: row 4j + l/16), clamped to the
  // tile's last row
  const int sel = lane >> 4;
#pragma unroll
  for (int q = 0; q < C::A_LOADS; ++q) {
    const int j = wave * C::A_LOADS + q;
    if (GATED) {
      int v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int r = 4 * j + u < m.item.rows ? 4 * j + u : m.item.rows - 1;
        v[u] = sload(p.sorted_pair, m.row_base + m.item.m0 + r) / p.k;
      }
      m.src_row[q] = sel == 0 ? v[0] : sel == 1 ? v[1] : sel == 2 ? v[2] : v[3];
    } else {
      const int r = 4 * j + sel < m.item.rows ? 4 * j + sel : m.item.rows - 1;
      m.src_row[q] = m.row_base + m.item.m0 + r;
    }
  }
  return m;
}

// Load sources of an item (see Fp4Ctx).
template <bool GATED>
__device__ __forceinline__ Fp4Ctx fp4_ctx(const FfnArgs& p, const Fp4Meta& m, int wave,
                                          int lane) {
  using C = Fp4Cfg;
  const Item& item = m.item;
  Fp4Ctx t;
  {
    const int left = item.rows - 4 * wave * C::A_LOADS;   // rows from this wave's first group
    const int groups = left <= 0 ? 0 : (left + 3) / 4;
    t.na = groups < C::A_LOADS ? groups : C::A_LOADS;
  }
  const bf16_t* A = static_cast<const bf16_t*>(p.a);
  const int arow = lane >> 4;
#pragma unroll
  for (int q = 0; q < C::A_LOADS; ++q) {
    const int rc = 4 * (wave * C::A_LOADS + q) + arow;
    t.a_src[q] = A + static_cast<size_t>(m.src_row[q]) * p.K + (((lane & 15) ^ (rc & 15)) << 3);
  }
  // code load j fills rows 16j..16j+15: lane l -> row 16j + l/4, slot l%4,
  // source chunk (l%4) ^ ((row >> 2) & 3)
  const int crow = lane >> 2;
  const int g = item.g;
  const size_t cstride = static_cast<size_t>(p.N) * (p.K / 2);   // bytes per expert
  const size_t sstride_e = static_cast<size_t>(p.K / 32) * p.N;
#pragma unroll
  for (int q = 0; q < C::C_LOADS; ++q) {
    const int j = wave * C::C_LOADS + q;
    const int R = 16 * j + crow;  // LDS B row
    int col;
    const uint8_t* base;
    if (GATED) {
      const int cg = R >> 6, rl = R & 63;
      base = static_cast<const uint8_t*>(rl >= 32 ? p.w1 : p.w0);
      col = item.n * (C::NB / 2) + cg * 32 + (rl & 31);
    } else {
      base = static_cast<const uint8_t*>(p.w0);
      col = item.n * C::NB + R;
    }
    t.c_src[q] = base + g * cstride + static_cast<size_t>(col) * (C::BK / 2) +
                 (((lane & 3) ^ ((R >> 2) & 3)) << 4);
  }
  {
    // scale load of rows 64 wave + l: LDS bytes 4R..4R+3 = row R's 4 K blocks
    const int R = 64 * wave + lane;
    int col;
    const uint8_t* sbase;
    if (GATED) {
      const int cg = R >> 6, rl = R & 63;
      sbase = rl >= 32 ? p.sc1 : p.sc0;
      col = item.n * (C::NB / 2) + cg * 32 + (rl & 31);
    } else {
      sbase = p.sc0;
      col = item.n * C::NB + R;
    }
    t.s_src = sbase + g * sstride_e + static_cast<size_t>(col) * 4;
  }
  return t;
}

// An item's outputs as bf16, packed two per register.  32x32 accumulator
// layout: lane l holds column l%32 and rows 8*(r/4) + 4*(l/32) + r%4.
// GATED: SwiGLU of the gate (acc[0]) and up (acc[1]) columns, 16 values;
// down: both column blocks, 32 values.
struct Fp4Out {
  uint32_t w[16];
};

template <bool GATED>
__device__ __forceinline__ void fp4_pack(const f32x16_t (&acc)[2], Fp4Out& o) {
  if (GATED) {
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      float v[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const float gt = acc[0][r + e];
        const float up = acc[1][r + e];
        v[e] = gt * __builtin_amdgcn_rcpf(1.0f + __expf(-gt)) * up;
      }
      o.w[r / 2] = static_cast<uint32_t>(f32_to_bf16(v[0])) |
                   (static_cast<uint32_t>(f32_to_bf16(v[1])) << 16);
    }
  } else {
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; r += 2)
        o.w[8 * j + r / 2] = static_cast<uint32_t>(f32_to_bf16(acc[j][r])) |
                             (static_cast<uint32_t>(f32_to_bf16(acc[j][r + 1])) << 16);
  }
}

template <bool GATED>
__device__ __forceinline__ void fp4_store(const FfnArgs& p, const Item& item, int row_base,
                                          int wave, int lane, const Fp4Out& o) {
  using C = Fp4Cfg;
  bf16_t* out = static_cast<bf16_t*>(p.out_routed);
  const size_t orow0 = static_cast<size_t>(row_base) + item.m0;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int row = 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
    if (row >= item.rows) continue;
    bf16_t* orow = out + (orow0 + row) * p.ldo;
    if (GATED) {
      const uint32_t w = o.w[r / 2];
      orow[item.n * (C::NB / 2) + wave * 32 + (lane & 31)] =
          static_cast<bf16_t>((r & 1) ? (w >> 16) : (w & 0xffffu));
    } else {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const uint32_t w = o.w[8 * j + r / 2];
        orow[item.n * C::NB + wave * 64 + j * 32 + (lane & 31)] =
            static_cast<bf16_t>((r & 1) ? (w >> 16) : (w & 0xffffu));
      }
    }
  }
}

// s_waitcnt vmcnt(n) for the n loads this wave issued after the stage waited
// for (one stage: the C + 1 code and scale loads and 0..A_LOADS A loads).
__device__ __forceinline__ void fp4_wait_stage(int n) {
  using C = Fp4Cfg;
  static_assert(C::A_LOADS == 2, "wait cases");
  if (n == C::LPW) wait_vm<C::LPW>();
  else if (n == C::LPW - 1) wait_vm<C::LPW - 1>();
  else wait_vm<C::LPW - 2>();
}

// The routed items first, first + stride, ... (< nr) of the list beg + i,
// with the ring run as one stream across items: the last two K steps of an
// item issue the first two stages of the next one, so a new item does not
// start by waiting a full HBM latency for its first stage.  An item's
// outputs are stored after the next item's first wait: a store counts in
// vmcnt like a load, and stores issued behind the next item's first stages
// would make that wait cover them too.  Needs nk >= 3 (the next item's
// metadata is read at the end of K step 0 and used at step nk - 2).
template <bool GATED>
__device__ __forceinline__ void fp4_routed_stream(const FfnArgs& p, const int* ts, const int* ofs,
                                                  long long beg, long long nr, long long first,
                                                  int stride, const uint8_t* ring,
                                                  uint32_t ring_base, int wave, int lane) {
  using C = Fp4Cfg;
  const int nk = p.K / C::BK;
  long long ic = first;
  Fp4Meta cur = fp4_meta<GATED>(p, ts, ofs, beg + ic, wave, lane);
  Fp4Ctx t = fp4_ctx<GATED>(p, cur, wave, lane);
  // every wave is done with the ring before it is refilled
  wait_vm<0>();
  lds_barrier();
  t.issue(0, ring_base, wave, p.N);
  t.issue(1, ring_base + C::STAGE, wave, p.N);
  int pend = t.na + C::C_LOADS + 1;  // loads of the last stage issued
  int sc = 0;                        // ring slot of the next stage computed
  int si = 2;                        // ring slot of the next stage issued
  Fp4Meta nxt = cur;
  bool more = false;

  // K step kt of the current item: wait for its stage, issue the stage two
  // ahead (of this item, else of the next, else a repeat of the last one,
  // which keeps the wait counts uniform), compute
  Fp4Out prev;
  Item prev_item = cur.item;
  int prev_base = cur.row_base;
  auto step = [&](int kt, f32x16_t (&acc)[2], bool store_prev) {
    fp4_wait_stage(pend);
    lds_barrier();
    if (store_prev) fp4_store<GATED>(p, prev_item, prev_base, wave, lane, prev);
    const int s2 = kt + C::NS - 1;
    if (s2 < nk) {
      t.issue(s2, ring_base + si * C::STAGE, wave, p.N);
    } else if (more) {
      if (s2 == nk) t = fp4_ctx<GATED>(p, nxt, wave, lane);
      t.issue(s2 - nk, ring_base + si * C::STAGE, wave, p.N);
    } else {
      t.issue(nk - 1, ring_base + si * C::STAGE, wave, p.N);
    }
    pend = t.na + C::C_LOADS + 1;
    si = si == C::NS - 1 ? 0 : si + 1;
    fp4_stage(ring + sc * C::STAGE, wave, lane, acc);
    sc = sc == C::NS - 1 ? 0 : sc + 1;
  };

  bool held = false;
  for (;;) {
    const long long in = ic + stride;
    more = in < nr;
    f32x16_t acc[2];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[j][r] = 0.0f;
    step(0, acc, held);
    if (more) nxt = fp4_meta<GATED>(p, ts, ofs, beg + in, wave, lane);
    for (int kt = 1; kt < nk; ++kt) step(kt, acc, false);
    fp4_pack<GATED>(acc, prev);
    prev_item = cur.item;
    prev_base = cur.row_base;
    if (!more) break;
    held = true;
    cur = nxt;
    ic = in;
  }
  fp4_store<GATED>(p, prev_item, prev_base, wave, lane, prev);
}

// One routed item with its own pipeline fill (items of fewer than 3 K steps).
template <bool GATED>
__device__ __forceinline__ void fp4_routed_item(const FfnArgs& p, const int* ts, const int* ofs,
                                                long long it, const uint8_t* ring,
                                                uint32_t ring_base, int wave, int lane) {
  using C = Fp4Cfg;
  const int nk = p.K / C::BK;
  const Fp4Meta m = fp4_meta<GATED>(p, ts, ofs, it, wave, lane);
  const Fp4Ctx t = fp4_ctx<GATED>(p, m, wave, lane);
  f32x16_t acc[2];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[j][r] = 0.0f;
  // every wave is done with the previous item's LDS before refilling it
  wait_vm<0>();
  lds_barrier();
#pragma unroll
  for (int s = 0; s < C::NS - 1; ++s)
    t.issue(s < nk ? s : nk - 1, ring_base + s * C::STAGE, wave, p.N);
  for (int kt = 0; kt < nk; ++kt) {
    fp4_wait_stage(t.na + C::C_LOADS + 1);
    lds_barrier();
    const int kn = kt + C::NS - 1 < nk ? kt + C::NS - 1 : nk - 1;
    t.issue(kn, ring_base + ((kt + C::NS - 1) % C::NS) * C::STAGE, wave, p.N);
    fp4_stage(ring + (kt % C::NS) * C::STAGE, wave, lane, acc);
  }
  Fp4Out o;
  fp4_pack<GATED>(acc, o);
  fp4_store<GATED>(p, m.item, m.row_base, wave, lane, o);
}

// Routed groups, then (p.ksplit > 0) the shared experts' bf16 tiles.
// Persistent workgroups over the items, cut into one contiguous chunk per
// XCD; workgroup slot s of an XCD takes items s, s + 64, ... of its chunk
// (routed first).  Two workgroups share each CU (a 3-stage ring each, 77 KiB
// of LDS), so one's stream covers the other's pipeline fills.
template <bool GATED>
__global__ __launch_bounds__(256, 2) void ffn_fp4_kernel(FfnArgs p) {
  using C = Fp4Cfg;
  __shared__ __attribute__((aligned(1024))) uint8_t ring[C::NS * C::STAGE];
  __shared__ int ts[kFp4MaxGroups + 1];   // tile plan
  __shared__ int ofs[kFp4MaxGroups + 1];  // group offsets of the routed rows

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = p.E + p.S;
  for (int g = tid; g <= G; g += 256) ts[g] = p.tile_start[g];
  for (int g = tid; g <= p.E; g += 256) ofs[g] = p.offsets[g];
  __syncthreads();

  // routed items, then the shared items; each XCD takes a contiguous chunk
  // of both, its routed chunk first
  const long long total = static_cast<long long>(ts[p.E]) * p.n_tiles;  // routed items
  const long long shared =
      p.ksplit > 0 ? static_cast<long long>(p.S) *
                         ((p.T + kFp4SharedRows - 1) / kFp4SharedRows) * p.n_tiles * p.ksplit
                   : 0;
  const int xcd = blockIdx.x & 7;
  const int per_xcd = gridDim.x >> 3;
  const int slot_id = blockIdx.x >> 3;
  const long long chunk = (total + 7) / 8;
  const long long beg = xcd * chunk < total ? xcd * chunk : total;
  const long long end = beg + chunk < total ? beg + chunk : total;
  const long long schunk = (shared + 7) / 8;
  const long long sbeg = xcd * schunk < shared ? xcd * schunk : shared;
  const long long send = sbeg + schunk < shared ? sbeg + schunk : shared;
  const long long nr = end - beg;
  const long long nitems = nr + (send - sbeg);
  const uint32_t ring_base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(LDS_PTR(ring)));

  long long i = slot_id;
  if (i < nr) {
    if (p.K / C::BK >= 3) {
      fp4_routed_stream<GATED>(p, ts, ofs, beg, nr, i, per_xcd, ring, ring_base, wave, lane);
      i += (nr - i + per_xcd - 1) / per_xcd * per_xcd;   // first index past the routed items
    } else {
      for (; i < nr; i += per_xcd)
        fp4_routed_item<GATED>(p, ts, ofs, beg + i, ring, ring_base, wave, lane);
    }
  }
  for (; i < nitems; i += per_xcd)
    fp4_shared_item<GATED>(p, sbeg + (i - nr), ring, ring_base, wave, lane);
  wait_vm<0>();  // no direct load may still be landing in LDS when the workgroup ends
}

hipError_t launch_fp4(const FfnArgs& a, bool gated, hipStream_t st) {
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    cus = 256;
  const int grid = 2 * ((cus + 7) / 8 * 8);  // two resident workgroups per CU
  if (gated) ffn_fp4_kernel<true><<<grid, 256, 0, st>>>(a);
  else ffn_fp4_kernel<false><<<grid, 256, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace moe
