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
// Layouts (one expert stack [E, N, K]):
//   codes  [E, N, K/2]  bytes; value 2i in the low nibble of byte i
//   scales [E, K/32, N] bytes X + 127; the scales of one K block of
//                        consecutive weight rows are contiguous
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
    *reinterpret_cast<uint4*>(codes + r * (K / 2) + kb * 16) =
        make_uint4(packed[0], packed[1], packed[2], packed[3]);
    const long long e = r / N;
    const long long n = r - e * N;
    scales[(e * kb_per_row + kb) * N + n] = static_cast<uint8_t>(X + 127);
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
//   scales 4 K blocks x 256 rows (bytes);
// all filled with direct global -> LDS loads: per wave up to 2 A loads and
// 4 code loads of 1 KiB and one 256-byte scale load (the scales of K block
// 4kt + wave).  An A load covers 4 rows and is skipped when none of them
// holds a row of the tile (decode tiles hold a row or two): the LDS rows it
// would fill only feed accumulator rows that are never stored, and the
// wave's wait counts follow its number of loads.  B fragments are read as 4 code bytes + 1 scale byte per lane and
// converted to bf16 in registers.
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
      dma16_lds(c_src[q] + kt * (C::BK / 2), slot + C::A_BYTES + (wave * C::C_LOADS + q) * 1024);
    dma4(s_src + static_cast<size_t>(kt) * 4 * sstride,
         slot + C::A_BYTES + C::C_BYTES + wave * 256);
  }
};

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// B fragment of substep kk for column block j of wave wn: lane l holds the
// 8 values k = 16kk + 8(l/32) .. of weight row 64wn + 32j + l%32.
__device__ __forceinline__ bf16x8_t fp4_frag(const uint8_t* st, int row, int kk, int half) {
  using C = Fp4Cfg;
  const int chunk = (kk >> 1) ^ ((row >> 2) & 3);   // 16-byte chunk holding bytes 8kk..
  const uint32_t word = *reinterpret_cast<const uint32_t*>(
      st + C::A_BYTES + row * 64 + chunk * 16 + (kk & 1) * 8 + half * 4);
  const uint32_t sb = st[C::A_BYTES + C::C_BYTES + (kk >> 1) * 256 + row];
  const float scale = __uint_as_float(sb == 0 ? 0x00400000u : sb << 23);  // 2^(sb-127)
  const bf16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, scale, 0);
  const bf16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, scale, 1);
  const bf16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, scale, 2);
  const bf16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, scale, 3);
  bf16x8_t r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

__device__ __forceinline__ void fp4_stage(const uint8_t* st, int wn, int lane,
                                          f32x16_t (&acc)[2]) {
  const int r32 = lane & 31;
  const int half = lane >> 5;
  const bf16_t* sa = reinterpret_cast<const bf16_t*>(st);
#pragma unroll
  for (int kk = 0; kk < Fp4Cfg::BK / 16; ++kk) {
    const int c = 2 * kk + half;  // 16-byte chunk of the A row
    const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(sa + r32 * 128 + ((c ^ (r32 & 15)) << 3));
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const bf16x8_t b = fp4_frag(st, wn * 64 + j * 32 + r32, kk, half);
      acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
    }
  }
}

// Routed groups only (the shared experts' weights are bf16 and go through
// the bf16 kernel).  Persistent workgroups over the items of groups
// 0..E-1, cut into one contiguous chunk per XCD.  Two workgroups share each
// CU (a 3-stage ring each, 77 KiB of LDS): every item starts by waiting a
// full HBM latency for its first stage, and the other workgroup's stream
// covers that wait (8% faster at T=64 than one workgroup with a 4-stage
// ring; 5 or 6 stages in one workgroup gain nothing).
template <bool GATED>
__global__ __launch_bounds__(256, 2) void ffn_fp4_kernel(FfnArgs p) {
  using C = Fp4Cfg;
  __shared__ __attribute__((aligned(1024))) uint8_t ring[C::NS * C::STAGE];
  __shared__ int ts[512];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = p.E + p.S;
  for (int g = tid; g <= G; g += 256) ts[g] = p.tile_start[g];
  __syncthreads();

  const long long total = static_cast<long long>(ts[p.E]) * p.n_tiles;  // routed items
  const int xcd = blockIdx.x & 7;
  const int per_xcd = gridDim.x >> 3;
  const int slot_id = blockIdx.x >> 3;
  const long long chunk = (total + 7) / 8;
  const long long beg = xcd * chunk;
  const long long end = beg + chunk < total ? beg + chunk : total;

  const bf16_t* A = static_cast<const bf16_t*>(p.a);
  const uint32_t ring_base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(LDS_PTR(ring)));
  const int nk = p.K / C::BK;
  const int kb_per_row = p.K / 32;
  // A load j fills rows 4j..4j+3: lane l -> row 4j + l/16, slot l%16,
  // source chunk (l%16) ^ (row & 15)
  const int arow = lane >> 4;
  // code load j fills rows 16j..16j+15: lane l -> row 16j + l/4, slot l%4,
  // source chunk (l%4) ^ ((row >> 2) & 3)
  const int crow = lane >> 2;

  for (long long it = beg + slot_id; it < end; it += per_xcd) {
    const Item item = decode_item(it, ts, G, p.n_tiles, C::MT, p.offsets, p.T, p.E);
    const int g = item.g;  // routed
    const size_t row_base = static_cast<size_t>(p.offsets[g]);
    Fp4Ctx t;
    {
      const int left = item.rows - 4 * wave * C::A_LOADS;   // rows from this wave's first group
      const int groups = left <= 0 ? 0 : (left + 3) / 4;
      t.na = groups < C::A_LOADS ? groups : C::A_LOADS;
    }
#pragma unroll
    for (int q = 0; q < C::A_LOADS; ++q) {
      const int j = wave * C::A_LOADS + q;
      int r = 4 * j + arow;
      const int rc = r;
      r = r < item.rows ? r : item.rows - 1;
      const int rr = item.m0 + r;
      const size_t src_row = GATED ? static_cast<size_t>(p.sorted_pair[row_base + rr] / p.k)
                                   : row_base + rr;
      t.a_src[q] = A + src_row * p.K + (((lane & 15) ^ (rc & 15)) << 3);
    }
    const size_t cstride = static_cast<size_t>(p.N) * (p.K / 2);   // bytes per expert
    const size_t sstride_e = static_cast<size_t>(kb_per_row) * p.N;
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
      t.c_src[q] = base + g * cstride + static_cast<size_t>(col) * (p.K / 2) +
                   (((lane & 3) ^ ((R >> 2) & 3)) << 4);
    }
    {
      // scale load of K block 4kt + wave: LDS bytes 4l..4l+3 = rows 4l..4l+3
      const int R = 4 * lane;
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
      t.s_src = sbase + g * sstride_e + static_cast<size_t>(wave) * p.N + col;
    }

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
    static_assert(C::NS == 3 && C::A_LOADS == 2, "wait cases");
    for (int kt = 0; kt < nk; ++kt) {
      if (t.na == 2) wait_vm<C::LPW>();
      else if (t.na == 1) wait_vm<C::LPW - 1>();
      else wait_vm<C::LPW - 2>();
      lds_barrier();
      const int kn = kt + C::NS - 1 < nk ? kt + C::NS - 1 : nk - 1;
      t.issue(kn, ring_base + ((kt + C::NS - 1) % C::NS) * C::STAGE, wave, p.N);
      fp4_stage(ring + (kt % C::NS) * C::STAGE, wave, lane, acc);
    }

    // ---- epilogue.  32x32 accumulator layout: lane l holds column l%32 and
    // rows 8*(r/4) + 4*(l/32) + r%4 for r = 0..15.
    bf16_t* out = static_cast<bf16_t*>(p.out_routed);
    const size_t orow0 = static_cast<size_t>(p.offsets[g]) + item.m0;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
      if (row >= item.rows) continue;
      bf16_t* orow = out + (orow0 + row) * p.ldo;
      if (GATED) {
        const float gt = acc[0][r];
        const float up = acc[1][r];
        orow[item.n * (C::NB / 2) + wave * 32 + (lane & 31)] =
            f32_to_bf16(gt * __builtin_amdgcn_rcpf(1.0f + __expf(-gt)) * up);
      } else {
#pragma unroll
        for (int j = 0; j < 2; ++j)
          orow[item.n * C::NB + wave * 64 + j * 32 + (lane & 31)] = f32_to_bf16(acc[j][r]);
      }
    }
  }
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
