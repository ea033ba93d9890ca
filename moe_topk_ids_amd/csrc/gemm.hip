// Grouped bf16 GEMMs of the expert FFN on CDNA4 matrix cores.
//
// Both products are "NT": the token operand and the weight operand are
// contiguous along the contraction dimension (hidden [T,H] and w1[e] [2I,H]
// for the gate/up projection; the bf16 intermediate [P,I] and w2[e] [H,I]
// for the down projection), so both are staged the same way.
//
// A workgroup owns one BM x BN output tile of one expert: BM consecutive rows
// of the expert-grouped padded layout produced by the routing step (all rows
// of a tile belong to one expert), and BN weight rows. The grid is sized for
// the largest possible number of row tiles; workgroups past the device-side
// tile count exit at once, so no host synchronisation is needed.
//
// The matrix-core instruction is v_mfma_f32_32x32x16_bf16 with the WEIGHT
// fragment as its first operand and the TOKEN fragment as its second, so the
// 16 accumulators of a lane hold 4 runs of 4 consecutive output columns for
// one token row: epilogues store 8-byte bf16 or 16-byte fp32 vectors.
//
// Staging: K is consumed 64 bf16 at a time. Global -> registers (16-byte
// loads, 8 lanes per 128-byte row segment) for step k+1 is in flight while
// the matrix cores work on step k out of LDS; LDS is double-buffered so one
// barrier per step suffices. Rows are stored in LDS as 8 chunks of 16 bytes
// permuted by an XOR of the row index, so that the fragment reads of any 16
// consecutive rows at the same logical chunk fall on distinct banks.
//
// Gate/up pairing (the epilogue needs silu(gate_i) * up_i in one lane): the
// BN weight rows of a GEMM1 tile are BN/2 gate rows [n0, n0+BN/2) and the
// BN/2 up rows I + [n0, n0+BN/2); each wave's column range covers matching
// gate and up sub-tiles. The same pairing is what tpu-inference's fused_moe
// kernel does when it fetches matching w1 and w3 blocks of one expert.
#include "moe_internal.h"

namespace moe {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int BK = 64;  // contraction elements per pipeline step (128 bytes per row)

enum Mode { kGateUpSilu = 0, kDownSlot = 1, kDownAtomic = 2 };

struct GemmArgs {
  const uint16_t* a;        // token operand: hidden [T,H] (gathered) or act [P,I]
  const uint16_t* w;        // weights: w1 [E,2I,H] or w2 [E,H,I]
  const int32_t* sorted;    // padded row -> slot
  const int32_t* tile_expert;
  const int32_t* num_tiles;
  const float* topk_weights;
  void* out;                // act bf16 [P,I] | y fp32 [T*K,H] | out fp32 [T,H]
  int64_t kdim;             // contraction length (H or I)
  int64_t n_out;            // output columns (I for GEMM1, H for GEMM2)
  int64_t w_expert_stride;  // elements per expert in w
  int64_t inter;            // I (GEMM1: offset of the up rows)
  int32_t topk;             // K
  int32_t max_tiles;        // row tiles the grid was sized for
};

__device__ __forceinline__ int swz(int r) { return (r ^ (r >> 3)) & 7; }

__device__ __forceinline__ float silu_mul(float g, float u) {
  // silu(g) * u = g * u / (1 + exp(-g)); exp via the hardware 2^x.
  const float e = __builtin_amdgcn_exp2f(-g * 1.4426950408889634f);
  return g * u * __builtin_amdgcn_rcpf(1.0f + e);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const __bf16 a = (__bf16)lo;  // round to nearest even
  const __bf16 b = (__bf16)hi;
  return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

template <int BM, int BN, int WGM, int WGN, int MODE>
__global__ __launch_bounds__(64 * WGM * WGN) void grouped_gemm(GemmArgs args) {
  constexpr int NT = 64 * WGM * WGN;
  constexpr int WTM = BM / WGM;  // token rows per wave
  constexpr int WTN = BN / WGN;  // weight rows per wave
  constexpr int TM = WTM / 32;
  constexpr int TN = WTN / 32;
  constexpr int CA = BM * 8 / NT;  // 16-byte token chunks per thread per step
  constexpr int CB = BN * 8 / NT;  // 16-byte weight chunks per thread per step
  constexpr int RSTEP = NT / 8;    // rows between a thread's consecutive chunks
  static_assert(CA >= 1 && CB >= 1 && TM >= 1 && TN >= 1, "tile too small");
  static_assert(MODE != kGateUpSilu || (TN % 2 == 0), "gate/up pairing needs even TN");

  __shared__ uint4 sA[2][BM * 8];
  __shared__ uint4 sW[2][BN * 8];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave % WGM;
  const int wn = wave / WGM;

  const int mt = blockIdx.x % args.max_tiles;
  const int ntile = blockIdx.x / args.max_tiles;
  if (mt >= args.num_tiles[0]) return;
  const int e = args.tile_expert[mt];
  const int64_t m0 = (int64_t)mt * BM;
  const int64_t kdim = args.kdim;

  // ---- per-thread global row pointers (fixed over the K loop) ----
  const int chunk = tid & 7;
  const uint16_t* arow[CA];
#pragma unroll
  for (int j = 0; j < CA; ++j) {
    const int64_t r = m0 + (tid >> 3) + j * RSTEP;
    if (MODE == kGateUpSilu) {
      const int32_t f = args.sorted[r];
      arow[j] = f >= 0 ? args.a + (int64_t)(f / args.topk) * kdim + chunk * 8 : nullptr;
    } else {
      arow[j] = args.a + r * kdim + chunk * 8;
    }
  }
  const uint16_t* wrow[CB];
  const uint16_t* wbase = args.w + (int64_t)e * args.w_expert_stride;
#pragma unroll
  for (int j = 0; j < CB; ++j) {
    const int nl = (tid >> 3) + j * RSTEP;
    int64_t row;
    bool ok;
    if (MODE == kGateUpSilu) {
      const int64_t n0g = (int64_t)ntile * (BN / 2);
      row = nl < BN / 2 ? n0g + nl : args.inter + n0g + (nl - BN / 2);
      ok = true;  // I is a multiple of BN/2
    } else {
      row = (int64_t)ntile * BN + nl;
      ok = row < args.n_out;
    }
    wrow[j] = ok ? wbase + row * kdim + chunk * 8 : nullptr;
  }

  uint4 ra[CA], rw[CB];
  const uint4 zero4 = make_uint4(0, 0, 0, 0);
  auto gload = [&](int64_t k0) {
#pragma unroll
    for (int j = 0; j < CA; ++j)
      ra[j] = arow[j] ? *reinterpret_cast<const uint4*>(arow[j] + k0) : zero4;
#pragma unroll
    for (int j = 0; j < CB; ++j)
      rw[j] = wrow[j] ? *reinterpret_cast<const uint4*>(wrow[j] + k0) : zero4;
  };
  auto sstore = [&](int st) {
#pragma unroll
    for (int j = 0; j < CA; ++j) {
      const int r = (tid >> 3) + j * RSTEP;
      sA[st][r * 8 + (chunk ^ swz(r))] = ra[j];
    }
#pragma unroll
    for (int j = 0; j < CB; ++j) {
      const int r = (tid >> 3) + j * RSTEP;
      sW[st][r * 8 + (chunk ^ swz(r))] = rw[j];
    }
  };

  f32x16_t acc[TN][TM];
#pragma unroll
  for (int a = 0; a < TN; ++a)
#pragma unroll
    for (int b = 0; b < TM; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.0f;

  // LDS row of each of this wave's weight sub-tiles
  int nrow[TN];
#pragma unroll
  for (int tn = 0; tn < TN; ++tn) {
    if (MODE == kGateUpSilu) {
      nrow[tn] = tn < TN / 2 ? wn * (WTN / 2) + tn * 32
                             : BN / 2 + wn * (WTN / 2) + (tn - TN / 2) * 32;
    } else {
      nrow[tn] = wn * WTN + tn * 32;
    }
  }

  const int nk = (int)(kdim / BK);
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) gload((int64_t)(kt + 1) * BK);
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      const int c = kk * 2 + (lane >> 5);
      bf16x8_t bt[TM], aw[TN];
#pragma unroll
      for (int tm = 0; tm < TM; ++tm) {
        const int r = wm * WTM + tm * 32 + (lane & 31);
        bt[tm] = __builtin_bit_cast(bf16x8_t, sA[cur][r * 8 + (c ^ swz(r))]);
      }
#pragma unroll
      for (int tn = 0; tn < TN; ++tn) {
        const int r = nrow[tn] + (lane & 31);
        aw[tn] = __builtin_bit_cast(bf16x8_t, sW[cur][r * 8 + (c ^ swz(r))]);
      }
#pragma unroll
      for (int tn = 0; tn < TN; ++tn)
#pragma unroll
        for (int tm = 0; tm < TM; ++tm)
          acc[tn][tm] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aw[tn], bt[tm], acc[tn][tm], 0, 0, 0);
    }
    if (kt + 1 < nk) sstore(cur ^ 1);
    __syncthreads();
  }

  // ---- epilogues ----
  // lane holds, for token row (lane & 31) of sub-tile tm, the weight columns
  // 8*j + 4*(lane >> 5) + {0,1,2,3} of sub-tile tn, in acc[tn][tm][4j..4j+3]
  const int csub = 4 * (lane >> 5);
  if (MODE == kGateUpSilu) {
    uint16_t* act = reinterpret_cast<uint16_t*>(args.out);
    const int64_t n0g = (int64_t)ntile * (BN / 2);
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) {
      const int64_t r = m0 + wm * WTM + tm * 32 + (lane & 31);
#pragma unroll
      for (int tn = 0; tn < TN / 2; ++tn) {
        const int64_t col = n0g + wn * (WTN / 2) + tn * 32 + csub;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const f32x16_t& g = acc[tn][tm];
          const f32x16_t& u = acc[tn + TN / 2][tm];
          uint2 v;
          v.x = pack_bf16x2(silu_mul(g[4 * j + 0], u[4 * j + 0]), silu_mul(g[4 * j + 1], u[4 * j + 1]));
          v.y = pack_bf16x2(silu_mul(g[4 * j + 2], u[4 * j + 2]), silu_mul(g[4 * j + 3], u[4 * j + 3]));
          *reinterpret_cast<uint2*>(act + r * args.n_out + col + 8 * j) = v;
        }
      }
    }
  } else {
    float* dst = reinterpret_cast<float*>(args.out);
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) {
      const int64_t r = m0 + wm * WTM + tm * 32 + (lane & 31);
      const int32_t f = args.sorted[r];
      if (f < 0) continue;
      float wgt = 1.0f;
      int64_t orow;
      if (MODE == kDownAtomic) {
        wgt = args.topk_weights[f];
        orow = (int64_t)(f / args.topk);
      } else {
        orow = f;
      }
#pragma unroll
      for (int tn = 0; tn < TN; ++tn) {
        const int64_t col = (int64_t)ntile * BN + wn * WTN + tn * 32 + csub;
        if (col >= args.n_out) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float* p = dst + orow * args.n_out + col + 8 * j;
          const f32x16_t& a = acc[tn][tm];
          if (MODE == kDownSlot) {
            *reinterpret_cast<f32x4_t*>(p) = f32x4_t{a[4 * j], a[4 * j + 1], a[4 * j + 2], a[4 * j + 3]};
          } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) unsafeAtomicAdd(p + i, wgt * a[4 * j + i]);
          }
        }
      }
    }
  }
}

template <int BM, int BN, int WGM, int WGN, int MODE>
hipError_t launch_cfg(const GemmArgs& a, int n_tiles, hipStream_t stream) {
  const int64_t blocks = (int64_t)a.max_tiles * n_tiles;
  if (blocks == 0) return hipSuccess;
  grouped_gemm<BM, BN, WGM, WGN, MODE><<<dim3((unsigned)blocks), dim3(64 * WGM * WGN), 0, stream>>>(a);
  return hipGetLastError();
}

template <int MODE>
hipError_t dispatch(GemmCfg cfg, const GemmArgs& a, int n_tiles, hipStream_t stream) {
  if (cfg.bm == 128 && cfg.bn == 128) return launch_cfg<128, 128, 2, 2, MODE>(a, n_tiles, stream);
  if (cfg.bm == 64 && cfg.bn == 128) return launch_cfg<64, 128, 2, 2, MODE>(a, n_tiles, stream);
  if (cfg.bm == 128 && cfg.bn == 256) return launch_cfg<128, 256, 2, 2, MODE>(a, n_tiles, stream);
  return hipErrorInvalidValue;
}

}  // namespace

GemmCfg pick_gemm1_cfg(int64_t n_slots, int64_t H, int64_t I, int64_t E) {
  (void)H;
  (void)I;
  const int64_t live = n_slots < E ? n_slots : E;
  const int64_t rows_per_expert = live > 0 ? n_slots / live : 0;
  if (rows_per_expert < 96) return GemmCfg{64, 128};
  return GemmCfg{128, 128};
}

GemmCfg pick_gemm2_cfg(int64_t n_slots, int64_t H, int64_t I, int64_t E, int bm) {
  (void)n_slots;
  (void)H;
  (void)I;
  (void)E;
  return GemmCfg{bm, 128};
}

hipError_t launch_gemm1_silu(GemmCfg cfg, const uint16_t* hidden, const uint16_t* w1,
                             const int32_t* sorted, const int32_t* tile_expert,
                             const int32_t* num_tiles, int64_t T, int64_t H, int64_t I,
                             int64_t K, int64_t max_tiles, uint16_t* act, hipStream_t stream) {
  (void)T;
  GemmArgs a{};
  a.a = hidden;
  a.w = w1;
  a.sorted = sorted;
  a.tile_expert = tile_expert;
  a.num_tiles = num_tiles;
  a.out = act;
  a.kdim = H;
  a.n_out = I;
  a.w_expert_stride = 2 * I * H;
  a.inter = I;
  a.topk = (int32_t)K;
  a.max_tiles = (int32_t)max_tiles;
  const int n_tiles = (int)(I / (cfg.bn / 2));
  return dispatch<kGateUpSilu>(cfg, a, n_tiles, stream);
}

hipError_t launch_gemm2(GemmCfg cfg, const uint16_t* act, const uint16_t* w2,
                        const int32_t* sorted, const int32_t* tile_expert,
                        const int32_t* num_tiles, const float* topk_weights, int64_t H,
                        int64_t I, int64_t K, int64_t max_tiles, float* y, float* out,
                        hipStream_t stream) {
  GemmArgs a{};
  a.a = act;
  a.w = w2;
  a.sorted = sorted;
  a.tile_expert = tile_expert;
  a.num_tiles = num_tiles;
  a.topk_weights = topk_weights;
  a.out = out ? (void*)out : (void*)y;
  a.kdim = I;
  a.n_out = H;
  a.w_expert_stride = H * I;
  a.inter = I;
  a.topk = (int32_t)K;
  a.max_tiles = (int32_t)max_tiles;
  const int n_tiles = (int)((H + cfg.bn - 1) / cfg.bn);
  if (out) return dispatch<kDownAtomic>(cfg, a, n_tiles, stream);
  return dispatch<kDownSlot>(cfg, a, n_tiles, stream);
}

}  // namespace moe
