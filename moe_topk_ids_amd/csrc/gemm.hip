// Grouped bf16 GEMMs of the expert FFN on CDNA4 matrix cores.
//
// Both products are "NT": the token operand and the weight operand are
// contiguous along the contraction dimension (hidden [T,H] and w1[e] [2I,H]
// for the gate/up projection; the bf16 intermediate [P,I] and w2[e] [H,I]
// for the down projection), so both are staged the same way.
//
// A workgroup owns one BM x BN output tile of one expert: BM consecutive rows
// of the expert-grouped padded layout produced by the routing step (all rows
// of a tile belong to one expert), and BN weight rows. The tile list is
// sized for the largest possible number of row tiles; tiles past the
// device-side tile count are skipped, so no host synchronisation is needed.
// The launch is persistent: as many workgroups as the chip holds at once,
// each looping over tiles.
//
// The matrix-core instruction is v_mfma_f32_32x32x16_bf16 with the WEIGHT
// fragment as its first operand and the TOKEN fragment as its second, so the
// 16 accumulators of a lane hold 4 runs of 4 consecutive output columns for
// one token row: epilogues store 8-byte bf16 or 16-byte fp32 vectors.
//
// Staging: K is consumed 64 bf16 (128 bytes per row) per step through an
// NS-deep ring of LDS stages. Each stage is filled by buffer_load_dwordx4
// with the LDS bit (global -> LDS directly, no register staging): a wave's
// load writes 1 KB of LDS, 16 bytes per lane, so the 8-chunk XOR permutation
// of each 128-byte row (chosen so that the fragment reads of any 16
// consecutive rows at one logical chunk hit distinct banks) is applied on
// the global side by choosing which chunk each lane fetches. While the
// matrix cores work on stage k, the loads of stages k+1 .. k+NS-1 are in
// flight; the vector-memory counter is waited on explicitly, one barrier per
// step. Rows outside the operand (pad rows of the routing layout, weight
// rows past N) are read through an out-of-range buffer offset and arrive as
// zeros.
//
// Gate/up pairing (the epilogue needs silu(gate_i) * up_i in one lane): the
// BN weight rows of a GEMM1 tile are BN/2 gate rows [n0, n0+BN/2) and the
// BN/2 up rows I + [n0, n0+BN/2); each wave's column range covers matching
// gate and up sub-tiles. The same pairing is what tpu-inference's fused_moe
// kernel does when it fetches matching w1 and w3 blocks of one expert.
#include <algorithm>

#include "device_util.h"
#include "moe_internal.h"

namespace moe {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));


// Workgroups of one round of the chip at one per CU (8 XCDs x 32 CUs).
constexpr int kRound = 256;

// kDownSlot writes fp32 slot rows; kDownSlotBf16 writes them rounded to bf16
// (round to nearest even), half the bytes for the combine to read back.
enum Mode { kGateUpSilu = 0, kDownSlot = 1, kDownAtomic = 2, kDownSlotBf16 = 3 };

struct GemmArgs {
  const uint16_t* a;        // token operand: hidden [T,H] (gathered) or act [P,I]
  const uint16_t* w;        // weights: w1 [E,2I,H] or w2 [E,H,I]
  const int32_t* sorted;    // padded row -> slot
  const int32_t* tile_expert;
  const int32_t* num_tiles;
  const float* topk_weights;
  void* out;                // act bf16 [P,I] | y fp32 or bf16 [T*K,H] | out fp32 [T,H]
  int64_t kdim;             // contraction length (H or I)
  int64_t n_out;            // output columns (I for GEMM1, H for GEMM2)
  int64_t w_expert_stride;  // elements per expert in w
  int64_t inter;            // I (GEMM1: offset of the up rows)
  uint32_t a_bytes;         // bytes of the token operand (GEMM1 gather bound)
  int32_t topk;             // K
  int32_t n_experts;        // E (a tile whose expert is outside [0, E) is skipped)
  int32_t max_tiles;        // row tiles the grid was sized for
  int32_t n_tiles;          // weight-row tiles
  int32_t group_m;          // row tiles per scheduling group
  int32_t xcd_slots;        // workgroups resident at once on one XCD
  int32_t nvb;              // virtual workgroups (tiles of the grid before persistence)
  // split of the down projection's contraction: split s of ksplit covers
  // stages [s*nk/ksplit, (s+1)*nk/ksplit) and writes its partial slot rows
  // to out + s*part_stride
  int32_t ksplit;
  int64_t part_stride;
  // Column-half tail of a tile order whose last round of the chip would be
  // at most half full (tiles of one workgroup per CU): phase 1 runs the whole
  // rounds of `rounds_of` workgroups, phase 2 (a second launch, BN half the
  // first's) runs the remaining tiles as two column halves each, so their
  // round takes about half a tile's time. 0: every tile in one launch.
  int32_t phase;
  int32_t rounds_of;
  // epilogue variants: activation kind and swigluoai parameters (GEMM1),
  // bias b1 [E, 2I] (GEMM1) or b2 [E, H] (GEMM2 with the atomic combine)
  int32_t act;
  float alpha, limit;
  const float* bias;
  // fp8 weights (instead of w): codes [E, rows, kdim] and one fp32 scale per
  // qblock codes along the contraction, [E, rows, nqb]
  const uint8_t* wq;
  const float* wscale;
  int32_t qblock;
  int32_t nqb;
};

// XOR permutation of the 16-byte chunks of a staged row (CPR chunks per
// row). With it the fragment reads of 8 consecutive rows cover a 128-byte
// bank window and those of 16 consecutive rows a 256-byte window without
// repeating a bank group, for both row widths used.
template <int CPR>
__device__ __forceinline__ int swz(int r) {
  if constexpr (CPR == 8) return (r ^ (r >> 3)) & 7;
  else return ((r >> 1) ^ (r >> 3)) & 3;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const __bf16 a = (__bf16)lo;  // round to nearest even
  const __bf16 b = (__bf16)hi;
  return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

// Pad rows and out-of-range weight rows are read through make_rsrc's
// out-of-range offset (kOutOfRange): they arrive as zeros without branches.

typedef __attribute__((address_space(3))) void lds_void_t;

// One 16-byte load per lane straight into LDS (buffer_load_dwordx4 with the
// LDS bit): lane i's bytes land at dst + 16*i, read from voffset + soffset.
// dst must be wave-uniform. (Plain functions: called from a template-
// dependent context, the builtin makes the host pass drop the kernel.)
__device__ __forceinline__ void load_lds_b128(__amdgpu_buffer_rsrc_t rsrc, const char* dst,
                                              uint32_t voffset, uint32_t soffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_t*)dst, 16, voffset, soffset, 0, 0);
}

// One 4-byte load per lane into LDS: lane i's word lands at dst + 4*i.
__device__ __forceinline__ void load_lds_b32(__amdgpu_buffer_rsrc_t rsrc, const char* dst,
                                             uint32_t voffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_t*)dst, 4, voffset, 0, 0, 0);
}

// 8 OCP E4M3 codes (k order: the bytes of lo, then of hi) to bf16 as
// bf16_rne(fp32(code) * scale): the decode is exact, the product is the fp32
// one, then one rounding to bf16.
__device__ __forceinline__ bf16x8_t fp8x8_to_bf16(uint32_t lo, uint32_t hi, float scale) {
  const f32x2_t a = __builtin_amdgcn_cvt_pk_f32_fp8((int)lo, false);
  const f32x2_t b = __builtin_amdgcn_cvt_pk_f32_fp8((int)lo, true);
  const f32x2_t c = __builtin_amdgcn_cvt_pk_f32_fp8((int)hi, false);
  const f32x2_t d = __builtin_amdgcn_cvt_pk_f32_fp8((int)hi, true);
  const float a0 = a[0], a1 = a[1], b0 = b[0], b1 = b[1];
  const float c0 = c[0], c1 = c[1], d0 = d[0], d1 = d[1];
  u32x4_t v;
  v[0] = pack_bf16x2(a0 * scale, a1 * scale);
  v[1] = pack_bf16x2(b0 * scale, b1 * scale);
  v[2] = pack_bf16x2(c0 * scale, c1 * scale);
  v[3] = pack_bf16x2(d0 * scale, d1 * scale);
  return __builtin_bit_cast(bf16x8_t, v);
}

// s_waitcnt on the vector-memory counter only (gfx9 encoding: vmcnt in bits
// 3:0 and 15:14, expcnt 6:4 and lgkmcnt 11:8 left at their no-wait maximum).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Workgroup barrier of a ring deeper than two stages: this wave's LDS reads
// complete, then the barrier, with no fence (a fence would make the compiler
// wait for every outstanding load, the later stages' included). The empty
// asm statements keep the compiler from moving memory accesses across it.
__device__ __forceinline__ void ring_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Epilogue of one wave's WTM x WTN sub-tile (wave position wm, wn in the
// tile): lane holds, for token row (lane & 31) of sub-tile tm, the weight
// columns 8*j + 4*(lane >> 5) + {0,1,2,3} of sub-tile tn, in
// acc[tn][tm][4j..4j+3].
// XOR key of the 16-byte chunks of a row staged for the epilogue's stores
// (CPR chunks per row): the 32 rows one write instruction covers land on
// distinct 16-byte bank groups of each 256-byte bank window, two rows per
// group (rows of 128 bytes share a window in pairs, hence row / 2 there).
template <int CPR>
__device__ __forceinline__ int stage_swz(int r) {
  return CPR >= 16 ? r % CPR : (r / (16 / CPR)) % CPR;
}

// STAGED: the tile (the gate/up product's bf16 intermediate, or bf16 slot
// rows) leaves through LDS, which must hold it.
template <int BM, int BN, int WTM, int WTN, int MODE, bool STAGED>
__device__ __forceinline__ void tile_epilogue(const GemmArgs& args,
                                              f32x16_t (&acc)[WTN / 32][WTM / 32], int64_t m0,
                                              int ntile, int e, int wm, int wn, int lane,
                                              int split, char* lds) {
  constexpr int TM = WTM / 32;
  constexpr int TN = WTN / 32;
  const int csub = 4 * (lane >> 5);
  if (MODE == kGateUpSilu) {
    uint16_t* act = reinterpret_cast<uint16_t*>(args.out);
    const int64_t n0g = (int64_t)ntile * (BN / 2);
    // the tile's intermediate: BM rows x BN/2 bf16 columns; with STAGED it
    // leaves through LDS (see the bf16 slot rows below)
    constexpr int CPRO = BN / 16;  // 16-byte chunks per staged row
    if constexpr (STAGED) {
      // every load of this wave has landed (the last step issues one stage
      // past the end, whose zeros go to the ring the tile is staged in) and
      // every wave is done with the last stage
      wait_vmcnt<0>();
      __syncthreads();
    }
    // v: columns col + 8j .. col + 8j + 3 of token row r (tile row tm*32 +
    // (lane & 31) of the wave, sub-tile tn)
    auto emit = [&](int64_t r, int64_t col, int tm, int tn, int j, uint2 v) {
      if constexpr (STAGED) {
        const int rl = wm * WTM + tm * 32 + (lane & 31);
        const int c = (wn * (WTN / 2) + tn * 32) / 8 + j;
        *reinterpret_cast<uint2*>(lds + rl * (BN / 2 * 2) + ((c ^ stage_swz<CPRO>(rl)) << 4) +
                                  (lane >> 5) * 8) = v;
      } else {
        *reinterpret_cast<uint2*>(act + r * args.n_out + col + 8 * j) = v;
      }
    };
    if (args.act == kActSilu && args.bias == nullptr) {
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
            emit(r, col, tm, tn, j, v);
          }
        }
      }
    } else {  // activation variant and/or gate/up bias
      const float* b1 = args.bias ? args.bias + (int64_t)e * 2 * args.inter : nullptr;
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
            float a[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              float gv = g[4 * j + q], uv = u[4 * j + q];
              if (b1) {
                gv += b1[col + 8 * j + q];
                uv += b1[args.inter + col + 8 * j + q];
              }
              a[q] = gated_act(gv, uv, args.act, args.alpha, args.limit);
            }
            uint2 v;
            v.x = pack_bf16x2(a[0], a[1]);
            v.y = pack_bf16x2(a[2], a[3]);
            emit(r, col, tm, tn, j, v);
          }
        }
      }
    }
    if constexpr (STAGED) {
      // every staged row leaves in 16-byte stores by consecutive lanes (pad
      // rows included: their zeros are part of the intermediate)
      constexpr int RPI = 64 / CPRO;
      constexpr int NWE = (BM / WTM) * (BN / WTN);
      constexpr int ITERS = BM / RPI / NWE;
      static_assert(64 % CPRO == 0 && (BM / RPI) % NWE == 0, "staged rows");
      const int wave = wn * (BM / WTM) + wm;
      const int cl = lane % CPRO;
      __syncthreads();
#pragma unroll
      for (int it = 0; it < ITERS; ++it) {
        const int r = (wave + it * NWE) * RPI + lane / CPRO;
        const uint4 v = *reinterpret_cast<const uint4*>(lds + r * (BN / 2 * 2) +
                                                        ((cl ^ stage_swz<CPRO>(r)) << 4));
        *reinterpret_cast<uint4*>(act + (m0 + r) * args.n_out + n0g + cl * 8) = v;
      }
    }
  } else if (MODE == kDownSlotBf16 && !STAGED) {
    // bf16 slot rows stored straight from the accumulators, 8 bytes per lane
    uint16_t* dst = reinterpret_cast<uint16_t*>(args.out);
    int32_t fr[TM];  // slot of each row, all looked up before the stores
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) fr[tm] = args.sorted[m0 + wm * WTM + tm * 32 + (lane & 31)];
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) {
      const int32_t f = fr[tm];
      if (f < 0) continue;
#pragma unroll
      for (int tn = 0; tn < TN; ++tn) {
        const int64_t col = (int64_t)ntile * BN + wn * WTN + tn * 32 + csub;
        if (col >= args.n_out) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const f32x16_t& a = acc[tn][tm];
          uint2 v;
          v.x = pack_bf16x2(a[4 * j], a[4 * j + 1]);
          v.y = pack_bf16x2(a[4 * j + 2], a[4 * j + 3]);
          *reinterpret_cast<uint2*>(dst + (int64_t)f * args.n_out + col + 8 * j) = v;
        }
      }
    }
  } else if (MODE == kDownSlotBf16) {
    // bf16 slot rows through LDS (free once every wave has read the last
    // stage): each lane writes its 4-column groups, then every staged row
    // leaves in 16-byte stores by consecutive lanes, so each line of a slot
    // row is written once and a tile takes half the store instructions of
    // 8-byte stores straight from the accumulators. The 16-byte chunks of a
    // staged row are XOR-permuted by the row, so the 32 rows one write
    // instruction covers spread over the banks.
    constexpr int CPRO = BN / 8;    // 16-byte chunks per staged row
    constexpr int RPI = 64 / CPRO;  // staged rows per store instruction
    constexpr int NWE = (BM / WTM) * (BN / WTN);
    constexpr int ITERS = BM / RPI / NWE;
    static_assert(64 % CPRO == 0 && (BM / RPI) % NWE == 0, "staged output rows");
    const int wave = wn * (BM / WTM) + wm;
    wait_vmcnt<0>();  // (as above: the past-the-end stage's zeros have landed)
    __syncthreads();
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) {
      const int r = wm * WTM + tm * 32 + (lane & 31);
#pragma unroll
      for (int tn = 0; tn < TN; ++tn) {
        const f32x16_t& a = acc[tn][tm];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int c = (wn * WTN + tn * 32) / 8 + j;  // chunk of columns 8j .. 8j+7
          uint2 v;
          v.x = pack_bf16x2(a[4 * j], a[4 * j + 1]);
          v.y = pack_bf16x2(a[4 * j + 2], a[4 * j + 3]);
          *reinterpret_cast<uint2*>(lds + r * (BN * 2) + ((c ^ stage_swz<CPRO>(r)) << 4) +
                                    (lane >> 5) * 8) = v;
        }
      }
    }
    __syncthreads();
    uint16_t* dst = reinterpret_cast<uint16_t*>(args.out);
    const int64_t n0 = (int64_t)ntile * BN;
    const int cl = lane % CPRO;
    const bool col_ok = n0 + cl * 8 < args.n_out;
    int32_t fr[ITERS];  // every slot lookup before the first store
#pragma unroll
    for (int it = 0; it < ITERS; ++it)
      fr[it] = args.sorted[m0 + (wave + it * NWE) * RPI + lane / CPRO];
#pragma unroll
    for (int it = 0; it < ITERS; ++it) {
      const int r = (wave + it * NWE) * RPI + lane / CPRO;
      const uint4 v =
          *reinterpret_cast<const uint4*>(lds + r * (BN * 2) + ((cl ^ stage_swz<CPRO>(r)) << 4));
      if (fr[it] >= 0 && col_ok)
        *reinterpret_cast<uint4*>(dst + (int64_t)fr[it] * args.n_out + n0 + cl * 8) = v;
    }
  } else {
    float* dst = reinterpret_cast<float*>(args.out) + (int64_t)split * args.part_stride;
    int32_t fr[TM];  // slot of each row, all looked up before the stores
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) fr[tm] = args.sorted[m0 + wm * WTM + tm * 32 + (lane & 31)];
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) {
      const int32_t f = fr[tm];
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
          } else if (args.bias == nullptr) {
#pragma unroll
            for (int i = 0; i < 4; ++i) unsafeAtomicAdd(p + i, wgt * a[4 * j + i]);
          } else {  // w * (y + b2[e]), the weight applied to the biased output
            const float* b2 = args.bias + (int64_t)e * args.n_out + col + 8 * j;
#pragma unroll
            for (int i = 0; i < 4; ++i) unsafeAtomicAdd(p + i, wgt * (a[4 * j + i] + b2[i]));
          }
        }
      }
    }
  }
}

template <int BM, int BN, int BK, int WGM, int WGN, int NS, int MODE, bool Q>
__global__ __launch_bounds__(64 * WGM * WGN) void grouped_gemm(GemmArgs args) {
  constexpr int NW = WGM * WGN;
  constexpr int WTM = BM / WGM;  // token rows per wave
  constexpr int WTN = BN / WGN;  // weight rows per wave
  constexpr int TM = WTM / 32;
  constexpr int TN = WTN / 32;
  constexpr int ROWB = BK * 2;            // bytes per staged token row
  constexpr int ROWW = Q ? BK : BK * 2;   // bytes per staged weight row (fp8 or bf16)
  constexpr int CPR = ROWB / 16;          // 16-byte chunks per staged row
  constexpr int CPW = ROWW / 16;
  constexpr int RPL = 1024 / ROWB;        // staged rows per 1 KB wave load
  constexpr int RPW = 1024 / ROWW;
  constexpr int LA = BM / (RPL * NW);     // 1 KB token-row loads per wave per stage
  constexpr int LB = BN / (RPW * NW);     // 1 KB weight-row loads per wave per stage
  static_assert(BK == 32 || BK == 64, "BK");
  static_assert(!Q || BK == 64, "fp8 weights are staged 64 codes per row");
  constexpr int A_BYTES = BM * ROWB;
  constexpr int STAGE = BM * ROWB + BN * ROWW;
  static_assert(LA >= 1 && LB >= 1 && TM >= 1 && TN >= 1, "tile too small");
  static_assert(MODE != kGateUpSilu || (TN % 2 == 0), "gate/up pairing needs even TN");
  static_assert(NS >= 2, "at least two stages");

  __shared__ __attribute__((aligned(1024))) char smem[NS * STAGE];
  // fp8 weights: the tile's per-block scales in dynamic LDS, [BN][nqb | 1]
  // (odd row stride: 32 consecutive rows read at one block hit distinct
  // banks), plus the overhang of the last 64-word load
  extern __shared__ __attribute__((aligned(256))) float scl[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: LDS load bases in M0
  const int wm = wave % WGM;
  const int wn = wave / WGM;

  // Persistent: the grid holds what the chip keeps resident, and each
  // workgroup walks the virtual workgroup ids vb = blockIdx.x, blockIdx.x +
  // gridDim.x, ... (gridDim.x is a multiple of 8, so every step stays on the
  // same XCD). A tile's first loads are then issued while the previous tile's
  // stores drain, instead of after the workgroup slot is freed and
  // dispatched again. The barrier at the top keeps the previous tile's last
  // LDS reads ahead of the next tile's loads.
  // the routing's live row tiles: fixed for the launch, read once
  const int live_m = min(args.num_tiles[0], args.max_tiles);
  for (int vb = blockIdx.x; vb < args.nvb; vb += gridDim.x) {
    __syncthreads();

    // XCD-aware tile order. Logical tiles are ordered in groups of GM row
    // tiles that sweep the weight tiles. Consecutive workgroup ids are dealt
    // round-robin to the 8 XCDs, so the workgroup in slot s of XCD x takes
    // tile w*8S + x*S + s%S of window w = s/S, S being the workgroups one XCD
    // holds at once: the XCDs work through the same window of 8S tiles
    // together (one expert's weights and token rows, which the last-level
    // cache then serves to all of them), each on a contiguous run of S tiles
    // that share rows in its own L2. The last, partial window is shared out
    // evenly over the XCDs. Only the routing's live row tiles are numbered,
    // so the rounds are the live tiles' rounds.
    const int n_tiles = args.n_tiles;
    // the tile order: live_m row tiles x n_ord column tiles (in phase 2 the
    // phase-1 launch's, twice this launch's width); phase 1 keeps its whole
    // rounds when the rest fills at most half a round, phase 2 takes that rest
    const int n_ord = args.phase == 2 ? n_tiles / 2 : n_tiles;
    const int ord_tiles = live_m * n_ord;
    int whole = ord_tiles;
    if (args.phase != 0) {
      const int w = (ord_tiles / args.rounds_of) * args.rounds_of;
      if (2 * (ord_tiles - w) <= args.rounds_of) whole = w;
    }
    const int per_split = args.phase == 2 ? 2 * (ord_tiles - whole) : whole;
    const int total = per_split * args.ksplit;
    const int S = args.xcd_slots;
    const int slot = vb / 8;
    const int nfull = total / (8 * S);
    const int chunk = (total - nfull * 8 * S + 7) / 8;  // per XCD in the partial window
    const int pid = slot < nfull * S
                        ? (slot / S) * 8 * S + (vb % 8) * S + slot % S
                        : nfull * 8 * S + (vb % 8) * chunk + (slot - nfull * S);
    // the grid was sized for every row tile the routing could produce: slots
    // past the live tiles' share (which would repeat another XCD's) do nothing
    if (pid >= total || (slot >= nfull * S && slot - nfull * S >= chunk)) continue;
    const int split = pid / per_split;  // the contraction split is the slowest index
    const int tpid = pid - split * per_split;
    const int opid = args.phase == 2 ? whole + tpid / 2 : tpid;  // position in the tile order
    const int group = opid / (args.group_m * n_ord);
    const int first_m = group * args.group_m;
    const int gsize = min(live_m - first_m, args.group_m);
    const int within = opid - group * args.group_m * n_ord;
    const int mt = first_m + within % gsize;
    const int ntile = args.phase == 2 ? 2 * (within / gsize) + (tpid & 1) : within / gsize;
    const int e = args.tile_expert[mt];
    if ((uint32_t)e >= (uint32_t)args.n_experts) continue;
    const int64_t m0 = (int64_t)mt * BM;
    const int64_t kdim = args.kdim;

    // weight row (within the expert) of staged row n of this tile, or -1
    auto weight_row = [&](int n) -> int64_t {
      if (MODE == kGateUpSilu) {
        const int64_t n0g = (int64_t)ntile * (BN / 2);
        return n < BN / 2 ? n0g + n : args.inter + n0g + (n - BN / 2);
      }
      const int64_t row = (int64_t)ntile * BN + n;
      return row < args.n_out ? row : -1;
    };

    // ---- per-lane load offsets (fixed over the K loop) ----
    // load j of this wave covers staged rows RPL*g .. RPL*g+RPL-1 (g = wave*L
    // + j); lane -> row RPL*g + lane/CPR, physical chunk lane%CPR, logical
    // chunk (lane%CPR) ^ swz(row): the XOR layout is applied on the global side.
    uint32_t aoff[LA], boff[LB];
    const uint16_t* a_base = MODE == kGateUpSilu ? args.a : args.a + m0 * kdim;
    const uint32_t a_num = MODE == kGateUpSilu ? args.a_bytes : (uint32_t)(BM * kdim * 2);
    const char* b_base =
        Q ? reinterpret_cast<const char*>(args.wq) + (int64_t)e * args.w_expert_stride
          : reinterpret_cast<const char*>(args.w + (int64_t)e * args.w_expert_stride);
    const uint32_t b_num = (uint32_t)(args.w_expert_stride * (Q ? 1 : 2));
    const __amdgpu_buffer_rsrc_t rsrc_a = make_rsrc(a_base, a_num);
    const __amdgpu_buffer_rsrc_t rsrc_b = make_rsrc(b_base, b_num);
    // token rows of the tile's slots: every lookup issued before the first
    // use, offsets computed without branches
    int32_t fsl[LA];
#pragma unroll
    for (int j = 0; j < LA; ++j)
      fsl[j] = MODE == kGateUpSilu ? args.sorted[m0 + RPL * (wave * LA + j) + lane / CPR] : 0;
#pragma unroll
    for (int j = 0; j < LA; ++j) {
      const int r = RPL * (wave * LA + j) + lane / CPR;
      const uint32_t cb = (uint32_t)(((lane % CPR) ^ swz<CPR>(r)) * 16);
      if (MODE == kGateUpSilu) {
        const int32_t f = fsl[j];
        const uint32_t t = (uint32_t)(f >= 0 ? f : 0) / (uint32_t)args.topk;
        aoff[j] = f >= 0 ? t * (uint32_t)(kdim * 2) + cb : kOutOfRange;
      } else {
        aoff[j] = (uint32_t)(r * kdim * 2) + cb;
      }
    }
#pragma unroll
    for (int j = 0; j < LB; ++j) {
      const int n = RPW * (wave * LB + j) + lane / CPW;
      const uint32_t cb = (uint32_t)(((lane % CPW) ^ swz<CPW>(n)) * 16);
      const int64_t row = weight_row(n);
      boff[j] = row >= 0 ? (uint32_t)(row * kdim * (Q ? 1 : 2)) + cb : kOutOfRange;
    }

    // fp8 weights: the tile's scales go to LDS ahead of stage 0's loads (and
    // so have landed once stage 0 has: loads complete in issue order)
    int sst = 1;
    if constexpr (Q) {
      const int nqb = args.nqb;
      sst = nqb | 1;
      const int64_t rows_pe = args.w_expert_stride / kdim;
      const __amdgpu_buffer_rsrc_t rsrc_s =
          make_rsrc(args.wscale + (int64_t)e * rows_pe * nqb, (uint32_t)(rows_pe * nqb * 4));
      for (int p0 = wave * 64; p0 < BN * sst; p0 += NW * 64) {
        const int p = p0 + lane;
        const int n = p / sst, b = p - n * sst;
        const int64_t row = n < BN ? weight_row(n) : -1;
        const uint32_t off = (row >= 0 && b < nqb) ? (uint32_t)((row * nqb + b) * 4) : kOutOfRange;
        load_lds_b32(rsrc_s, reinterpret_cast<const char*>(scl) + p0 * 4, off);
      }
    }

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

    f32x16_t acc[TN][TM];
#pragma unroll
    for (int a = 0; a < TN; ++a)
#pragma unroll
      for (int b = 0; b < TM; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.0f;

    const int nk = (int)(kdim / BK) / args.ksplit;  // stages of this split
    const int kt0 = split * nk;                     // its first stage

    // Loads of stage kt into LDS buffer `buf`; stages past the last one read
    // out of range (nothing is fetched, the buffer, which is not read again,
    // receives zeros), so the issue needs no branch.
#define MOE_ISSUE_STAGE(buf, kt)                                                              \
    do {                                                                                        \
      const bool live_ = (kt) < nk;                                                             \
      const uint32_t sa_ = live_ ? (uint32_t)(kt0 + (kt)) * ROWB : kOutOfRange;                 \
      const uint32_t sw_ = live_ ? (uint32_t)(kt0 + (kt)) * ROWW : kOutOfRange;                 \
      const char* sb_ = smem + (buf) * STAGE;                                                   \
      _Pragma("unroll") for (int j = 0; j < LA; ++j)                                           \
          load_lds_b128(rsrc_a, sb_ + (wave * LA + j) * 1024, aoff[j], sa_);                    \
      _Pragma("unroll") for (int j = 0; j < LB; ++j)                                           \
          load_lds_b128(rsrc_b, sb_ + A_BYTES + (wave * LB + j) * 1024, boff[j], sw_);          \
    } while (0)

    // Fragment reads of sub-step kk of stage kt (in LDS buffer `buf`); the
    // lane holds 8 k values of its row. bf16 weights: chunk 2*kk + lane/32 of
    // both 128-byte rows. fp8 weights: one 16-byte chunk of a 64-byte weight
    // row holds 8 codes for each of two sub-steps, so sub-steps 2j and 2j+1
    // take the two halves of chunk 2j + lane/32, and the token fragment reads
    // the matching k values (a fixed permutation of k inside the stage, the
    // same on both operands). Both chunks of a stage are read with its first
    // sub-step; each sub-step's codes are widened, as bf16(fp32(code) * scale),
    // after the matrix ops of the sub-step before it have been issued, so the
    // conversion overlaps them.
    uint32_t qraw[Q ? 2 : 1][Q ? TN : 1][4];
    float qsc[Q ? TN : 1];
#define MOE_LOAD_FRAGS(F, buf, kk, ktv)                                                        \
    do {                                                                                         \
      const char* sa_ = smem + (buf) * STAGE;                                                    \
      const char* sw_ = sa_ + A_BYTES;                                                           \
      const int h_ = lane >> 5;                                                                  \
      const int c_ = Q ? 4 * ((kk) / 2) + 2 * h_ + ((kk) % 2) : (kk) * 2 + h_;                   \
      _Pragma("unroll") for (int tm = 0; tm < TM; ++tm) {                                        \
        const int r = wm * WTM + tm * 32 + (lane & 31);                                          \
        F##b[tm] = *reinterpret_cast<const bf16x8_t*>(sa_ + r * ROWB + ((c_ ^ swz<CPR>(r)) << 4)); \
      }                                                                                          \
      if constexpr (!Q) {                                                                        \
        _Pragma("unroll") for (int tn = 0; tn < TN; ++tn) {                                      \
          const int r = nrow[tn] + (lane & 31);                                                  \
          F##a[tn] =                                                                           \
              *reinterpret_cast<const bf16x8_t*>(sw_ + r * ROWW + ((c_ ^ swz<CPW>(r)) << 4));  \
        }                                                                                        \
      } else if ((kk) == 0) {                                                                    \
        const int qb_ = (kt0 + (ktv)) * BK / args.qblock;                                        \
        _Pragma("unroll") for (int tn = 0; tn < TN; ++tn) {                                      \
          const int r = nrow[tn] + (lane & 31);                                                  \
          qsc[tn] = scl[r * sst + qb_];                                                          \
          _Pragma("unroll") for (int pr = 0; pr < 2; ++pr) {                                     \
            const u32x4_t v_ = *reinterpret_cast<const u32x4_t*>(                                \
                sw_ + r * ROWW + (((2 * pr + h_) ^ swz<CPW>(r)) << 4));                          \
            qraw[pr][tn][0] = v_[0];                                                             \
            qraw[pr][tn][1] = v_[1];                                                             \
            qraw[pr][tn][2] = v_[2];                                                             \
            qraw[pr][tn][3] = v_[3];                                                             \
          }                                                                                      \
        }                                                                                        \
      }                                                                                          \
    } while (0)
    // fp8 weights: widen the codes of sub-step kk into F##a
#define MOE_WIDEN(F, kk)                                                                       \
    do {                                                                                         \
      if constexpr (Q) {                                                                         \
        _Pragma("unroll") for (int tn = 0; tn < TN; ++tn)                                        \
            F##a[tn] = fp8x8_to_bf16(qraw[(kk) / 2][tn][2 * ((kk) % 2)],                         \
                                     qraw[(kk) / 2][tn][2 * ((kk) % 2) + 1], qsc[tn]);           \
      }                                                                                          \
    } while (0)

    constexpr int KK = BK / 16;  // matrix-core sub-steps per stage (even)
    static_assert(KK % 2 == 0, "fragment double buffer alternates per sub-step");
    static_assert(NS == 2 || NS == 4, "two- or four-stage ring");
    static_assert(!Q || NS == 2, "fp8 weights: two-stage ring");
    // Matrix ops of a stage's last sub-step issued ahead of the stage
    // boundary: a quarter of them in the bf16 gate/up product with 256-row
    // tiles (measured 3-4 % faster there); elsewhere none (equal or slower).
    constexpr int PRE = (Q || MODE != kGateUpSilu || BM != 256) ? 0 : TM * TN / 4;

    // matrix ops [first, first + count) of one sub-step (op i: weight sub-tile
    // i / TM, token sub-tile i % TM)
#define MOE_MMA(F, first, count)                                                               \
    do {                                                                                         \
      _Pragma("unroll") for (int i_ = 0; i_ < TM * TN; ++i_) {                                   \
        if (i_ >= (first) && i_ < (first) + (count)) {                                           \
          const int tn_ = i_ / TM, tm_ = i_ % TM;                                                \
          acc[tn_][tm_] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(F##a[tn_], F##b[tm_],         \
                                                                  acc[tn_][tm_], 0, 0, 0);       \
        }                                                                                        \
      }                                                                                          \
    } while (0)
    // sub-steps 0 .. KK-2 of stage kt: the fragments of the next sub-step are
    // read (and fp8 codes widened) around this sub-step's matrix ops
#define MOE_SUBSTEPS(buf, kt)                                                                  \
    do {                                                                                         \
      _Pragma("unroll") for (int kk = 0; kk + 1 < KK; ++kk) {                                    \
        if (kk % 2 == 0) {                                                                       \
          MOE_LOAD_FRAGS(f1, buf, kk + 1, kt);                                                   \
          MOE_MMA(f0, 0, TM * TN);                                                               \
          MOE_WIDEN(f1, kk + 1);                                                                 \
        } else {                                                                                 \
          MOE_LOAD_FRAGS(f0, buf, kk + 1, kt);                                                   \
          MOE_MMA(f1, 0, TM * TN);                                                               \
          MOE_WIDEN(f0, kk + 1);                                                                 \
        }                                                                                        \
      }                                                                                          \
    } while (0)

    // prologue: stages 0 .. NS-1 in flight (one per buffer; missing stages
    // read out of range), stage 0 landed, its first fragments read
#pragma unroll
    for (int s0 = 0; s0 < NS; ++s0) MOE_ISSUE_STAGE(s0, s0);
    wait_vmcnt<(NS - 1) * (LA + LB)>();
    ring_barrier();  // no fence: the later stages stay in flight
    bf16x8_t f0a[TN], f0b[TM], f1a[TN], f1b[TM];
    MOE_LOAD_FRAGS(f0, 0, 0, 0);
    MOE_WIDEN(f0, 0);

    // Every stage but the last. Its last sub-step's fragments are already in
    // registers, so the stage boundary is interleaved with that sub-step's
    // matrix ops: the first PRE of them, then the wait (stage kt+1 landed;
    // with four buffers stages kt+2 and kt+3 stay in flight) and the barrier
    // (every wave is done reading stage kt), then the loads of stage kt+NS
    // into the buffer stage kt leaves (issued first: they have the longest way
    // to go), the reads of stage kt+1's first fragments, then the rest of the
    // matrix ops. The last stage is peeled off, so the loop body has no branch
    // (with one, the accumulators are copied between register files around
    // it).
    for (int kt = 0; kt + 1 < nk; ++kt) {
      const int buf = kt & (NS - 1);
      MOE_SUBSTEPS(buf, kt);
      MOE_MMA(f1, 0, PRE);
      if constexpr (NS == 2) {
        wait_vmcnt<0>();
        __syncthreads();
      } else {
        wait_vmcnt<(NS - 2) * (LA + LB)>();
        ring_barrier();
      }
      MOE_ISSUE_STAGE(buf, kt + NS);
      MOE_LOAD_FRAGS(f0, (kt + 1) & (NS - 1), 0, kt + 1);
      MOE_MMA(f1, PRE, TM * TN - PRE);
      MOE_WIDEN(f0, 0);
    }
    MOE_SUBSTEPS((nk - 1) & (NS - 1), nk - 1);
    MOE_MMA(f1, 0, TM * TN);
#undef MOE_SUBSTEPS
#undef MOE_MMA
#undef MOE_WIDEN
#undef MOE_LOAD_FRAGS
#undef MOE_ISSUE_STAGE

    // bf16 intermediates and bf16 slot rows leave through the ring's LDS
    // where the tile fits it (the intermediate always does; with FP8 weights
    // the gate/up kernel keeps direct stores: staging there spills)
    constexpr bool kStaged = (MODE == kGateUpSilu && !Q && BM * BN <= NS * STAGE) ||
                             (MODE == kDownSlotBf16 && BM * BN * 2 <= NS * STAGE);
    tile_epilogue<BM, BN, WTM, WTN, MODE, kStaged>(args, acc, m0, ntile, e, wm, wn, lane, split,
                                                   smem);
  }  // persistent tile loop
}

template <int BM, int BN, int BK, int WGM, int WGN, int NS, int MODE, bool Q>
hipError_t launch_cfg(GemmArgs a, hipStream_t stream) {
  if (a.ksplit < 1) a.ksplit = 1;
  // phase 2: at most two halves of each tile short of a round
  const int64_t total =
      a.phase == 2 ? 2 * (int64_t)a.rounds_of : (int64_t)a.max_tiles * a.n_tiles * a.ksplit;
  if (total == 0) return hipSuccess;
  const size_t scl_bytes = Q ? ((size_t)BN * (a.nqb | 1) + 64) * sizeof(float) : 0;
  // workgroups one CU holds at once (LDS-bound: 160 KB per CU), 32 CUs per XCD;
  // the column halves of a tail go one to a CU
  constexpr size_t kStageBytes = (size_t)BM * BK * 2 + (size_t)BN * BK * (Q ? 1 : 2);
  const int64_t per_cu =
      a.phase == 2 ? 1 : (int64_t)((160 * 1024) / (NS * kStageBytes + scl_bytes));
  a.xcd_slots = (int32_t)(32 * (per_cu < 1 ? 1 : per_cu));
  const int64_t S = a.xcd_slots, nfull = total / (8 * S);
  const int64_t blocks = 8 * (nfull * S + (total - nfull * 8 * S + 7) / 8);
  // virtual workgroups: the tile order's grid; launched: what one round of
  // the chip holds (both multiples of 8)
  a.nvb = (int32_t)blocks;
  const int64_t grid = blocks < 8 * S ? blocks : 8 * S;
  grouped_gemm<BM, BN, BK, WGM, WGN, NS, MODE, Q>
      <<<dim3((unsigned)grid), dim3(64 * WGM * WGN), scl_bytes, stream>>>(a);
  return hipGetLastError();
}

template <int MODE, bool Q>
hipError_t dispatch(GemmCfg cfg, GemmArgs a, hipStream_t stream) {
  a.group_m = 8;
  // (token rows, weight rows, waves): the variants kept after sweeping tile
  // shape, pipeline depth and wave layout on the workloads' shapes
  if constexpr (!Q) {
    // four-stage rings for launches of at most one tile per CU (a stage's
    // latency is then not covered by other workgroups' work)
    if (cfg.ns == 4) {
      if (cfg.bm == 64 && cfg.bn == 256) return launch_cfg<64, 256, 64, 1, 4, 4, MODE, Q>(a, stream);
      if (cfg.bm == 64 && cfg.bn == 128) return launch_cfg<64, 128, 64, 2, 2, 4, MODE, Q>(a, stream);
      if (cfg.bm == 128 && cfg.bn == 128) return launch_cfg<128, 128, 64, 2, 2, 4, MODE, Q>(a, stream);
    }
  }
  if (cfg.bm == 64 && cfg.bn == 256) return launch_cfg<64, 256, 64, 1, 4, 2, MODE, Q>(a, stream);
  if (cfg.bm == 64 && cfg.bn == 128) return launch_cfg<64, 128, 64, 2, 2, 2, MODE, Q>(a, stream);
  if (cfg.bm == 128 && cfg.bn == 128) return launch_cfg<128, 128, 64, 2, 2, 2, MODE, Q>(a, stream);
  if (cfg.bm == 192 && cfg.bn == 256) return launch_cfg<192, 256, 64, 2, 4, 2, MODE, Q>(a, stream);
  if (cfg.bm == 256 && cfg.bn == 256) return launch_cfg<256, 256, 64, 2, 4, 2, MODE, Q>(a, stream);
  if constexpr (MODE != kGateUpSilu && !Q) {
    // column halves of the down projection's tail: the 192x256 and 256x256
    // tiles' per-wave shapes on four waves (one workgroup per CU; the
    // 192-row halves hold a four-stage ring in the CU's 160 KB of LDS)
    if (cfg.ns == 4 && cfg.bm == 192 && cfg.bn == 128)
      return launch_cfg<192, 128, 64, 2, 2, 4, MODE, Q>(a, stream);
    if (cfg.bm == 192 && cfg.bn == 128) return launch_cfg<192, 128, 64, 2, 2, 2, MODE, Q>(a, stream);
    if (cfg.bm == 256 && cfg.bn == 128) return launch_cfg<256, 128, 64, 2, 2, 2, MODE, Q>(a, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace

// Tile choice from a cost model of the two grouped products.
//
// Expected row tiles: with K distinct experts drawn per token, an expert's
// row count is binomial (mean T*K/E, variance T*(K/E)*(1-K/E)); the expected
// number of BM-row tiles it needs is averaged over five points of the
// normal approximation. A product's time is then taken as (tiles per CU) x
// (flops per tile) / (relative tile efficiency). Tiles that share a CU
// (64x128 three to a CU, 64x256 and 128x128 two) overlap their tail rounds,
// so the count stays fractional; 192x256 and 256x256 tiles fill a CU alone,
// so they are rounded up to whole rounds. The down-projection term uses the
// tile that product runs (64x256 on the 64-row layout).
//
// The efficiencies (64x256 0.91, 128x128 1, 256x256 1.23) were fitted to
// measured times of those three configurations on every shape of the
// atrex-bench shapes table; against the fastest configuration per shape the
// model gives up at most 1-2 %, except at T=4195 with E=128, I=768, where
// 128x128 is 3 % faster than its 64x256. 192x256 (0.9 the padding of
// 256-row tiles on ~1050-row experts, and exactly three rounds for the
// prefill shape) takes 1.15: with it the model picks 192x256 where it
// measured fastest (T=4195 and T=4098 with E=8, T=2400 with E=128: 12-19 %
// less than the previous pick) and keeps 256x256 where that stays ahead
// (T >= 8192 with E=128, the large E=8 shapes). 64x128 gate/up tiles take
// 0.925, between the 0.91 that T=520 and T=668 need and the 0.938 above
// which they would displace 128x128 at T=277 (14 % faster there), and are a
// candidate only while they fit one round: picked at T=135 and T=668 with
// E=8 (81 -> 76 and 111 -> 105-110 us per call) and T=520 with E=128 (-2 %).
namespace {
double expected_row_tiles(int64_t T, int64_t K, int64_t E, int bm) {
  const int64_t n = T * K;
  const double live = (double)(n < E ? n : E);
  const double mean = (double)n / live;
  const double p = (double)K / (double)E;
  const double sd = sqrt((double)T * p * (1.0 - p));
  const double z[5] = {-2.0, -1.0, 0.0, 1.0, 2.0};
  const double w[5] = {0.054, 0.242, 0.399, 0.242, 0.054};
  double acc = 0.0, wsum = 0.0;
  for (int i = 0; i < 5; ++i) {
    const double rows = fmax(1.0, mean + z[i] * sd);
    acc += w[i] * ceil(rows / bm);
    wsum += w[i];
  }
  return live * acc / wsum;
}

double tile_eff(GemmCfg c) {
  if (c.bm == 64) return c.bn == 128 ? 0.925 : 0.91;
  return c.bm == 128 ? 1.0 : c.bm == 192 ? 1.15 : 1.23;
}

// c: the gate/up tile; the down projection runs pick_gemm2_cfg's tile on the
// same row layout.
double model_cost(int64_t T, int64_t K, int64_t H, int64_t I, int64_t E, GemmCfg c) {
  const double rt = expected_row_tiles(T, K, E, c.bm);
  const GemmCfg c2 = pick_gemm2_cfg(T * K, H, I, E, c.bm);
  const GemmCfg cg[2] = {c, c2};
  const double prod[2][2] = {{(double)H, (double)(2 * I / c.bn)},                   // gate/up
                             {(double)I, (double)((H + c2.bn - 1) / c2.bn)}};  // down
  double t = 0.0;
  for (int g = 0; g < 2; ++g) {
    const double per_cu = rt * prod[g][1] / 256.0;
    const double rounds = cg[g].bm >= 192 ? fmax(1.0, ceil(per_cu - 0.02)) : fmax(1.0, per_cu);
    t += rounds * (double)cg[g].bm * cg[g].bn * prod[g][0] * 2.0 / tile_eff(cg[g]);
  }
  return t;
}
}  // namespace

// A four-stage ring where a launch expects at most one tile per CU: with no
// other workgroup's work to cover a stage's latency, each tile then keeps
// three stages in flight instead of one. For the 64- and 128-row tiles,
// whose four stages fit a CU's LDS.
int pick_ring_stages(GemmCfg cfg, int64_t T, int64_t K, int64_t E, int64_t n_tiles) {
  const bool fits =
      (cfg.bm == 64 && (cfg.bn == 128 || cfg.bn == 256)) || (cfg.bm == 128 && cfg.bn == 128);
  return fits && expected_row_tiles(T, K, E, cfg.bm) * (double)n_tiles <= 256.0 ? 4 : 2;
}

GemmCfg pick_gemm1_cfg(int64_t T, int64_t K, int64_t H, int64_t I, int64_t E) {
  const GemmCfg cands[5] = {{64, 128}, {64, 256}, {128, 128}, {192, 256}, {256, 256}};
  GemmCfg best = cands[2];
  double best_t = model_cost(T, K, H, I, E, best);
  for (const GemmCfg& c : cands) {
    // 64x128 gate/up tiles (three workgroups per CU) only while all of them
    // fit one round of the chip: beyond it they measured 6-14 % slower than
    // 64x256 (E=128: T=1019, 2044; T=4195 with I=768)
    if (c.bn == 128 && c.bm == 64 && expected_row_tiles(T, K, E, 64) * (2 * I / 128) > 3 * 256)
      continue;
    const double t = model_cost(T, K, H, I, E, c);
    if (t < best_t) {
      best = c;
      best_t = t;
    }
  }
  best.ns = pick_ring_stages(best, T, K, E, I / (best.bn / 2));
  return best;
}

// Split of the down projection's contraction for problems whose tiles
// cannot fill the chip (few tokens per expert: at T = 135, E = 8, top-2 its
// 128 tiles would occupy a quarter of the workgroup slots, each a chain of
// 32 dependent stages). Splitting it in two gives twice the tiles, each
// with half the chain; the combine adds the two partial rows in a fixed
// order (deterministic). Taken while the doubled tile count stays within the
// workgroups the chip holds at once and each half keeps at least 4 stages.
// Measured with the weights streamed from HBM, 128-row tiles: T = 135
// 32.1 -> 22.9 us, T = 277 33.6 -> 25.9 us; four parts measured slower
// (26.2, 30.5 us). The gate/up projection is not split: with an extra pass
// for the activation it measured no faster.
int pick_ksplit(GemmCfg cfg, int64_t T, int64_t K, int64_t E, int64_t n_tiles, int64_t kdim) {
  const int64_t per_cu = cfg.bm >= 192 ? 1 : 2;  // LDS-bound residency of the tile shapes
  const double slots = 256.0 * per_cu;
  const double tiles = expected_row_tiles(T, K, E, cfg.bm) * (double)n_tiles;
  const int64_t nk = kdim / 64;
  return (tiles * 2 <= slots && nk % 2 == 0 && nk / 2 >= 4) ? 2 : 1;
}

// Whether the down projection runs its last partial round as column halves
// (a second launch): 192- and 256-row tiles fill a CU alone, so R whole
// rounds plus a fraction f of one take R + 1 tile times; with f <= 1/2 the
// leftover tiles split into at most one round of half-width tiles, about
// R + 1/2 (measured efficiency of the halves aside). Each output element
// still sums its whole contraction in the same order: the results are the
// same bits. The kernels decide again from the routing's own tile count.
// n_rows: the weight rows per expert (H); kdim: the contraction (I). Only for
// contractions of at least 16 stages: with fewer, a half-width tile pays a
// whole tile's prologue and epilogue for half the work (measured slower on
// the E=128, I=384 and I=768 rows). The same split of the gate/up product
// measured slower on the E=128, I=768 rows and is not offered.
// The tile count is estimated here as sum_j P(rows > j*bm) per expert under
// the normal approximation of the binomial row count (the cost model's five
// points misplace experts whose mean sits on a tile boundary, as at T=8192,
// E=128: 512 rows per expert on 256-row tiles); if the routing's own count
// leaves more than half a round, the kernels run it whole and the second
// launch has nothing to do.
bool pick_tail_split(GemmCfg cfg, int64_t T, int64_t K, int64_t E, int64_t n_rows,
                     int64_t kdim, int64_t max_tiles) {
  if (cfg.bm < 192 || cfg.bn != 256 || n_rows % 256 != 0 || kdim < 16 * 64) return false;
  const int64_t n_tiles = n_rows / 256;
  if (max_tiles * n_tiles < kRound) return false;  // one launch never fills a round
  const int64_t n = T * K;
  const double live = (double)(n < E ? n : E);
  const double mean = (double)n / live;
  const double p = (double)K / (double)E;
  const double sd = fmax(sqrt((double)T * p * (1.0 - p)), 1e-9);
  double per_expert = 0.0;  // E[ceil(rows / bm)] for rows >= 1
  for (int64_t j = 0; (double)j * cfg.bm < mean + 8.0 * sd; ++j)
    per_expert += j == 0 ? 1.0 : 0.5 * erfc(((double)j * cfg.bm + 0.5 - mean) / (sd * sqrt(2.0)));
  const double rounds = live * per_expert * (double)n_tiles / kRound;
  const double f = rounds - floor(rounds);  // (a few hundredths: whole rounds but for rare experts)
  return rounds >= 1.0 && f > 0.03 && f <= 0.5;
}

GemmCfg pick_gemm2_cfg(int64_t n_slots, int64_t H, int64_t I, int64_t E, int bm) {
  (void)n_slots;
  (void)H;
  (void)I;
  (void)E;
  if (bm == 256) return GemmCfg{256, 256};
  if (bm == 192) return GemmCfg{192, 256};
  if (bm == 128) return GemmCfg{128, 128};
  return GemmCfg{64, 256};
}

hipError_t launch_gemm1_silu(GemmCfg cfg, const uint16_t* hidden, const uint16_t* w1,
                             const int32_t* sorted, const int32_t* tile_expert,
                             const int32_t* num_tiles, int64_t T, int64_t H, int64_t I,
                             int64_t E, int64_t K, int64_t max_tiles, uint16_t* act,
                             const Epilogue& ep, hipStream_t stream) {
  GemmArgs a{};
  a.n_experts = (int32_t)E;
  a.ksplit = 1;
  a.act = ep.act;
  a.alpha = ep.alpha;
  a.limit = ep.limit;
  a.bias = ep.b1;
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
  a.a_bytes = (uint32_t)(T * H * 2);
  a.n_tiles = (int)(I / (cfg.bn / 2));
  return dispatch<kGateUpSilu, false>(cfg, a, stream);
}

hipError_t launch_gemm2(GemmCfg cfg, const uint16_t* act, const uint16_t* w2,
                        const int32_t* sorted, const int32_t* tile_expert,
                        const int32_t* num_tiles, const float* topk_weights, int64_t H,
                        int64_t I, int64_t E, int64_t K, int64_t max_tiles, float* y,
                        float* out, const float* b2, hipStream_t stream, int ksplit,
                        int64_t n_slots, uint16_t* y16, bool tail) {
  if (out && ksplit > 1) return hipErrorInvalidValue;  // atomic adds of partial sums
  if (y16 && (out || ksplit > 1)) return hipErrorInvalidValue;  // whole rows, rounded once
  GemmArgs a{};
  a.n_experts = (int32_t)E;
  a.ksplit = ksplit;
  a.part_stride = n_slots * H;
  a.bias = out ? b2 : nullptr;  // on the slot path the combine adds b2
  a.a = act;
  a.w = w2;
  a.sorted = sorted;
  a.tile_expert = tile_expert;
  a.num_tiles = num_tiles;
  a.topk_weights = topk_weights;
  a.out = out ? (void*)out : y16 ? (void*)y16 : (void*)y;
  a.kdim = I;
  a.n_out = H;
  a.w_expert_stride = H * I;
  a.inter = I;
  a.topk = (int32_t)K;
  a.max_tiles = (int32_t)max_tiles;
  a.n_tiles = (int)((H + cfg.bn - 1) / cfg.bn);
  auto run = [&](GemmCfg c, const GemmArgs& g) {
    if (out) return dispatch<kDownAtomic, false>(c, g, stream);
    if (y16) return dispatch<kDownSlotBf16, false>(c, g, stream);
    return dispatch<kDownSlot, false>(c, g, stream);
  };
  if (!tail || ksplit != 1 || cfg.bm < 192 || cfg.bn != 256 || H % 256 != 0 ||
      (int64_t)a.max_tiles * a.n_tiles < kRound)
    return run(cfg, a);
  // whole rounds of the chip (one 192- or 256-row tile per CU), then the
  // rest as column halves
  a.phase = 1;
  a.rounds_of = kRound;
  hipError_t st = run(cfg, a);
  if (st != hipSuccess) return st;
  a.phase = 2;
  a.n_tiles = (int)(H / 128);
  GemmCfg half{cfg.bm, 128};
  half.ns = cfg.bm == 192 ? 4 : 2;  // 4 x 40 KB stages fill the LDS; 256-row stages do not fit
  return run(half, a);
}

bool fp8_gemm_supported(int64_t H, int64_t I, int64_t block) {
  return block % 64 == 0 && H / block <= kMaxScaleBlocks && I / block <= kMaxScaleBlocks;
}

hipError_t launch_gemm1_silu_fp8(GemmCfg cfg, const uint16_t* hidden, const uint8_t* w1q,
                                 const float* w1s, int64_t block, const int32_t* sorted,
                                 const int32_t* tile_expert, const int32_t* num_tiles, int64_t T,
                                 int64_t H, int64_t I, int64_t E, int64_t K, int64_t max_tiles,
                                 uint16_t* act, const Epilogue& ep, hipStream_t stream) {
  if (!fp8_gemm_supported(H, I, block)) return hipErrorInvalidValue;
  GemmArgs a{};
  a.n_experts = (int32_t)E;
  a.ksplit = 1;
  a.act = ep.act;
  a.alpha = ep.alpha;
  a.limit = ep.limit;
  a.bias = ep.b1;
  a.a = hidden;
  a.wq = w1q;
  a.wscale = w1s;
  a.qblock = (int32_t)block;
  a.nqb = (int32_t)(H / block);
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
  a.a_bytes = (uint32_t)(T * H * 2);
  a.n_tiles = (int)(I / (cfg.bn / 2));
  return dispatch<kGateUpSilu, true>(cfg, a, stream);
}

hipError_t launch_gemm2_fp8(GemmCfg cfg, const uint16_t* act, const uint8_t* w2q,
                            const float* w2s, int64_t block, const int32_t* sorted,
                            const int32_t* tile_expert, const int32_t* num_tiles,
                            const float* topk_weights, int64_t H, int64_t I, int64_t E,
                            int64_t K, int64_t max_tiles, float* y, float* out, const float* b2,
                            hipStream_t stream, int ksplit, int64_t n_slots, uint16_t* y16) {
  if (!fp8_gemm_supported(H, I, block)) return hipErrorInvalidValue;
  if (out && ksplit > 1) return hipErrorInvalidValue;
  if (y16 && (out || ksplit > 1)) return hipErrorInvalidValue;
  GemmArgs a{};
  a.n_experts = (int32_t)E;
  a.ksplit = ksplit;
  a.part_stride = n_slots * H;
  a.bias = out ? b2 : nullptr;  // on the slot path the combine adds b2
  a.a = act;
  a.wq = w2q;
  a.wscale = w2s;
  a.qblock = (int32_t)block;
  a.nqb = (int32_t)(I / block);
  a.sorted = sorted;
  a.tile_expert = tile_expert;
  a.num_tiles = num_tiles;
  a.topk_weights = topk_weights;
  a.out = out ? (void*)out : y16 ? (void*)y16 : (void*)y;
  a.kdim = I;
  a.n_out = H;
  a.w_expert_stride = H * I;
  a.inter = I;
  a.topk = (int32_t)K;
  a.max_tiles = (int32_t)max_tiles;
  a.n_tiles = (int)((H + cfg.bn - 1) / cfg.bn);
  if (out) return dispatch<kDownAtomic, true>(cfg, a, stream);
  if (y16) return dispatch<kDownSlotBf16, true>(cfg, a, stream);
  return dispatch<kDownSlot, true>(cfg, a, stream);
}

}  // namespace moe
