// Small-batch path with each routed expert streamed once (a few tokens to a
// few hundred slots): where several slots of the batch chose the same
// expert, the per-slot weight streaming of the single-token kernels would
// read that expert's rows once per slot. Here the work is split by expert:
//
//   sb_gateup  workgroup (expert r-th present, 4 columns i): every wave
//              streams gate row i and up row I+i of the expert once, then
//              for each slot routed to the expert reads the slot's token
//              row and stores act[f, i] = bf16(silu(g) * u);
//   sb_down    workgroup (expert, 4*R output rows): each wave streams R rows
//              w2[e, h, :] once, then for each routed slot writes the
//              unscaled y[f, h] = w2[e, h, :] . act[f, :] (fp32);
//   combine    out[t, :] = sum over k, in order, of w[t,k] * y[t*K+k, :]
//              (the grouped path's deterministic combine, combine.hip).
//
// This is the small-batch regime the metrale forward_k2 dispatch serves
// (one expert weight stream feeding several rows) and the grouping that
// tpu-inference's start_a2a_scatter performs, without the padded layout:
// the slots of an expert are found per workgroup from an LDS bitmap of the
// experts present and an LDS list of the expert's slots. Dot products use
// the packed bf16 dot instruction (two products per lane per instruction,
// fp32 accumulation), so weights and token rows stay packed in registers.
#include "device_util.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kBitmapWords = kMaxExperts / 32;

// (the vector elements are copied to scalars first: a bit cast applied to a
// vector element expression itself reads element 0 whatever the index)
__device__ __forceinline__ float dot8(u32x4_t a, u32x4_t b, float acc) {
  const uint32_t a0 = a[0], a1 = a[1], a2 = a[2], a3 = a[3];
  const uint32_t b0 = b[0], b1 = b[1], b2 = b[2], b3 = b[3];
  acc = dot2(a0, b0, acc);
  acc = dot2(a1, b1, acc);
  acc = dot2(a2, b2, acc);
  return dot2(a3, b3, acc);
}

// Shared prologue: find the expert this workgroup serves (the r-th expert
// present among the n slot ids, in ascending expert id) and list its slots
// in LDS. Returns the expert, or -1 if fewer than r+1 experts are present.
// Slots with an id outside [0, E) belong to no expert.
__device__ __forceinline__ int32_t find_expert(const int32_t* __restrict__ ids, int32_t n,
                                               int32_t E, int32_t r, uint32_t* s_bits,
                                               int32_t* s_slots, int32_t* s_count) {
  for (int w = threadIdx.x; w < kBitmapWords; w += kThreads) s_bits[w] = 0;
  if (threadIdx.x == 0) *s_count = 0;
  __syncthreads();
  for (int32_t q = threadIdx.x; q < n; q += kThreads) {
    const int32_t e = ids[q];
    if (e >= 0 && e < E) atomicOr(&s_bits[e >> 5], 1u << (e & 31));
  }
  __syncthreads();
  // every thread walks the bitmap (E/32 words) to the r-th set bit
  int32_t expert = -1, seen = 0;
  for (int w = 0; w < (E + 31) / 32; ++w) {
    const uint32_t b = s_bits[w];
    const int c = __builtin_popcount(b);
    if (seen + c > r) {
      uint32_t m = b;
      for (int skip = r - seen; skip > 0; --skip) m &= m - 1;  // drop the lowest bits
      expert = w * 32 + __builtin_ctz(m);
      break;
    }
    seen += c;
  }
  if (expert < 0) return -1;
  for (int32_t q = threadIdx.x; q < n; q += kThreads)
    if (ids[q] == expert) s_slots[atomicAdd(s_count, 1)] = q;
  __syncthreads();
  return expert;
}

struct SbArgs {
  const uint16_t* hidden;
  const uint16_t* w1;
  const uint16_t* w2;
  const int32_t* topk_ids;
  uint16_t* act;  // bf16 [n, I]
  float* y;       // fp32 [n, H]
  int64_t H, I;
  int32_t E, K, n;
  Epilogue ep;  // activation variant and gate/up bias (b2 is the combine's)
};

// NC: 16-byte chunks per lane per gate/up row (H / 512 rounded up). WIDE:
// the batch averages 8+ slots per expert.
template <int NC, bool WIDE>
__global__ __launch_bounds__(kThreads) void sb_gateup(SbArgs a) {
  __shared__ uint32_t s_bits[kBitmapWords];
  __shared__ int32_t s_slots[kSmallBatchMaxSlots];
  __shared__ int32_t s_count;
  const int32_t e = find_expert(a.topk_ids, a.n, a.E, blockIdx.y, s_bits, s_slots, &s_count);
  if (e < 0) return;
  const int lane = threadIdx.x & 63;
  const int64_t i = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
  const int64_t H = a.H, I = a.I;
  if (i >= I) return;
  const int64_t nc = H / 8;
  const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.w1 + (int64_t)e * 2 * I * H), (short)0, (int)(2 * I * H * 2), 0x00020000);
  u32x4_t gv[NC], uv[NC];
#pragma unroll
  for (int j = 0; j < NC; ++j) {
    const int64_t c = lane + 64 * j;
    const bool ok = c < nc;
    gv[j] = __builtin_amdgcn_raw_buffer_load_b128(
        wr, ok ? (uint32_t)((i * H + c * 8) * 2) : kOutOfRange, 0, 0);
    uv[j] = __builtin_amdgcn_raw_buffer_load_b128(
        wr, ok ? (uint32_t)(((I + i) * H + c * 8) * 2) : kOutOfRange, 0, 0);
  }
  // token rows of SB slots are loaded together, so their latency overlaps;
  // with many slots per expert up to 16 chunks per lane, so that a batch pays
  // about one L2 round trip for its rows (with one or two, the extra rows
  // would be repeats)
  constexpr int SB = WIDE ? (NC >= 16 ? 1 : 16 / NC) : (NC <= 2 ? 4 : (NC <= 4 ? 2 : 1));
  const int32_t count = s_count;
  for (int32_t m0 = 0; m0 < count; m0 += SB) {
    u32x4_t xv[SB][NC];
#pragma unroll
    for (int b = 0; b < SB; ++b) {
      const int32_t m = m0 + b < count ? m0 + b : count - 1;  // a repeat, not stored
      const int64_t t = s_slots[m] / a.K;
      const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(a.hidden + t * H), (short)0, (int)(H * 2), 0x00020000);
#pragma unroll
      for (int j = 0; j < NC; ++j) {
        const int64_t c = lane + 64 * j;
        xv[b][j] = __builtin_amdgcn_raw_buffer_load_b128(
            xr, c < nc ? (uint32_t)(c * 16) : kOutOfRange, 0, 0);
      }
    }
    float g[SB], u[SB];
#pragma unroll
    for (int b = 0; b < SB; ++b) {
      g[b] = 0.f;
      u[b] = 0.f;
#pragma unroll
      for (int j = 0; j < NC; ++j) {
        g[b] = dot8(gv[j], xv[b][j], g[b]);
        u[b] = dot8(uv[j], xv[b][j], u[b]);
      }
    }
#pragma unroll
    for (int b = 0; b < SB; ++b) {  // independent reductions, interleaved
      g[b] = group_sum<64>(g[b]);
      u[b] = group_sum<64>(u[b]);
    }
#pragma unroll
    for (int b = 0; b < SB; ++b) {
      if (lane == 63 && m0 + b < count) {
        if (a.ep.b1) {
          g[b] += a.ep.b1[(int64_t)e * 2 * I + i];
          u[b] += a.ep.b1[(int64_t)e * 2 * I + I + i];
        }
        const float v = a.ep.act == kActSilu
                            ? g[b] / (1.0f + __expf(-g[b])) * u[b]
                            : gated_act(g[b], u[b], a.ep.act, a.ep.alpha, a.ep.limit);
        const __bf16 bv = (__bf16)v;  // round to nearest even
        a.act[(int64_t)s_slots[m0 + b] * I + i] = __builtin_bit_cast(uint16_t, bv);
      }
    }
  }
}

// G lanes per w2 row, R = 64 / G rows per wave, JD chunks per lane per row
// (G * JD >= I / 8); WIDE as for sb_gateup.
template <int G, int JD, bool WIDE>
__global__ __launch_bounds__(kThreads) void sb_down(SbArgs a) {
  __shared__ uint32_t s_bits[kBitmapWords];
  __shared__ int32_t s_slots[kSmallBatchMaxSlots];
  __shared__ int32_t s_count;
  constexpr int R = 64 / G;
  const int32_t e = find_expert(a.topk_ids, a.n, a.E, blockIdx.y, s_bits, s_slots, &s_count);
  if (e < 0) return;
  const int lane = threadIdx.x & 63;
  const int gl = lane % G;  // lane inside the row group
  const int64_t H = a.H, I = a.I;
  const int64_t h = ((int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6)) * R + lane / G;
  if (h - lane / G >= H) return;  // the wave's first row is past the end
  const bool h_ok = h < H;
  const int64_t cpr = I / 8;  // 16-byte chunks per row
  const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.w2 + (int64_t)e * H * I), (short)0, (int)(H * I * 2), 0x00020000);
  u32x4_t wv[JD];
#pragma unroll
  for (int j = 0; j < JD; ++j) {
    const int64_t c = gl + G * j;
    wv[j] = __builtin_amdgcn_raw_buffer_load_b128(
        wr, (h_ok && c < cpr) ? (uint32_t)((h * I + c * 8) * 2) : kOutOfRange, 0, 0);
  }
  // activation rows loaded together
  constexpr int SB = WIDE ? (JD >= 16 ? 1 : 16 / JD) : (JD <= 8 ? 2 : 1);
  const int32_t count = s_count;
  for (int32_t m0 = 0; m0 < count; m0 += SB) {
    u32x4_t av[SB][JD];
#pragma unroll
    for (int b = 0; b < SB; ++b) {
      const int32_t m = m0 + b < count ? m0 + b : count - 1;  // a repeat, not stored
      const __amdgpu_buffer_rsrc_t ar = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(a.act + (int64_t)s_slots[m] * I), (short)0, (int)(I * 2), 0x00020000);
#pragma unroll
      for (int j = 0; j < JD; ++j) {
        const int64_t c = gl + G * j;
        av[b][j] = __builtin_amdgcn_raw_buffer_load_b128(
            ar, c < cpr ? (uint32_t)(c * 16) : kOutOfRange, 0, 0);
      }
    }
    float sum[SB];
#pragma unroll
    for (int b = 0; b < SB; ++b) {
      sum[b] = 0.f;
#pragma unroll
      for (int j = 0; j < JD; ++j) sum[b] = dot8(wv[j], av[b][j], sum[b]);
    }
#pragma unroll
    for (int b = 0; b < SB; ++b) sum[b] = group_sum<G>(sum[b]);
#pragma unroll
    for (int b = 0; b < SB; ++b)
      if (gl == G - 1 && h_ok && m0 + b < count) a.y[(int64_t)s_slots[m0 + b] * H + h] = sum[b];
  }
}

template <int G, bool WIDE>
hipError_t launch_down_g(const SbArgs& a, int64_t jd, int64_t rows_per_block, unsigned gy,
                         hipStream_t stream) {
  const dim3 grid((unsigned)((a.H + rows_per_block - 1) / rows_per_block), gy);
  if (jd <= 2) sb_down<G, 2, WIDE><<<grid, kThreads, 0, stream>>>(a);
  else if (jd <= 4) sb_down<G, 4, WIDE><<<grid, kThreads, 0, stream>>>(a);
  else if (jd <= 6) sb_down<G, 6, WIDE><<<grid, kThreads, 0, stream>>>(a);
  else if (jd <= 8) sb_down<G, 8, WIDE><<<grid, kThreads, 0, stream>>>(a);
  else if (jd <= 16) sb_down<G, 16, WIDE><<<grid, kThreads, 0, stream>>>(a);
  else sb_down<G, 32, WIDE><<<grid, kThreads, 0, stream>>>(a);
  return hipGetLastError();
}

template <bool WIDE>
hipError_t launch_down(const SbArgs& a, int64_t g, int64_t jd, int64_t rows_per_block,
                       unsigned gy, hipStream_t stream) {
  switch (g) {
    case 1: return launch_down_g<1, WIDE>(a, jd, rows_per_block, gy, stream);
    case 2: return launch_down_g<2, WIDE>(a, jd, rows_per_block, gy, stream);
    case 4: return launch_down_g<4, WIDE>(a, jd, rows_per_block, gy, stream);
    case 8: return launch_down_g<8, WIDE>(a, jd, rows_per_block, gy, stream);
    case 16: return launch_down_g<16, WIDE>(a, jd, rows_per_block, gy, stream);
    case 32: return launch_down_g<32, WIDE>(a, jd, rows_per_block, gy, stream);
    default: return launch_down_g<64, WIDE>(a, jd, rows_per_block, gy, stream);
  }
}

template <bool WIDE>
void launch_gateup(const SbArgs& a, int64_t nc, dim3 g1, hipStream_t stream) {
  if (nc <= 1) sb_gateup<1, WIDE><<<g1, kThreads, 0, stream>>>(a);
  else if (nc <= 2) sb_gateup<2, WIDE><<<g1, kThreads, 0, stream>>>(a);
  else if (nc <= 4) sb_gateup<4, WIDE><<<g1, kThreads, 0, stream>>>(a);
  else if (nc <= 8) sb_gateup<8, WIDE><<<g1, kThreads, 0, stream>>>(a);
  else sb_gateup<16, WIDE><<<g1, kThreads, 0, stream>>>(a);
}

}  // namespace

bool small_batch_supported(int64_t T, int64_t H, int64_t I, int64_t K) {
  return T * K <= kSmallBatchMaxSlots && H / 8 <= 64 * 16 && I / 8 <= 64 * 32;
}

hipError_t launch_small_batch(const uint16_t* hidden, const uint16_t* w1, const uint16_t* w2,
                              const int32_t* topk_ids, int64_t T, int64_t H, int64_t I,
                              int64_t E, int64_t K, uint16_t* act, float* y,
                              const Epilogue& ep, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  if (!small_batch_supported(T, H, I, K)) return hipErrorInvalidValue;
  SbArgs a;
  a.hidden = hidden;
  a.w1 = w1;
  a.w2 = w2;
  a.topk_ids = topk_ids;
  a.act = act;
  a.y = y;
  a.H = H;
  a.I = I;
  a.E = (int32_t)E;
  a.K = (int32_t)K;
  a.n = (int32_t)(T * K);
  a.ep = ep;
  // one workgroup row per possibly-present expert; absent ranks exit
  const unsigned gy = (unsigned)(a.n < E ? a.n : E);
  const int64_t nc = (H / 8 + 63) / 64;
  const dim3 g1((unsigned)((I + kWaves - 1) / kWaves), gy);
  // 8+ slots per present expert on average and small experts (H*I <= 2^20,
  // where the call is latency-bound): load more slot rows at once. T=64,
  // H=512, I=256, E=8, top-2: 32.1 -> 27.2 us per call. On every batch the
  // same widening measured 5-65 % slower at H=2048 (E=8 and E=128: each wave
  // re-reads more activation rows from L2), and 1-3 % faster at H=I=4096.
  const bool wide = a.n >= 8 * (int64_t)gy && H * I <= (int64_t)1 << 20;
  if (wide) launch_gateup<true>(a, nc, g1, stream);
  else launch_gateup<false>(a, nc, g1, stream);
  hipError_t st = hipGetLastError();
  if (st != hipSuccess) return st;
  // lanes per w2 row: the smallest power of two giving at most 8 chunks per
  // lane (2 for a wide batch, so that a wave loads 8 slots' activation rows
  // at once; more once all 64 lanes share one row)
  const int64_t cpr = I / 8;
  const int64_t per_lane = wide ? 2 : 8;
  int64_t g = 1;
  while (g < 64 && g * per_lane < cpr) g *= 2;
  const int64_t jd = (cpr + g - 1) / g;
  const int64_t rows_per_block = kWaves * (64 / g);
  return wide ? launch_down<true>(a, g, jd, rows_per_block, gy, stream)
              : launch_down<false>(a, g, jd, rows_per_block, gy, stream);
}

}  // namespace moe
