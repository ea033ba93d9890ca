// Small-batch path (a handful of tokens, e.g. one decode token with top-8
// of 128 experts): the work is streaming the chosen experts' weights once,
// so it is organised for HBM bandwidth, not matrix cores.
//
// This is the regime the metrale forward_k2 dispatch serves with separate
// gate/up, silu/down and weighted-sum kernels per row pair; here two
// launches do it for any small T:
//   decode_gateup  one wave per (slot, i pair): streams the gate rows i, i+1
//                  and up rows I+i, I+i+1 of the slot's expert (16-byte loads,
//                  64 lanes over consecutive chunks, all issued up front),
//                  reduces across the wave and stores act = bf16(silu(g) * u);
//   decode_down    one wave per (token, output row h): streams w2[e_k, h, :]
//                  for every k of the token together with the token's K
//                  activation rows, and writes
//                  out[t, h] = sum_k w_k * (w2[e_k, h, :] . act[t*K+k, :]).
// No atomics: each output element is produced by exactly one wave.
#include "device_util.h"
#include "moe_internal.h"


namespace moe {
namespace {

// Cache policy of the expert-weight loads: non-temporal (each weight is read
// once per call; measured on the decode workload, 20.2 -> 19.6 us per call).
// The per-expert streaming kernels keep default loads (non-temporal measured
// 2 % slower there).
constexpr int kNonTemporal = 2;  // the NT bit of the gfx950 cache-policy field

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kMaxDownIter = 32;  // 16-byte chunks per lane held in registers

__device__ __forceinline__ float dot8(u32x4_t a, u32x4_t b) {
  float s = bf16lo(a[0]) * bf16lo(b[0]);
  s = fmaf(bf16hi(a[0]), bf16hi(b[0]), s);
  s = fmaf(bf16lo(a[1]), bf16lo(b[1]), s);
  s = fmaf(bf16hi(a[1]), bf16hi(b[1]), s);
  s = fmaf(bf16lo(a[2]), bf16lo(b[2]), s);
  s = fmaf(bf16hi(a[2]), bf16hi(b[2]), s);
  s = fmaf(bf16lo(a[3]), bf16lo(b[3]), s);
  s = fmaf(bf16hi(a[3]), bf16hi(b[3]), s);
  return s;
}
__device__ __forceinline__ float dot8(uint4 a, uint4 b) {
  return dot8(u32x4_t{a.x, a.y, a.z, a.w}, u32x4_t{b.x, b.y, b.z, b.w});
}

// One wave per (slot, IPW consecutive intermediate columns): the IPW gate
// rows and the IPW up rows of H bf16 each. NC = 16-byte chunks per lane per
// row; every load of the wave is issued before the first use.
template <int NC, int IPW>
__global__ __launch_bounds__(kThreads) void decode_gateup(
    const uint16_t* __restrict__ hidden, const uint16_t* __restrict__ w1,
    const int32_t* __restrict__ topk_ids, int64_t H, int64_t I, int32_t E, int32_t K,
    uint16_t* __restrict__ act, Epilogue ep) {
  const int lane = threadIdx.x & 63;
  const int64_t i0 = ((int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6)) * IPW;
  const int64_t f = blockIdx.y;
  if (i0 >= I) return;
  const int32_t e = topk_ids[f];
  if (e < 0 || e >= E) {
    if (lane < IPW && i0 + lane < I) act[f * I + i0 + lane] = 0;
    return;
  }
  const int64_t t = f / K;
  const int64_t nc = H / 8;
  // buffer loads: offsets past the end read zeros (no branches, no scratch)
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(hidden + t * H, (uint32_t)(H * 2));
  const __amdgpu_buffer_rsrc_t wr = make_rsrc(w1 + (int64_t)e * 2 * I * H, (uint32_t)(2 * I * H * 2));
  u32x4_t wv[2 * IPW][NC], xv[NC];
#pragma unroll
  for (int j = 0; j < NC; ++j) {
    const int64_t c = lane + 64 * j;
    const bool ok = c < nc;
#pragma unroll
    for (int r = 0; r < IPW; ++r) {
      const bool okr = ok && (i0 + r < I);
      const uint32_t og = okr ? (uint32_t)(((i0 + r) * H + c * 8) * 2) : kOutOfRange;
      const uint32_t ou = okr ? (uint32_t)(((I + i0 + r) * H + c * 8) * 2) : kOutOfRange;
      wv[r][j] = __builtin_amdgcn_raw_buffer_load_b128(wr, og, 0, kNonTemporal);
      wv[IPW + r][j] = __builtin_amdgcn_raw_buffer_load_b128(wr, ou, 0, kNonTemporal);
    }
    xv[j] = __builtin_amdgcn_raw_buffer_load_b128(xr, ok ? (uint32_t)(c * 16) : kOutOfRange, 0, 0);
  }
  float s[2 * IPW];
#pragma unroll
  for (int r = 0; r < 2 * IPW; ++r) s[r] = 0.f;
#pragma unroll
  for (int j = 0; j < NC; ++j)
#pragma unroll
    for (int r = 0; r < 2 * IPW; ++r) s[r] += dot8(wv[r][j], xv[j]);
#pragma unroll
  for (int r = 0; r < 2 * IPW; ++r) s[r] = wave_sum(s[r]);
#pragma unroll
  for (int r = 0; r < IPW; ++r) {
    if (lane == 63 && i0 + r < I) {
      float g = s[r], u = s[IPW + r];
      if (ep.b1) {
        g += ep.b1[(int64_t)e * 2 * I + i0 + r];
        u += ep.b1[(int64_t)e * 2 * I + I + i0 + r];
      }
      const float a = ep.act == kActSilu ? g / (1.0f + __expf(-g)) * u
                                         : gated_act(g, u, ep.act, ep.alpha, ep.limit);
      const __bf16 b = (__bf16)a;  // round to nearest even
      act[f * I + i0 + r] = __builtin_bit_cast(uint16_t, b);
    }
  }
}

// One wave per (token, output row h): streams w2[e_k, h, :] for every k of
// the token. J = 16-byte chunks per lane over the K activation rows.
template <int J>
__global__ __launch_bounds__(kThreads) void decode_down(
    const uint16_t* __restrict__ w2, const float* __restrict__ topk_weights,
    const int32_t* __restrict__ topk_ids, const uint16_t* __restrict__ act, int64_t H,
    int64_t I, int32_t E, int32_t K, const float* __restrict__ b2, float* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int64_t h = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
  const int64_t t = blockIdx.y;
  if (h >= H) return;
  const int64_t cpr = I / 8;   // 16-byte chunks per row
  const int64_t nq = K * cpr;  // chunks over the token's K activation rows
  // row h of each chosen expert's w2 and the token's activation rows; a
  // dropped slot or a lane past the end loads from a valid address and its
  // product is discarded (no branches around the loads)
  const int32_t cpr32 = (int32_t)cpr, nq32 = (int32_t)nq;
  const uint4* w2v = reinterpret_cast<const uint4*>(w2);
  const uint4* av_base = reinterpret_cast<const uint4*>(act + t * K * I);
  uint4 wv[J], av[J];
  float wk[J];
  bool okj[J];
  int32_t ej[J], qj[J], cj[J];
  // first every routing lookup, then every weight/activation load, so the
  // wave has all its row loads in flight at once
#pragma unroll
  for (int j = 0; j < J; ++j) {
    // 32-bit index math (a 64-bit division would branch per chunk)
    const int32_t q = lane + 64 * j;
    const int32_t k = q < nq32 ? (int32_t)((uint32_t)q / (uint32_t)cpr32) : K - 1;  // clamped
    qj[j] = q;
    cj[j] = q - k * cpr32;
    ej[j] = topk_ids[t * K + k];
    wk[j] = topk_weights[t * K + k];
  }
#pragma unroll
  for (int j = 0; j < J; ++j) {
    okj[j] = qj[j] < nq32 && ej[j] >= 0 && ej[j] < E;
    {
      const u32x4_t q = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(
          &w2v[okj[j] ? ((int64_t)ej[j] * H + h) * cpr + cj[j] : 0]));
      wv[j] = make_uint4(q[0], q[1], q[2], q[3]);
    }
    av[j] = av_base[okj[j] ? qj[j] : 0];
  }
  float s = 0.f;
  if (b2) {
    // expert bias before the routing weight: w_k * (partial + b2[e_k, h]),
    // added by the lane holding the first chunk of row k
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const float bj = (okj[j] && cj[j] == 0) ? b2[(int64_t)ej[j] * H + h] : 0.f;
      const float d = wk[j] * (dot8(wv[j], av[j]) + bj);
      s += okj[j] ? d : 0.f;
    }
  } else {
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const float d = wk[j] * dot8(wv[j], av[j]);
      s += okj[j] ? d : 0.f;
    }
  }
  s = wave_sum(s);
  if (lane == 63) out[t * H + h] = s;
}

}  // namespace

hipError_t launch_decode(const uint16_t* hidden, const uint16_t* w1, const uint16_t* w2,
                         const float* topk_weights, const int32_t* topk_ids, int64_t T,
                         int64_t H, int64_t I, int64_t E, int64_t K, uint16_t* act,
                         float* out, const Epilogue& ep, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const int64_t nc = (H / 8 + 63) / 64;           // chunks per lane per gate/up row
  const int64_t iters = (K * (I / 8) + 63) / 64;  // chunks per lane in the down kernel
  if (nc > 16 || iters > kMaxDownIter) return hipErrorInvalidValue;
  constexpr int kIPW = 1;  // one gate/up column pair per wave measured fastest
  dim3 g1((unsigned)((I + kIPW * kWaves - 1) / (kIPW * kWaves)), (unsigned)(T * K));
#define MOE_GATEUP(NN) \
  decode_gateup<NN, kIPW><<<g1, kThreads, 0, stream>>>(hidden, w1, topk_ids, H, I, (int32_t)E, \
                                                       (int32_t)K, act, ep)
  if (nc <= 1) MOE_GATEUP(1);
  else if (nc <= 2) MOE_GATEUP(2);
  else if (nc <= 4) MOE_GATEUP(4);
  else if (nc <= 8) MOE_GATEUP(8);
  else MOE_GATEUP(16);
#undef MOE_GATEUP
  hipError_t st = hipGetLastError();
  if (st != hipSuccess) return st;
  dim3 g2((unsigned)((H + kWaves - 1) / kWaves), (unsigned)T);
#define MOE_DOWN(JJ)                                                                     \
  decode_down<JJ><<<g2, kThreads, 0, stream>>>(w2, topk_weights, topk_ids, act, H, I, \
                                               (int32_t)E, (int32_t)K, ep.b2, out)
  if (iters <= 4) MOE_DOWN(4);
  else if (iters <= 8) MOE_DOWN(8);
  else if (iters <= 12) MOE_DOWN(12);
  else if (iters <= 16) MOE_DOWN(16);
  else if (iters <= 24) MOE_DOWN(24);
  else MOE_DOWN(32);
#undef MOE_DOWN
  return hipGetLastError();
}

// Largest K * I the decode path can hold in registers.
bool decode_supported(int64_t H, int64_t I, int64_t K) {
  return K * (I / 8) <= 64 * kMaxDownIter && H / 8 <= 64 * 16;
}

}  // namespace moe
