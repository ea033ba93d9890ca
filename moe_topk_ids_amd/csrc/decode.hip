// Small-batch path (a handful of tokens, e.g. one decode token with top-8
// of 128 experts): the work is streaming the chosen experts' weights once,
// so it is organised for HBM bandwidth, not matrix cores.
//
// This is the regime the metrale forward_k2 dispatch serves with separate
// gate/up, silu/down and weighted-sum kernels per row pair; here two
// launches do it for any small T:
//   decode_gateup  one wave per (slot, i): streams the gate row i and the up
//                  row I+i of the slot's expert (16-byte loads, 64 lanes over
//                  consecutive chunks), reduces across the wave and stores
//                  act[slot, i] = bf16(silu(g) * u);
//   decode_down    one wave per (token, pair of output rows h): streams
//                  w2[e_k, h, :] for every k of the token, with the token's
//                  K activation rows held in registers, and writes
//                  out[t, h] = sum_k w_k * (w2[e_k, h, :] . act[t*K+k, :]).
// No atomics: each output element is produced by exactly one wave.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kDownRows = 2;    // output rows per wave in decode_down
constexpr int kMaxDownIter = 32;  // 16-byte chunks per lane held in registers

__device__ __forceinline__ float bf16lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }

__device__ __forceinline__ float dot8(uint4 a, uint4 b) {
  float s = bf16lo(a.x) * bf16lo(b.x);
  s = fmaf(bf16hi(a.x), bf16hi(b.x), s);
  s = fmaf(bf16lo(a.y), bf16lo(b.y), s);
  s = fmaf(bf16hi(a.y), bf16hi(b.y), s);
  s = fmaf(bf16lo(a.z), bf16lo(b.z), s);
  s = fmaf(bf16hi(a.z), bf16hi(b.z), s);
  s = fmaf(bf16lo(a.w), bf16lo(b.w), s);
  s = fmaf(bf16hi(a.w), bf16hi(b.w), s);
  return s;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

__global__ __launch_bounds__(kThreads) void decode_gateup(
    const uint16_t* __restrict__ hidden, const uint16_t* __restrict__ w1,
    const int32_t* __restrict__ topk_ids, int64_t H, int64_t I, int32_t E, int32_t K,
    uint16_t* __restrict__ act) {
  const int lane = threadIdx.x & 63;
  const int64_t i = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
  const int64_t f = blockIdx.y;
  if (i >= I) return;
  const int32_t e = topk_ids[f];
  if (e < 0 || e >= E) {
    if (lane == 0) act[f * I + i] = 0;
    return;
  }
  const int64_t t = f / K;
  const uint4* x = reinterpret_cast<const uint4*>(hidden + t * H);
  const uint4* wg = reinterpret_cast<const uint4*>(w1 + ((int64_t)e * 2 * I + i) * H);
  const uint4* wu = reinterpret_cast<const uint4*>(w1 + ((int64_t)e * 2 * I + I + i) * H);
  const int64_t nc = H / 8;
  float g = 0.f, u = 0.f;
  for (int64_t c = lane; c < nc; c += 64) {
    const uint4 xv = x[c];
    g += dot8(wg[c], xv);
    u += dot8(wu[c], xv);
  }
  g = wave_sum(g);
  u = wave_sum(u);
  if (lane == 0) {
    const float a = g / (1.0f + __expf(-g)) * u;
    const __bf16 b = (__bf16)a;  // round to nearest even
    act[f * I + i] = __builtin_bit_cast(uint16_t, b);
  }
}

template <int J>
__global__ __launch_bounds__(kThreads) void decode_down(
    const uint16_t* __restrict__ w2, const float* __restrict__ topk_weights,
    const int32_t* __restrict__ topk_ids, const uint16_t* __restrict__ act, int64_t H,
    int64_t I, int32_t E, int32_t K, float* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int64_t h0 = ((int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6)) * kDownRows;
  const int64_t t = blockIdx.y;
  if (h0 >= H) return;
  const int64_t cpr = I / 8;   // 16-byte chunks per row
  const int64_t nq = K * cpr;  // chunks over the token's K activation rows
  uint4 av[J];
  const uint4* wp[J];  // chunk of w2[e_k, 0, :]; row h adds h * I
  float wk[J];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int64_t q = lane + 64 * j;
    wp[j] = nullptr;
    wk[j] = 0.f;
    av[j] = make_uint4(0, 0, 0, 0);
    if (q < nq) {
      const int64_t k = q / cpr;
      const int64_t c = q - k * cpr;
      const int32_t e = topk_ids[t * K + k];
      if (e >= 0 && e < E) {
        wp[j] = reinterpret_cast<const uint4*>(w2 + (int64_t)e * H * I) + c;
        wk[j] = topk_weights[t * K + k];
        av[j] = reinterpret_cast<const uint4*>(act + (t * K + k) * I)[c];
      }
    }
  }
  const int64_t row_stride = I / 8;  // in uint4
#pragma unroll
  for (int r = 0; r < kDownRows; ++r) {
    const int64_t h = h0 + r;
    if (h >= H) break;
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < J; ++j) {
      if (wp[j]) s = fmaf(wk[j], dot8(wp[j][h * row_stride], av[j]), s);
    }
    s = wave_sum(s);
    if (lane == 0) out[t * H + h] = s;
  }
}

}  // namespace

hipError_t launch_decode(const uint16_t* hidden, const uint16_t* w1, const uint16_t* w2,
                         const float* topk_weights, const int32_t* topk_ids, int64_t T,
                         int64_t H, int64_t I, int64_t E, int64_t K, uint16_t* act,
                         float* out, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const int64_t iters = (K * (I / 8) + 63) / 64;
  if (iters > kMaxDownIter) return hipErrorInvalidValue;
  dim3 g1((unsigned)((I + kWaves - 1) / kWaves), (unsigned)(T * K));
  decode_gateup<<<g1, kThreads, 0, stream>>>(hidden, w1, topk_ids, H, I, (int32_t)E,
                                             (int32_t)K, act);
  hipError_t st = hipGetLastError();
  if (st != hipSuccess) return st;
  const int64_t rows_per_block = (int64_t)kWaves * kDownRows;
  dim3 g2((unsigned)((H + rows_per_block - 1) / rows_per_block), (unsigned)T);
#define MOE_DOWN(JJ)                                                                     \
  decode_down<JJ><<<g2, kThreads, 0, stream>>>(w2, topk_weights, topk_ids, act, H, I, \
                                               (int32_t)E, (int32_t)K, out)
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
bool decode_supported(int64_t I, int64_t K) { return K * (I / 8) <= 64 * kMaxDownIter; }

}  // namespace moe
