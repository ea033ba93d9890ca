// Weighted top-k combine and output zeroing.
//
// combine: out[t, :] = sum over k = 0..K-1, in that order and starting from
// zero, of topk_weights[t,k] * (y[t*K + k, :] + b2[e, :]) (fp32; no b2 term
// without expert biases), skipping dropped slots
// (slot_of[f] < 0 on the grouped path, an id outside [0, E) otherwise).
// This is the weighted sum over a token's chosen experts of the
// atrex-bench #009 "Reference Implementation" (its index_add_ of the
// weighted expert outputs) and of ref_moe in tpu-inference's fused_moe
// kernel.py. Products and sums are rounded separately (contraction into
// fused multiply-adds is switched off), in the oracle's order; as the
// hardware fp32 atomic add rounds to nearest even too, for K <= 2 this gives
// the same bits as the atomic path's 0 + a + b in either order.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void combine_kernel(
    const float* __restrict__ y, const float* __restrict__ topk_weights,
    const int32_t* __restrict__ slot_of, const int32_t* __restrict__ ids, int32_t E, int64_t T,
    int64_t H, int32_t K, const float* __restrict__ b2, float* __restrict__ out) {
#pragma clang fp contract(off)
  const int64_t h4 = H / 4;
  const int64_t n = T * h4;
  for (int64_t q = (int64_t)blockIdx.x * kThreads + threadIdx.x; q < n;
       q += (int64_t)gridDim.x * kThreads) {
    const int64_t t = q / h4;
    const int64_t c = q - t * h4;
    float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int k = 0; k < K; ++k) {
      const int64_t f = t * K + k;
      if (slot_of ? slot_of[f] < 0 : (uint32_t)ids[f] >= (uint32_t)E) continue;
      const float w = topk_weights[f];
      float4 v = reinterpret_cast<const float4*>(y + f * H)[c];
      if (b2) {  // w * (y + b2[e]): the expert's bias before its routing weight
        const float4 b = reinterpret_cast<const float4*>(b2 + (int64_t)ids[f] * H)[c];
        v.x = v.x + b.x;
        v.y = v.y + b.y;
        v.z = v.z + b.z;
        v.w = v.w + b.w;
      }
      o.x = o.x + w * v.x;
      o.y = o.y + w * v.y;
      o.z = o.z + w * v.z;
      o.w = o.w + w * v.w;
    }
    reinterpret_cast<float4*>(out + t * H)[c] = o;
  }
}

__global__ __launch_bounds__(kThreads) void zero_kernel(float* __restrict__ out, int64_t n4) {
  for (int64_t q = (int64_t)blockIdx.x * kThreads + threadIdx.x; q < n4;
       q += (int64_t)gridDim.x * kThreads)
    reinterpret_cast<float4*>(out)[q] = make_float4(0.f, 0.f, 0.f, 0.f);
}

unsigned grid_for(int64_t work) {
  int64_t blocks = (work + kThreads - 1) / kThreads;
  const int64_t cap = 256 * 16;  // enough resident workgroups to cover the chip
  return (unsigned)(blocks < cap ? (blocks > 0 ? blocks : 1) : cap);
}

}  // namespace

hipError_t launch_combine(const float* y, const float* topk_weights, const int32_t* slot_of,
                          const int32_t* topk_ids, int64_t E, int64_t T, int64_t H, int64_t K,
                          const float* b2, float* out, hipStream_t stream) {
  const int64_t n = T * (H / 4);
  if (n == 0) return hipSuccess;
  combine_kernel<<<grid_for(n), kThreads, 0, stream>>>(y, topk_weights, slot_of, topk_ids,
                                                         (int32_t)E, T, H, (int32_t)K, b2, out);
  return hipGetLastError();
}

hipError_t launch_zero(float* out, int64_t n, hipStream_t stream) {
  const int64_t n4 = n / 4;  // n is a multiple of 4 (H is a multiple of 128)
  if (n4 == 0) return hipSuccess;
  zero_kernel<<<grid_for(n4), kThreads, 0, stream>>>(out, n4);
  return hipGetLastError();
}

}  // namespace moe
