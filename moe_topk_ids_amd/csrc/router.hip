// Router: fp32 logits [T,E] -> softmax over experts -> the K largest
// (ties to the lowest expert id) -> optional renormalisation, producing the
// topk_weights / topk_ids the fused forward consumes.
//
// This is the step the atrex-bench #009 "Input Generation" section performs
// with softmax and topk, that tpu-inference's get_top_k performs with K
// rounds of max/argmax (argmax keeps the first index) masking each chosen
// expert, and that metrale's forward_k2 launches as moe_topk_softmax_batched
// with norm_topk_prob. Here one wave owns one token: lane l holds experts
// l, l+64, ... in registers; each round is a wave-wide (value, id) argmax.
// Selection compares the fp32 logits themselves (softmax is increasing), so
// the chosen ids do not depend on how exp() rounds.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

template <int EPL>
__global__ __launch_bounds__(kThreads) void topk_softmax_kernel(
    const float* __restrict__ logits, int64_t T, int32_t E, int32_t K, int renormalize,
    float* __restrict__ weights, int32_t* __restrict__ ids) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* l = logits + t * E;
  float v[EPL];
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    const int e = lane + 64 * j;
    const float x = l[e < E ? e : 0];  // valid address; padding replaced below
    v[j] = e < E ? x : -INFINITY;
  }
  float m = -INFINITY;
#pragma unroll
  for (int j = 0; j < EPL; ++j) m = fmaxf(m, v[j]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
  float d = 0.f;
#pragma unroll
  for (int j = 0; j < EPL; ++j)
    if (lane + 64 * j < E) d += expf(v[j] - m);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) d += __shfl_xor(d, off, 64);

  uint32_t taken = 0;  // bit j: expert lane + 64*j already chosen
  float chosen_sum = 0.f;
  for (int k = 0; k < K; ++k) {
    // best candidate of this lane: largest value, lowest id on ties
    float bv = -INFINITY;
    int be = 0x7fffffff;
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
      const int e = lane + 64 * j;
      const bool cand = e < E && !((taken >> j) & 1u);
      if (cand && (v[j] > bv || be == 0x7fffffff)) {
        bv = v[j];
        be = e;
      }
    }
    // wave argmax over (value desc, id asc)
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(bv, off, 64);
      const int oe = __shfl_xor(be, off, 64);
      const bool better = oe != 0x7fffffff &&
                          (be == 0x7fffffff || ov > bv || (ov == bv && oe < be));
      if (better) {
        bv = ov;
        be = oe;
      }
    }
    if ((be & 63) == lane) taken |= 1u << (be >> 6);
    const float p = expf(bv - m) / d;
    chosen_sum += p;
    if (lane == 0) {
      weights[t * K + k] = p;
      ids[t * K + k] = be;
    }
  }
  if (renormalize && lane == 0)
    for (int k = 0; k < K; ++k) weights[t * K + k] = weights[t * K + k] / chosen_sum;
}

}  // namespace

hipError_t launch_topk_softmax(const float* logits, int64_t T, int64_t E, int64_t K,
                               bool renormalize, float* weights, int32_t* ids,
                               hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const dim3 grid((unsigned)((T + kWaves - 1) / kWaves));
  const int r = renormalize ? 1 : 0;
#define MOE_TOPK(EPL) \
  topk_softmax_kernel<EPL><<<grid, kThreads, 0, stream>>>(logits, T, (int32_t)E, (int32_t)K, r, weights, ids)
  if (E <= 64) MOE_TOPK(1);
  else if (E <= 128) MOE_TOPK(2);
  else if (E <= 256) MOE_TOPK(4);
  else if (E <= 512) MOE_TOPK(8);
  else MOE_TOPK(16);
#undef MOE_TOPK
  return hipGetLastError();
}

}  // namespace moe
