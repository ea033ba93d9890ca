// Router: fp32 logits [T,E] -> softmax over experts -> the K largest
// (ties to the lowest expert id) -> optional renormalisation, producing the
// topk_weights / topk_ids the fused forward consumes.
//
// This is the step the atrex-bench #009 "Input Generation" section performs
// with softmax and topk, that tpu-inference's get_top_k performs with K
// rounds of max/argmax (argmax keeps the first index) masking each chosen
// expert, and that metrale's forward_k2 launches as moe_topk_softmax_batched
// with norm_topk_prob.
//
// Layout: a group of G lanes owns one token, lane s of the group holds
// experts EPL*s .. EPL*s+EPL-1 in registers (EPL 4 up to 64 experts, 8 up to
// 128, else 16; G the smallest power of two with EPL*G >= E), so a wave
// serves 64/G tokens (4 at E=128). Every reduction over the group uses DPP
// moves inside a row of 16 lanes (cross-lane permutes through LDS only for
// groups of 32 and 64 lanes, E > 256). Each of the K
// rounds is a group-wide maximum of a 64-bit key: the logit in an
// order-preserving integer encoding above the complement of the expert id,
// so the largest logit wins and, among equal logits, the lowest id. Selection
// compares the fp32 logits themselves (softmax is increasing), so the chosen
// ids do not depend on how exp() rounds. The K weights are computed at the
// end, choice k on lane k mod G of the group, and renormalised by a group
// sum.
#include <type_traits>

#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;

// fp32 -> uint32 with the same order (non-NaN inputs; -0 is taken as +0).
__device__ __forceinline__ uint32_t ordered_bits(float v) {
  const uint32_t u = __float_as_uint(v + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float from_ordered_bits(uint32_t o) {
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}

// The value lane (i ^ m) holds, for the exchange patterns used below: CTRL a
// DPP control inside a row of 16 lanes, or a permute across rows.
template <int CTRL>
__device__ __forceinline__ uint32_t xchg(uint32_t v) {
  if constexpr (CTRL == 16 || CTRL == 32)
    return (uint32_t)__shfl_xor((int)v, CTRL, 64);
  else
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xf, 0xf, false);
}

// Group-wide combine of a value over aligned groups of G lanes; every lane
// of the group ends with the result (the pairings are perfect matchings,
// and both partners combine the same two values, so they agree bitwise):
// quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror, row_mirror,
// then lanes 16 and 32 apart.
template <int G, typename F>
__device__ __forceinline__ uint64_t group_reduce_u64(uint64_t k, F&& pick) {
  auto step = [&](auto ctrl) {
    constexpr int C = decltype(ctrl)::value;
    const uint32_t lo = xchg<C>((uint32_t)k), hi = xchg<C>((uint32_t)(k >> 32));
    k = pick(k, ((uint64_t)hi << 32) | lo);
  };
  if constexpr (G >= 2) step(std::integral_constant<int, 0xB1>{});
  if constexpr (G >= 4) step(std::integral_constant<int, 0x4E>{});
  if constexpr (G >= 8) step(std::integral_constant<int, 0x141>{});
  if constexpr (G >= 16) step(std::integral_constant<int, 0x140>{});
  if constexpr (G >= 32) step(std::integral_constant<int, 16>{});
  if constexpr (G >= 64) step(std::integral_constant<int, 32>{});
  return k;
}

template <int G>
__device__ __forceinline__ float group_max_f32(float v) {
  return __uint_as_float((uint32_t)group_reduce_u64<G>(
      __float_as_uint(v),
      [](uint64_t a, uint64_t b) {
        return (uint64_t)__float_as_uint(fmaxf(__uint_as_float((uint32_t)a),
                                               __uint_as_float((uint32_t)b)));
      }));
}

template <int G>
__device__ __forceinline__ float group_sum_f32(float v) {
  return __uint_as_float((uint32_t)group_reduce_u64<G>(
      __float_as_uint(v),
      [](uint64_t a, uint64_t b) {
        return (uint64_t)__float_as_uint(__uint_as_float((uint32_t)a) +
                                         __uint_as_float((uint32_t)b));
      }));
}

// G lanes per token, EPL logits per lane, at most KMAX choices, VEC: E a
// multiple of 4 (16-byte loads).
template <int G, int EPL, int KMAX, bool VEC>
__global__ __launch_bounds__(kThreads) void topk_softmax_kernel(
    const float* __restrict__ logits, int64_t T, int32_t E, int32_t K, int renormalize,
    float* __restrict__ weights, int32_t* __restrict__ ids) {
  constexpr int kTokensPerBlock = kThreads / G;
  const int sub = threadIdx.x % G;
  const int64_t t = (int64_t)blockIdx.x * kTokensPerBlock + threadIdx.x / G;
  const bool live_tok = t < T;
  const int e0 = sub * EPL;
  const float* row = logits + (live_tok ? t : 0) * E;

  float v[EPL];
  if constexpr (VEC) {
#pragma unroll
    for (int q = 0; q < EPL / 4; ++q) {
      const int e = e0 + 4 * q;
      const float4 x = (live_tok && e < E) ? *reinterpret_cast<const float4*>(row + e)
                                           : make_float4(-INFINITY, -INFINITY, -INFINITY,
                                                         -INFINITY);
      v[4 * q] = x.x;
      v[4 * q + 1] = x.y;
      v[4 * q + 2] = x.z;
      v[4 * q + 3] = x.w;
    }
  } else {
#pragma unroll
    for (int j = 0; j < EPL; ++j) v[j] = (live_tok && e0 + j < E) ? row[e0 + j] : -INFINITY;
  }

  // softmax: max, then the sum of exp(v - max) (lane terms in order, then
  // the group tree)
  float m = -INFINITY;
#pragma unroll
  for (int j = 0; j < EPL; ++j) m = fmaxf(m, v[j]);
  m = group_max_f32<G>(m);
  float d = 0.f;
#pragma unroll
  for (int j = 0; j < EPL; ++j)
    if (e0 + j < E) d += expf(v[j] - m);
  d = group_sum_f32<G>(d);

  // selection keys: order-preserving logit bits above the complemented id;
  // 0 marks an expert already chosen or past E (below every real key)
  uint32_t key_hi[EPL];
#pragma unroll
  for (int j = 0; j < EPL; ++j) key_hi[j] = (e0 + j < E) ? ordered_bits(v[j]) : 0u;

  // K rounds; every lane of the group learns each winner. Lane sub keeps the
  // winners of rounds sub, sub + G, ... for the weights below.
  constexpr int kMine = (KMAX + G - 1) / G;
  uint64_t mine[kMine];
#pragma unroll
  for (int r = 0; r < kMine; ++r) mine[r] = 0;
#pragma unroll
  for (int k = 0; k < KMAX; ++k) {
    if (k < K) {
      uint64_t best = 0;
#pragma unroll
      for (int j = 0; j < EPL; ++j) {
        const uint64_t key = ((uint64_t)key_hi[j] << 32) | (0xffffffffu - (uint32_t)(e0 + j));
        best = (key_hi[j] != 0u && key > best) ? key : best;
      }
      best = group_reduce_u64<G>(best, [](uint64_t a, uint64_t b) { return a > b ? a : b; });
      const int jj = (int)(0xffffffffu - (uint32_t)best) - e0;
#pragma unroll
      for (int j = 0; j < EPL; ++j)
        if (j == jj) key_hi[j] = 0u;  // the owner lane removes the chosen expert
      if (k % G == sub) mine[k / G] = best;
    }
  }

  // weights: p = exp(logit - max) / denominator for each choice, on the lane
  // that keeps it; the renormalising sum over the K choices is a group sum
  float p[kMine];
  float psum = 0.f;
#pragma unroll
  for (int r = 0; r < kMine; ++r) {
    const int k = sub + G * r;
    p[r] = k < K ? expf(from_ordered_bits((uint32_t)(mine[r] >> 32)) - m) / d : 0.f;
    psum += p[r];
  }
  if (renormalize) psum = group_sum_f32<G>(psum);
  if (live_tok) {
#pragma unroll
    for (int r = 0; r < kMine; ++r) {
      const int k = sub + G * r;
      if (k < K) {
        weights[t * K + k] = renormalize ? p[r] / psum : p[r];
        ids[t * K + k] = (int32_t)(0xffffffffu - (uint32_t)mine[r]);
      }
    }
  }
}

}  // namespace

hipError_t launch_topk_softmax(const float* logits, int64_t T, int64_t E, int64_t K,
                               bool renormalize, float* weights, int32_t* ids,
                               hipStream_t stream) {
  if (T == 0) return hipSuccess;
  if (E > 64 * 16 || K > 32) return hipErrorInvalidValue;
  const int r = renormalize ? 1 : 0;
  const bool vec = E % 4 == 0;
  // logits per lane: 4 up to 64 experts, 8 up to 128, then 16, so that a
  // token's group stays within a row of 16 lanes up to 256 experts and each
  // lane's serial work stays short
#define MOE_TOPK(GG, EE, KM, VV)                                                          \
  topk_softmax_kernel<GG, EE, KM, VV>                                                     \
      <<<dim3((unsigned)((T + kThreads / GG - 1) / (kThreads / GG))), kThreads, 0, stream>>>( \
          logits, T, (int32_t)E, (int32_t)K, r, weights, ids)
#define MOE_TOPK_K(GG, EE, VV)               \
  do {                                       \
    if (K <= 8) MOE_TOPK(GG, EE, 8, VV);     \
    else MOE_TOPK(GG, EE, 32, VV);           \
  } while (0)
#define MOE_TOPK_G(VV)                              \
  do {                                              \
    if (E <= 4) MOE_TOPK_K(1, 4, VV);               \
    else if (E <= 8) MOE_TOPK_K(2, 4, VV);          \
    else if (E <= 16) MOE_TOPK_K(4, 4, VV);         \
    else if (E <= 32) MOE_TOPK_K(8, 4, VV);         \
    else if (E <= 64) MOE_TOPK_K(16, 4, VV);        \
    else if (E <= 128) MOE_TOPK_K(16, 8, VV);       \
    else if (E <= 256) MOE_TOPK_K(16, 16, VV);      \
    else if (E <= 512) MOE_TOPK_K(32, 16, VV);      \
    else MOE_TOPK_K(64, 16, VV);                    \
  } while (0)
  if (vec) MOE_TOPK_G(true);
  else MOE_TOPK_G(false);
#undef MOE_TOPK_G
#undef MOE_TOPK_K
#undef MOE_TOPK
  return hipGetLastError();
}

}  // namespace moe
