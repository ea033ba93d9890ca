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
// serves 64/G tokens (4 at E=128). Each lane first sorts its EPL experts by
// logit, largest first, the lower id first among equal logits (a Batcher
// odd-even merge network on a 64-bit key: the logit in an order-preserving
// integer encoding above the complemented position). Each of the K rounds
// is then a group-wide maximum of the lanes' heads (32-bit, DPP moves inside
// a row of 16 lanes, cross-row permutes only for groups of 32 and 64 lanes)
// and a ballot: the lowest lane whose head reaches it holds the winner (the
// largest logit, ties to the lowest id, as lanes hold ascending ids) and
// pops its head. Selection compares the fp32 logits themselves (softmax is
// increasing), so the chosen ids do not depend on how exp() rounds. A lane's
// chosen experts are the first ones of its sorted list, won in the rounds
// its bit mask records; their weights are computed at the end: exp(l - max)
// over the softmax denominator, or, renormalised, over the group's sum of the
// chosen exps (the denominator cancels there and is not formed).
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

// Group-wide combine of a 32-bit value over aligned groups of G lanes; every
// lane of the group ends with the result (the pairings are perfect
// matchings, and both partners combine the same two values, so they agree
// bitwise): quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror,
// row_mirror, then lanes 16 and 32 apart.
template <int G, typename F>
__device__ __forceinline__ uint32_t group_reduce(uint32_t k, F&& pick) {
  if constexpr (G >= 2) k = pick(k, xchg<0xB1>(k));
  if constexpr (G >= 4) k = pick(k, xchg<0x4E>(k));
  if constexpr (G >= 8) k = pick(k, xchg<0x141>(k));
  if constexpr (G >= 16) k = pick(k, xchg<0x140>(k));
  if constexpr (G >= 32) k = pick(k, xchg<16>(k));
  if constexpr (G >= 64) k = pick(k, xchg<32>(k));
  return k;
}

template <int G>
__device__ __forceinline__ float group_sum_f32(float v) {
  return __uint_as_float(group_reduce<G>(__float_as_uint(v), [](uint32_t a, uint32_t b) {
    return __float_as_uint(__uint_as_float(a) + __uint_as_float(b));
  }));
}

// Sorts the N composite keys (hi, lo) into descending order with Batcher's
// odd-even merge network (N a power of two; the loops unroll to a fixed
// list of compare-exchanges).
template <int N>
__device__ __forceinline__ void sort_desc(uint32_t (&hi)[N], uint32_t (&lo)[N]) {
#pragma unroll
  for (int p = 1; p < N; p <<= 1) {
#pragma unroll
    for (int k = p; k >= 1; k >>= 1) {
#pragma unroll
      for (int j = k % p; j + k < N; j += 2 * k) {
#pragma unroll
        for (int i = 0; i < k; ++i) {
          const int a = i + j, b = i + j + k;
          if (b < N && a / (2 * p) == b / (2 * p)) {
            const uint64_t ka = ((uint64_t)hi[a] << 32) | lo[a];
            const uint64_t kb = ((uint64_t)hi[b] << 32) | lo[b];
            const bool sw = kb > ka;
            const uint32_t h = hi[a], l = lo[a];
            hi[a] = sw ? hi[b] : hi[a];
            lo[a] = sw ? lo[b] : lo[a];
            hi[b] = sw ? h : hi[b];
            lo[b] = sw ? l : lo[b];
          }
        }
      }
    }
  }
}

// G lanes per token, EPL logits per lane, at most KMAX choices, VEC: E a
// multiple of 4 (16-byte loads).
template <int G, int EPL, int KMAX, bool VEC>
__global__ __launch_bounds__(kThreads) void topk_softmax_kernel(
    const float* __restrict__ logits, int64_t T, int32_t E, int32_t K, int renormalize,
    float* __restrict__ weights, int32_t* __restrict__ ids) {
  constexpr int kTokensPerBlock = kThreads / G;
  constexpr int kOut = EPL < KMAX ? EPL : KMAX;  // choices one lane can hold
  const int lane = threadIdx.x & 63;
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

  // this lane's experts sorted: logit order bits (0 past E, below every real
  // key) above 255 - position (the lower id first among equal logits)
  uint32_t hi[EPL], lo[EPL];
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    hi[j] = (e0 + j < E) ? ordered_bits(v[j]) : 0u;
    lo[j] = 255u - (uint32_t)j;
  }
  sort_desc<EPL>(hi, lo);
  uint32_t shi[kOut], slo[kOut];  // the head of the sorted list, kept for the output
#pragma unroll
  for (int i = 0; i < kOut; ++i) {
    shi[i] = hi[i];
    slo[i] = lo[i];
  }

  // K rounds: the group's largest head; the lowest lane holding it pops it
  const int gbase = lane & ~(G - 1);
  uint32_t won = 0;  // bit k: this lane won round k
  uint32_t top = 0;  // the token's largest logit (order bits), round 0's maximum
#pragma unroll 1
  for (int k = 0; k < K; ++k) {
    const uint32_t gmax =
        group_reduce<G>(hi[0], [](uint32_t a, uint32_t b) { return a > b ? a : b; });
    top = k == 0 ? gmax : top;
    const uint64_t hit = __ballot(hi[0] == gmax);
    int wsub;
    if constexpr (G == 64) wsub = __builtin_ctzll(hit);
    else wsub = __builtin_ctz((uint32_t)(hit >> gbase) & (uint32_t)((1ull << G) - 1));
    // the owner pops its head: a bitwise select on an all-ones mask (kept
    // opaque: as selects on `owner` the optimiser turns the shift into
    // selects by a pop count, each a compare chain over the list)
    uint32_t pop = sub == wsub ? ~0u : 0u;
    asm volatile("" : "+v"(pop));
#pragma unroll
    for (int j = 0; j + 1 < EPL; ++j) hi[j] = (hi[j + 1] & pop) | (hi[j] & ~pop);
    hi[EPL - 1] &= ~pop;
    won |= pop & (1u << k);
  }

  // weights: exp(l - max) of each chosen expert, over the softmax
  // denominator (lane terms in order, then the group tree) or, renormalised,
  // over the group's sum of the chosen exps
  const float m = from_ordered_bits(top);
  float den = 0.f;
  if (!renormalize) {
#pragma unroll
    for (int j = 0; j < EPL; ++j)
      if (e0 + j < E) den += expf(v[j] - m);
    den = group_sum_f32<G>(den);
  }
  float x[kOut];
  int r[kOut];
  uint32_t rest = won;
  float xsum = 0.f;
#pragma unroll
  for (int i = 0; i < kOut; ++i) {
    r[i] = -1;
    x[i] = 0.f;
    if (rest != 0u) {  // the lane's i-th choice, won in round r[i]
      r[i] = __builtin_ctz(rest);
      rest &= rest - 1u;
      x[i] = expf(from_ordered_bits(shi[i]) - m);
      xsum += x[i];
    }
  }
  if (renormalize) den = group_sum_f32<G>(xsum);
  if (live_tok) {
#pragma unroll
    for (int i = 0; i < kOut; ++i) {
      if (r[i] >= 0) {
        weights[t * K + r[i]] = x[i] / den;
        ids[t * K + r[i]] = e0 + (int32_t)(255u - slo[i]);
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
