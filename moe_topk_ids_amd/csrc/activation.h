// Gated activations and expert biases, device side.
//
// The activations are those of the later tpu-inference fused_moe
// kernel.py's activation_fn: silu(g) * u; gelu(g) * u in jax.nn.gelu's
// default tanh form (and the erf form, for callers of that convention); and
// swigluoai: the gate clipped from above at `limit`, the up projection
// clipped to [-limit, limit], then (up + 1) * gate * sigmoid(alpha * gate).
// Biases (ref_moe of the same page): b1 [E, 2I] fp32 is added to the gate
// (first I) and up (last I) projections before the activation; b2 [E, H]
// fp32 is added to an expert's down projection before the routing weight.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

enum ActKind : int32_t { kActSilu = 0, kActGeluTanh = 1, kActSwigluOai = 2, kActGeluErf = 3 };

// Everything the epilogues need beyond the plain silu path.
struct Epilogue {
  int32_t act = kActSilu;
  float alpha = 1.702f;  // swigluoai
  float limit = 7.0f;    // swigluoai
  const float* b1 = nullptr;
  const float* b2 = nullptr;
  bool plain() const { return act == kActSilu && b1 == nullptr && b2 == nullptr; }
};

// silu(g) * u = g * u / (1 + exp(-g)), exp via the hardware 2^x: the plain
// epilogue of the gate/up projection.
__device__ __forceinline__ float silu_mul(float g, float u) {
  const float e = __builtin_amdgcn_exp2f(-g * 1.4426950408889634f);
  return g * u * __builtin_amdgcn_rcpf(1.0f + e);
}

// act(g, u) for the variants (silu included). tanh(z) = 1 - 2 / (e^{2z} + 1)
// and the sigmoid use the hardware exp and reciprocal; the error is far
// inside the bf16 rounding of the stored activation.
__device__ __forceinline__ float gated_act(float g, float u, int32_t act, float alpha,
                                           float limit) {
  if (act == kActGeluTanh) {
    const float z = 0.7978845608028654f * (g + 0.044715f * (g * g * g));
    const float t = 1.0f - 2.0f * __builtin_amdgcn_rcpf(1.0f + __expf(2.0f * z));
    return 0.5f * g * (1.0f + t) * u;
  }
  if (act == kActGeluErf) return 0.5f * g * (1.0f + erff(g * 0.7071067811865476f)) * u;
  if (act == kActSwigluOai) {
    const float gc = fminf(g, limit);
    const float uc = fminf(fmaxf(u, -limit), limit);
    return (uc + 1.0f) * gc * __builtin_amdgcn_rcpf(1.0f + __expf(-alpha * gc));
  }
  return g * u * __builtin_amdgcn_rcpf(1.0f + __expf(-g));
}

}  // namespace moe
