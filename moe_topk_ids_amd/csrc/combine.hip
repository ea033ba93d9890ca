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
// the same bits as the atomic path's 0 + a + b in either order (when the
// down projection's contraction is not split: the atomic path never splits
// it, and its partial rows would be summed before the weight here).
#include "device_util.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;

// Slot rows are read exactly once: non-temporal loads keep them from
// displacing other lines in the L2 and last-level caches (measured on the
// bf16 combine: wide, 537 MB of rows, 135 -> 105 us; large 91 -> 89 us).
// Non-temporal stores of the output measured slower (+5 to +14 %) and are
// not used.
__device__ __forceinline__ uint4 stream_load(const uint4* p) {
  const u32x4_t q = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(q[0], q[1], q[2], q[3]);
}
__device__ __forceinline__ float4 stream_load(const float4* p) {
  typedef float f32x4_v __attribute__((ext_vector_type(4)));
  const f32x4_v q = __builtin_nontemporal_load(reinterpret_cast<const f32x4_v*>(p));
  return make_float4(q[0], q[1], q[2], q[3]);
}
// A workgroup loops over tokens t = blockIdx.x, blockIdx.x + gridDim.x, ...;
// its lanes cover NC float4 columns each of the row's blockIdx.y-th block of
// 256 * NC columns. Per token, the slot lookups and weights are wave-uniform
// (scalar loads), and each lane issues the loads of KP slot rows x NC
// columns before the first use, then adds them in k order. A dropped slot is
// skipped by a select, never by a branch around its load (its row is loaded
// from a valid address and discarded).
template <int KP, int NC>
__global__ __launch_bounds__(kThreads) void combine_kernel(
    const float* __restrict__ y, const float* __restrict__ topk_weights,
    const int32_t* __restrict__ slot_of, const int32_t* __restrict__ ids, int32_t E, int64_t T,
    int64_t H, int32_t K, const float* __restrict__ b2, float* __restrict__ out,
    int32_t ksplit) {
#pragma clang fp contract(off)
  const int64_t h4 = H / 4;
  const int64_t split4 = T * K * h4;  // float4s per partial slot buffer
  const float4* y4 = reinterpret_cast<const float4*>(y);
  const float4* b4 = reinterpret_cast<const float4*>(b2);
  const int64_t c0 = (int64_t)blockIdx.y * kThreads * NC + threadIdx.x;
  int64_t col[NC];
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const int64_t c = c0 + (int64_t)kThreads * i;
    col[i] = c < h4 ? c : h4 - 1;  // lanes past the row end load a valid column
  }
  for (int64_t t = blockIdx.x; t < T; t += gridDim.x) {
    float4 o[NC];
#pragma unroll
    for (int i = 0; i < NC; ++i) o[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int k0 = 0; k0 < K; k0 += KP) {
      float4 v[KP][NC];
      float w[KP];
      bool live[KP];
#pragma unroll
      for (int j = 0; j < KP; ++j) {
        const int k = k0 + j < K ? k0 + j : K - 1;
        const int64_t f = t * K + k;
        const int32_t e = ids[f];
        const bool in = (uint32_t)e < (uint32_t)E;
        live[j] = k0 + j < K && (slot_of ? slot_of[f] >= 0 : in);
        w[j] = topk_weights[f];
#pragma unroll
        for (int i = 0; i < NC; ++i) v[j][i] = stream_load(y4 + f * h4 + col[i]);
        for (int s = 1; s < ksplit; ++s) {  // partial sums of a split contraction, in order
#pragma unroll
          for (int i = 0; i < NC; ++i) {
            const float4 p = stream_load(y4 + s * split4 + f * h4 + col[i]);
            v[j][i].x = v[j][i].x + p.x;
            v[j][i].y = v[j][i].y + p.y;
            v[j][i].z = v[j][i].z + p.z;
            v[j][i].w = v[j][i].w + p.w;
          }
        }
        if (b2) {  // w * (y + b2[e]): the expert's bias before its routing weight
#pragma unroll
          for (int i = 0; i < NC; ++i) {
            const float4 b = b4[(in ? (int64_t)e : 0) * h4 + col[i]];
            v[j][i].x = v[j][i].x + b.x;
            v[j][i].y = v[j][i].y + b.y;
            v[j][i].z = v[j][i].z + b.z;
            v[j][i].w = v[j][i].w + b.w;
          }
        }
      }
#pragma unroll
      for (int j = 0; j < KP; ++j) {
#pragma unroll
        for (int i = 0; i < NC; ++i) {
          // component-wise selects (a select of the whole vector would
          // go through private memory)
          const float nx = o[i].x + w[j] * v[j][i].x;
          const float ny = o[i].y + w[j] * v[j][i].y;
          const float nz = o[i].z + w[j] * v[j][i].z;
          const float nw = o[i].w + w[j] * v[j][i].w;
          o[i].x = live[j] ? nx : o[i].x;
          o[i].y = live[j] ? ny : o[i].y;
          o[i].z = live[j] ? nz : o[i].z;
          o[i].w = live[j] ? nw : o[i].w;
        }
      }
    }
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const int64_t c = c0 + (int64_t)kThreads * i;
      if (c < h4) reinterpret_cast<float4*>(out + t * H)[c] = o[i];
    }
  }
}

// The same weighted sum over bf16 slot rows (each y_{t,k} rounded to bf16
// once by the down projection): out[t, :] = sum over k, in order from zero,
// of w[t,k] * (y16[t*K + k, :] + b2[e, :]). A lane covers NC groups of 8
// columns of the row's blockIdx.y-th block of 2048 * NC columns: one
// 16-byte load of 8 bf16 per slot row and group, widened exactly to fp32.
template <int KP, int NC>
__global__ __launch_bounds__(kThreads) void combine_bf16_kernel(
    const uint16_t* __restrict__ y16, const float* __restrict__ topk_weights,
    const int32_t* __restrict__ slot_of, const int32_t* __restrict__ ids, int32_t E, int64_t T,
    int64_t H, int32_t K, const float* __restrict__ b2, float* __restrict__ out) {
#pragma clang fp contract(off)
  const int64_t h8 = H / 8;
  const uint4* y8 = reinterpret_cast<const uint4*>(y16);
  const float4* b4 = reinterpret_cast<const float4*>(b2);
  const int64_t c0 = (int64_t)blockIdx.y * kThreads * NC + threadIdx.x;
  int64_t col[NC];
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const int64_t c = c0 + (int64_t)kThreads * i;
    col[i] = c < h8 ? c : h8 - 1;  // lanes past the row end load a valid group
  }
  for (int64_t t = blockIdx.x; t < T; t += gridDim.x) {
    float o[NC][8];
#pragma unroll
    for (int i = 0; i < NC; ++i)
#pragma unroll
      for (int q = 0; q < 8; ++q) o[i][q] = 0.f;
    for (int k0 = 0; k0 < K; k0 += KP) {
      uint4 v[KP][NC];
      float w[KP];
      bool live[KP];
      int32_t ev[KP];
#pragma unroll
      for (int j = 0; j < KP; ++j) {
        const int k = k0 + j < K ? k0 + j : K - 1;
        const int64_t f = t * K + k;
        const int32_t e = ids[f];
        const bool in = (uint32_t)e < (uint32_t)E;
        live[j] = k0 + j < K && (slot_of ? slot_of[f] >= 0 : in);
        ev[j] = in ? e : 0;
        w[j] = topk_weights[f];
#pragma unroll
        for (int i = 0; i < NC; ++i) v[j][i] = stream_load(y8 + f * h8 + col[i]);
      }
#pragma unroll
      for (int j = 0; j < KP; ++j) {
#pragma unroll
        for (int i = 0; i < NC; ++i) {
          float yv[8] = {bf16lo(v[j][i].x), bf16hi(v[j][i].x), bf16lo(v[j][i].y),
                         bf16hi(v[j][i].y), bf16lo(v[j][i].z), bf16hi(v[j][i].z),
                         bf16lo(v[j][i].w), bf16hi(v[j][i].w)};
          if (b2) {  // w * (y + b2[e]): the expert's bias before its routing weight
            const float4 ba = b4[(int64_t)ev[j] * (H / 4) + 2 * col[i]];
            const float4 bb = b4[(int64_t)ev[j] * (H / 4) + 2 * col[i] + 1];
            yv[0] = yv[0] + ba.x;
            yv[1] = yv[1] + ba.y;
            yv[2] = yv[2] + ba.z;
            yv[3] = yv[3] + ba.w;
            yv[4] = yv[4] + bb.x;
            yv[5] = yv[5] + bb.y;
            yv[6] = yv[6] + bb.z;
            yv[7] = yv[7] + bb.w;
          }
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            const float n = o[i][q] + w[j] * yv[q];
            o[i][q] = live[j] ? n : o[i][q];
          }
        }
      }
    }
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const int64_t c = c0 + (int64_t)kThreads * i;
      if (c < h8) {
        float4* dst = reinterpret_cast<float4*>(out + t * H) + 2 * c;
        dst[0] = make_float4(o[i][0], o[i][1], o[i][2], o[i][3]);
        dst[1] = make_float4(o[i][4], o[i][5], o[i][6], o[i][7]);
      }
    }
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
                          const float* b2, float* out, hipStream_t stream, int ksplit) {
  const int64_t n = T * (H / 4);
  if (n == 0) return hipSuccess;
  const int64_t nc = (H / 4 + kThreads - 1) / kThreads;  // float4 columns per lane
  // rows wider than 8192 floats: column blocks of 8192 along grid.y
  const dim3 grid((unsigned)(T < 2048 ? T : 2048), (unsigned)((nc + 7) / 8));
#define MOE_COMBINE(KP, NC)                                                                    \
  combine_kernel<KP, NC><<<grid, kThreads, 0, stream>>>(y, topk_weights, slot_of, topk_ids,    \
                                                        (int32_t)E, T, H, (int32_t)K, b2, out, \
                                                        ksplit)
#define MOE_COMBINE_NC(KP)            \
  do {                                \
    if (nc <= 1) MOE_COMBINE(KP, 1);  \
    else if (nc <= 2) MOE_COMBINE(KP, 2); \
    else if (nc <= 4) MOE_COMBINE(KP, 4); \
    else MOE_COMBINE(KP, 8);          \
  } while (0)
  if (K <= 1) MOE_COMBINE_NC(1);
  else if (K <= 2) MOE_COMBINE_NC(2);
  else if (K <= 4 || nc > 4) MOE_COMBINE_NC(4);  // at most 16 float4 loads in flight per lane
  else MOE_COMBINE_NC(8);
#undef MOE_COMBINE_NC
#undef MOE_COMBINE
  return hipGetLastError();
}

hipError_t launch_combine_bf16(const uint16_t* y16, const float* topk_weights,
                               const int32_t* slot_of, const int32_t* topk_ids, int64_t E,
                               int64_t T, int64_t H, int64_t K, const float* b2, float* out,
                               hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const int64_t nc = (H / 8 + kThreads - 1) / kThreads;  // 8-column groups per lane
  // rows wider than 16384 floats: column blocks along grid.y
  const dim3 grid((unsigned)(T < 2048 ? T : 2048), (unsigned)((nc + 3) / 4));
#define MOE_COMBINE16(KP, NC)                                                               \
  combine_bf16_kernel<KP, NC><<<grid, kThreads, 0, stream>>>(y16, topk_weights, slot_of,     \
                                                             topk_ids, (int32_t)E, T, H,     \
                                                             (int32_t)K, b2, out)
#define MOE_COMBINE16_NC(KP)               \
  do {                                     \
    if (nc <= 1) MOE_COMBINE16(KP, 1);     \
    else if (nc <= 2) MOE_COMBINE16(KP, 2); \
    else MOE_COMBINE16(KP, 4);             \
  } while (0)
  // at most 16 loads of 16 bytes in flight per lane
  if (K <= 1) MOE_COMBINE16_NC(1);
  else if (K <= 2) MOE_COMBINE16_NC(2);
  else if (K <= 4 || nc > 2) MOE_COMBINE16_NC(4);
  else MOE_COMBINE16_NC(8);
#undef MOE_COMBINE16_NC
#undef MOE_COMBINE16
  return hipGetLastError();
}

hipError_t launch_zero(float* out, int64_t n, hipStream_t stream) {
  const int64_t n4 = n / 4;  // n is a multiple of 4 (H is a multiple of 128)
  if (n4 == 0) return hipSuccess;
  zero_kernel<<<grid_for(n4), kThreads, 0, stream>>>(out, n4);
  return hipGetLastError();
}

}  // namespace moe
