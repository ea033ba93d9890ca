// Expert weights quantised to OCP FP8 E4M3 with an fp32 scale per block of
// `block` consecutive elements along the contraction axis (the sub-channel
// quantisation of the later tpu-inference fused_moe kernel.py: ref_moe's
// w1_scale / w2_scale). A weight is fp8(code) * scale[row, col / block].
// Layouts: w1q uint8 [E, 2I, H] with w1s fp32 [E, 2I, H/block]; w2q uint8
// [E, H, I] with w2s fp32 [E, H, I/block].
//
// The weight-streaming paths read the fp8 codes directly, so a decode step
// moves half the bytes of the bf16 weights:
//   decode_gateup_q / decode_down_q   the per-token kernels of decode.hip
//       with 16 weights per 16-byte load; each chunk lies inside one scale
//       block (block is a multiple of 128), so its dot product is taken
//       unscaled and multiplied by the chunk's scale;
//   sb_gateup_q / sb_down_q           the per-expert kernels of
//       small_batch.hip; the expert's rows are widened to packed bf16 once
//       (every E4M3 value is exact in bf16) and reused for all its slots.
// The grouped path first widens the weights to bf16 (dequant_fp8: the
// fp32 product rounded to bf16, the one extra rounding of this path) and
// then runs the bf16 MFMA GEMMs unchanged.
#include <algorithm>

#include "device_util.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kBitmapWords = kMaxExperts / 32;
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// 16 fp8 codes (one 16-byte chunk) times 16 bf16 values (two chunks), fp32.
__device__ __forceinline__ float dot16(u32x4_t q, u32x4_t xa, u32x4_t xb) {
  float s = 0.f;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t qw = q[w];
    const uint32_t x0 = w < 2 ? xa[2 * w] : xb[2 * w - 4];
    const uint32_t x1 = w < 2 ? xa[2 * w + 1] : xb[2 * w - 3];
    const f32x2_t lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)qw, false);
    const f32x2_t hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)qw, true);
    const float l0 = lo[0], l1 = lo[1], h0 = hi[0], h1 = hi[1];
    s = fmaf(l0, bf16lo(x0), s);
    s = fmaf(l1, bf16hi(x0), s);
    s = fmaf(h0, bf16lo(x1), s);
    s = fmaf(h1, bf16hi(x1), s);
  }
  return s;
}

// Four fp8 codes to two packed bf16 pairs (exact).
__device__ __forceinline__ void fp8x4_to_bf16(uint32_t qw, uint32_t& p0, uint32_t& p1) {
  const f32x2_t lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)qw, false);
  const f32x2_t hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)qw, true);
  const float l0 = lo[0], l1 = lo[1], h0 = hi[0], h1 = hi[1];
  p0 = (__float_as_uint(l0) >> 16) | (__float_as_uint(l1) & 0xffff0000u);
  p1 = (__float_as_uint(h0) >> 16) | (__float_as_uint(h1) & 0xffff0000u);
}

// 16 bf16 weights (8 packed pairs) times 16 bf16 values (two chunks).
__device__ __forceinline__ float dot16_bf16(const uint32_t (&w)[8], u32x4_t xa, u32x4_t xb) {
  const uint32_t a0 = xa[0], a1 = xa[1], a2 = xa[2], a3 = xa[3];
  const uint32_t b0 = xb[0], b1 = xb[1], b2 = xb[2], b3 = xb[3];
  float s = dot2(w[0], a0, 0.f);
  s = dot2(w[1], a1, s);
  s = dot2(w[2], a2, s);
  s = dot2(w[3], a3, s);
  s = dot2(w[4], b0, s);
  s = dot2(w[5], b1, s);
  s = dot2(w[6], b2, s);
  return dot2(w[7], b3, s);
}

// ---- grouped path: widen to bf16 ----

// out[r, c] = bf16(fp8(q[r, c]) * s[r, c / block]) for r < rows, c < cols;
// one thread per 16 codes.
__global__ __launch_bounds__(kThreads) void dequant_fp8(const uint8_t* __restrict__ q,
                                                        const float* __restrict__ s,
                                                        int64_t rows, int64_t cols,
                                                        int64_t block,
                                                        uint16_t* __restrict__ out) {
  const int64_t cpr = cols / 16;
  const int64_t n = rows * cpr;
  const int64_t nb = cols / block;
  for (int64_t z = (int64_t)blockIdx.x * kThreads + threadIdx.x; z < n;
       z += (int64_t)gridDim.x * kThreads) {
    const int64_t r = z / cpr, c = z - r * cpr;
    const u32x4_t v = *reinterpret_cast<const u32x4_t*>(q + r * cols + 16 * c);
    const float sc = s[r * nb + (16 * c) / block];
    u32x4_t o0, o1;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t qw = v[w];
      const f32x2_t lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)qw, false);
      const f32x2_t hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)qw, true);
      const float l0 = lo[0] * sc, l1 = lo[1] * sc, h0 = hi[0] * sc, h1 = hi[1] * sc;
      const uint32_t p0 = (uint32_t)to_bf16_bits(l0) | ((uint32_t)to_bf16_bits(l1) << 16);
      const uint32_t p1 = (uint32_t)to_bf16_bits(h0) | ((uint32_t)to_bf16_bits(h1) << 16);
      if (w < 2) {
        o0[2 * w] = p0;
        o0[2 * w + 1] = p1;
      } else {
        o1[2 * w - 4] = p0;
        o1[2 * w - 3] = p1;
      }
    }
    u32x4_t* dst = reinterpret_cast<u32x4_t*>(out + r * cols + 16 * c);
    dst[0] = o0;
    dst[1] = o1;
  }
}

// ---- per-token path ----

struct QArgs {
  const uint16_t* hidden;
  const uint8_t* w1q;
  const float* w1s;
  const uint8_t* w2q;
  const float* w2s;
  const float* topk_weights;
  const int32_t* topk_ids;
  uint16_t* act;
  float* out;  // per-token path: out [T, H]; per-expert path: y [n, H]
  int64_t H, I, block;
  int32_t E, K, n;
  Epilogue ep;
};

// One wave per (slot, i): gate row i and up row I+i of the slot's expert,
// NC 16-byte chunks (16 codes each) per lane per row, all loads up front.
template <int NC>
__global__ __launch_bounds__(kThreads) void decode_gateup_q(QArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t i = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
  const int64_t f = blockIdx.y;
  const int64_t H = a.H, I = a.I;
  if (i >= I) return;
  const int32_t e = a.topk_ids[f];
  if (e < 0 || e >= a.E) {
    if (lane == 63) a.act[f * I + i] = 0;
    return;
  }
  const int64_t t = f / a.K;
  const int64_t nc = H / 16, nb = H / a.block;
  const int64_t rg = (int64_t)e * 2 * I + i, ru = rg + I;
  const __amdgpu_buffer_rsrc_t wr = make_rsrc(a.w1q + (int64_t)e * 2 * I * H, (uint32_t)(2 * I * H));
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(a.hidden + t * H, (uint32_t)(H * 2));
  u32x4_t gq[NC], uq[NC], xa[NC], xb[NC];
  float sg[NC], su[NC];
#pragma unroll
  for (int j = 0; j < NC; ++j) {
    const int64_t c = lane + 64 * j;
    const bool ok = c < nc;
    gq[j] = __builtin_amdgcn_raw_buffer_load_b128(wr, ok ? (uint32_t)(i * H + 16 * c) : kOutOfRange, 0, 0);
    uq[j] = __builtin_amdgcn_raw_buffer_load_b128(wr, ok ? (uint32_t)((I + i) * H + 16 * c) : kOutOfRange, 0, 0);
    xa[j] = __builtin_amdgcn_raw_buffer_load_b128(xr, ok ? (uint32_t)(32 * c) : kOutOfRange, 0, 0);
    xb[j] = __builtin_amdgcn_raw_buffer_load_b128(xr, ok ? (uint32_t)(32 * c + 16) : kOutOfRange, 0, 0);
    const int64_t blk = ok ? (16 * c) / a.block : 0;
    sg[j] = a.w1s[rg * nb + blk];
    su[j] = a.w1s[ru * nb + blk];
  }
  float g = 0.f, u = 0.f;
#pragma unroll
  for (int j = 0; j < NC; ++j) {
    g = fmaf(sg[j], dot16(gq[j], xa[j], xb[j]), g);
    u = fmaf(su[j], dot16(uq[j], xa[j], xb[j]), u);
  }
  g = group_sum<64>(g);
  u = group_sum<64>(u);
  if (lane == 63) {
    if (a.ep.b1) {
      g += a.ep.b1[(int64_t)e * 2 * I + i];
      u += a.ep.b1[(int64_t)e * 2 * I + I + i];
    }
    a.act[f * I + i] = to_bf16_bits(gated_act(g, u, a.ep.act, a.ep.alpha, a.ep.limit));
  }
}

// One wave per (token, output row h): w2 row h of every chosen expert, J
// chunks (16 codes each) per lane over the K rows, and the token's K
// activation rows; writes out[t, h] = sum_k w_k * (y_k[h] + b2[e_k, h]).
template <int J>
__global__ __launch_bounds__(kThreads) void decode_down_q(QArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t h = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
  const int64_t t = blockIdx.y;
  const int64_t H = a.H, I = a.I;
  if (h >= H) return;
  const int32_t K = a.K;
  const int32_t cpr = (int32_t)(I / 16);  // chunks per row
  const int32_t nq = K * cpr;
  const int64_t nb = I / a.block;
  const u32x4_t* wq = reinterpret_cast<const u32x4_t*>(a.w2q);
  const u32x4_t* av = reinterpret_cast<const u32x4_t*>(a.act + t * K * I);
  u32x4_t wv[J], xa[J], xb[J];
  float wk[J], sc[J];
  bool okj[J];
  int32_t ej[J], cj[J];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int32_t q = lane + 64 * j;
    const int32_t k = q < nq ? (int32_t)((uint32_t)q / (uint32_t)cpr) : K - 1;  // clamped
    cj[j] = q - k * cpr;
    ej[j] = a.topk_ids[t * K + k];
    wk[j] = a.topk_weights[t * K + k];
    okj[j] = q < nq;
  }
#pragma unroll
  for (int j = 0; j < J; ++j) {
    okj[j] = okj[j] && ej[j] >= 0 && ej[j] < a.E;
    const int64_t row = okj[j] ? (int64_t)ej[j] * H + h : 0;
    const int64_t c = okj[j] ? cj[j] : 0;
    wv[j] = wq[row * cpr + c];
    sc[j] = a.w2s[row * nb + (16 * c) / a.block];
    const int32_t q = okj[j] ? lane + 64 * j : 0;
    xa[j] = av[2 * q];
    xb[j] = av[2 * q + 1];
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < J; ++j) {
    float d = sc[j] * dot16(wv[j], xa[j], xb[j]);
    if (a.ep.b2 && cj[j] == 0 && okj[j]) d += a.ep.b2[(int64_t)ej[j] * H + h];
    s += okj[j] ? wk[j] * d : 0.f;
  }
  s = group_sum<64>(s);
  if (lane == 63) a.out[t * H + h] = s;
}

// ---- per-expert path ----

// The r-th expert present among the n slot ids and its slots, in LDS (the
// same prologue as small_batch.hip).
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
  int32_t expert = -1, seen = 0;
  for (int w = 0; w < (E + 31) / 32; ++w) {
    const uint32_t b = s_bits[w];
    const int c = __builtin_popcount(b);
    if (seen + c > r) {
      uint32_t m = b;
      for (int skip = r - seen; skip > 0; --skip) m &= m - 1;
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

// Workgroup (r-th present expert, 4 columns i): gate row i and up row I+i
// widened to bf16 once, then act[f, i] for every slot f of the expert.
template <int NC>
__global__ __launch_bounds__(kThreads) void sb_gateup_q(QArgs a) {
  __shared__ uint32_t s_bits[kBitmapWords];
  __shared__ int32_t s_slots[kSmallBatchMaxSlots];
  __shared__ int32_t s_count;
  const int32_t e = find_expert(a.topk_ids, a.n, a.E, blockIdx.y, s_bits, s_slots, &s_count);
  if (e < 0) return;
  const int lane = threadIdx.x & 63;
  const int64_t i = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
  const int64_t H = a.H, I = a.I;
  if (i >= I) return;
  const int64_t nc = H / 16, nb = H / a.block;
  const int64_t rg = (int64_t)e * 2 * I + i, ru = rg + I;
  const __amdgpu_buffer_rsrc_t wr = make_rsrc(a.w1q + (int64_t)e * 2 * I * H, (uint32_t)(2 * I * H));
  uint32_t gw[NC][8], uw[NC][8];
  float sg[NC], su[NC];
#pragma unroll
  for (int j = 0; j < NC; ++j) {
    const int64_t c = lane + 64 * j;
    const bool ok = c < nc;
    const u32x4_t g4 = __builtin_amdgcn_raw_buffer_load_b128(wr, ok ? (uint32_t)(i * H + 16 * c) : kOutOfRange, 0, 0);
    const u32x4_t u4 = __builtin_amdgcn_raw_buffer_load_b128(wr, ok ? (uint32_t)((I + i) * H + 16 * c) : kOutOfRange, 0, 0);
    const int64_t blk = ok ? (16 * c) / a.block : 0;
    sg[j] = a.w1s[rg * nb + blk];
    su[j] = a.w1s[ru * nb + blk];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t gq = g4[w], uq = u4[w];
      fp8x4_to_bf16(gq, gw[j][2 * w], gw[j][2 * w + 1]);
      fp8x4_to_bf16(uq, uw[j][2 * w], uw[j][2 * w + 1]);
    }
  }
  const int32_t count = s_count;
  for (int32_t m = 0; m < count; ++m) {
    const int32_t f = s_slots[m];
    const __amdgpu_buffer_rsrc_t xr = make_rsrc(a.hidden + (int64_t)(f / a.K) * H, (uint32_t)(H * 2));
    float g = 0.f, u = 0.f;
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      const int64_t c = lane + 64 * j;
      const bool ok = c < nc;
      const u32x4_t xa = __builtin_amdgcn_raw_buffer_load_b128(xr, ok ? (uint32_t)(32 * c) : kOutOfRange, 0, 0);
      const u32x4_t xb = __builtin_amdgcn_raw_buffer_load_b128(xr, ok ? (uint32_t)(32 * c + 16) : kOutOfRange, 0, 0);
      g = fmaf(sg[j], dot16_bf16(gw[j], xa, xb), g);
      u = fmaf(su[j], dot16_bf16(uw[j], xa, xb), u);
    }
    g = group_sum<64>(g);
    u = group_sum<64>(u);
    if (lane == 63) {
      if (a.ep.b1) {
        g += a.ep.b1[(int64_t)e * 2 * I + i];
        u += a.ep.b1[(int64_t)e * 2 * I + I + i];
      }
      a.act[(int64_t)f * I + i] = to_bf16_bits(gated_act(g, u, a.ep.act, a.ep.alpha, a.ep.limit));
    }
  }
}

// Workgroup (expert, 4*R rows of w2), G = 64/R lanes per row, JD chunks of
// 16 codes per lane; unscaled-by-routing rows y[f, h] for every slot f.
template <int G, int JD>
__global__ __launch_bounds__(kThreads) void sb_down_q(QArgs a) {
  __shared__ uint32_t s_bits[kBitmapWords];
  __shared__ int32_t s_slots[kSmallBatchMaxSlots];
  __shared__ int32_t s_count;
  constexpr int R = 64 / G;
  const int32_t e = find_expert(a.topk_ids, a.n, a.E, blockIdx.y, s_bits, s_slots, &s_count);
  if (e < 0) return;
  const int lane = threadIdx.x & 63;
  const int gl = lane % G;
  const int64_t H = a.H, I = a.I;
  const int64_t h = ((int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6)) * R + lane / G;
  if (h - lane / G >= H) return;  // the wave's first row is past the end
  const bool h_ok = h < H;
  const int64_t cpr = I / 16, nb = I / a.block;
  const int64_t row = (int64_t)e * H + (h_ok ? h : 0);
  const __amdgpu_buffer_rsrc_t wr = make_rsrc(a.w2q + (int64_t)e * H * I, (uint32_t)(H * I));
  uint32_t ww[JD][8];
  float sc[JD];
#pragma unroll
  for (int j = 0; j < JD; ++j) {
    const int64_t c = gl + G * j;
    const bool ok = h_ok && c < cpr;
    const u32x4_t w4 = __builtin_amdgcn_raw_buffer_load_b128(wr, ok ? (uint32_t)(h * I + 16 * c) : kOutOfRange, 0, 0);
    sc[j] = a.w2s[row * nb + (ok ? (16 * c) / a.block : 0)];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t wq = w4[w];
      fp8x4_to_bf16(wq, ww[j][2 * w], ww[j][2 * w + 1]);
    }
  }
  const int32_t count = s_count;
  for (int32_t m = 0; m < count; ++m) {
    const int32_t f = s_slots[m];
    const __amdgpu_buffer_rsrc_t ar = make_rsrc(a.act + (int64_t)f * I, (uint32_t)(I * 2));
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < JD; ++j) {
      const int64_t c = gl + G * j;
      const bool ok = c < cpr;
      const u32x4_t xa = __builtin_amdgcn_raw_buffer_load_b128(ar, ok ? (uint32_t)(32 * c) : kOutOfRange, 0, 0);
      const u32x4_t xb = __builtin_amdgcn_raw_buffer_load_b128(ar, ok ? (uint32_t)(32 * c + 16) : kOutOfRange, 0, 0);
      s = fmaf(sc[j], dot16_bf16(ww[j], xa, xb), s);
    }
    s = group_sum<G>(s);
    if (gl == G - 1 && h_ok) a.out[(int64_t)f * H + h] = s;
  }
}

template <int G>
hipError_t launch_sb_down_q(const QArgs& a, int64_t jd, unsigned gy, hipStream_t stream) {
  const int64_t rows_per_block = kWaves * (64 / G);
  const dim3 grid((unsigned)((a.H + rows_per_block - 1) / rows_per_block), gy);
  if (jd <= 1) sb_down_q<G, 1><<<grid, kThreads, 0, stream>>>(a);
  else if (jd <= 2) sb_down_q<G, 2><<<grid, kThreads, 0, stream>>>(a);
  else if (jd <= 4) sb_down_q<G, 4><<<grid, kThreads, 0, stream>>>(a);
  else sb_down_q<G, 8><<<grid, kThreads, 0, stream>>>(a);
  return hipGetLastError();
}

QArgs make_qargs(const uint16_t* hidden, const Fp8Weights& w, const float* topk_weights,
                 const int32_t* topk_ids, int64_t T, int64_t H, int64_t I, int64_t E,
                 int64_t K, uint16_t* act, float* out, const Epilogue& ep) {
  QArgs a;
  a.hidden = hidden;
  a.w1q = w.w1q;
  a.w1s = w.w1s;
  a.w2q = w.w2q;
  a.w2s = w.w2s;
  a.topk_weights = topk_weights;
  a.topk_ids = topk_ids;
  a.act = act;
  a.out = out;
  a.H = H;
  a.I = I;
  a.block = w.block;
  a.E = (int32_t)E;
  a.K = (int32_t)K;
  a.n = (int32_t)(T * K);
  a.ep = ep;
  return a;
}

}  // namespace

bool fp8_block_ok(int64_t H, int64_t I, int64_t block) {
  return block >= 128 && block % 128 == 0 && H % block == 0 && I % block == 0;
}

bool fp8_decode_supported(int64_t H, int64_t I, int64_t K) {
  return H / 16 <= 64 * 16 && K * (I / 16) <= 64 * 16;
}

bool fp8_small_batch_supported(int64_t T, int64_t H, int64_t I, int64_t K) {
  return T * K <= kSmallBatchMaxSlots && H / 16 <= 64 * 8 && I / 16 <= 64 * 8;
}

hipError_t launch_dequant_fp8(const Fp8Weights& w, int64_t E, int64_t H, int64_t I,
                              uint16_t* w1, uint16_t* w2, hipStream_t stream) {
  const int64_t n1 = E * 2 * I * (H / 16), n2 = E * H * (I / 16);
  const unsigned g1 = (unsigned)std::min<int64_t>((n1 + kThreads - 1) / kThreads, 256 * 32);
  const unsigned g2 = (unsigned)std::min<int64_t>((n2 + kThreads - 1) / kThreads, 256 * 32);
  dequant_fp8<<<g1, kThreads, 0, stream>>>(w.w1q, w.w1s, E * 2 * I, H, w.block, w1);
  hipError_t st = hipGetLastError();
  if (st != hipSuccess) return st;
  dequant_fp8<<<g2, kThreads, 0, stream>>>(w.w2q, w.w2s, E * H, I, w.block, w2);
  return hipGetLastError();
}

hipError_t launch_decode_fp8(const uint16_t* hidden, const Fp8Weights& w,
                             const float* topk_weights, const int32_t* topk_ids, int64_t T,
                             int64_t H, int64_t I, int64_t E, int64_t K, uint16_t* act,
                             float* out, const Epilogue& ep, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  if (!fp8_decode_supported(H, I, K)) return hipErrorInvalidValue;
  const QArgs a = make_qargs(hidden, w, topk_weights, topk_ids, T, H, I, E, K, act, out, ep);
  const int64_t nc = (H / 16 + 63) / 64;
  const dim3 g1((unsigned)((I + kWaves - 1) / kWaves), (unsigned)(T * K));
  if (nc <= 1) decode_gateup_q<1><<<g1, kThreads, 0, stream>>>(a);
  else if (nc <= 2) decode_gateup_q<2><<<g1, kThreads, 0, stream>>>(a);
  else if (nc <= 4) decode_gateup_q<4><<<g1, kThreads, 0, stream>>>(a);
  else if (nc <= 8) decode_gateup_q<8><<<g1, kThreads, 0, stream>>>(a);
  else decode_gateup_q<16><<<g1, kThreads, 0, stream>>>(a);
  hipError_t st = hipGetLastError();
  if (st != hipSuccess) return st;
  const int64_t iters = (K * (I / 16) + 63) / 64;
  const dim3 g2((unsigned)((H + kWaves - 1) / kWaves), (unsigned)T);
  if (iters <= 2) decode_down_q<2><<<g2, kThreads, 0, stream>>>(a);
  else if (iters <= 4) decode_down_q<4><<<g2, kThreads, 0, stream>>>(a);
  else if (iters <= 6) decode_down_q<6><<<g2, kThreads, 0, stream>>>(a);
  else if (iters <= 8) decode_down_q<8><<<g2, kThreads, 0, stream>>>(a);
  else if (iters <= 12) decode_down_q<12><<<g2, kThreads, 0, stream>>>(a);
  else decode_down_q<16><<<g2, kThreads, 0, stream>>>(a);
  return hipGetLastError();
}

hipError_t launch_small_batch_fp8(const uint16_t* hidden, const Fp8Weights& w,
                                  const int32_t* topk_ids, int64_t T, int64_t H, int64_t I,
                                  int64_t E, int64_t K, uint16_t* act, float* y,
                                  const Epilogue& ep, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  if (!fp8_small_batch_supported(T, H, I, K)) return hipErrorInvalidValue;
  const QArgs a = make_qargs(hidden, w, nullptr, topk_ids, T, H, I, E, K, act, y, ep);
  const unsigned gy = (unsigned)(a.n < E ? a.n : E);
  const int64_t nc = (H / 16 + 63) / 64;
  const dim3 g1((unsigned)((I + kWaves - 1) / kWaves), gy);
  if (nc <= 1) sb_gateup_q<1><<<g1, kThreads, 0, stream>>>(a);
  else if (nc <= 2) sb_gateup_q<2><<<g1, kThreads, 0, stream>>>(a);
  else if (nc <= 4) sb_gateup_q<4><<<g1, kThreads, 0, stream>>>(a);
  else sb_gateup_q<8><<<g1, kThreads, 0, stream>>>(a);
  hipError_t st = hipGetLastError();
  if (st != hipSuccess) return st;
  // lanes per w2 row: the smallest power of two giving at most 4 chunks of
  // 16 codes per lane (at most 8 once all 64 lanes share one row)
  const int64_t cpr = I / 16;
  int64_t g = 1;
  while (g < 64 && g * 4 < cpr) g *= 2;
  const int64_t jd = (cpr + g - 1) / g;
  switch (g) {
    case 1: return launch_sb_down_q<1>(a, jd, gy, stream);
    case 2: return launch_sb_down_q<2>(a, jd, gy, stream);
    case 4: return launch_sb_down_q<4>(a, jd, gy, stream);
    case 8: return launch_sb_down_q<8>(a, jd, gy, stream);
    case 16: return launch_sb_down_q<16>(a, jd, gy, stream);
    case 32: return launch_sb_down_q<32>(a, jd, gy, stream);
    default: return launch_sb_down_q<64>(a, jd, gy, stream);
  }
}

}  // namespace moe
