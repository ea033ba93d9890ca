// Device helpers shared by the streaming kernels (decode, small batch, fp8,
// router) and the grouped GEMMs: buffer resources whose out-of-range bytes
// read as zero, bf16 unpacking, the packed bf16 dot product and lane
// reductions built from DPP moves (no LDS round trips).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// A buffer offset at or past num_records of every resource used here: a load
// through it returns zeros and fetches nothing, so rows outside an operand
// need no branch around their load.
constexpr uint32_t kOutOfRange = 0x80000000u;

// Raw buffer resource over [base, base + bytes); bytes past the end read as zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

// The two bf16 values packed in a 32-bit word, as fp32 (exact).
__device__ __forceinline__ float bf16lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }

// acc + a.lo * b.lo + a.hi * b.hi with the packed bf16 dot instruction
// (v_dot2c_f32_bf16: fp32 accumulation).
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), acc, false);
}

// fp32 -> bf16 bits, round to nearest even.
__device__ __forceinline__ uint16_t to_bf16_bits(float v) {
  const __bf16 b = (__bf16)v;
  return __builtin_bit_cast(uint16_t, b);
}

// v + the value DPP control CTRL moves into this lane (0 where ROW_MASK
// leaves a row of 16 lanes out).
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ float dpp_add(float v) {
  const int m = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROW_MASK, 0xf,
                                            false);
  return v + __builtin_bit_cast(float, m);
}

// Sum over aligned groups of G lanes. The group's total ends up in its last
// lane (and, for G <= 16, in every lane of the group).
template <int G>
__device__ __forceinline__ float group_sum(float v) {
  if (G >= 2) v = dpp_add<0xB1>(v);         // quad_perm [1,0,3,2]: pairs
  if (G >= 4) v = dpp_add<0x4E>(v);         // quad_perm [2,3,0,1]: quads
  if (G >= 8) v = dpp_add<0x141>(v);        // row_half_mirror: 8 lanes
  if (G >= 16) v = dpp_add<0x140>(v);       // row_mirror: 16 lanes
  if (G >= 32) v = dpp_add<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3: 32 lanes
  if (G >= 64) v = dpp_add<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3: 64 lanes
  return v;
}

// Sum over the wave; the total is in lane 63.
__device__ __forceinline__ float wave_sum(float v) { return group_sum<64>(v); }

}  // namespace moe
