// Internal declarations shared by the HIP translation units of the library.
// Every launcher enqueues on `stream` and returns the launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "activation.h"

namespace moe {

// Records the message moe_last_error() returns on this thread; returns code.
int set_last_error(int code, const char* msg);

// Slots handled by one routing workgroup (grows with T*K so that the number
// of routing workgroups stays at most kRouteMaxBlocks).
constexpr int kRouteThreads = 256;
// Problems up to this size are routed in one launch (a workgroup per 1024
// slots).
constexpr int64_t kRouteOnePassMaxSlots = 65536;
constexpr int64_t kRouteOnePassMaxExperts = 512;
constexpr int kRouteMaxBlocks = 128;
constexpr int kMaxExperts = 1024;

inline int64_t route_block_slots(int64_t n_slots) {
  int64_t rb = 1024;
  while ((n_slots + rb - 1) / rb > kRouteMaxBlocks) rb *= 2;
  return rb;
}
inline int64_t route_blocks(int64_t n_slots) {
  int64_t rb = route_block_slots(n_slots);
  return n_slots == 0 ? 0 : (n_slots + rb - 1) / rb;
}

// Row capacity of the padded, expert-grouped layout: every non-empty expert
// adds at most m_tile - 1 pad rows, and at most min(E, n_slots) experts are
// non-empty.
inline int64_t padded_capacity(int64_t n_slots, int64_t E, int64_t m_tile) {
  int64_t live = n_slots < E ? n_slots : E;
  int64_t cap = n_slots + live * (m_tile - 1);
  return (cap + m_tile - 1) / m_tile * m_tile;
}

hipError_t launch_route(const int32_t* ids, int64_t T, int64_t K, int64_t E, int32_t m_tile,
                        int32_t* block_hist, int32_t* counts, int32_t* offsets, int32_t* sorted, int32_t* slot_of,
                        int32_t* tile_expert, int32_t* num_tiles, hipStream_t stream);

// Tile configuration of the grouped GEMMs, chosen per problem on the host.
// Every grouped GEMM skips a row tile whose tile_expert entry is outside
// [0, E) rather than address weights past the end of w1/w2.
struct GemmCfg {
  int bm;      // token rows per tile (the routing m_tile)
  int bn;      // weight rows per tile (GEMM1: half gate, half up)
  int ns = 2;  // stages of the global->LDS ring (pick_ring_stages)
};

GemmCfg pick_gemm1_cfg(int64_t T, int64_t K, int64_t H, int64_t I, int64_t E);
// 4 (a four-stage ring) where a launch of n_tiles column tiles per row tile
// expects at most one tile per CU and the tile's stages fit, else 2.
int pick_ring_stages(GemmCfg cfg, int64_t T, int64_t K, int64_t E, int64_t n_tiles);
GemmCfg pick_gemm2_cfg(int64_t n_slots, int64_t H, int64_t I, int64_t E, int bm);

// FP8-weight grouped GEMMs: the weight tiles are staged as codes and widened
// to bf16 (bf16_rne(fp32(code) * scale)) at fragment read; supported while
// H/block and I/block are at most kMaxScaleBlocks (the tile's scales sit in LDS).
constexpr int kMaxScaleBlocks = 32;
bool fp8_gemm_supported(int64_t H, int64_t I, int64_t block);
hipError_t launch_gemm1_silu_fp8(GemmCfg cfg, const uint16_t* hidden, const uint8_t* w1q,
                                 const float* w1s, int64_t block, const int32_t* sorted,
                                 const int32_t* tile_expert, const int32_t* num_tiles, int64_t T,
                                 int64_t H, int64_t I, int64_t E, int64_t K, int64_t max_tiles,
                                 uint16_t* act, const Epilogue& ep, hipStream_t stream);
hipError_t launch_gemm2_fp8(GemmCfg cfg, const uint16_t* act, const uint8_t* w2q,
                            const float* w2s, int64_t block, const int32_t* sorted,
                            const int32_t* tile_expert, const int32_t* num_tiles,
                            const float* topk_weights, int64_t H, int64_t I, int64_t E,
                            int64_t K, int64_t max_tiles, float* y, float* out, const float* b2,
                            hipStream_t stream, int ksplit = 1, int64_t n_slots = 0,
                            uint16_t* y16 = nullptr);

hipError_t launch_gemm1_silu(GemmCfg cfg, const uint16_t* hidden, const uint16_t* w1,
                             const int32_t* sorted, const int32_t* tile_expert,
                             const int32_t* num_tiles, int64_t T, int64_t H, int64_t I,
                             int64_t E, int64_t K, int64_t max_tiles, uint16_t* act,
                             const Epilogue& ep, hipStream_t stream);

// Down projection. If `out` is non-null the tile results (plus b2[e], if
// given) are scaled by the routing weight and atomically added to out[t, :];
// otherwise they are written unscaled and unbiased to y[f, :] (f = t*K + k),
// or, if `y16` is non-null (no split), rounded to bf16 into y16[f, :].
hipError_t launch_gemm2(GemmCfg cfg, const uint16_t* act, const uint16_t* w2,
                        const int32_t* sorted, const int32_t* tile_expert,
                        const int32_t* num_tiles, const float* topk_weights, int64_t H,
                        int64_t I, int64_t E, int64_t K, int64_t max_tiles, float* y,
                        float* out, const float* b2, hipStream_t stream, int ksplit = 1,
                        int64_t n_slots = 0, uint16_t* y16 = nullptr, bool tail = false);
// tail: with ksplit 1, run a last partial round of at most half the chip as
// column halves in a second launch (pick_tail_split; same results bit for bit).
bool pick_tail_split(GemmCfg cfg, int64_t T, int64_t K, int64_t E, int64_t n_rows,
                     int64_t kdim, int64_t max_tiles);

// Split of the down projection's contraction (1 or 2; see gemm.hip):
// with ksplit > 1, launch_gemm2 writes ksplit partial slot buffers y + s*n_slots*H.
int pick_ksplit(GemmCfg cfg, int64_t T, int64_t K, int64_t E, int64_t n_tiles, int64_t kdim);

// out[t, :] = sum_k w[t,k] * (y[t*K+k, :] + b2[e_k, :]) (b2 may be null),
// where with a split contraction y[f, :] is the sum over s = 0..ksplit-1 (in
// that order) of the partial rows y + s*T*K*H.
// A slot is dropped if slot_of[f] < 0, or, without slot_of, if its id is
// outside [0, E).
hipError_t launch_combine(const float* y, const float* topk_weights, const int32_t* slot_of,
                          const int32_t* topk_ids, int64_t E, int64_t T, int64_t H, int64_t K,
                          const float* b2, float* out, hipStream_t stream, int ksplit = 1);
// The same weighted sum over bf16 slot rows y16 [T*K, H] (no split).
hipError_t launch_combine_bf16(const uint16_t* y16, const float* topk_weights,
                               const int32_t* slot_of, const int32_t* topk_ids, int64_t E,
                               int64_t T, int64_t H, int64_t K, const float* b2, float* out,
                               hipStream_t stream);
hipError_t launch_zero(float* out, int64_t n, hipStream_t stream);

// Sets *err_flag to 1 if any id is outside [0, E) or repeats within a token.
hipError_t launch_validate_ids(const int32_t* ids, int64_t T, int64_t K, int64_t E,
                               int32_t* err_flag, hipStream_t stream);

bool decode_supported(int64_t H, int64_t I, int64_t K);

// Expert-deduplicated small-batch path (small_batch.hip): act bf16 [T*K, I]
// and unscaled per-slot outputs y fp32 [T*K, H], then launch_combine.
constexpr int kSmallBatchMaxSlots = 1024;
bool small_batch_supported(int64_t T, int64_t H, int64_t I, int64_t K);
hipError_t launch_small_batch(const uint16_t* hidden, const uint16_t* w1, const uint16_t* w2,
                              const int32_t* topk_ids, int64_t T, int64_t H, int64_t I,
                              int64_t E, int64_t K, uint16_t* act, float* y,
                              const Epilogue& ep, hipStream_t stream);

// Expert weights as OCP FP8 E4M3 codes with an fp32 scale per `block`
// elements of the contraction axis (fp8.hip).
struct Fp8Weights {
  const uint8_t* w1q;  // [E, 2I, H]
  const float* w1s;    // [E, 2I, H / block]
  const uint8_t* w2q;  // [E, H, I]
  const float* w2s;    // [E, H, I / block]
  int64_t block;
};
bool fp8_block_ok(int64_t H, int64_t I, int64_t block);
bool fp8_decode_supported(int64_t H, int64_t I, int64_t K);
bool fp8_small_batch_supported(int64_t T, int64_t H, int64_t I, int64_t K);
// Widen both weight tensors to bf16 (w1 [E, 2I, H], w2 [E, H, I]).
hipError_t launch_dequant_fp8(const Fp8Weights& w, int64_t E, int64_t H, int64_t I,
                              uint16_t* w1, uint16_t* w2, hipStream_t stream);
hipError_t launch_decode_fp8(const uint16_t* hidden, const Fp8Weights& w,
                             const float* topk_weights, const int32_t* topk_ids, int64_t T,
                             int64_t H, int64_t I, int64_t E, int64_t K, uint16_t* act,
                             float* out, const Epilogue& ep, hipStream_t stream);
hipError_t launch_small_batch_fp8(const uint16_t* hidden, const Fp8Weights& w,
                                  const int32_t* topk_ids, int64_t T, int64_t H, int64_t I,
                                  int64_t E, int64_t K, uint16_t* act, float* y,
                                  const Epilogue& ep, hipStream_t stream);

hipError_t launch_topk_softmax(const float* logits, int64_t T, int64_t E, int64_t K,
                               bool renormalize, float* weights, int32_t* ids,
                               hipStream_t stream);

hipError_t launch_decode(const uint16_t* hidden, const uint16_t* w1, const uint16_t* w2,
                         const float* topk_weights, const int32_t* topk_ids, int64_t T,
                         int64_t H, int64_t I, int64_t E, int64_t K, uint16_t* act,
                         float* out, const Epilogue& ep, hipStream_t stream);

}  // namespace moe
