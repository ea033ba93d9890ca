/*
 * moe_topk_ids: fused Mixture-of-Experts forward for AMD Instinct MI355X
 * (gfx950), as a C ABI over plain device pointers.
 *
 * What is computed (atrex-bench operator #009 "fused_moe", section
 * "Reference Implementation"; the same computation as ref_moe in
 * tpu-inference's fused_moe v1 kernel.py): for every token t and each of its
 * K chosen experts e = topk_ids[t,k] with routing weight w = topk_weights[t,k],
 *
 *     g = x[t] . W1[e, 0:I, :]^T          (gate, fp32 accumulation)
 *     u = x[t] . W1[e, I:2I, :]^T         (up)
 *     a = silu(g) * u                     (stored as bf16, round-to-nearest-even)
 *     y = a . W2[e]^T                     (fp32 accumulation)
 *     out[t] = sum over k of w * y        (fp32)
 *
 * The routing ids and weights are inputs: the softmax / top-k / renormalise
 * step that produces them (the "Input Generation" section of the same page)
 * happens before this library is called. Weights are used as given.
 *
 * Conventions shared by every entry point:
 *  - All array arguments are DEVICE pointers on the current HIP device,
 *    owned by the caller; nothing is retained after the call returns.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream)
 *    and the call returns without waiting for it, unless a flag says
 *    otherwise. Buffers must stay alive until the stream has passed the work.
 *  - Return value: MOE_OK (0) or a negative MOE_ERR_* code; moe_last_error()
 *    then gives a message for the calling thread.
 *  - Layouts are dense row-major:
 *      hidden        bf16  [T, H]
 *      w1            bf16  [E, 2I, H]   rows 0..I-1 gate, rows I..2I-1 up
 *      w2            bf16  [E, H, I]
 *      topk_weights  fp32  [T, K]
 *      topk_ids      int32 [T, K]
 *      out           fp32  [T, H]       fully overwritten
 *  - Preconditions: H and I are multiples of 128 (the same alignment rule
 *    the tpu-inference kernel enforces on hidden and intermediate sizes);
 *    1 <= K <= E <= 1024; T >= 0. T == 0 is a successful no-op.
 *  - Ids are expected distinct per token and inside [0, E). An id outside
 *    [0, E) never causes an out-of-bounds access: that (t,k) pair is dropped
 *    (contributes nothing). With MOE_FLAG_VALIDATE_IDS the call additionally
 *    synchronises the stream and returns MOE_ERR_INVALID_ARG if any id was
 *    out of range or repeated within a token.
 */
#ifndef MOE_TOPK_IDS_H
#define MOE_TOPK_IDS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_OK 0
#define MOE_ERR_INVALID_ARG (-1) /* null pointer with T > 0, bad sizes, K > E, bad ids */
#define MOE_ERR_UNSUPPORTED (-2) /* H or I not a multiple of 128, E > 1024, ... */
#define MOE_ERR_HIP (-3)         /* a HIP runtime call failed */
#define MOE_ERR_ALLOC (-4)       /* internal workspace: allocation failed or above MOE_WORKSPACE_LIMIT */
#define MOE_ERR_WORKSPACE (-5)   /* caller workspace too small or misaligned */

/* Combine the K expert outputs with fp32 atomic adds straight from the down
 * projection into a zeroed `out`, instead of the default deterministic
 * per-(token,k) slot write followed by a weighted sum in k order. The order
 * of the adds is not fixed; for K <= 2 the result is still run-to-run
 * identical and equal to the default path's bits (0 + a + b in either order,
 * every add rounded to nearest even). */
#define MOE_FLAG_ATOMIC_COMBINE 1u
/* Force the grouped (routing + two grouped GEMMs) path. */
#define MOE_FLAG_FORCE_GROUPED 2u
/* Force the per-token weight-streaming path (each slot streams its own
 * expert's rows; meant for one or two tokens). */
#define MOE_FLAG_FORCE_DECODE 4u
/* Synchronise the stream after every stage and name the first stage whose
 * kernels failed in moe_last_error(). The workspace layout then also holds a
 * 256-byte guard band after every region (moe_workspace_bytes with this flag
 * counts them), filled before the first stage and compared after each: a
 * stage that wrote past its region returns MOE_ERR_WORKSPACE naming the
 * stage and the region. */
#define MOE_FLAG_DEBUG_SYNC 8u
/* Check ids on the device; see the preconditions above. Synchronises. */
#define MOE_FLAG_VALIDATE_IDS 16u
/* Force the expert-deduplicated small-batch path (each routed expert's rows
 * streamed once for all slots routed to it; T*K <= 1024). */
#define MOE_FLAG_FORCE_SMALL_BATCH 32u
/* For moe_workspace_bytes and moe_path: the sizes and path of
 * moe_forward_fp8 (FP8 weights). moe_forward_fp8 sets it itself; the bf16
 * entry points ignore it. */
#define MOE_FLAG_FP8_WEIGHTS 64u
/* Expert outputs on the grouped path's default (slot) combine: with
 * MOE_FLAG_BF16_Y each down-projection result y_{t,k} is stored rounded to
 * bf16 (round to nearest even) and the weighted sum reads it back, half the
 * bytes of fp32 rows; with MOE_FLAG_FP32_Y it stays fp32. Without either
 * flag the library chooses (moe_y_bf16 says which). The bf16 rounding is
 * the one tpu-inference's fused_moe kernel applies to its down projection's
 * results: out[t] = sum_k w * (bf16(y_{t,k}) + b2[e_k]) in fp32, k order. */
#define MOE_FLAG_BF16_Y 128u
#define MOE_FLAG_FP32_Y 256u
/* Grouped path: run the down projection in one launch even where its last
 * round of 192- or 256-row tiles would leave half the chip idle (by default
 * those tiles then run as column halves in a second launch). The results
 * are the same bits either way; for measurement. */
#define MOE_FLAG_NO_TAIL_SPLIT 512u

/* Paths, as returned by moe_path. A FORCE flag whose path does not support
 * the sizes falls back to the grouped path. */
#define MOE_PATH_GROUPED 0     /* routing + two grouped MFMA GEMMs + combine */
#define MOE_PATH_DECODE 1      /* per-token weight streaming, two kernels */
#define MOE_PATH_SMALL_BATCH 2 /* per-expert weight streaming + combine */

/*
 * The fused forward: out = sum_k topk_weights[:,k] * Expert_{topk_ids[:,k]}(hidden).
 * Uses a per-device workspace that the library allocates on first use and
 * grows as needed (freed by moe_release); the first call for a new maximum
 * size allocates and is therefore not graph-capture safe. Calls that use the
 * internal workspace of one device share it: they must be ordered (one
 * stream, or synchronised), else give each concurrent caller its own
 * workspace through moe_forward_ex. Two environment variables, read once
 * per process, set its flags: MOE_COMBINE ("slot", the default, or "atomic":
 * MOE_FLAG_ATOMIC_COMBINE) and MOE_DEBUG_SYNC (any value but "" or "0":
 * MOE_FLAG_DEBUG_SYNC). A third, MOE_WORKSPACE_LIMIT (bytes; unset or 0 for
 * none), caps the internal workspace of every entry point that uses it: a
 * call that would need more returns MOE_ERR_ALLOC before any device work.
 */
int moe_forward(const void* hidden, const void* w1, const void* w2,
                const float* topk_weights, const int32_t* topk_ids,
                int64_t T, int64_t H, int64_t I, int64_t E, int64_t K,
                float* out, void* stream);

/*
 * As moe_forward, with explicit flags (MOE_FLAG_*) and an optional caller
 * workspace. If `workspace` is NULL the internal workspace is used; else it
 * must be a device buffer of at least moe_workspace_bytes(...) bytes, 256-byte
 * aligned, used exclusively by this call until the stream passes it. With a
 * caller workspace the call performs no allocation.
 */
int moe_forward_ex(const void* hidden, const void* w1, const void* w2,
                   const float* topk_weights, const int32_t* topk_ids,
                   int64_t T, int64_t H, int64_t I, int64_t E, int64_t K,
                   float* out, uint32_t flags, void* workspace, size_t workspace_bytes,
                   void* stream);

/*
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc. The same
 * forward as moe_forward_ex (same kernels, same bits) with no allocation and
 * no caller workspace: its workspace is a static device array of
 * MOE_NOALLOC_SCRATCH_BYTES, which every GPU the library runs on holds from
 * the first call on that device until the process ends. Sizes whose
 * workspace (moe_workspace_bytes(T, H, I, E, K, flags)) exceeds it return
 * MOE_ERR_WORKSPACE with a message naming both sizes; 128 MiB holds every
 * per-token and small-batch call and grouped calls up to T=4195, H=I=2048,
 * E=8, top-2. Every call on one GPU uses that GPU's one array: calls that
 * overlap on one GPU (different streams, or threads without ordering) race;
 * order them on one stream. The array keeps the last call's contents; no
 * kernel relies on it starting at zero. Flags as moe_forward_ex (bf16
 * weights; MOE_FLAG_VALIDATE_IDS and MOE_FLAG_DEBUG_SYNC synchronise the
 * stream and so do not belong in a captured graph).
 */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
int moe_forward_noalloc(const void* hidden, const void* w1, const void* w2,
                        const float* topk_weights, const int32_t* topk_ids,
                        int64_t T, int64_t H, int64_t I, int64_t E, int64_t K,
                        float* out, uint32_t flags, void* stream);

/* Gated activations (the later tpu-inference fused_moe kernel.py,
 * activation_fn and swigluoai): */
#define MOE_ACT_SILU 0      /* silu(g) * u                                    */
#define MOE_ACT_GELU_TANH 1 /* gelu(g) * u, tanh form (jax.nn.gelu's default) */
#define MOE_ACT_SWIGLUOAI 2 /* (clip(u, -limit, limit) + 1) * gc * sigmoid(alpha * gc),
                               gc = min(g, limit); alpha 1.702, limit 7 there */
#define MOE_ACT_GELU_ERF 3  /* gelu(g) * u, erf form                          */

/*
 * As moe_forward_ex, with a gated activation variant and optional fp32 expert
 * biases (ref_moe of the later tpu-inference fused_moe kernel.py):
 *   b1  fp32 [E, 2I] or NULL: b1[e, 0:I] is added to the gate projection and
 *       b1[e, I:2I] to the up projection, before the activation;
 *   b2  fp32 [E, H] or NULL: added to expert e's down projection before its
 *       routing weight: out[t] = sum_k w[t,k] * (y_{t,k} + b2[e_k]).
 * `alpha` and `limit` are read for MOE_ACT_SWIGLUOAI only (limit >= 0).
 * Returns MOE_ERR_INVALID_ARG for an unknown activation. moe_forward_ex is
 * this call with MOE_ACT_SILU and no biases.
 */
int moe_forward_act(const void* hidden, const void* w1, const void* w2,
                    const float* topk_weights, const int32_t* topk_ids,
                    int64_t T, int64_t H, int64_t I, int64_t E, int64_t K,
                    int32_t activation, float alpha, float limit,
                    const float* b1, const float* b2,
                    float* out, uint32_t flags, void* workspace, size_t workspace_bytes,
                    void* stream);

/*
 * As moe_forward_act, with expert weights quantised to OCP FP8 E4M3 (1 byte
 * per weight: sign, 4 exponent bits with bias 7, 3 mantissa bits; 0x7F and
 * 0xFF are NaN) and one fp32 scale per `block` consecutive weights along the
 * contraction axis (the sub-channel quantisation of the later tpu-inference
 * fused_moe kernel.py, ref_moe's w1_scale and w2_scale):
 *   w1q       uint8 [E, 2I, H]         w1[e,n,h] = fp8(w1q[e,n,h]) * w1_scale[e,n,h/block]
 *   w1_scale  fp32  [E, 2I, H/block]
 *   w2q       uint8 [E, H, I]          w2[e,h,i] = fp8(w2q[e,h,i]) * w2_scale[e,h,i/block]
 *   w2_scale  fp32  [E, H, I/block]
 * `block` must be a multiple of 128 dividing H and I (MOE_ERR_UNSUPPORTED
 * otherwise). The per-token and small-batch paths read the codes directly;
 * the grouped path widens all weights to bf16 in its workspace first (the
 * fp32 product rounded to bf16), so its workspace holds a bf16 copy of w1 and
 * w2: size it with moe_workspace_bytes(..., flags | MOE_FLAG_FP8_WEIGHTS).
 */
int moe_forward_fp8(const void* hidden, const uint8_t* w1q, const float* w1_scale,
                    const uint8_t* w2q, const float* w2_scale, int64_t block,
                    const float* topk_weights, const int32_t* topk_ids,
                    int64_t T, int64_t H, int64_t I, int64_t E, int64_t K,
                    int32_t activation, float alpha, float limit,
                    const float* b1, const float* b2,
                    float* out, uint32_t flags, void* workspace, size_t workspace_bytes,
                    void* stream);

/* Bytes of workspace moe_forward_ex needs for these sizes and flags
 * (0 for T == 0). Returns 0 and sets the last error on invalid sizes. */
size_t moe_workspace_bytes(int64_t T, int64_t H, int64_t I, int64_t E, int64_t K,
                           uint32_t flags);

/* The row tile M that the grouped path pads each expert's rows to, for these
 * sizes and flags (the value moe_route must be given to reproduce the
 * forward's routing). Returns a negative MOE_ERR_* code on invalid sizes. */
int32_t moe_m_tile(int64_t T, int64_t H, int64_t I, int64_t E, int64_t K, uint32_t flags);

/* 1 if moe_forward_ex would take the per-token weight-streaming path for
 * these sizes and flags, 0 otherwise, negative MOE_ERR_* on invalid sizes. */
int moe_uses_decode_path(int64_t T, int64_t H, int64_t I, int64_t E, int64_t K, uint32_t flags);

/* The MOE_PATH_* moe_forward_ex takes for these sizes and flags, or a
 * negative MOE_ERR_* code on invalid sizes. */
int moe_path(int64_t T, int64_t H, int64_t I, int64_t E, int64_t K, uint32_t flags);

/* 1 if moe_forward_ex (and moe_forward_act / moe_forward_fp8 with these
 * flags) rounds each expert output y_{t,k} to bf16 before the weighted sum
 * for these sizes and flags (grouped path, slot combine), 0 if it keeps
 * them fp32, negative MOE_ERR_* on invalid sizes. */
int moe_y_bf16(int64_t T, int64_t H, int64_t I, int64_t E, int64_t K, uint32_t flags);

/* 1 if moe_forward_ex, for these sizes and flags, plans the down
 * projection's last partial round as column halves in a second launch (see
 * MOE_FLAG_NO_TAIL_SPLIT; the kernels confirm it from the routing's tile
 * count), 0 if not, negative MOE_ERR_* on invalid sizes. */
int moe_down_tail_split(int64_t T, int64_t H, int64_t I, int64_t E, int64_t K, uint32_t flags);

/*
 * The routing step alone (the grouping that tpu-inference's start_a2a_scatter
 * performs when it places each (token, k) pair into its expert's contiguous
 * buffer, walking tokens in order and k in order inside a token). With slot
 * f = t*K + k:
 *   counts[E]        slots per expert (ids outside [0,E) are not counted)
 *   offsets[E+1]     exclusive prefix sums of counts rounded up to m_tile
 *   sorted[cap]      padded row -> slot f, grouped by expert, ascending f
 *                    inside an expert; rows past an expert's count up to
 *                    its padded end hold -1. Only rows < offsets[E] are written.
 *   slot_of[T*K]     slot -> padded row; -1 for a dropped (out-of-range) id
 *   tile_expert[cap/m_tile]  expert of each m_tile-row tile
 *   num_tiles[1]     offsets[E] / m_tile
 * `capacity` is the length of `sorted`; it must be at least
 * T*K + min(E, T*K)*(m_tile-1). m_tile must be a multiple of 16 in [16, 256].
 * `scratch` is a device buffer of at least moe_route_scratch_bytes(T,K,E)
 * bytes. Deterministic: the output is a pure function of the ids.
 */
int moe_route(const int32_t* topk_ids, int64_t T, int64_t K, int64_t E, int32_t m_tile,
              int32_t* counts, int32_t* offsets, int32_t* sorted, int32_t* slot_of,
              int32_t* tile_expert, int32_t* num_tiles, int64_t capacity,
              void* scratch, void* stream);
size_t moe_route_scratch_bytes(int64_t T, int64_t K, int64_t E);

/*
 * The first grouped GEMM with its fused activation, on routing arrays from
 * moe_route (same m_tile): for every padded row r < offsets[E] holding slot
 * f = sorted[r] >= 0, act[r, :] = bf16_rne(silu(g) * u) for token f / K and
 * expert tile_expert[r / m_tile]; pad rows get zeros. act is bf16
 * [capacity, I] (row-major); rows >= offsets[E] are not written.
 * `max_tiles` = capacity / m_tile bounds the launch. m_tile must be 64, 128,
 * 192 or 256 (the row tiles the grouped GEMMs are built for; moe_m_tile
 * returns one of them). sorted, tile_expert and num_tiles must come from
 * moe_route called with the same E and m_tile (and these T, K); a tile whose
 * expert is outside [0, E) is skipped, never read past w1. When m_tile equals
 * moe_m_tile(T, H, I, E, K, 0) this runs exactly the gate/up kernel (tile
 * width included) that moe_forward runs for these sizes.
 */
int moe_gemm1_silu(const void* hidden, const void* w1, const int32_t* sorted,
                   const int32_t* tile_expert, const int32_t* num_tiles,
                   int64_t T, int64_t H, int64_t I, int64_t E, int64_t K, int32_t m_tile,
                   int64_t max_tiles, void* act, void* stream);

/*
 * moe_gemm1_silu with FP8 E4M3 gate/up weights (the layout of
 * moe_forward_fp8: w1q uint8 [E, 2I, H], w1_scale fp32 [E, 2I, H/block]):
 * the weight tiles are read as codes and each fragment is widened in
 * registers to bf16_rne(fp32(code) * scale) before the bf16 matrix ops, the
 * step tpu-inference's fused_moe kernel.py (sub-channel quantisation)
 * performs when it scales each contraction block of its w1/w3 product.
 * Also MOE_ERR_UNSUPPORTED when H/block or I/block exceeds 32.
 */
int moe_gemm1_silu_fp8(const void* hidden, const uint8_t* w1q, const float* w1_scale,
                       int64_t block, const int32_t* sorted, const int32_t* tile_expert,
                       const int32_t* num_tiles, int64_t T, int64_t H, int64_t I, int64_t E,
                       int64_t K, int32_t m_tile, int64_t max_tiles, void* act, void* stream);

/* With FP8 weights the grouped path either widens fragments inside its GEMMs
 * (returns 1) or first widens every expert to bf16 in the workspace and runs
 * the bf16 GEMMs (returns 0), whichever is cheaper for these sizes; negative
 * MOE_ERR_* on invalid sizes or block. */
int moe_fp8_widens_in_gemm(int64_t T, int64_t H, int64_t I, int64_t E, int64_t K,
                           int64_t block);

/*
 * The router that produces topk_weights / topk_ids from fp32 router logits
 * [T,E] (the softmax-then-top-k step of the atrex-bench #009 "Input
 * Generation" section, tpu-inference get_top_k, metrale
 * moe_topk_softmax_batched):
 *   p[e] = softmax over the E logits of the token (fp32);
 *   ids[t, 0..K-1] = the K experts with the largest logits, in descending
 *       order, ties to the lower id (the same order as the probabilities);
 *   weights[t,k] = p[ids[t,k]], divided by sum_k p[ids[t,k]] if
 *       `renormalize` is non-zero.
 * logits fp32 [T,E] row-major (finite values); weights fp32 [T,K]; ids int32
 * [T,K]. 1 <= K <= min(E, 32), E <= 1024. Asynchronous on `stream`.
 */
int moe_topk_softmax(const float* router_logits, int64_t T, int64_t E, int64_t K,
                     int renormalize, float* topk_weights, int32_t* topk_ids, void* stream);

/* Message for the last failing call on this thread ("" if none). */
const char* moe_last_error(void);

/* Free the internal workspaces of every device (after synchronising them). */
void moe_release(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_TOPK_IDS_H */
