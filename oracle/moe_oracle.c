/*
 * Plain CPU oracle for the fused Mixture-of-Experts forward.
 *
 * TEST INFRASTRUCTURE ONLY. This file is the slow, obviously correct
 * definition that the GPU library is checked against. Only the test suite,
 * the smoke check and the benchmark's CPU-baseline leg may load it. It shares
 * no code, header, table or helper with the HIP library, and the HIP library
 * never calls it.
 *
 * Sources (cited by page title and section):
 *   [atrex-009]  atrex-bench operator #009 "fused_moe", section "Reference
 *                Implementation" (Model.forward): for each expert, the tokens
 *                routed to it are taken in fp32, multiplied by w1[e] (rows
 *                0..I-1 gate, rows I..2I-1 up; F.linear, i.e. x times w1[e]
 *                transposed), activated as silu(gate)*up, multiplied by w2[e]
 *                (again F.linear) and added, scaled by the routing weight,
 *                into an fp32 zero-initialised [T,H] output.
 *   [tpu-ref]    tpu-inference fused_moe v1 kernel.py, function ref_moe: the
 *                same computation walked per token, per chosen expert, with
 *                the per-token outputs summed with the top-k weights.
 *   [tpu-v2]     tpu-inference fused_moe kernel.py, the later version:
 *                activation_fn (silu(g)*u, gelu(g)*u with jax.nn.gelu's
 *                default tanh form, swigluoai), swigluoai (gate clipped from
 *                above and up clipped to [-limit, limit], then
 *                (up + 1) * gate * sigmoid(alpha * gate), alpha 1.702 and
 *                limit 7 by default), and ref_moe's optional fp32 biases: b1
 *                added to the gate and up projections before the
 *                activation, b2 added to each expert's down projection
 *                before the routing weight. Its ref_moe also takes quantised
 *                expert weights with per-block fp32 scales ("sub-channel"
 *                quantisation): each weight is its quantised value, widened
 *                to fp32, times the scale of its block of subc_quant_wsz
 *                consecutive elements along the contraction axis, for its
 *                own output column.
 *   [tpu-scatter] tpu-inference fused_moe v1 kernel.py, start_a2a_scatter:
 *                (token, k) pairs are placed into per-expert contiguous
 *                buffers by walking tokens in order and, inside a token, the
 *                k choices in order, bumping a per-expert cursor. This fixes
 *                the stable order used by the routing oracle below.
 *
 * Readings taken where the pages are silent (each restated in the design
 * notes): the combine adds the K weighted expert outputs in k order from 0;
 * the dot products accumulate in fp32 in ascending index order; silu(g) is
 * g / (1 + exp(-g)); the routing weights are used as given (never
 * renormalised here); in bf16-intermediate mode the activation silu(g)*u is
 * rounded to bf16 (round to nearest, ties to even) before the down
 * projection, mirroring the GPU's declared storage precision.
 *
 * Modes (the `mode` argument of the fp32 forwards, a bit mask):
 *   ORA_MODE_BF16_INTER (1)  the activation rounded to bf16, as above;
 *   ORA_MODE_BF16_Y     (2)  each expert's down-projection result y_{t,k}
 *                            rounded to bf16 (round to nearest, ties to even)
 *                            before its bias b2 and its routing weight are
 *                            applied, then accumulated in fp32 as before.
 *                            [tpu-ffn2] tpu-inference fused_moe v1 kernel.py,
 *                            dynamic_ffn2, brings the down projection's fp32
 *                            results to bf16 before accumulating them (by bit
 *                            truncation, with bf16 additions); the reading
 *                            here keeps one round-to-nearest-even per y_{t,k}
 *                            and fp32 accumulation.
 *
 * Build: gcc -O2 -ffp-contract=off -fopenmp -shared -fPIC (no fast-math), so
 * every fp32 operation is a separately rounded IEEE operation.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ */
/* bf16 <-> fp32 (bf16 is the upper half of an IEEE binary32)          */
/* ------------------------------------------------------------------ */

static float ora_bf16_to_f32(uint16_t b) {
  uint32_t u = ((uint32_t)b) << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* Round to nearest even. NaN stays NaN (quiet bit forced). */
static uint16_t ora_f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu) != 0u) {
    return (uint16_t)((u >> 16) | 0x0040u);
  }
  uint32_t lsb = (u >> 16) & 1u;
  uint32_t rounded = u + 0x7fffu + lsb;
  return (uint16_t)(rounded >> 16);
}

void oracle_f32_to_bf16(const float* in, uint16_t* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = ora_f32_to_bf16_rne(in[i]);
}

void oracle_bf16_to_f32(const uint16_t* in, float* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = ora_bf16_to_f32(in[i]);
}

/* ------------------------------------------------------------------ */
/* Routing oracle                                                      */
/* ------------------------------------------------------------------ */

/*
 * Groups the T*K (token, k) slots by expert, in the stable token-major,
 * k-minor order of [tpu-scatter], each expert's group padded up to a
 * multiple of the row tile M.
 *
 *   counts[e]      number of slots f = t*K + k with ids[f] == e
 *   offsets[e]     exclusive prefix sum of roundup(counts, M); offsets[E]
 *                  is the padded total P
 *   sorted[r]      slot f at padded row r; pad rows hold -1   (length P)
 *   slot_of[f]     padded row of slot f; -1 if ids[f] is outside [0, E)
 *   tile_expert[j] expert owning rows [j*M, (j+1)*M), j < P/M
 *   *num_tiles     P / M
 *
 * Returns 0, or -1 if sorted_cap < P or tile_cap < P/M.
 */
int oracle_route(const int32_t* ids, int64_t T, int64_t K, int64_t E, int64_t M,
                 int32_t* counts, int32_t* offsets, int32_t* sorted, int64_t sorted_cap,
                 int32_t* slot_of, int32_t* tile_expert, int64_t tile_cap,
                 int32_t* num_tiles) {
  const int64_t n = T * K;
  for (int64_t e = 0; e < E; ++e) counts[e] = 0;
  for (int64_t f = 0; f < n; ++f) {
    int32_t e = ids[f];
    if (e >= 0 && e < E) counts[e] += 1;
  }
  offsets[0] = 0;
  for (int64_t e = 0; e < E; ++e) {
    int64_t padded = ((counts[e] + M - 1) / M) * M;
    offsets[e + 1] = (int32_t)(offsets[e] + padded);
  }
  const int64_t P = offsets[E];
  if (P > sorted_cap || P / M > tile_cap) return -1;
  for (int64_t r = 0; r < P; ++r) sorted[r] = -1;
  int32_t* fill = (int32_t*)calloc((size_t)(E > 0 ? E : 1), sizeof(int32_t));
  for (int64_t f = 0; f < n; ++f) { /* ascending f: token-major, k-minor */
    int32_t e = ids[f];
    if (e < 0 || e >= E) {
      slot_of[f] = -1;
      continue;
    }
    int64_t r = offsets[e] + fill[e];
    fill[e] += 1;
    sorted[r] = (int32_t)f;
    slot_of[f] = (int32_t)r;
  }
  free(fill);
  for (int64_t e = 0; e < E; ++e)
    for (int64_t j = offsets[e] / M; j < offsets[e + 1] / M; ++j) tile_expert[j] = (int32_t)e;
  *num_tiles = (int32_t)(P / M);
  return 0;
}

/* ------------------------------------------------------------------ */
/* Gated activations ([atrex-009] silu; [tpu-v2] activation_fn)        */
/* ------------------------------------------------------------------ */

enum { ORA_ACT_SILU = 0, ORA_ACT_GELU_TANH = 1, ORA_ACT_SWIGLUOAI = 2, ORA_ACT_GELU_ERF = 3 };

/* act(g, u) in fp32, each operation rounded separately. */
static float ora_act_f32(float g, float u, int act, float alpha, float limit) {
  if (act == ORA_ACT_GELU_TANH) {
    /* 0.5 g (1 + tanh(sqrt(2/pi) (g + 0.044715 g^3))) */
    const float inner = 0.7978845608028654f * (g + 0.044715f * (g * g * g));
    return (0.5f * g * (1.0f + tanhf(inner))) * u;
  }
  if (act == ORA_ACT_GELU_ERF) /* 0.5 g (1 + erf(g / sqrt 2)) */
    return (0.5f * g * (1.0f + erff(g * 0.7071067811865476f))) * u;
  if (act == ORA_ACT_SWIGLUOAI) {
    const float gc = g < limit ? g : limit;
    const float uc = u < -limit ? -limit : (u > limit ? limit : u);
    const float glu = gc / (1.0f + expf(-(alpha * gc)));
    return (uc + 1.0f) * glu;
  }
  return (g / (1.0f + expf(-g))) * u; /* silu(g) * u */
}

static double ora_act_f64(double g, double u, int act, double alpha, double limit) {
  if (act == ORA_ACT_GELU_TANH) {
    const double inner = 0.79788456080286535588 * (g + 0.044715 * g * g * g);
    return 0.5 * g * (1.0 + tanh(inner)) * u;
  }
  if (act == ORA_ACT_GELU_ERF) return 0.5 * g * (1.0 + erf(g * 0.70710678118654752440)) * u;
  if (act == ORA_ACT_SWIGLUOAI) {
    const double gc = g < limit ? g : limit;
    const double uc = u < -limit ? -limit : (u > limit ? limit : u);
    return (uc + 1.0) * (gc / (1.0 + exp(-alpha * gc)));
  }
  return g / (1.0 + exp(-g)) * u;
}

/* ------------------------------------------------------------------ */
/* One expert applied to one token, fp32 ([atrex-009] Model.forward)   */
/* ------------------------------------------------------------------ */

/*
 * act[i] = act(g[i], u[i]) with g[i] = sum_h x[h]*w1[e,i,h] (+ b1e[i]) and
 * u[i] = sum_h x[h]*w1[e,I+i,h] (+ b1e[I+i]), fp32, h ascending; b1e may be
 * NULL (no bias). If bf16_inter, act is rounded to bf16 (RNE) and returned
 * widened back to fp32.
 */
static void ora_expert_act_f32(const uint16_t* x, const uint16_t* w1e, int64_t H, int64_t I,
                               int act_kind, float alpha, float limit, const float* b1e,
                               int bf16_inter, float* act) {
  for (int64_t i = 0; i < I; ++i) {
    const uint16_t* wg = w1e + i * H;
    const uint16_t* wu = w1e + (I + i) * H;
    float g = 0.0f, u = 0.0f;
    for (int64_t h = 0; h < H; ++h) {
      float xv = ora_bf16_to_f32(x[h]);
      g = g + xv * ora_bf16_to_f32(wg[h]);
      u = u + xv * ora_bf16_to_f32(wu[h]);
    }
    if (b1e) {
      g = g + b1e[i];
      u = u + b1e[I + i];
    }
    float a = ora_act_f32(g, u, act_kind, alpha, limit);
    if (bf16_inter) a = ora_bf16_to_f32(ora_f32_to_bf16_rne(a));
    act[i] = a;
  }
}

/* y[h] = sum_i act[i] * w2[e,h,i], fp32, i ascending. */
static void ora_expert_down_f32(const float* act, const uint16_t* w2e, int64_t H, int64_t I,
                                float* y) {
  for (int64_t h = 0; h < H; ++h) {
    const uint16_t* wr = w2e + h * I;
    float acc = 0.0f;
    for (int64_t i = 0; i < I; ++i) acc = acc + act[i] * ora_bf16_to_f32(wr[i]);
    y[h] = acc;
  }
}

/*
 * Full forward, fp32 ([atrex-009] Model.forward, [tpu-ref] ref_moe):
 *   out[t,h] = sum over k = 0..K-1 (in that order, from 0) of
 *              topk_weights[t,k] * y_{t,k}[h]
 * Slots whose id lies outside [0, E) contribute nothing.
 * x: bf16 [T,H]; w1: bf16 [E,2I,H]; w2: bf16 [E,H,I]; out: fp32 [T,H].
 */
/*
 * With an activation variant and optional biases ([tpu-v2] ref_moe):
 * act_kind 0 silu, 1 gelu (tanh form), 2 swigluoai(alpha, limit), 3 gelu
 * (erf form); b1 fp32 [E, 2I] (gate biases, then up biases) or NULL; b2 fp32
 * [E, H] or NULL, added to y before the routing weight:
 *   out[t,h] = sum_k topk_weights[t,k] * (y_{t,k}[h] + b2[e,h]).
 * mode: ORA_MODE_* bits (bf16 activation; bf16 y_{t,k} before b2 and w).
 */
#define ORA_MODE_BF16_INTER 1
#define ORA_MODE_BF16_Y 2

void oracle_moe_forward_act(const uint16_t* x, const uint16_t* w1, const uint16_t* w2,
                            const float* topk_weights, const int32_t* topk_ids, int64_t T,
                            int64_t H, int64_t I, int64_t E, int64_t K, int act_kind,
                            float alpha, float limit, const float* b1, const float* b2,
                            int mode, float* out) {
  const int bf16_inter = (mode & ORA_MODE_BF16_INTER) != 0;
  const int bf16_y = (mode & ORA_MODE_BF16_Y) != 0;
#pragma omp parallel
  {
    float* act = (float*)malloc((size_t)I * sizeof(float));
    float* y = (float*)malloc((size_t)H * sizeof(float));
#pragma omp for schedule(dynamic, 1)
    for (int64_t t = 0; t < T; ++t) {
      float* o = out + t * H;
      for (int64_t h = 0; h < H; ++h) o[h] = 0.0f;
      for (int64_t k = 0; k < K; ++k) {
        int32_t e = topk_ids[t * K + k];
        if (e < 0 || e >= E) continue;
        float w = topk_weights[t * K + k];
        ora_expert_act_f32(x + t * H, w1 + (int64_t)e * 2 * I * H, H, I, act_kind, alpha, limit,
                           b1 ? b1 + (int64_t)e * 2 * I : NULL, bf16_inter, act);
        ora_expert_down_f32(act, w2 + (int64_t)e * H * I, H, I, y);
        if (bf16_y)
          for (int64_t h = 0; h < H; ++h) y[h] = ora_bf16_to_f32(ora_f32_to_bf16_rne(y[h]));
        if (b2)
          for (int64_t h = 0; h < H; ++h) y[h] = y[h] + b2[(int64_t)e * H + h];
        for (int64_t h = 0; h < H; ++h) o[h] = o[h] + w * y[h];
      }
    }
    free(act);
    free(y);
  }
}

void oracle_moe_forward(const uint16_t* x, const uint16_t* w1, const uint16_t* w2,
                        const float* topk_weights, const int32_t* topk_ids, int64_t T,
                        int64_t H, int64_t I, int64_t E, int64_t K, int mode, float* out) {
  oracle_moe_forward_act(x, w1, w2, topk_weights, topk_ids, T, H, I, E, K, ORA_ACT_SILU, 0.0f,
                         0.0f, NULL, NULL, mode, out);
}

/*
 * The activation of every slot f = t*K + k as bf16 bits [T*K, I]
 * (bf16-intermediate mode), for checking the stored intermediate. Slots
 * with an out-of-range id are left as zero.
 */
void oracle_slot_act_bf16(const uint16_t* x, const uint16_t* w1, const int32_t* topk_ids,
                          int64_t T, int64_t H, int64_t I, int64_t E, int64_t K,
                          uint16_t* act_out) {
#pragma omp parallel
  {
    float* act = (float*)malloc((size_t)I * sizeof(float));
#pragma omp for schedule(dynamic, 1)
    for (int64_t f = 0; f < T * K; ++f) {
      int64_t t = f / K;
      int32_t e = topk_ids[f];
      uint16_t* dst = act_out + f * I;
      if (e < 0 || e >= E) {
        for (int64_t i = 0; i < I; ++i) dst[i] = 0;
        continue;
      }
      ora_expert_act_f32(x + t * H, w1 + (int64_t)e * 2 * I * H, H, I, ORA_ACT_SILU, 0.0f, 0.0f,
                         NULL, 0, act);
      for (int64_t i = 0; i < I; ++i) dst[i] = ora_f32_to_bf16_rne(act[i]);
    }
    free(act);
  }
}

/* ------------------------------------------------------------------ */
/* fp64 version of the same definition, for pinning the fp32 oracle    */
/* ------------------------------------------------------------------ */

void oracle_moe_forward_act_f64(const uint16_t* x, const uint16_t* w1, const uint16_t* w2,
                                const double* topk_weights, const int32_t* topk_ids, int64_t T,
                                int64_t H, int64_t I, int64_t E, int64_t K, int act_kind,
                                double alpha, double limit, const double* b1, const double* b2,
                                double* out) {
#pragma omp parallel
  {
    double* act = (double*)malloc((size_t)I * sizeof(double));
#pragma omp for schedule(dynamic, 1)
    for (int64_t t = 0; t < T; ++t) {
      double* o = out + t * H;
      for (int64_t h = 0; h < H; ++h) o[h] = 0.0;
      for (int64_t k = 0; k < K; ++k) {
        int32_t e = topk_ids[t * K + k];
        if (e < 0 || e >= E) continue;
        double w = topk_weights[t * K + k];
        const uint16_t* w1e = w1 + (int64_t)e * 2 * I * H;
        const uint16_t* w2e = w2 + (int64_t)e * H * I;
        for (int64_t i = 0; i < I; ++i) {
          double g = 0.0, u = 0.0;
          for (int64_t h = 0; h < H; ++h) {
            double xv = (double)ora_bf16_to_f32(x[t * H + h]);
            g += xv * (double)ora_bf16_to_f32(w1e[i * H + h]);
            u += xv * (double)ora_bf16_to_f32(w1e[(I + i) * H + h]);
          }
          if (b1) {
            g += b1[(int64_t)e * 2 * I + i];
            u += b1[(int64_t)e * 2 * I + I + i];
          }
          act[i] = ora_act_f64(g, u, act_kind, alpha, limit);
        }
        for (int64_t h = 0; h < H; ++h) {
          double acc = 0.0;
          for (int64_t i = 0; i < I; ++i) acc += act[i] * (double)ora_bf16_to_f32(w2e[h * I + i]);
          if (b2) acc += b2[(int64_t)e * H + h];
          o[h] += w * acc;
        }
      }
    }
    free(act);
  }
}

void oracle_moe_forward_f64(const uint16_t* x, const uint16_t* w1, const uint16_t* w2,
                            const double* topk_weights, const int32_t* topk_ids, int64_t T,
                            int64_t H, int64_t I, int64_t E, int64_t K, double* out) {
  oracle_moe_forward_act_f64(x, w1, w2, topk_weights, topk_ids, T, H, I, E, K, ORA_ACT_SILU, 0.0,
                             0.0, NULL, NULL, out);
}

/* ------------------------------------------------------------------ */
/* Quantised expert weights ([tpu-v2] ref_moe with w1_scale/w2_scale)  */
/* ------------------------------------------------------------------ */

/*
 * The quantised values are OCP FP8 E4M3 ("e4m3fn"): 1 sign bit, 4 exponent
 * bits (bias 7), 3 mantissa bits, no infinities, 0x7F and 0xFF NaN, exponent
 * field 0 for subnormals m * 2^-9. (The page leaves the quantised dtype
 * open; this is the format the matrix and conversion units of the target
 * read.)
 */
float oracle_fp8_e4m3_to_f32(uint8_t c) {
  const int sgn = c >> 7, ex = (c >> 3) & 15, m = c & 7;
  float v;
  if (ex == 15 && m == 7)
    v = NAN;
  else if (ex == 0)
    v = ldexpf((float)m, -9);
  else
    v = ldexpf(1.0f + (float)m / 8.0f, ex - 7);
  return sgn ? -v : v;
}

/*
 * Forward with quantised weights, fp32 ([tpu-v2] ref_moe):
 *   w1[e, n, h] = fp8(w1q[e, n, h]) * w1s[e, n, h / block]   (fp32 product)
 *   w2[e, h, i] = fp8(w2q[e, h, i]) * w2s[e, h, i / block]
 * then exactly oracle_moe_forward_act with those weights. Layouts: w1q uint8
 * [E, 2I, H], w1s fp32 [E, 2I, H/block], w2q uint8 [E, H, I], w2s fp32
 * [E, H, I/block]; block divides H and I.
 */
void oracle_moe_forward_q(const uint16_t* x, const uint8_t* w1q, const float* w1s,
                          const uint8_t* w2q, const float* w2s, int64_t block,
                          const float* topk_weights, const int32_t* topk_ids, int64_t T,
                          int64_t H, int64_t I, int64_t E, int64_t K, int act_kind, float alpha,
                          float limit, const float* b1, const float* b2, int mode,
                          float* out) {
  const int bf16_inter = (mode & ORA_MODE_BF16_INTER) != 0;
  const int bf16_y = (mode & ORA_MODE_BF16_Y) != 0;
  float lut[256];
  for (int c = 0; c < 256; ++c) lut[c] = oracle_fp8_e4m3_to_f32((uint8_t)c);
  const int64_t nb1 = H / block, nb2 = I / block;
#pragma omp parallel
  {
    float* act = (float*)malloc((size_t)I * sizeof(float));
#pragma omp for schedule(dynamic, 1)
    for (int64_t t = 0; t < T; ++t) {
      float* o = out + t * H;
      for (int64_t h = 0; h < H; ++h) o[h] = 0.0f;
      for (int64_t k = 0; k < K; ++k) {
        const int32_t e = topk_ids[t * K + k];
        if (e < 0 || e >= E) continue;
        const float w = topk_weights[t * K + k];
        for (int64_t i = 0; i < I; ++i) {
          const int64_t rg = (int64_t)e * 2 * I + i, ru = rg + I;
          float g = 0.0f, u = 0.0f;
          for (int64_t h = 0; h < H; ++h) {
            const float xv = ora_bf16_to_f32(x[t * H + h]);
            const float wg = lut[w1q[rg * H + h]] * w1s[rg * nb1 + h / block];
            const float wu = lut[w1q[ru * H + h]] * w1s[ru * nb1 + h / block];
            g = g + xv * wg;
            u = u + xv * wu;
          }
          if (b1) {
            g = g + b1[(int64_t)e * 2 * I + i];
            u = u + b1[(int64_t)e * 2 * I + I + i];
          }
          float a = ora_act_f32(g, u, act_kind, alpha, limit);
          if (bf16_inter) a = ora_bf16_to_f32(ora_f32_to_bf16_rne(a));
          act[i] = a;
        }
        for (int64_t h = 0; h < H; ++h) {
          const int64_t r = (int64_t)e * H + h;
          float acc = 0.0f;
          for (int64_t i = 0; i < I; ++i)
            acc = acc + act[i] * (lut[w2q[r * I + i]] * w2s[r * nb2 + i / block]);
          if (bf16_y) acc = ora_bf16_to_f32(ora_f32_to_bf16_rne(acc));
          if (b2) acc = acc + b2[(int64_t)e * H + h];
          o[h] = o[h] + w * acc;
        }
      }
    }
    free(act);
  }
}

/* ------------------------------------------------------------------ */
/* Router: softmax -> top-K -> renormalise                            */
/* ------------------------------------------------------------------ */

/*
 * For each token t (logits fp32 [T,E]):
 *   m = max_e logits[t,e];  p[e] = exp(logits[t,e] - m) / sum_e' exp(logits[t,e'] - m)
 *   ([atrex-009] Input Generation: softmax over experts; [tpu-ref] ref_moe and
 *   get_top_k in tpu-inference kernel.py apply softmax to the gating logits).
 *   K rounds of: pick the largest remaining expert, ties to the lowest id
 *   (get_top_k's argmax takes the first index), remove it.
 *   Selection compares the fp32 logits: softmax is strictly increasing, so
 *   this is the order of the exact probabilities, and it does not depend on
 *   how exp() rounds.
 *   ids[t,k] = chosen expert k (descending); weights[t,k] = p of that expert,
 *   divided, if renormalize, by the sum of the K chosen p added in k order
 *   (get_top_k's renormalisation; [atrex-009] divides by the sum of the top
 *   values). All arithmetic fp32, exp() from libm, sums in ascending order.
 */
void oracle_topk_softmax(const float* logits, int64_t T, int64_t E, int64_t K, int renormalize,
                         float* weights, int32_t* ids) {
#pragma omp parallel
  {
    unsigned char* taken = (unsigned char*)malloc((size_t)E);
#pragma omp for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
      const float* l = logits + t * E;
      float m = l[0];
      for (int64_t e = 1; e < E; ++e)
        if (l[e] > m) m = l[e];
      float denom = 0.0f;
      for (int64_t e = 0; e < E; ++e) denom = denom + expf(l[e] - m);
      for (int64_t e = 0; e < E; ++e) taken[e] = 0;
      float chosen_sum = 0.0f;
      for (int64_t k = 0; k < K; ++k) {
        int64_t best = -1;
        for (int64_t e = 0; e < E; ++e) {
          if (taken[e]) continue;
          if (best < 0 || l[e] > l[best]) best = e; /* strict: ties keep the lower id */
        }
        taken[best] = 1;
        ids[t * K + k] = (int32_t)best;
        const float p = expf(l[best] - m) / denom;
        weights[t * K + k] = p;
        chosen_sum = chosen_sum + p;
      }
      if (renormalize)
        for (int64_t k = 0; k < K; ++k) weights[t * K + k] = weights[t * K + k] / chosen_sum;
    }
    free(taken);
  }
}
