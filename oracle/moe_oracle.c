/*
 * CPU oracle of the fused MoE layer.  TEST INFRASTRUCTURE ONLY: it is used by
 * tests/, by the smoke check and by the CPU-baseline leg of the benchmark, and
 * never by the library's product path.  It shares no code with the HIP path.
 *
 * Plain, slow and obviously correct: loops in the order the method states,
 * float64 arithmetic, no blocking, fusion or reordering.  Where a float decides
 * an integer (top-k selection, fp8 codes) the decision is taken in float32,
 * the precision the kernels use, so both sides can agree bit for bit.
 *
 * Sources ("the pages"):
 *  [MK]  vllm/model_executor/layers/fused_moe/modular_kernel.py (vllm-cpu
 *        0.11.0.post2 wheel listing): the header comment that splits the layer
 *        into [Router] -> [Quantize-Dispatch] -> [Permute-Experts-Unpermute]
 *        -> [Combine]; _moe_problem_size; FusedMoEActivationFormat;
 *        ExpertTokensMetadata; FusedMoEPrepareAndFinalize.prepare / finalize;
 *        FusedMoEPermuteExpertsUnpermute.activation / apply;
 *        FusedMoEModularKernel.forward.
 *  [WT]  "EP: CUDA-graph-safe HT internode dispatch+combine (worst-tokens
 *        mode)": per-expert counts in a device int32 tensor, masked grouped
 *        GEMM over padded per-expert buffers.
 *  [SE]  SharedExperts (vllm fused_moe/runner/shared_experts): the shared
 *        expert is a separate dense layer whose output is returned beside the
 *        routed output.
 *
 * Readings where the pages are silent (each is listed with its reason in the
 * design notes):
 *  - router: score = softmax over all E logits, or sigmoid; the k experts with
 *    the largest logits are picked, ties to the lower index, emitted in
 *    descending order; optional renormalisation over the k picks.
 *  - w1 holds the gate rows [0, I) then the up rows [I, 2I).
 *  - token-group fp8: scale = max(amax, 1e-10) / 448 in fp32, code = OCP
 *    e4m3fn round-to-nearest-even of clamp(x / scale, -448, 448).
 *  - Standard layout: expert segments padded to a multiple of `align`, pad
 *    slots hold -1; inside a segment pairs keep ascending flat index m*k+j.
 *  - Batched layout: a pair's slot is its rank among the pairs of its expert
 *    (ascending flat index); ranks >= capacity are dropped.
 *  - gelu_and_mul: the exact GELU, g * Phi(g) = 0.5 g (1 + erf(g / sqrt 2)).
 *  - Expert-parallel shard (expert_map: global -> local expert, -1 = held by
 *    another shard): the router runs over the global experts; pairs of other
 *    shards are neither counted nor computed and add nothing to this shard's
 *    output, so the shards' outputs sum to the unsharded layer's.
 *  - Router weight on the input (topk = 1): the weight multiplies the input
 *    row, which is then held in the activation dtype (the exact product
 *    rounded to fp32, and to bf16 for bf16 activations) before any
 *    quantisation; the combine then adds the expert output unweighted.
 *
 * Parity unpinned (conventions the pages leave open, shared by both sides):
 * the gate/up half order, the 1e-10 floor in the fp8 scale and the Zipf
 * construction of the skewed workload's logits.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { OR_F32 = 0, OR_BF16 = 1, OR_FP8 = 2 };
enum { OR_SOFTMAX = 0, OR_SIGMOID = 1 };
enum { OR_STANDARD = 0, OR_BATCHED = 1 };
enum { OR_SILU = 0, OR_GELU = 1 };

/* ---------------------------------------------------------------- formats */

/* bfloat16 is the top half of an IEEE float32. */
static double bf16_value(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* OCP e4m3fn: 1 sign, 4 exponent (bias 7), 3 mantissa bits; exponent 0 is
 * subnormal (m/8 * 2^-6); 0x7f / 0xff are NaN; no infinities; max 448. */
double oracle_e4m3_decode(uint8_t c) {
  int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    v = ldexp((double)m, -9);
  else
    v = ldexp((double)(8 + m), e - 10);
  return s ? -v : v;
}

/* Nearest e4m3fn code, ties to the even code (mantissa LSB 0), by plain search
 * over the 127 finite magnitudes.  Magnitudes >= 448 saturate to 448 (callers
 * clamp before encoding, so this branch only guards misuse). */
uint8_t oracle_e4m3_encode(float v) {
  if (isnan(v)) return 0x7f;
  uint8_t sign = signbit(v) ? 0x80 : 0;
  double a = fabs((double)v);
  if (a >= 448.0) return sign | 0x7e;
  int best = 0;
  double bestd = INFINITY;
  for (int c = 0; c <= 0x7e; ++c) {
    double d = fabs(oracle_e4m3_decode((uint8_t)c) - a);
    if (d < bestd || (d == bestd && (c & 1) == 0)) {
      best = c;
      bestd = d;
    }
  }
  return sign | (uint8_t)best;
}

/* Element-wise forms of the two functions above, for whole arrays. */
void oracle_e4m3_encode_array(int64_t n, const float *v, uint8_t *out) {
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_e4m3_encode(v[i]);
}

void oracle_e4m3_decode_array(int64_t n, const uint8_t *c, double *out) {
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_e4m3_decode(c[i]);
}

/* Per-token-group quantisation with group 128 ([MK] FusedMoEPrepareAndFinalize
 * .prepare, which quantises the input as the quant config asks (block_shape /
 * per_act_token_quant); the a2 scale keeps the second GEMM's input quantised
 * the same way).  x is [rows, cols] fp32, q [rows, cols], s [rows, cols/128]. */
void oracle_quant_g128(int64_t rows, int64_t cols, const float *x, uint8_t *q, float *s) {
  int64_t G = cols / 128;
  for (int64_t r = 0; r < rows; ++r) {
    for (int64_t g = 0; g < G; ++g) {
      const float *xg = x + r * cols + g * 128;
      float amax = 0.0f;
      for (int i = 0; i < 128; ++i) {
        float a = fabsf(xg[i]);
        if (a > amax) amax = a;
      }
      float sc = fmaxf(amax, 1e-10f) / 448.0f;
      s[r * G + g] = sc;
      for (int i = 0; i < 128; ++i) {
        float t = xg[i] / sc;
        if (t > 448.0f) t = 448.0f;
        if (t < -448.0f) t = -448.0f;
        q[r * cols + g * 128 + i] = oracle_e4m3_encode(t);
      }
    }
  }
}

/* Element (r, c) of expert e of a weight tensor [E, R, C] as float64; fp8
 * weights carry one fp32 scale per 128x128 block, scale [E, R/128, C/128]. */
static double weight_at(int dtype, const void *w, const float *scale, int64_t e, int64_t R,
                        int64_t C, int64_t r, int64_t c) {
  int64_t idx = (e * R + r) * C + c;
  switch (dtype) {
    case OR_F32:
      return (double)((const float *)w)[idx];
    case OR_BF16:
      return bf16_value(((const uint16_t *)w)[idx]);
    default: {
      double sc = scale[(e * (R / 128) + r / 128) * (C / 128) + c / 128];
      return oracle_e4m3_decode(((const uint8_t *)w)[idx]) * sc;
    }
  }
}

static double act_at(int dtype, const void *x, int64_t idx) {
  return dtype == OR_F32 ? (double)((const float *)x)[idx] : bf16_value(((const uint16_t *)x)[idx]);
}

/* ----------------------------------------------------------------- router */

/* [Router] of the [MK] header comment; forward() consumes its topk_weights
 * [M, k] and topk_ids [M, k].  Selection compares the fp32 logits (both score
 * maps are increasing, so this is top-k of the scores). */
void oracle_route(int64_t M, int64_t E, int64_t k, const float *logits, int scoring,
                  int renormalize, int32_t *ids, double *weights) {
  char *taken = (char *)malloc((size_t)E);
  for (int64_t m = 0; m < M; ++m) {
    const float *l = logits + m * E;
    memset(taken, 0, (size_t)E);
    for (int64_t j = 0; j < k; ++j) {
      int64_t best = -1;
      for (int64_t e = 0; e < E; ++e)
        if (!taken[e] && (best < 0 || l[e] > l[best])) best = e;
      taken[best] = 1;
      ids[m * k + j] = (int32_t)best;
    }
    double mx = -INFINITY, den = 0.0;
    if (scoring == OR_SOFTMAX) {
      for (int64_t e = 0; e < E; ++e)
        if ((double)l[e] > mx) mx = (double)l[e];
      for (int64_t e = 0; e < E; ++e) den += exp((double)l[e] - mx);
    }
    double sum = 0.0;
    for (int64_t j = 0; j < k; ++j) {
      double z = (double)l[ids[m * k + j]];
      double p = scoring == OR_SOFTMAX ? exp(z - mx) / den : 1.0 / (1.0 + exp(-z));
      weights[m * k + j] = p;
      sum += p;
    }
    if (renormalize)
      for (int64_t j = 0; j < k; ++j) weights[m * k + j] /= sum;
  }
  free(taken);
}

/* ------------------------------------------------- counting and permutation */

/* ExpertTokensMetadata.expert_num_tokens ([MK]): tokens routed to each
 * (local) expert.  A negative id is a pair held by another expert-parallel
 * shard and is not counted. */
void oracle_count(int64_t n, const int32_t *ids, int64_t E, int32_t *counts) {
  for (int64_t e = 0; e < E; ++e) counts[e] = 0;
  for (int64_t f = 0; f < n; ++f)
    if (ids[f] >= 0) counts[ids[f]]++;
}

/* Standard activation format ([MK] FusedMoEActivationFormat.Standard; the
 * "Permute" of [Permute-Experts-Unpermute]): a stable counting sort of the
 * n = M*k (token, slot) pairs by expert.  Expert e's segment starts at
 * offsets[e], the exclusive prefix sum of the counts rounded up to `align`;
 * perm[slot] = flat pair index m*k+j (-1 on pad slots), inv[pair] = slot.
 * Returns offsets[E] (the padded row total). */
int64_t oracle_permute_standard(int64_t n, const int32_t *ids, int64_t E, int64_t align,
                                int32_t *counts, int32_t *offsets, int32_t *perm,
                                int64_t perm_len, int32_t *inv) {
  oracle_count(n, ids, E, counts);
  offsets[0] = 0;
  for (int64_t e = 0; e < E; ++e)
    offsets[e + 1] = offsets[e] + (int32_t)(((counts[e] + align - 1) / align) * align);
  for (int64_t s = 0; s < perm_len; ++s) perm[s] = -1;
  int32_t *next = (int32_t *)malloc(sizeof(int32_t) * (size_t)E);
  for (int64_t e = 0; e < E; ++e) next[e] = offsets[e];
  for (int64_t f = 0; f < n; ++f) {
    if (ids[f] < 0) {          /* another shard's pair: no slot */
      inv[f] = -1;
      continue;
    }
    int32_t s = next[ids[f]]++;
    perm[s] = (int32_t)f;
    inv[f] = s;
  }
  free(next);
  return offsets[E];
}

/* BatchedExperts format ([MK] FusedMoEActivationFormat.BatchedExperts:
 * (num experts, max tokens per expert, hidden); [WT] worst-tokens buffers):
 * pair f goes to row e*cap + r of the padded buffer, r its rank among expert
 * e's pairs in ascending f; ranks >= cap do not fit and are dropped (-1).
 * counts[e] is the full number of pairs routed to e. */
void oracle_permute_batched(int64_t n, const int32_t *ids, int64_t E, int64_t cap,
                            int32_t *counts, int32_t *inv) {
  for (int64_t e = 0; e < E; ++e) counts[e] = 0;
  for (int64_t f = 0; f < n; ++f) {
    int32_t e = ids[f];
    if (e < 0) {               /* another shard's pair */
      inv[f] = -1;
      continue;
    }
    int32_t r = counts[e]++;
    inv[f] = r < cap ? (int32_t)(e * cap + r) : -1;
  }
}

/* ------------------------------------------------------------ expert MLP */

/* One expert on one input row ([MK] header comment: a GEMM, the gated
 * activation, optional quantisation, a second GEMM;
 * FusedMoEPermuteExpertsUnpermute.activation: silu_and_mul, whose output is
 * half the width of its input).
 *   h   = W1[e] a            (2I values; gate = h[0:I], up = h[I:2I])
 *   act = silu(gate) * up,   silu(z) = z / (1 + exp(-z))
 *      or gelu(gate) * up,   gelu(z) = 0.5 z (1 + erf(z / sqrt 2))  (gelu_and_mul)
 *   [fp8: act is re-quantised per group of 128 before the second GEMM]
 *   y   = W2[e] act          (K values)
 * a is [K]; act_out [I] receives act before any re-quantisation. */
void oracle_expert_row(int w_dtype, const void *w1, const float *w1_scale, const void *w2,
                       const float *w2_scale, int64_t e, int64_t K, int64_t I, int activation,
                       const double *a, int requant_fp8, double *act_out, double *y_out) {
  double *act = (double *)malloc(sizeof(double) * (size_t)I);
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < I; ++j) {
    double g = 0.0, u = 0.0;
    for (int64_t c = 0; c < K; ++c) {
      g += weight_at(w_dtype, w1, w1_scale, e, 2 * I, K, j, c) * a[c];
      u += weight_at(w_dtype, w1, w1_scale, e, 2 * I, K, I + j, c) * a[c];
    }
    if (activation == OR_GELU)
      act[j] = 0.5 * g * (1.0 + erf(g / sqrt(2.0))) * u;
    else
      act[j] = g / (1.0 + exp(-g)) * u;
  }
  if (act_out) memcpy(act_out, act, sizeof(double) * (size_t)I);
  if (requant_fp8) {
    float *af = (float *)malloc(sizeof(float) * (size_t)I);
    uint8_t *q = (uint8_t *)malloc((size_t)I);
    float *s = (float *)malloc(sizeof(float) * (size_t)(I / 128));
    for (int64_t j = 0; j < I; ++j) af[j] = (float)act[j];
    oracle_quant_g128(1, I, af, q, s);
    for (int64_t j = 0; j < I; ++j) act[j] = oracle_e4m3_decode(q[j]) * (double)s[j / 128];
    free(af);
    free(q);
    free(s);
  }
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < K; ++r) {
    double acc = 0.0;
    for (int64_t j = 0; j < I; ++j) acc += weight_at(w_dtype, w2, w2_scale, e, K, I, r, j) * act[j];
    y_out[r] = acc;
  }
  free(act);
}

/* bfloat16 round-to-nearest-even of a float32 (NaN kept quiet). */
static float round_bf16(float v) {
  uint32_t u;
  memcpy(&u, &v, 4);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) u |= 0x00400000u;
  else u += 0x7fffu + ((u >> 16) & 1u);
  u &= 0xffff0000u;
  float r;
  memcpy(&r, &u, 4);
  return r;
}

/* Element c of token m's input row: x itself, or with the router weight on
 * the input ([MK] prepare: with the flag set, the weights scale the
 * activations ahead of quantisation and dispatch) w * x held in the
 * activation dtype. */
static double input_value(int act_dtype, const void *x, int64_t K, int64_t m, int64_t c, int weighted,
                          float w) {
  double v = act_at(act_dtype, x, m * K + c);
  if (!weighted) return v;
  float p = (float)((double)w * v);   /* exact product, one rounding to fp32 */
  return act_dtype == OR_BF16 ? (double)round_bf16(p) : (double)p;
}

/* Input row of token m as the experts see it: x itself (weighted or not),
 * or with token-group fp8 quantisation the dequantised codes q*s ([MK]
 * prepare).  weighted != 0 applies router weight w to the input first. */
void oracle_input_row(int act_dtype, int act_quant, const void *x, int64_t K, int64_t m, int weighted,
                      float w, double *a) {
  if (!act_quant) {
    for (int64_t c = 0; c < K; ++c) a[c] = input_value(act_dtype, x, K, m, c, weighted, w);
    return;
  }
  float *xf = (float *)malloc(sizeof(float) * (size_t)K);
  uint8_t *q = (uint8_t *)malloc((size_t)K);
  float *s = (float *)malloc(sizeof(float) * (size_t)(K / 128));
  for (int64_t c = 0; c < K; ++c) xf[c] = (float)input_value(act_dtype, x, K, m, c, weighted, w);
  oracle_quant_g128(1, K, xf, q, s);
  for (int64_t c = 0; c < K; ++c) a[c] = oracle_e4m3_decode(q[c]) * (double)s[c / 128];
  free(xf);
  free(q);
  free(s);
}

/* --------------------------------------------------------------- combine */

/* [Combine]: TopKWeightAndReduce as described by FusedMoEPrepareAndFinalize
 * .finalize ([MK]): out[m] = sum_j w[m,j] * y[m,j,:], y being the unweighted,
 * unreduced (M, topk, K) expert output.  keep[m*k+j] == 0 drops a pair (a
 * batched row that did not fit); keep may be NULL. */
void oracle_combine(int64_t M, int64_t k, int64_t K, const double *w, const double *y,
                    const int32_t *keep, double *out) {
  for (int64_t m = 0; m < M; ++m) {
    for (int64_t c = 0; c < K; ++c) out[m * K + c] = 0.0;
    for (int64_t j = 0; j < k; ++j) {
      if (keep && !keep[m * k + j]) continue;
      for (int64_t c = 0; c < K; ++c) out[m * K + c] += w[m * k + j] * y[(m * k + j) * K + c];
    }
  }
}

/* --------------------------------------------------------------- layer */

/* The whole layer ([MK] FusedMoEModularKernel.forward) for a chosen subset of
 * tokens: route all M tokens over the Eg global experts (the batched format
 * needs every token's rank), map each pick to a local expert (expert_map;
 * NULL: global == local, Eg == E), then for each chosen token run the local
 * experts of its picks and combine; picks held by other shards add nothing.
 * weight_on_input (topk = 1): the router weight scales the input row and the
 * combine adds the expert output unweighted.  out is [ntok, K]; ids_out /
 * w_out ([ntok, k], global ids) may be NULL. */
int oracle_moe_tokens(int64_t M, int64_t K, int64_t I, int64_t E, int64_t Eg, int64_t k, int scoring,
                      int renormalize, int act_dtype, int w_dtype, int act_quant, int format,
                      int64_t cap, int activation, int weight_on_input, const int32_t *expert_map,
                      const float *logits, const void *x, const void *w1, const float *w1_scale,
                      const void *w2, const float *w2_scale, int64_t ntok, const int64_t *tokens,
                      double *out, int32_t *ids_out, double *w_out) {
  for (int64_t t = 0; t < ntok; ++t)
    if (tokens[t] < 0 || tokens[t] >= M) return -1;
  if (weight_on_input && k != 1) return -2;
  int32_t *ids = (int32_t *)malloc(sizeof(int32_t) * (size_t)(M * k));
  int32_t *lids = (int32_t *)malloc(sizeof(int32_t) * (size_t)(M * k));
  double *wts = (double *)malloc(sizeof(double) * (size_t)(M * k));
  int32_t *inv = NULL, *counts = NULL;
  oracle_route(M, Eg, k, logits, scoring, renormalize, ids, wts);
  for (int64_t f = 0; f < M * k; ++f) lids[f] = expert_map ? expert_map[ids[f]] : ids[f];
  if (format == OR_BATCHED) {
    inv = (int32_t *)malloc(sizeof(int32_t) * (size_t)(M * k));
    counts = (int32_t *)malloc(sizeof(int32_t) * (size_t)E);
    oracle_permute_batched(M * k, lids, E, cap, counts, inv);
  }
  double *a = (double *)malloc(sizeof(double) * (size_t)K);
  double *y = (double *)malloc(sizeof(double) * (size_t)(k * K));
  double *wc = (double *)malloc(sizeof(double) * (size_t)k);
  int32_t *keep = (int32_t *)malloc(sizeof(int32_t) * (size_t)k);
  for (int64_t t = 0; t < ntok; ++t) {
    int64_t m = tokens[t];
    oracle_input_row(act_dtype, act_quant, x, K, m, weight_on_input, (float)wts[m * k], a);
    for (int64_t j = 0; j < k; ++j) {
      if (ids_out) ids_out[t * k + j] = ids[m * k + j];
      if (w_out) w_out[t * k + j] = wts[m * k + j];
      wc[j] = weight_on_input ? 1.0 : wts[m * k + j];
      keep[j] = lids[m * k + j] >= 0 && !(inv && inv[m * k + j] < 0);
      if (keep[j])
        oracle_expert_row(w_dtype, w1, w1_scale, w2, w2_scale, lids[m * k + j], K, I, activation, a,
                          act_quant != 0, NULL, y + j * K);
    }
    oracle_combine(1, k, K, wc, y, keep, out + t * K);
  }
  free(a);
  free(y);
  free(wc);
  free(keep);
  free(ids);
  free(lids);
  free(wts);
  free(inv);
  free(counts);
  return 0;
}

/* Shared expert ([SE]; [MK] forward returns (shared_output, output)): the
 * same gated MLP (same activation) with one expert, applied to every token,
 * not routed and not weighted.  w1 [2I, K], w2 [K, I]; out [ntok, K]. */
int oracle_dense_mlp_tokens(int64_t M, int64_t K, int64_t I, int dtype, int activation, const void *x,
                            const void *w1, const void *w2, int64_t ntok, const int64_t *tokens,
                            double *out) {
  for (int64_t t = 0; t < ntok; ++t)
    if (tokens[t] < 0 || tokens[t] >= M) return -1;
  double *a = (double *)malloc(sizeof(double) * (size_t)K);
  for (int64_t t = 0; t < ntok; ++t) {
    int64_t m = tokens[t];
    oracle_input_row(dtype, 0, x, K, m, 0, 1.0f, a);
    oracle_expert_row(dtype, w1, NULL, w2, NULL, 0, K, I, activation, a, 0, NULL, out + t * K);
  }
  free(a);
  return 0;
}
