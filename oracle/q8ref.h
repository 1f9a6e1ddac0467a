/*
 * q8ref: the CPU oracle for the Q8_0 block-quantized matmul.
 *
 * TEST INFRASTRUCTURE ONLY.  Plain, slow, scalar C that states the method's
 * definition directly.  Only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark may load it.  It shares no code, header,
 * table or constant with the HIP library, and the HIP library never calls it.
 *
 * Sources of the definition (the three pages studied for this project):
 *  - Q8_0 block: one fp16 scale followed by 32 int8 values, 34 bytes
 *    ("Ember packed Q8 decode" post, row-contiguous source diagram).
 *  - Quantization: per 32-value block, scale d = amax / 127, values rounded to
 *    the nearest integer; activations are quantized with the same per-block
 *    scheme as the weights ("ferro" README, "How the iGPU path is fast",
 *    item 1; weights converted to Q8_0 at load time, "Using LFM2.5").
 *  - Block dot: exact int32 sum of 32 int8 products scaled by both fp16
 *    scales, block results reduced in fp32 per output row.
 *  - Packed tiles hold the same bytes as the row-contiguous blocks, only
 *    reordered: 544 bytes per 16 blocks ("Ember packed Q8 decode" post).
 *
 * Readings where the pages are silent (each is listed in the project's
 * design notes):
 *  - "round to nearest" ties go away from zero (C roundf);
 *  - x / d is one correctly rounded fp32 division by the fp32 scale d; the
 *    stored scale is d rounded to fp16 (round to nearest even, gradual
 *    underflow);
 *  - an all-zero block has d = 0, every q = 0 and a +0 stored scale;
 *  - the oracle's output is sum_b t_b accumulated in fp64 and rounded once to
 *    fp32, where t_b = fp32(s_b * (D_w * D_x)) (the fp16 x fp16 product is
 *    exact in fp32, so t_b carries one rounding); any fp32 summation order is
 *    within |err| <= 1e-5 * sum_b |t_b|, which is the acceptance bound.
 *
 * Layout codes (the oracle's own copies of the format definitions):
 *  0 ROWS   : row-contiguous Q8_0, rows x (k/32) blocks of [fp16 d][32 x int8].
 *  1 PACKED : records of 64 rows x 8 blocks (17,408 bytes = 512 blocks x 34),
 *             record (T, G) at byte (T * (k/256) + G) * 17408; inside it the
 *             int8 value of row 64T+r, column 256G + 32bb + 16h + j sits at
 *             bb*2048 + h*1024 + r*16 + j, and the fp16 scale of (r, bb) at
 *             16384 + r*16 + bb*2.  Needs n % 64 == 0 and k % 256 == 0.
 *  2 ACT    : planar activations, int8 [rows][k] followed by fp16
 *             [rows][k/32]; rows * k / 32 * 34 bytes in all.
 */
#ifndef Q8REF_H
#define Q8REF_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes. */
#define Q8REF_OK 0
#define Q8REF_EARG 1
#define Q8REF_ESHAPE 2

/* IEEE binary16 <-> binary32 from the bit definitions. */
uint16_t q8ref_f32_to_f16(float f);
float q8ref_f16_to_f32(uint16_t h);
void q8ref_f32_to_f16_n(const float *in, uint16_t *out, int64_t n);
void q8ref_f16_to_f32_n(const uint16_t *in, float *out, int64_t n);

/* One 32-value block: writes q[32], returns the stored fp16 scale bits and
 * (if d_out) the fp32 scale d used for the division. */
uint16_t q8ref_quantize_block(const float *x, int8_t *q, float *d_out);

/* The sum of n non-negative finite doubles, rounded once to fp64 (to nearest,
 * ties to even).  Every term is added exactly into a fixed-point integer that
 * holds every fp64 bit position, and that integer is rounded at the end, so
 * the result does not depend on the order of the terms.  A negative,
 * infinite or NaN term returns NaN. */
double q8ref_exact_sum(const double *v, int64_t n);

/* rows x k fp32 (row stride ld_x elements) -> layout 0 (ROWS) or 2 (ACT). */
int q8ref_quantize_rows(const float *x, int64_t ld_x, int64_t rows, int64_t k, int layout, uint8_t *out);

/* Fused producer: residual add + RMSNorm + Q8_0 quantization of each row
 * ("ferro" README, "How the iGPU path is fast", item 3: residual + norm +
 * int8 quantization in one pass, emitting the next GEMM's int8 input).  The
 * pages name the fusion but not the norm's formula or precision; the reading
 * taken (Llama's RMSNorm):
 *   h_j   = fp32(res_in_j + x_j), or x_j when res_in is NULL (a norm with
 *           no residual add, as before a model's first layer); written to
 *           res_out unless res_out is NULL
 *   ss    = sum_j (double)h_j^2, rounded once to fp64 (every square of an
 *           fp32 is exact in fp64; the sum is q8ref_exact_sum's, so no
 *           summation order enters the definition)
 *   r     = fp32(1.0 / sqrt(ss / k + eps)), all in correctly rounded fp64
 *   n_j   = fp32(fp32(h_j * r) * w_j)
 * and n is quantized per 32-value block as q8ref_quantize_block does, into
 * the ACT layout.  res_out may be the same buffer as res_in or x.  Returns Q8REF_OK, Q8REF_EARG or
 * Q8REF_ESHAPE (k % 32). */
int q8ref_rmsnorm_quantize(const float *x, const float *res_in, const float *w, int64_t rows, int64_t k, float eps,
                           float *res_out, uint8_t *q_out);

/* ROWS <-> PACKED byte permutations. */
int q8ref_pack(const uint8_t *w_rows, int64_t n, int64_t k, uint8_t *w_packed);
int q8ref_unpack(const uint8_t *w_packed, int64_t n, int64_t k, uint8_t *w_rows);

/* Per-block integer dots s[m][n][b] and terms t[m][n][b] (tiny shapes). */
int q8ref_block_terms(const uint8_t *x_act, int64_t m, const uint8_t *w_rows, int64_t n, int64_t k,
                      int32_t *s, float *t);

/* y[m][n] (row stride ld_y) and S[m][n] = sum_b |t_b| (may be NULL),
 * threads >= 1 split the output rows n; results do not depend on threads. */
int q8ref_matmul(const uint8_t *x_act, int64_t m, const uint8_t *w_rows, int64_t n, int64_t k,
                 float *y, int64_t ld_y, double *S, int threads);

/* Selected outputs: y[i] = output (mi[i], ni[i]) for i < count. */
int q8ref_matmul_points(const uint8_t *x_act, int64_t m, const uint8_t *w_rows, int64_t n, int64_t k,
                        const int64_t *mi, const int64_t *ni, int64_t count, float *y, double *S);

/* Routed experts: pair p = t * topk + j uses expert ids[p] and activation
 * row (x_per_pair ? p : t); y is [tokens * topk][n].  Expert e's ROWS
 * weights start at byte e * expert_stride of w_rows. */
int q8ref_grouped_matmul(const uint8_t *x_act, int64_t x_rows, int x_per_pair, const int32_t *ids,
                         int64_t tokens, int topk, const uint8_t *w_rows, int64_t n_experts,
                         int64_t expert_stride, int64_t n, int64_t k, float *y, double *S, int threads);

/* ---- around the routed experts: router, SwiGLU, weighted combine ---------
 * The pages name device routing, the real router's expert ids and weights,
 * and a sparse-MoE layer ("Ferrule" README: completed foundation, "device
 * routing"; runtime decision: the real router determines expert ids and
 * weights; status table: an OLMoE sparse-MoE path), without formulas.  The
 * readings taken (Mixtral/DeepSeek/OLMoE-style MoE):
 *  - exp is evaluated by one fixed fp64 algorithm for x <= 0, so that both
 *    sides reach the same fp32 results where they decide integer codes and
 *    expert weights (q8ref_exp_nonpos below);
 *  - top-k: the k largest logits, ties to the lower expert id, slots in
 *    descending logit order (ties ascending id);
 *  - weights: softmax, either over the k selected logits (normalize = 1) or
 *    over all experts, keeping the selected ones (normalize = 0);
 *  - SwiGLU: h = silu(gate) * up, silu(g) = g / (1 + e^-g);
 *  - combine: out_t = sum_j w_tj * y_(t*topk+j). */

/* e^x for x <= 0 (x < -745.5 gives +0), fp64: k = rint(x * fp64(1/ln2));
 * r = (x - k*C1) - k*C2 with C1 = ln2 truncated to a multiple of 2^-32 (k*C1
 * is exact) and C2 = fp64(ln2 - C1); p = Horner evaluation of
 * sum_{i=0..13} r^i / i! (coefficients fp64(1 / i!), each step one multiply
 * and one add, no fused operations); result ldexp(p, k).  Truncation error
 * below 1e-17 relative; a few fp64 ulps in all. */
double q8ref_exp_nonpos(double x);

/* Router: logits fp32 [tokens][n_experts] -> ids int32 [tokens][topk] and
 * weights fp32 [tokens][topk].  With m = the largest logit of the token and
 * e_i = q8ref_exp_nonpos((double)l_i - (double)m):
 *   normalize = 1: D = sum of e over the selected experts
 *   normalize = 0: D = sum of e over all experts
 * each sum rounded once to fp64 (q8ref_exact_sum: no summation order enters)
 *   w_j = fp32(e_{id_j} / D).
 * Returns Q8REF_OK or Q8REF_EARG (sizes, topk outside 1..n_experts). */
int q8ref_moe_route(const float *logits, int64_t tokens, int64_t n_experts, int topk, int normalize, int32_t *ids,
                    float *weights);

/* SwiGLU + quantization: gate, up fp32 [rows][n] (row strides ld_gate,
 * ld_up) -> ACT buffer of h [rows][n]:
 *   e = q8ref_exp_nonpos(-|g|); s = g >= 0 ? g / (1 + e) : (g * e) / (1 + e)
 *   (fp64, the same value as g / (1 + e^-g) up to rounding);
 *   h = fp32(s * (double)u); then the block quantizer.  n % 32 == 0. */
int q8ref_swiglu_quantize(const float *gate, int64_t ld_gate, const float *up, int64_t ld_up, int64_t rows, int64_t n,
                          uint8_t *q_out);

/* Weighted combine: out[t][c] = sum_j w[t][j] * y[t*topk + j][c] accumulated
 * in fp64, rounded once; Sc (may be NULL) receives sum_j |w[t][j] * y[..][c]|. */
int q8ref_moe_combine(const float *y, int64_t ld_y, const float *w, int64_t tokens, int topk, int64_t n, float *out,
                      double *Sc);

/* ---- Q8_0 KV cache ("ferro" README, "KV cache": K/V rows stored as int8 with
 * one fp32 scale per 32 values, quantized in the fused norm + rope +
 * cache-write kernel and dequantized in the attention kernels).  Readings:
 *  - a KV block: d = fp32(amax / 127) kept as fp32 (not rounded to fp16),
 *    q = roundf(x / d) (ties away from zero), d = 0 for an all-zero block;
 *  - qkv rows hold n_heads query heads, then n_kv key heads, then n_kv value
 *    heads, each head_dim values (one fused QKV projection per token);
 *  - optional per-head RMSNorm of q and k (gains of head_dim values, NULL for
 *    none): ss = sum of the exact fp64 squares x^2 rounded once to fp64
 *    (q8ref_exact_sum); r = fp32(1 / sqrt(ss / head_dim + eps));
 *    n = fp32(fp32(x * r) * g);
 *  - rotary embedding of q and k (after the norm) in the half-split layout:
 *    for i < head_dim/2, with c = cos_tab[pos][i], s = sin_tab[pos][i]:
 *      y_i        = fp32(fp32(x_i * c) - fp32(x_{i+h} * s))
 *      y_{i+h}    = fp32(fp32(x_{i+h} * c) + fp32(x_i * s)),  h = head_dim/2;
 *    the tables are inputs (model constants), fp32 [positions][head_dim/2];
 *  - cache layout, head-major (one head's positions contiguous): int8
 *    [n_kv][n_slots][head_dim] and fp32 scales [n_kv][n_slots][head_dim/32],
 *    for K and V alike; token t writes slot slots[t] of every head; v is
 *    quantized as is (no norm, no rotation). */

/* The fused norm + rope + cache write for `tokens` rows of qkv (fp32,
 * [tokens][(n_heads + 2 n_kv) head_dim]); q_out fp32 [tokens][n_heads][head_dim]
 * receives the normalized, rotated queries.  head_dim in {64, 128, 256}. */
int q8ref_kv_write(const float *qkv, int64_t tokens, int n_heads, int n_kv, int head_dim, const int32_t *positions,
                   const float *cos_tab, const float *sin_tab, const float *q_gain, const float *k_gain, float eps,
                   const int32_t *slots, int64_t n_slots, float *q_out, int8_t *k_cache, float *k_scale,
                   int8_t *v_cache, float *v_scale);

/* Decode attention over the Q8 KV cache, one query row per sequence:
 *   for query head h (kv head h / (n_heads / n_kv)), keys j < len[s] at slot
 *   base[s] + j (base[s] + len[s] <= n_slots), dequantized k = q * d and
 *   v = q * d (exact in fp64):
 *   s_j = scale * sum_d q_d k_jd;  p_j = exp(s_j - max);  out = sum p_j v_j / sum p_j
 * all in fp64, out rounded once to fp32.  bound (may be NULL) receives, per
 * output, an fp64 error budget for any fp32 evaluation, whatever its
 * summation order: each dot product is a sum of head_dim + 2 rounded terms,
 * each softmax sum and weighted sum a sum of len terms in any order (at most
 * len - 1 roundings, Higham's bound for recursive summation in any order),
 * plus a few roundings for the exponential, the maximum and the division (an
 * error common to every p_j, such as that of the maximum, cancels in the
 * normalization):
 *   (sum_j p_j |v_jd| * (scale * S_j * 2 (head_dim + 2) u + (len + 8) u))
 *   / sum_j p_j + 2 u |out|,  S_j = sum_d |q_d k_jd|,  u = 2^-24. */
int q8ref_attention_decode(const float *q, int64_t seqs, int n_heads, int n_kv, int head_dim, const int8_t *k_cache,
                           const float *k_scale, const int8_t *v_cache, const float *v_scale, int64_t n_slots,
                           const int32_t *base, const int32_t *len, float scale, float *out, double *bound);

#ifdef __cplusplus
}
#endif
#endif
