/*
 * q8ref.c: the CPU oracle.  TEST INFRASTRUCTURE ONLY (see q8ref.h for what it
 * follows and for the readings it takes where the pages are silent).
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math -fPIC -shared
 * (x86-64 evaluates float arithmetic in SSE single precision, so every fp32
 * operation below is one IEEE-754 rounding; -ffp-contract=off forbids fused
 * multiply-adds).
 */
#include "q8ref.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

#define QK 32        /* values per block */
#define BLK 34       /* bytes per block: fp16 scale + 32 int8 */
#define PR 64        /* rows per packed record */
#define PB 8         /* blocks per packed record */
#define REC (PR * PB * BLK) /* 17408 bytes */

/* ------------------------------------------------------------------------ */
/* binary16 codec                                                           */
/* ------------------------------------------------------------------------ */

static uint32_t f2u(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static float u2f(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

/* fp32 -> fp16, round to nearest, ties to even; results too large become
 * infinity, results too small become subnormal or zero. */
uint16_t q8ref_f32_to_f16(float f) {
    uint32_t u = f2u(f);
    uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
    uint32_t e32 = (u >> 23) & 0xffu;
    uint32_t man = u & 0x7fffffu;
    if (e32 == 0xffu) {
        if (man == 0) return sign | 0x7c00u;              /* infinity */
        return (uint16_t)(sign | 0x7e00u | (man >> 13));   /* quiet NaN, payload kept */
    }
    if (e32 == 0) return sign;  /* fp32 zero/subnormal: below half the smallest fp16 subnormal */
    int e = (int)e32 - 127;     /* unbiased exponent, value = 1.man * 2^e */
    if (e > 15) return sign | 0x7c00u;
    uint32_t full = man | 0x800000u; /* 24-bit significand, value = full * 2^(e-23) */
    if (e >= -14) {
        /* normal fp16: keep 11 significant bits */
        uint32_t h = ((uint32_t)(e + 15) << 10) | (man >> 13);
        uint32_t rem = man & 0x1fffu;
        if (rem > 0x1000u || (rem == 0x1000u && (h & 1u))) h += 1; /* carry may reach inf: correct */
        return (uint16_t)(sign | h);
    }
    /* subnormal fp16: value / 2^-24 = full * 2^(e+1); shift right by s = -(e+1) */
    int s = -(e + 1);
    if (s > 25) return sign;
    uint32_t kq = full >> s;
    uint32_t rem = full & ((1u << s) - 1u);
    uint32_t half = 1u << (s - 1);
    if (rem > half || (rem == half && (kq & 1u))) kq += 1; /* may become the smallest normal: correct */
    return (uint16_t)(sign | kq);
}

float q8ref_f16_to_f32(uint16_t h) {
    uint32_t sign = ((uint32_t)h & 0x8000u) << 16;
    uint32_t e = (h >> 10) & 0x1fu;
    uint32_t man = h & 0x3ffu;
    if (e == 0x1fu) return u2f(sign | 0x7f800000u | (man << 13));
    if (e == 0) {
        if (man == 0) return u2f(sign);
        /* subnormal: man * 2^-24; normalise into an fp32 normal */
        int shift = 0;
        while (!(man & 0x400u)) { man <<= 1; shift++; }
        man &= 0x3ffu;
        uint32_t e32 = (uint32_t)(127 - 15 - shift + 1);
        return u2f(sign | (e32 << 23) | (man << 13));
    }
    return u2f(sign | ((e - 15 + 127) << 23) | (man << 13));
}

void q8ref_f32_to_f16_n(const float *in, uint16_t *out, int64_t n) {
    for (int64_t i = 0; i < n; i++) out[i] = q8ref_f32_to_f16(in[i]);
}

void q8ref_f16_to_f32_n(const uint16_t *in, float *out, int64_t n) {
    for (int64_t i = 0; i < n; i++) out[i] = q8ref_f16_to_f32(in[i]);
}

/* ------------------------------------------------------------------------ */
/* quantization                                                             */
/* ------------------------------------------------------------------------ */

uint16_t q8ref_quantize_block(const float *x, int8_t *q, float *d_out) {
    float amax = 0.0f;
    for (int j = 0; j < QK; j++) {
        float a = fabsf(x[j]);
        if (a > amax) amax = a;
    }
    float d = amax / 127.0f;
    for (int j = 0; j < QK; j++) {
        if (d == 0.0f) {
            q[j] = 0;
        } else {
            float r = x[j] / d;       /* one correctly rounded division */
            q[j] = (int8_t)roundf(r); /* nearest integer, halves away from zero */
        }
    }
    if (d_out) *d_out = d;
    return q8ref_f32_to_f16(d);
}

static void put16(uint8_t *p, uint16_t v) { p[0] = (uint8_t)(v & 0xffu); p[1] = (uint8_t)(v >> 8); }
static uint16_t get16(const uint8_t *p) { return (uint16_t)(p[0] | (p[1] << 8)); }

int q8ref_quantize_rows(const float *x, int64_t ld_x, int64_t rows, int64_t k, int layout, uint8_t *out) {
    if (!x || !out || rows < 0 || k <= 0 || ld_x < k) return Q8REF_EARG;
    if (k % QK) return Q8REF_ESHAPE;
    if (layout != 0 && layout != 2) return Q8REF_EARG;
    int64_t nb = k / QK;
    for (int64_t r = 0; r < rows; r++) {
        for (int64_t b = 0; b < nb; b++) {
            int8_t q[QK];
            uint16_t d = q8ref_quantize_block(x + r * ld_x + b * QK, q, NULL);
            if (layout == 0) {
                uint8_t *blk = out + (r * nb + b) * BLK;
                put16(blk, d);
                memcpy(blk + 2, q, QK);
            } else {
                memcpy(out + r * k + b * QK, q, QK);
                put16(out + rows * k + (r * nb + b) * 2, d);
            }
        }
    }
    return Q8REF_OK;
}

/* ------------------------------------------------------------------------ */
/* exactly rounded fp64 sum of non-negative terms                            */
/* ------------------------------------------------------------------------ */

/* Bit p of the accumulator stands for 2^(p - 1074), the fp64 subnormal unit;
 * the largest finite fp64 has its top bit at p = 2097, and 34 limbs of 64 bits
 * (2176 positions) leave 78 bits of headroom for carries. */
#define XS_LIMBS 34
#define XS_BIAS 1074

static void xs_add_bits(uint64_t *acc, uint64_t v, int pos) {
    /* acc += v * 2^pos (v < 2^53), carrying upwards */
    int li = pos / 64, sh = pos % 64;
    uint64_t lo = v << sh;
    uint64_t hi = sh ? (v >> (64 - sh)) : 0;
    uint64_t old = acc[li];
    acc[li] = old + lo;
    uint64_t carry = (acc[li] < old) ? 1 : 0;
    for (int i = li + 1; i < XS_LIMBS && (hi || carry); i++) {
        old = acc[i];
        uint64_t add = hi + carry; /* hi < 2^53, no wrap */
        acc[i] = old + add;
        carry = (acc[i] < old) ? 1 : 0;
        hi = 0;
    }
}

static int xs_bit(const uint64_t *acc, int p) { return (int)((acc[p / 64] >> (p % 64)) & 1u); }

double q8ref_exact_sum(const double *v, int64_t n) {
    uint64_t acc[XS_LIMBS];
    memset(acc, 0, sizeof(acc));
    for (int64_t i = 0; i < n; i++) {
        const double x = v[i];
        if (!(x >= 0.0) || x > 1.7976931348623157e308) return NAN; /* outside the contract */
        uint64_t u;
        memcpy(&u, &x, 8);
        const int eb = (int)((u >> 52) & 0x7ffu);
        uint64_t mant = u & 0xfffffffffffffull;
        int pos; /* bit position of mant's least significant bit */
        if (eb == 0) {
            pos = 0; /* subnormal (or zero): mant * 2^-1074 */
        } else {
            mant |= 1ull << 52;
            pos = eb - 1; /* value = mant * 2^(eb - 1075) = mant * 2^(pos - 1074) */
        }
        if (mant) xs_add_bits(acc, mant, pos);
    }
    int top = -1;
    for (int p = XS_LIMBS * 64 - 1; p >= 0; p--)
        if (xs_bit(acc, p)) {
            top = p;
            break;
        }
    if (top < 0) return 0.0;
    if (top < 53) { /* at most 53 bits: exactly representable */
        uint64_t m = 0;
        for (int p = top; p >= 0; p--) m = (m << 1) | (uint64_t)xs_bit(acc, p);
        return ldexp((double)m, -XS_BIAS);
    }
    /* keep the top 53 bits, round to nearest with ties to even */
    uint64_t m = 0;
    for (int p = top; p > top - 53; p--) m = (m << 1) | (uint64_t)xs_bit(acc, p);
    const int lsb = top - 52;
    const int round = xs_bit(acc, lsb - 1);
    int sticky = 0;
    for (int p = lsb - 2; p >= 0 && !sticky; p--) sticky = xs_bit(acc, p);
    if (round && (sticky || (m & 1u))) m += 1; /* 2^53 after the carry is still exact */
    return ldexp((double)m, lsb - XS_BIAS);
}

/* ------------------------------------------------------------------------ */
/* fused residual + RMSNorm + quantization ("ferro" README, item 3)          */
/* ------------------------------------------------------------------------ */

int q8ref_rmsnorm_quantize(const float *x, const float *res_in, const float *w, int64_t rows, int64_t k, float eps,
                           float *res_out, uint8_t *q_out) {
    if (!x || !w || !q_out || rows < 0 || k <= 0) return Q8REF_EARG;
    if (k % QK) return Q8REF_ESHAPE;
    int64_t nb = k / QK;
    float *h = malloc(sizeof(float) * (size_t)k);
    float *n = malloc(sizeof(float) * (size_t)k);
    double *sq = malloc(sizeof(double) * (size_t)k);
    if (!h || !n || !sq) {
        free(h);
        free(n);
        free(sq);
        return Q8REF_EARG;
    }
    for (int64_t r = 0; r < rows; r++) {
        for (int64_t j = 0; j < k; j++) h[j] = res_in ? res_in[r * k + j] + x[r * k + j] : x[r * k + j];
        /* ss: the exactly rounded sum of the squares (each square of an fp32 is exact in fp64) */
        for (int64_t j = 0; j < k; j++) sq[j] = (double)h[j] * (double)h[j];
        const double ss = q8ref_exact_sum(sq, k);
        const double mean = ss / (double)k;
        const float rs = (float)(1.0 / sqrt(mean + (double)eps));
        for (int64_t j = 0; j < k; j++) {
            const float hr = h[j] * rs;
            n[j] = hr * w[j];
        }
        if (res_out)
            for (int64_t j = 0; j < k; j++) res_out[r * k + j] = h[j];
        for (int64_t b = 0; b < nb; b++) {
            int8_t q[QK];
            uint16_t d = q8ref_quantize_block(n + b * QK, q, NULL);
            memcpy(q_out + r * k + b * QK, q, QK);
            put16(q_out + rows * k + (r * nb + b) * 2, d);
        }
    }
    free(h);
    free(n);
    free(sq);
    return Q8REF_OK;
}

/* ------------------------------------------------------------------------ */
/* packed layout                                                            */
/* ------------------------------------------------------------------------ */

static int64_t packed_q_offset(int64_t row, int64_t col, int64_t k) {
    int64_t T = row / PR, r = row % PR;
    int64_t G = col / (QK * PB), c = col % (QK * PB);
    int64_t bb = c / QK, h = (c % QK) / 16, j = c % 16;
    return (T * (k / (QK * PB)) + G) * REC + bb * 2048 + h * 1024 + r * 16 + j;
}

static int64_t packed_d_offset(int64_t row, int64_t block, int64_t k) {
    int64_t T = row / PR, r = row % PR;
    int64_t G = block / PB, bb = block % PB;
    return (T * (k / (QK * PB)) + G) * REC + PR * PB * QK + r * 16 + bb * 2;
}

int q8ref_pack(const uint8_t *w_rows, int64_t n, int64_t k, uint8_t *w_packed) {
    if (!w_rows || !w_packed || n <= 0 || k <= 0) return Q8REF_EARG;
    if (n % PR || k % (QK * PB)) return Q8REF_ESHAPE;
    int64_t nb = k / QK;
    for (int64_t row = 0; row < n; row++) {
        for (int64_t b = 0; b < nb; b++) {
            const uint8_t *blk = w_rows + (row * nb + b) * BLK;
            memcpy(w_packed + packed_d_offset(row, b, k), blk, 2);
            for (int64_t j = 0; j < QK; j++)
                w_packed[packed_q_offset(row, b * QK + j, k)] = blk[2 + j];
        }
    }
    return Q8REF_OK;
}

int q8ref_unpack(const uint8_t *w_packed, int64_t n, int64_t k, uint8_t *w_rows) {
    if (!w_rows || !w_packed || n <= 0 || k <= 0) return Q8REF_EARG;
    if (n % PR || k % (QK * PB)) return Q8REF_ESHAPE;
    int64_t nb = k / QK;
    for (int64_t row = 0; row < n; row++) {
        for (int64_t b = 0; b < nb; b++) {
            uint8_t *blk = w_rows + (row * nb + b) * BLK;
            memcpy(blk, w_packed + packed_d_offset(row, b, k), 2);
            for (int64_t j = 0; j < QK; j++)
                blk[2 + j] = w_packed[packed_q_offset(row, b * QK + j, k)];
        }
    }
    return Q8REF_OK;
}

/* ------------------------------------------------------------------------ */
/* block dot and matmul                                                     */
/* ------------------------------------------------------------------------ */

/* Integer dot of block b of activation row mi with block b of weight row ni. */
static int32_t block_dot(const uint8_t *x_act, int64_t k, int64_t mi, const uint8_t *w_rows, int64_t ni, int64_t b) {
    const int8_t *qx = (const int8_t *)(x_act + mi * k + b * QK);
    const int8_t *qw = (const int8_t *)(w_rows + (ni * (k / QK) + b) * BLK + 2);
    int32_t s = 0;
    for (int j = 0; j < QK; j++) s += (int32_t)qx[j] * (int32_t)qw[j];
    return s;
}

/* t = fp32(s * (Dw * Dx)): Dw * Dx is exact in fp32, so one rounding. */
static float block_term(const uint8_t *x_act, int64_t m, int64_t k, int64_t mi, const uint8_t *w_rows, int64_t ni,
                        int64_t b, int32_t *s_out) {
    int64_t nb = k / QK;
    int32_t s = block_dot(x_act, k, mi, w_rows, ni, b);
    float dx = q8ref_f16_to_f32(get16(x_act + m * k + (mi * nb + b) * 2));
    float dw = q8ref_f16_to_f32(get16(w_rows + (ni * nb + b) * BLK));
    float scale = dw * dx;
    if (s_out) *s_out = s;
    return (float)s * scale;
}

static void output(const uint8_t *x_act, int64_t m, const uint8_t *w_rows, int64_t k, int64_t mi, int64_t ni,
                   float *y, double *S) {
    double acc = 0.0, mag = 0.0;
    for (int64_t b = 0; b < k / QK; b++) {
        float t = block_term(x_act, m, k, mi, w_rows, ni, b, NULL);
        acc += (double)t;
        mag += fabs((double)t);
    }
    *y = (float)acc;
    if (S) *S = mag;
}

int q8ref_block_terms(const uint8_t *x_act, int64_t m, const uint8_t *w_rows, int64_t n, int64_t k,
                      int32_t *s, float *t) {
    if (!x_act || !w_rows || m <= 0 || n <= 0 || k <= 0) return Q8REF_EARG;
    if (k % QK) return Q8REF_ESHAPE;
    int64_t nb = k / QK;
    for (int64_t mi = 0; mi < m; mi++)
        for (int64_t ni = 0; ni < n; ni++)
            for (int64_t b = 0; b < nb; b++) {
                int32_t sv;
                float tv = block_term(x_act, m, k, mi, w_rows, ni, b, &sv);
                if (s) s[(mi * n + ni) * nb + b] = sv;
                if (t) t[(mi * n + ni) * nb + b] = tv;
            }
    return Q8REF_OK;
}

typedef struct {
    const uint8_t *x_act;
    int64_t m;
    const uint8_t *w_rows;
    int64_t n, k, ld_y;
    float *y;
    double *S;
    int64_t n0, n1;
} mm_job;

static void *mm_worker(void *arg) {
    mm_job *j = (mm_job *)arg;
    for (int64_t ni = j->n0; ni < j->n1; ni++)
        for (int64_t mi = 0; mi < j->m; mi++)
            output(j->x_act, j->m, j->w_rows, j->k, mi, ni, &j->y[mi * j->ld_y + ni],
                   j->S ? &j->S[mi * j->n + ni] : NULL);
    return NULL;
}

int q8ref_matmul(const uint8_t *x_act, int64_t m, const uint8_t *w_rows, int64_t n, int64_t k,
                 float *y, int64_t ld_y, double *S, int threads) {
    if (!x_act || !w_rows || !y || m <= 0 || n <= 0 || k <= 0 || ld_y < n) return Q8REF_EARG;
    if (k % QK) return Q8REF_ESHAPE;
    if (threads < 1) threads = 1;
    if (threads > n) threads = (int)n;
    mm_job *jobs = (mm_job *)calloc((size_t)threads, sizeof(mm_job));
    pthread_t *tid = (pthread_t *)calloc((size_t)threads, sizeof(pthread_t));
    if (!jobs || !tid) { free(jobs); free(tid); return Q8REF_EARG; }
    for (int i = 0; i < threads; i++) {
        mm_job jb = {x_act, m, w_rows, n, k, ld_y, y, S, n * i / threads, n * (i + 1) / threads};
        jobs[i] = jb;
    }
    for (int i = 1; i < threads; i++) pthread_create(&tid[i], NULL, mm_worker, &jobs[i]);
    mm_worker(&jobs[0]);
    for (int i = 1; i < threads; i++) pthread_join(tid[i], NULL);
    free(jobs);
    free(tid);
    return Q8REF_OK;
}

int q8ref_matmul_points(const uint8_t *x_act, int64_t m, const uint8_t *w_rows, int64_t n, int64_t k,
                        const int64_t *mi, const int64_t *ni, int64_t count, float *y, double *S) {
    if (!x_act || !w_rows || !mi || !ni || !y || m <= 0 || n <= 0 || k <= 0 || count < 0) return Q8REF_EARG;
    if (k % QK) return Q8REF_ESHAPE;
    for (int64_t i = 0; i < count; i++) {
        if (mi[i] < 0 || mi[i] >= m || ni[i] < 0 || ni[i] >= n) return Q8REF_EARG;
        output(x_act, m, w_rows, k, mi[i], ni[i], &y[i], S ? &S[i] : NULL);
    }
    return Q8REF_OK;
}

int q8ref_grouped_matmul(const uint8_t *x_act, int64_t x_rows, int x_per_pair, const int32_t *ids,
                         int64_t tokens, int topk, const uint8_t *w_rows, int64_t n_experts,
                         int64_t expert_stride, int64_t n, int64_t k, float *y, double *S, int threads) {
    if (!x_act || !ids || !w_rows || !y || tokens <= 0 || topk <= 0 || n_experts <= 0 || n <= 0 || k <= 0)
        return Q8REF_EARG;
    if (k % QK) return Q8REF_ESHAPE;
    int64_t pairs = tokens * topk;
    if (x_rows != (x_per_pair ? pairs : tokens)) return Q8REF_ESHAPE;
    if (threads < 1) threads = 1;
    int64_t nb = k / QK;
    /* One single-row activation view per pair: the row's int8 values and its
     * scales, copied into a 1-row ACT buffer so the matmul above applies. */
    uint8_t *one = (uint8_t *)malloc((size_t)(nb * BLK));
    if (!one) return Q8REF_EARG;
    for (int64_t p = 0; p < pairs; p++) {
        int32_t e = ids[p];
        if (e < 0 || e >= n_experts) { free(one); return Q8REF_EARG; }
        int64_t xr = x_per_pair ? p : p / topk;
        memcpy(one, x_act + xr * k, (size_t)k);
        memcpy(one + k, x_act + x_rows * k + xr * nb * 2, (size_t)(nb * 2));
        int rc = q8ref_matmul(one, 1, w_rows + (int64_t)e * expert_stride, n, k, y + p * n, n,
                              S ? S + p * n : NULL, threads);
        if (rc) { free(one); return rc; }
    }
    free(one);
    return Q8REF_OK;
}

/* ------------------------------------------------------------------------ */
/* around the routed experts: exp, router, SwiGLU, combine                  */
/* ------------------------------------------------------------------------ */

double q8ref_exp_nonpos(double x) {
    if (x < -745.5) return 0.0;
    /* C1: ln 2 truncated to a multiple of 2^-32; C2: the rest, rounded */
    const double inv_ln2 = 0x1.71547652b82fep+0, C1 = 0x1.62e42fee00000p-1, C2 = 0x1.a39ef35793c76p-33;
    const double kd = rint(x * inv_ln2);
    const double r = (x - kd * C1) - kd * C2;
    double fact = 1.0;
    double c[14];
    for (int i = 0; i < 14; i++) {
        if (i > 0) fact *= (double)i; /* i! is exact in fp64 for i <= 22 */
        c[i] = 1.0 / fact;
    }
    double p = c[13];
    for (int i = 12; i >= 0; i--) p = p * r + c[i];
    return ldexp(p, (int)kd);
}

int q8ref_moe_route(const float *logits, int64_t tokens, int64_t n_experts, int topk, int normalize, int32_t *ids,
                    float *weights) {
    if (!logits || !ids || !weights || tokens < 0 || n_experts <= 0 || topk < 1 || topk > n_experts)
        return Q8REF_EARG;
    char *taken = malloc((size_t)n_experts);
    double *e = malloc(sizeof(double) * (size_t)n_experts);
    if (!taken || !e) {
        free(taken);
        free(e);
        return Q8REF_EARG;
    }
    for (int64_t t = 0; t < tokens; t++) {
        const float *l = logits + t * n_experts;
        memset(taken, 0, (size_t)n_experts);
        /* selection: repeatedly the largest remaining logit, ties to the lower id */
        for (int j = 0; j < topk; j++) {
            int64_t best = -1;
            for (int64_t e = 0; e < n_experts; e++)
                if (!taken[e] && (best < 0 || l[e] > l[best])) best = e;
            taken[best] = 1;
            ids[t * topk + j] = (int32_t)best;
        }
        const double m = (double)l[ids[t * topk]];
        /* D: the exactly rounded sum of the e's (selected experts, or all of them) */
        int64_t ne = 0;
        if (normalize) {
            for (int j = 0; j < topk; j++) e[ne++] = q8ref_exp_nonpos((double)l[ids[t * topk + j]] - m);
        } else {
            for (int64_t x = 0; x < n_experts; x++) e[ne++] = q8ref_exp_nonpos((double)l[x] - m);
        }
        const double D = q8ref_exact_sum(e, ne);
        for (int j = 0; j < topk; j++)
            weights[t * topk + j] = (float)(q8ref_exp_nonpos((double)l[ids[t * topk + j]] - m) / D);
    }
    free(taken);
    free(e);
    return Q8REF_OK;
}

int q8ref_swiglu_quantize(const float *gate, int64_t ld_gate, const float *up, int64_t ld_up, int64_t rows, int64_t n,
                          uint8_t *q_out) {
    if (!gate || !up || !q_out || rows < 0 || n <= 0 || ld_gate < n || ld_up < n) return Q8REF_EARG;
    if (n % QK) return Q8REF_ESHAPE;
    const int64_t nb = n / QK;
    float h[QK];
    for (int64_t r = 0; r < rows; r++) {
        for (int64_t b = 0; b < nb; b++) {
            for (int j = 0; j < QK; j++) {
                const double g = (double)gate[r * ld_gate + b * QK + j];
                const double u = (double)up[r * ld_up + b * QK + j];
                const double e = q8ref_exp_nonpos(-fabs(g));
                const double s = g >= 0.0 ? g / (1.0 + e) : (g * e) / (1.0 + e);
                h[j] = (float)(s * u);
            }
            int8_t q[QK];
            const uint16_t d = q8ref_quantize_block(h, q, NULL);
            memcpy(q_out + r * n + b * QK, q, QK);
            put16(q_out + rows * n + (r * nb + b) * 2, d);
        }
    }
    return Q8REF_OK;
}

int q8ref_moe_combine(const float *y, int64_t ld_y, const float *w, int64_t tokens, int topk, int64_t n, float *out,
                      double *Sc) {
    if (!y || !w || !out || tokens < 0 || topk < 1 || n <= 0 || ld_y < n) return Q8REF_EARG;
    for (int64_t t = 0; t < tokens; t++)
        for (int64_t c = 0; c < n; c++) {
            double acc = 0.0, S = 0.0;
            for (int j = 0; j < topk; j++) {
                const double v = (double)w[t * topk + j] * (double)y[(t * topk + j) * ld_y + c];
                acc += v;
                S += fabs(v);
            }
            out[t * n + c] = (float)acc;
            if (Sc) Sc[t * n + c] = S;
        }
    return Q8REF_OK;
}

/* ------------------------------------------------------------------------ */
/* Q8_0 KV cache: fused norm + rope + cache write; decode attention         */
/* ------------------------------------------------------------------------ */

/* KV block: fp32 scale kept as is */
static float kv_quantize_block(const float *x, int8_t *q) {
    float amax = 0.0f;
    for (int j = 0; j < QK; j++) {
        const float a = fabsf(x[j]);
        if (a > amax) amax = a;
    }
    const float d = amax / 127.0f;
    for (int j = 0; j < QK; j++) q[j] = d == 0.0f ? 0 : (int8_t)roundf(x[j] / d);
    return d;
}

static void head_norm(float *x, int hd, const float *g, float eps) {
    double sq[256];
    for (int i = 0; i < hd; i++) sq[i] = (double)x[i] * (double)x[i];
    const double ss = q8ref_exact_sum(sq, hd); /* exactly rounded sum of the exact squares */
    const float r = (float)(1.0 / sqrt(ss / (double)hd + (double)eps));
    for (int i = 0; i < hd; i++) {
        const float xr = x[i] * r;
        x[i] = xr * g[i];
    }
}

static void head_rope(float *x, int hd, const float *c, const float *s) {
    const int h = hd / 2;
    for (int i = 0; i < h; i++) {
        const float a = x[i], b = x[i + h];
        const float ac = a * c[i], bs = b * s[i], bc = b * c[i], as = a * s[i];
        x[i] = ac - bs;
        x[i + h] = bc + as;
    }
}

int q8ref_kv_write(const float *qkv, int64_t tokens, int n_heads, int n_kv, int head_dim, const int32_t *positions,
                   const float *cos_tab, const float *sin_tab, const float *q_gain, const float *k_gain, float eps,
                   const int32_t *slots, int64_t n_slots, float *q_out, int8_t *k_cache, float *k_scale,
                   int8_t *v_cache, float *v_scale) {
    if (!qkv || !positions || !cos_tab || !sin_tab || !slots || !q_out || !k_cache || !k_scale || !v_cache ||
        !v_scale || tokens < 0 || n_heads <= 0 || n_kv <= 0 || n_heads % n_kv || n_slots <= 0)
        return Q8REF_EARG;
    if (head_dim != 64 && head_dim != 128 && head_dim != 256) return Q8REF_ESHAPE;
    const int hd = head_dim, nb = hd / QK, h2 = hd / 2;
    const int64_t row = (int64_t)(n_heads + 2 * n_kv) * hd;
    float x[256];
    for (int64_t t = 0; t < tokens; t++) {
        const float *r = qkv + t * row;
        const float *c = cos_tab + (int64_t)positions[t] * h2, *s = sin_tab + (int64_t)positions[t] * h2;
        for (int h = 0; h < n_heads; h++) {
            memcpy(x, r + (int64_t)h * hd, sizeof(float) * hd);
            if (q_gain) head_norm(x, hd, q_gain, eps);
            head_rope(x, hd, c, s);
            memcpy(q_out + (t * n_heads + h) * hd, x, sizeof(float) * hd);
        }
        const int64_t slot = slots[t];
        if (slot < 0 || slot >= n_slots) return Q8REF_EARG;
        for (int h = 0; h < n_kv; h++) {
            const int64_t row = (int64_t)h * n_slots + slot; /* head-major cache rows */
            memcpy(x, r + (int64_t)(n_heads + h) * hd, sizeof(float) * hd);
            if (k_gain) head_norm(x, hd, k_gain, eps);
            head_rope(x, hd, c, s);
            for (int b = 0; b < nb; b++)
                k_scale[row * nb + b] = kv_quantize_block(x + b * QK, k_cache + row * hd + b * QK);
            memcpy(x, r + (int64_t)(n_heads + n_kv + h) * hd, sizeof(float) * hd);
            for (int b = 0; b < nb; b++)
                v_scale[row * nb + b] = kv_quantize_block(x + b * QK, v_cache + row * hd + b * QK);
        }
    }
    return Q8REF_OK;
}

int q8ref_attention_decode(const float *q, int64_t seqs, int n_heads, int n_kv, int head_dim, const int8_t *k_cache,
                           const float *k_scale, const int8_t *v_cache, const float *v_scale, int64_t n_slots,
                           const int32_t *base, const int32_t *len, float scale, float *out, double *bound) {
    if (!q || !k_cache || !k_scale || !v_cache || !v_scale || !base || !len || !out || seqs < 0 || n_heads <= 0 ||
        n_kv <= 0 || n_heads % n_kv || head_dim <= 0 || head_dim % QK || n_slots <= 0)
        return Q8REF_EARG;
    const int hd = head_dim, nb = hd / QK, G = n_heads / n_kv;
    const double u = ldexp(1.0, -24);
    for (int64_t sq = 0; sq < seqs; sq++) {
        const int64_t L = len[sq];
        if (L <= 0 || base[sq] < 0 || base[sq] + L > n_slots) return Q8REF_EARG;
        double *sc = malloc(sizeof(double) * (size_t)L), *Sj = malloc(sizeof(double) * (size_t)L);
        if (!sc || !Sj) {
            free(sc);
            free(Sj);
            return Q8REF_EARG;
        }
        for (int h = 0; h < n_heads; h++) {
            const int kvh = h / G;
            const float *qh = q + (sq * n_heads + h) * hd;
            double mx = -INFINITY;
            for (int64_t j = 0; j < L; j++) {
                const int64_t row = (int64_t)kvh * n_slots + base[sq] + j;
                const int8_t *kr = k_cache + row * hd;
                const float *ks = k_scale + row * nb;
                double acc = 0.0, aabs = 0.0;
                for (int d = 0; d < hd; d++) {
                    const double kv = (double)kr[d] * (double)ks[d / QK];
                    acc += (double)qh[d] * kv;
                    aabs += fabs((double)qh[d] * kv);
                }
                sc[j] = (double)scale * acc;
                Sj[j] = aabs;
                if (sc[j] > mx) mx = sc[j];
            }
            double l = 0.0;
            for (int64_t j = 0; j < L; j++) {
                sc[j] = exp(sc[j] - mx);
                l += sc[j];
            }
            for (int d = 0; d < hd; d++) {
                double o = 0.0, ob = 0.0;
                for (int64_t j = 0; j < L; j++) {
                    const int64_t row = (int64_t)kvh * n_slots + base[sq] + j;
                    const double vv = (double)v_cache[row * hd + d] * (double)v_scale[row * nb + d / QK];
                    o += sc[j] * vv;
                    ob += sc[j] * fabs(vv) *
                          ((double)scale * Sj[j] * 2.0 * (hd + 2) * u + ((double)L + 8.0) * u);
                }
                const double r = o / l;
                out[(sq * n_heads + h) * hd + d] = (float)r;
                if (bound) bound[(sq * n_heads + h) * hd + d] = ob / l + 2.0 * u * fabs(r);
            }
        }
        free(sc);
        free(Sj);
    }
    return Q8REF_OK;
}
