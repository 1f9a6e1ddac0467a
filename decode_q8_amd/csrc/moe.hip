// The steps either side of the routed-expert GEMVs of a mixture-of-experts
// layer: the router (top-k over the router logits and the experts' softmax
// weights), SwiGLU between the gate/up and the down GEMVs (its output
// quantized to the down GEMV's Q8_0 input), and the weighted combine of the
// down outputs ("Ferrule" README: device routing, the real router deciding
// expert ids and weights, a sparse-MoE execution path).
//
// Where the results decide integers (expert ids, the SwiGLU codes) or are
// meant to be reproducible bit for bit (the weights), every floating-point
// step is fixed: e^x (x <= 0) is evaluated by one stated fp64 algorithm built
// from correctly rounded basic operations only (no fused operations: the
// library is compiled with contraction off), so its value does not depend on
// the device's math library:
//   k = rint(x * fp64(1/ln 2)),  r = (x - k*C1) - k*C2  (C1 = ln 2 truncated
//   to a multiple of 2^-32, so k*C1 is exact; C2 = the rest, rounded),
//   e^r = Horner sum of r^i / i!, i = 0..13 (coefficients fp64(1 / i!)),
//   e^x = ldexp(e^r, k);   x < -745.5 gives +0.
// |r| <= ln2 / 2 bounds the truncation error below 1e-17 relative.
#include "device.hpp"
#include "launch.hpp"

namespace q8k {

__device__ __forceinline__ double exp_nonpos(double x) {
    if (x < -745.5) return 0.0;
    const double inv_ln2 = 0x1.71547652b82fep+0;
    const double C1 = 0x1.62e42fee00000p-1, C2 = 0x1.a39ef35793c76p-33;
    const double kd = __builtin_rint(x * inv_ln2);
    const double r = (x - kd * C1) - kd * C2;
    // 1 / i!, i = 13 .. 0 (each a correctly rounded quotient of exact integers)
    double p = 1.0 / 6227020800.0;
    p = p * r + 1.0 / 479001600.0;
    p = p * r + 1.0 / 39916800.0;
    p = p * r + 1.0 / 3628800.0;
    p = p * r + 1.0 / 362880.0;
    p = p * r + 1.0 / 40320.0;
    p = p * r + 1.0 / 5040.0;
    p = p * r + 1.0 / 720.0;
    p = p * r + 1.0 / 120.0;
    p = p * r + 1.0 / 24.0;
    p = p * r + 1.0 / 6.0;
    p = p * r + 1.0 / 2.0;
    p = p * r + 1.0;
    p = p * r + 1.0;
    return __builtin_ldexp(p, (int)kd);
}

// ---------------------------------------------------------------------------
// Router: one wavefront per token.  Lane l holds the logits of experts
// l, l + 64, ... (n_experts <= 1024).  Slot j is the arg-max over the experts
// not yet taken, ties to the lower id: a wave-wide maximum of the logits'
// order-preserving keys, then the minimum id among the lanes that hold it.
// ---------------------------------------------------------------------------

constexpr int ROUTE_MAX_PER_LANE = 16;  // n_experts <= 1024

// Order-preserving image of a finite fp32 value in uint32 (larger value,
// larger key; -0 and +0 share a key since they compare equal).  Every key is
// above 0, which therefore serves as "nothing left".
__device__ __forceinline__ uint32_t value_key(float v) {
    if (v == 0.0f) v = 0.0f;
    const uint32_t b = __builtin_bit_cast(uint32_t, v);
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Wave-wide max / min of a uint32 through DPP lane moves (no LDS round trip):
// swaps inside quads, mirrors inside half rows and rows, then the row
// broadcasts 15 and 31; lane 63 ends with the result.
template <bool MAX>
__device__ __forceinline__ uint32_t dpp_op(uint32_t a, uint32_t b) {
    return MAX ? (a > b ? a : b) : (a < b ? a : b);
}

template <bool MAX>
__device__ __forceinline__ uint32_t wave_reduce(uint32_t x) {
#define Q8_DPP(ctrl, rows) \
    x = dpp_op<MAX>(x, (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, ctrl, rows, 0xf, false))
    Q8_DPP(0xb1, 0xf);   // quad_perm [1, 0, 3, 2]
    Q8_DPP(0x4e, 0xf);   // quad_perm [2, 3, 0, 1]
    Q8_DPP(0x141, 0xf);  // row_half_mirror
    Q8_DPP(0x140, 0xf);  // row_mirror
    Q8_DPP(0x142, 0xa);  // row_bcast:15 into rows 1 and 3
    Q8_DPP(0x143, 0xc);  // row_bcast:31 into rows 2 and 3
#undef Q8_DPP
    return (uint32_t)__builtin_amdgcn_readlane((int)x, 63);
}

__global__ __launch_bounds__(256) void moe_route_kernel(const float *__restrict__ logits, int32_t tokens,
                                                        int32_t n_experts, int32_t topk, int32_t normalize,
                                                        int32_t *__restrict__ ids, float *__restrict__ weights) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= tokens) return;  // whole waves leave together
    const float *l = logits + (int64_t)t * n_experts;
    const int per = (n_experts + 63) >> 6;
    float v[ROUTE_MAX_PER_LANE];
    uint32_t taken = 0u;
#pragma unroll
    for (int i = 0; i < ROUTE_MAX_PER_LANE; i++) {
        const int e = lane + 64 * i;
        v[i] = (i < per && e < n_experts) ? l[e] : 0.0f;
    }
    int32_t *ids_t = ids + (int64_t)t * topk;
    float *w_t = weights + (int64_t)t * topk;
    float top = 0.0f;       // the largest logit (slot 0)
    float mine = 0.0f;      // lane j < topk: the logit of slot j
    for (int j = 0; j < topk; j++) {
        // this lane's best remaining expert (ascending ids, so ties keep the lower)
        uint32_t bk = 0u, bid = 0xffffffffu;
#pragma unroll
        for (int i = 0; i < ROUTE_MAX_PER_LANE; i++) {
            const int e = lane + 64 * i;
            if (i < per && e < n_experts && !((taken >> i) & 1u)) {
                const uint32_t k = value_key(v[i]);
                if (k > bk) {
                    bk = k;
                    bid = (uint32_t)e;
                }
            }
        }
        // the largest value over the wave, then the lowest id holding it
        const uint32_t kmax = wave_reduce<true>(bk);
        const int e = (int)wave_reduce<false>(bk == kmax ? bid : 0xffffffffu);
        if ((e & 63) == lane) taken |= 1u << (e >> 6);
        // the winning logit, from its owner lane
        float lv = 0.0f;
#pragma unroll
        for (int i = 0; i < ROUTE_MAX_PER_LANE; i++)
            if ((e >> 6) == i) lv = v[i];
        lv = __shfl(lv, e & 63);
        if (j == 0) top = lv;
        if (lane == j) mine = lv;
        if (lane == 0) ids_t[j] = e;
    }
    const double m = (double)top;
    const double ej = exp_nonpos((double)mine - m);  // lane j < topk: slot j's term, all slots at once
    double D;
    if (normalize) {
        // sum over the selected experts in slot order (every lane, sequentially)
        D = 0.0;
        for (int j = 0; j < topk; j++) D += __shfl(ej, j);
    } else {
        // all experts: lane partials in ascending expert order, then a halving tree
        double P = 0.0;
#pragma unroll
        for (int i = 0; i < ROUTE_MAX_PER_LANE; i++) {
            const int e = lane + 64 * i;
            if (i < per && e < n_experts) P += exp_nonpos((double)v[i] - m);
        }
#pragma unroll
        for (int s = 32; s >= 1; s >>= 1) P += __shfl_down(P, s);
        D = __shfl(P, 0);
    }
    if (lane < topk) w_t[lane] = (float)(ej / D);
}

// ---------------------------------------------------------------------------
// SwiGLU + quantization: 4 values per lane, a 32-value block on 8 lanes.
//   e = e^-|g|,  s = g >= 0 ? g / (1 + e) : (g * e) / (1 + e)   (fp64)
//   h = fp32(s * u), then the block quantizer (d = amax / 127, q = round(h / d)).
// ---------------------------------------------------------------------------

__device__ __forceinline__ float swiglu(float g, float u) {
    const double gd = (double)g;
    const double e = exp_nonpos(-__builtin_fabs(gd));
    const double s = gd >= 0.0 ? gd / (1.0 + e) : (gd * e) / (1.0 + e);
    return (float)(s * (double)u);
}

__global__ __launch_bounds__(256) void swiglu_quantize_kernel(const float *__restrict__ gate, int64_t ld_gate,
                                                              const float *__restrict__ up, int64_t ld_up,
                                                              int64_t rows, int64_t n, uint8_t *__restrict__ q) {
    const int64_t chunks = n >> 2;  // 4-value chunks per row
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const bool valid = gid < rows * chunks;
    const int64_t r = valid ? gid / chunks : 0;
    const int64_t c = valid ? gid - r * chunks : 0;
    float h[4] = {0.f, 0.f, 0.f, 0.f};
    if (valid) {
        const float4 g4 = *reinterpret_cast<const float4 *>(gate + r * ld_gate + 4 * c);
        const float4 u4 = *reinterpret_cast<const float4 *>(up + r * ld_up + 4 * c);
        h[0] = swiglu(g4.x, u4.x);
        h[1] = swiglu(g4.y, u4.y);
        h[2] = swiglu(g4.z, u4.z);
        h[3] = swiglu(g4.w, u4.w);
    }
    // a block is 8 consecutive chunks of one row: 8 aligned lanes (n % 32 == 0)
    float amax = fmaxf(fmaxf(fabsf(h[0]), fabsf(h[1])), fmaxf(fabsf(h[2]), fabsf(h[3])));
    amax = fmaxf(amax, __shfl_xor(amax, 1));
    amax = fmaxf(amax, __shfl_xor(amax, 2));
    amax = fmaxf(amax, __shfl_xor(amax, 4));
    const float d = amax / 127.0f;
    uint32_t packed = 0u;
#pragma unroll
    for (int i = 0; i < 4; i++) {
        int qi = 0;
        if (d != 0.0f) qi = (int)roundf(h[i] / d);  // |qi| <= 127 since |h| <= amax
        packed |= ((uint32_t)qi & 0xffu) << (8 * i);
    }
    if (!valid) return;
    *reinterpret_cast<uint32_t *>(q + r * n + 4 * c) = packed;
    if ((c & 7) == 0) *reinterpret_cast<uint16_t *>(q + rows * n + (r * (n >> 5) + (c >> 3)) * 2) =
        float_to_half_bits(d);
}

// ---------------------------------------------------------------------------
// Weighted combine: out[t][c] = sum_j w[t][j] * y[t*topk + j][c], fp32, slot
// order, each product and each addition rounded separately.
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(256) void moe_combine_kernel(const float *__restrict__ y, int64_t ld_y,
                                                          const float *__restrict__ w, int64_t tokens, int32_t topk,
                                                          int64_t n, float *__restrict__ out, int64_t ld_out) {
    const int64_t chunks = n >> 2;
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid >= tokens * chunks) return;
    const int64_t t = gid / chunks, c = gid - t * chunks;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j = 0; j < topk; j++) {
        const float wj = w[t * topk + j];
        const float4 v = *reinterpret_cast<const float4 *>(y + (t * topk + j) * ld_y + 4 * c);
        acc.x = acc.x + wj * v.x;
        acc.y = acc.y + wj * v.y;
        acc.z = acc.z + wj * v.z;
        acc.w = acc.w + wj * v.w;
    }
    *reinterpret_cast<float4 *>(out + t * ld_out + 4 * c) = acc;
}

// Host side ---------------------------------------------------------------

hipError_t launch_moe_route(const float *logits, int64_t tokens, int64_t n_experts, int topk, int normalize,
                            int32_t *ids, float *weights, hipStream_t s) {
    if (tokens == 0) return hipSuccess;
    const dim3 grid((unsigned)((tokens + 3) / 4));
    hipLaunchKernelGGL(moe_route_kernel, grid, dim3(256), 0, s, logits, (int32_t)tokens, (int32_t)n_experts,
                       (int32_t)topk, (int32_t)normalize, ids, weights);
    return hipGetLastError();
}

hipError_t launch_swiglu_quantize(const float *gate, int64_t ld_gate, const float *up, int64_t ld_up, int64_t rows,
                                  int64_t n, void *q_out, hipStream_t s) {
    const int64_t threads = rows * (n / 4);
    if (threads == 0) return hipSuccess;
    hipLaunchKernelGGL(swiglu_quantize_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, gate,
                       ld_gate, up, ld_up, rows, n, (uint8_t *)q_out);
    return hipGetLastError();
}

hipError_t launch_moe_combine(const float *y, int64_t ld_y, const float *w, int64_t tokens, int topk, int64_t n,
                              float *out, int64_t ld_out, hipStream_t s) {
    const int64_t threads = tokens * (n / 4);
    if (threads == 0) return hipSuccess;
    hipLaunchKernelGGL(moe_combine_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, y, ld_y, w,
                       tokens, (int32_t)topk, n, out, ld_out);
    return hipGetLastError();
}

}  // namespace q8k
