// Fused producer of a quantized GEMM input: residual add + RMSNorm + Q8_0
// quantization of each row in one pass ("ferro" README, "How the iGPU path is
// fast", item 3: the norm and the int8 quantization of the next matmul's
// input fused with the residual add).
//
// Per row (the pages name the fusion, not the norm; the reading is Llama's
// RMSNorm with a fixed fp64 sum order):
//   h_j = fp32(res_in_j + x_j)   (x_j without a residual), stored to res_out
//   ss  = sum of (double)h_j^2: thread t of 512 sums the 4-value chunks
//         t, t + 512, t + 1024, ... in increasing j, then the 512 partials
//         are folded p_t += p_{t+s} for s = 256, 128, ..., 1
//   r   = fp32(1 / sqrt(ss / k + eps)), every step a correctly rounded fp64
//         operation
//   n_j = fp32(fp32(h_j * r) * w_j), quantized per 32-value block exactly as
//         the block quantizer does (d = amax / 127, q = round(n / d)).
//
// Mapping: one 512-thread workgroup per row, each thread a 16-byte chunk of
// every 2048 values (coalesced 1 KB per wave and load), the row kept in
// registers between the sum and the quantization (k <= 16384).  A 32-value
// block is the chunks of 8 consecutive lanes, so its amax is a 3-step
// butterfly; its 32 codes leave as 8 coalesced 4-byte stores.  The kernel is
// HBM-bound: 13 + 1/16 bytes per value (x, residual in and out, code, scale),
// the gain staying in L2 across rows.  The row data is touched once, so it
// is loaded and stored non-temporally (streamed past the caches; measured
// 12-14% faster than ordinary accesses on the 2048-row launch), and 512
// threads per row rather than 256 keep more loads in flight per workgroup,
// which matters when the rows are too few to fill the GPU (188 rows: 22%).
#include "device.hpp"
#include "launch.hpp"

namespace q8k {

constexpr int NORM_THREADS = 512;
constexpr int NORM_SPAN = NORM_THREADS * 4;  // values per pass of the workgroup

static_assert(NORM_THREADS == 512, "the partial-sum fold below is written for 512 partials");

typedef float v4f __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float4 load_stream(const float *p) {
    const v4f v = __builtin_nontemporal_load(reinterpret_cast<const v4f *>(p));
    return make_float4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ void store_stream(float *p, const float4 &v) {
    const v4f u = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(u, reinterpret_cast<v4f *>(p));
}

template <int P>  // passes over the row: NORM_SPAN * P >= k
__global__ __launch_bounds__(NORM_THREADS) void rmsnorm_quantize_kernel(const float *x,
                                                                        const float *res_in, float *res_out,
                                                                        const float *__restrict__ w, int32_t rows,
                                                                        int32_t k, float eps, uint8_t *__restrict__ q) {
    __shared__ double sp[NORM_THREADS];
    __shared__ float r_bcast;
    const int t = threadIdx.x;
    const int64_t row = blockIdx.x;
    const int64_t base = row * k;

    float4 h[P], wv[P];
    double p = 0.0;
#pragma unroll
    for (int i = 0; i < P; i++) {
        const int j0 = 4 * t + NORM_SPAN * i;
        h[i] = make_float4(0.f, 0.f, 0.f, 0.f);
        wv[i] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (j0 < k) {
            // the gain is loaded with the row, off the critical path after the reduction
            wv[i] = *reinterpret_cast<const float4 *>(w + j0);
            const float4 xv = load_stream(x + base + j0);
            if (res_in) {
                const float4 rv = load_stream(res_in + base + j0);
                h[i] = make_float4(rv.x + xv.x, rv.y + xv.y, rv.z + xv.z, rv.w + xv.w);
            } else {
                h[i] = xv;
            }
            if (res_out) store_stream(res_out + base + j0, h[i]);
            // squares are exact in fp64; only the additions round
            p += (double)h[i].x * (double)h[i].x;
            p += (double)h[i].y * (double)h[i].y;
            p += (double)h[i].z * (double)h[i].z;
            p += (double)h[i].w * (double)h[i].w;
        }
    }
    // fold the 512 partials: wave 0 takes strides 256, 128 and 64 from LDS
    // (lane t forms p_{t+u} + p_{t+u+256} for u = 0, 128, 64, 192, sums the
    // pairs as strides 128 and 64 would), then strides 32 .. 1 by shuffles
    sp[t] = p;
    __syncthreads();
    if (t < 64) {
        const double a0 = sp[t] + sp[t + 256], a1 = sp[t + 128] + sp[t + 384];
        const double a2 = sp[t + 64] + sp[t + 320], a3 = sp[t + 192] + sp[t + 448];
        p = (a0 + a1) + (a2 + a3);
#pragma unroll
        for (int s = 32; s >= 1; s >>= 1) p += __shfl_down(p, s);
        if (t == 0) {
            const double mean = p / (double)k;
            r_bcast = (float)(1.0 / sqrt(mean + (double)eps));
        }
    }
    __syncthreads();
    const float rs = r_bcast;

    const int64_t nb = k / QK;
    uint8_t *scales = q + (int64_t)rows * k;
#pragma unroll
    for (int i = 0; i < P; i++) {
        const int j0 = 4 * t + NORM_SPAN * i;
        const bool valid = j0 < k;  // uniform over each block's 8 lanes (k % 32 == 0)
        float v[4] = {0.f, 0.f, 0.f, 0.f};
        if (valid) {
            v[0] = (h[i].x * rs) * wv[i].x;
            v[1] = (h[i].y * rs) * wv[i].y;
            v[2] = (h[i].z * rs) * wv[i].z;
            v[3] = (h[i].w * rs) * wv[i].w;
        }
        float amax = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
        amax = fmaxf(amax, __shfl_xor(amax, 1));
        amax = fmaxf(amax, __shfl_xor(amax, 2));
        amax = fmaxf(amax, __shfl_xor(amax, 4));
        const float d = amax / 127.0f;
        uint32_t packed = 0u;
#pragma unroll
        for (int c = 0; c < 4; c++) {
            int qc = 0;
            if (d != 0.0f) qc = (int)roundf(v[c] / d);  // |qc| <= 127 since |v| <= amax
            packed |= ((uint32_t)qc & 0xffu) << (8 * c);
        }
        if (valid) {
            __builtin_nontemporal_store(packed, reinterpret_cast<uint32_t *>(q + base + j0));
            if ((t & 7) == 0)
                *reinterpret_cast<uint16_t *>(scales + (row * nb + j0 / QK) * 2) = float_to_half_bits(d);
        }
    }
}

hipError_t launch_rmsnorm_quantize(const float *x, const float *res_in, float *res_out, const float *w,
                                   int64_t rows, int64_t k, float eps, void *q_out, hipStream_t s) {
    if (rows == 0) return hipSuccess;
    const int passes = (int)((k + NORM_SPAN - 1) / NORM_SPAN);
    const dim3 grid((unsigned)rows), block(NORM_THREADS);
    uint8_t *q = (uint8_t *)q_out;
#define Q8_NORM_CASE(PP)                                                                                            \
    if (passes <= PP) {                                                                                             \
        hipLaunchKernelGGL(rmsnorm_quantize_kernel<PP>, grid, block, 0, s, x, res_in, res_out, w, (int32_t)rows,    \
                           (int32_t)k, eps, q);                                                                     \
        return hipGetLastError();                                                                                   \
    }
    Q8_NORM_CASE(1) Q8_NORM_CASE(2) Q8_NORM_CASE(4) Q8_NORM_CASE(8)
#undef Q8_NORM_CASE
    return hipErrorInvalidValue;
}

}  // namespace q8k
