// Q8_0 quantizer for gfx950: fp32 rows -> 32-value blocks (fp16 scale + int8).
//
// Per block, d = amax / 127 (one correctly rounded fp32 division), each value
// becomes the nearest integer to x / d (one correctly rounded division, ties
// away from zero) and the stored scale is fp16(d) ("ferro" README, "How the
// iGPU path is fast", item 1: activations quantized per 32-value block;
// "Ember packed Q8 decode" post: [scale][q0 ... q31] blocks).
//
// Mapping: 4 consecutive lanes own one block (8 values each, two 16-byte
// loads); the block amax is a 2-step butterfly inside the 4-lane group, so a
// wavefront quantizes 16 blocks per pass with fully coalesced 1 KB reads.
#include "device.hpp"
#include "launch.hpp"

namespace q8k {

template <int LAYOUT>  // 0: ROWS (34-byte blocks), 2: ACT (int8 plane + fp16 plane)
__global__ __launch_bounds__(256) void quantize_kernel(const float *__restrict__ x, int64_t ld_x, int64_t rows,
                                                       int64_t k, uint8_t *__restrict__ out) {
    const int64_t nb = k / QK;
    const int64_t total = rows * nb;
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t blk = gid >> 2;
    const int sub = (int)(gid & 3);
    const bool valid = blk < total;
    const int64_t r = valid ? blk / nb : 0;
    const int64_t b = valid ? blk - r * nb : 0;

    float v[8];
    if (valid) {
        const float4 *p = reinterpret_cast<const float4 *>(x + r * ld_x + b * QK + sub * 8);
        const float4 a0 = p[0], a1 = p[1];  // plain loads: a line spans both (see load_nt)
        v[0] = a0.x; v[1] = a0.y; v[2] = a0.z; v[3] = a0.w;
        v[4] = a1.x; v[5] = a1.y; v[6] = a1.z; v[7] = a1.w;
    } else {
#pragma unroll
        for (int j = 0; j < 8; j++) v[j] = 0.0f;
    }
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; j++) amax = fmaxf(amax, fabsf(v[j]));
    // max is exact and order-free: a butterfly over the 4 lanes of the block
    amax = fmaxf(amax, __shfl_xor(amax, 1));
    amax = fmaxf(amax, __shfl_xor(amax, 2));

    const float d = amax / 127.0f;
    uint32_t packed[2] = {0u, 0u};
#pragma unroll
    for (int j = 0; j < 8; j++) {
        int q = 0;
        if (d != 0.0f) q = (int)roundf(v[j] / d);  // |q| <= 127 since |v| <= amax
        packed[j >> 2] |= ((uint32_t)q & 0xffu) << (8 * (j & 3));
    }
    if (!valid) return;
    const uint16_t dh = float_to_half_bits(d);
    if (LAYOUT == 2) {
        *reinterpret_cast<uint2 *>(out + r * k + b * QK + sub * 8) = make_uint2(packed[0], packed[1]);
        if (sub == 0) *reinterpret_cast<uint16_t *>(out + rows * k + (r * nb + b) * 2) = dh;
    } else {
        uint8_t *base = out + blk * BLOCK_BYTES;  // 2-byte aligned
        if (sub == 0) *reinterpret_cast<uint16_t *>(base) = dh;
        uint16_t *qp = reinterpret_cast<uint16_t *>(base + 2 + sub * 8);
        qp[0] = (uint16_t)packed[0];
        qp[1] = (uint16_t)(packed[0] >> 16);
        qp[2] = (uint16_t)packed[1];
        qp[3] = (uint16_t)(packed[1] >> 16);
    }
}

hipError_t launch_quantize(const float *x, int64_t ld_x, int64_t rows, int64_t k, int layout, void *out,
                           hipStream_t s) {
    const int64_t threads = rows * (k / QK) * 4;
    if (threads == 0) return hipSuccess;
    const dim3 grid((unsigned)((threads + 255) / 256));
    if (layout == 2)
        hipLaunchKernelGGL(quantize_kernel<2>, grid, dim3(256), 0, s, x, ld_x, rows, k, (uint8_t *)out);
    else
        hipLaunchKernelGGL(quantize_kernel<0>, grid, dim3(256), 0, s, x, ld_x, rows, k, (uint8_t *)out);
    return hipGetLastError();
}

}  // namespace q8k
