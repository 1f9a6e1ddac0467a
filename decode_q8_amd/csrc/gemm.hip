// Prefill GEMM (m > 8) for gfx950 on int8 MFMA.
//
// The Q8_0 block dot is a dense int8 contraction per 32-value block ("ferro"
// README, "How the iGPU path is fast", item 1: int8 GEMMs with activations
// quantized per 32-block).  One v_mfma_i32_32x32x32_i8 covers exactly one
// block for a 32 x 32 output tile, so its int32 results are the exact block
// dots s; the per-block fp32 epilogue applies Dw * Dx:
//   group accumulator  a = fma(float(s), Dw * Dx, a)  over the 8 blocks of a
//                          256-value group (the first block multiplies),
//   output             y = ((a_0 + a_1) + a_2) + ...   over the groups.
// The order depends on k only, so each row is bit-identical for any m and
// any row order.
//
// Tiling: a 256-thread workgroup owns a 128 x 128 output tile; each wave a
// 64 x 64 quarter (2 x 2 MFMA tiles).  Operands are read straight from global
// memory in the MFMA register layout: activation rows are row-major int8, and
// the packed weight layout already places 32 rows x 16 values of one block
// half contiguously (one 16-byte load per lane).  Activation scales of the
// group are staged once per workgroup in LDS as fp32.
#include "device.hpp"
#include "launch.hpp"

namespace q8k {

constexpr int GT_M = 128;
constexpr int GT_N = 128;

__global__ __launch_bounds__(256) void gemm_kernel(const int8_t *__restrict__ xq, const uint16_t *__restrict__ xs,
                                                   int64_t M, const uint8_t *__restrict__ w, int64_t N, int64_t K,
                                                   float *__restrict__ y, int64_t ld_y) {
    __shared__ float sx[GROUP_BLOCKS][GT_M];
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave & 1, wn = wave >> 1;
    const int half = lane >> 5, l32 = lane & 31;
    const int64_t m_tile = (int64_t)blockIdx.y * GT_M;
    const int64_t n_wave = (int64_t)blockIdx.x * GT_N + wn * 64;
    const bool n_ok = n_wave < N;  // N % 64 == 0: a wave is either fully in range or idle
    const int64_t G = K / GROUP_K;
    const int64_t nb = K / QK;
    const int64_t T = n_ok ? n_wave / TILE_ROWS : 0;

    // activation rows this lane feeds to the MFMA (clamped into range)
    const int8_t *arow[2];
#pragma unroll
    for (int i = 0; i < 2; i++) {
        int64_t r = m_tile + wm * 64 + i * 32 + l32;
        r = r < M ? r : M - 1;
        arow[i] = xq + r * K + half * 16;
    }

    float acc[2][2][16];
    for (int64_t g = 0; g < G; g++) {
        __syncthreads();
        {
            // stage Dx of 128 rows x 8 blocks: thread -> (row, 4 blocks)
            const int r = tid >> 1, b4 = (tid & 1) * 4;
            const int64_t row = m_tile + r;
            uint2 v = make_uint2(0u, 0u);
            if (row < M) v = *reinterpret_cast<const uint2 *>(xs + row * nb + g * GROUP_BLOCKS + b4);
            sx[b4 + 0][r] = half_bits_to_float(v.x & 0xffffu);
            sx[b4 + 1][r] = half_bits_to_float(v.x >> 16);
            sx[b4 + 2][r] = half_bits_to_float(v.y & 0xffffu);
            sx[b4 + 3][r] = half_bits_to_float(v.y >> 16);
        }
        __syncthreads();
        if (!n_ok) continue;
        const uint8_t *rec = w + (T * G + g) * RECORD_BYTES;
        uint4 wsc[2];
#pragma unroll
        for (int j = 0; j < 2; j++) wsc[j] = *reinterpret_cast<const uint4 *>(rec + RECORD_Q_BYTES + (j * 32 + l32) * 16);
        float ga[2][2][16];
#pragma unroll
        for (int bb = 0; bb < GROUP_BLOCKS; bb++) {
            v4i a[2], b[2];
#pragma unroll
            for (int i = 0; i < 2; i++) a[i] = *reinterpret_cast<const v4i *>(arow[i] + g * GROUP_K + bb * QK);
#pragma unroll
            for (int j = 0; j < 2; j++)
                b[j] = *reinterpret_cast<const v4i *>(rec + bb * 2048 + half * 1024 + (j * 32 + l32) * 16);
            float dw[2];
#pragma unroll
            for (int j = 0; j < 2; j++)
                dw[j] = half_bits_to_float((word_of(wsc[j], bb >> 1) >> (16 * (bb & 1))) & 0xffffu);
#pragma unroll
            for (int i = 0; i < 2; i++) {
                // Dx of the 16 output rows this lane holds: rows 8q + 4*half + p
                float dx[16];
#pragma unroll
                for (int q = 0; q < 4; q++) {
                    const float4 v = *reinterpret_cast<const float4 *>(&sx[bb][wm * 64 + i * 32 + 8 * q + 4 * half]);
                    dx[4 * q] = v.x; dx[4 * q + 1] = v.y; dx[4 * q + 2] = v.z; dx[4 * q + 3] = v.w;
                }
#pragma unroll
                for (int j = 0; j < 2; j++) {
                    const v16i zero = {0};
                    const v16i s = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[i], b[j], zero, 0, 0, 0);
#pragma unroll
                    for (int r = 0; r < 16; r++) {
                        const float sp = dx[r] * dw[j];  // exact
                        ga[i][j][r] = bb == 0 ? (float)s[r] * sp : __builtin_fmaf((float)s[r], sp, ga[i][j][r]);
                    }
                }
            }
        }
#pragma unroll
        for (int i = 0; i < 2; i++)
#pragma unroll
            for (int j = 0; j < 2; j++)
#pragma unroll
                for (int r = 0; r < 16; r++) acc[i][j][r] = g == 0 ? ga[i][j][r] : acc[i][j][r] + ga[i][j][r];
    }
    if (!n_ok) return;
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
        for (int r = 0; r < 16; r++) {
            const int64_t row = m_tile + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
            if (row >= M) continue;
#pragma unroll
            for (int j = 0; j < 2; j++) y[row * ld_y + n_wave + j * 32 + l32] = acc[i][j][r];
        }
}

hipError_t launch_gemm(const void *x_q, int64_t m, const void *w, int64_t n, int64_t k, float *y, int64_t ld_y,
                       hipStream_t s) {
    const int8_t *xq = (const int8_t *)x_q;
    const uint16_t *xs = (const uint16_t *)((const uint8_t *)x_q + m * k);
    const dim3 grid((unsigned)((n + GT_N - 1) / GT_N), (unsigned)((m + GT_M - 1) / GT_M));
    hipLaunchKernelGGL(gemm_kernel, grid, dim3(256), 0, s, xq, xs, m, (const uint8_t *)w, n, k, y, ld_y);
    return hipGetLastError();
}

}  // namespace q8k
