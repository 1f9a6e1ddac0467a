// Prefill GEMM (m > 8) for gfx950 on int8 MFMA.
//
// The Q8_0 block dot is a dense int8 contraction per 32-value block ("ferro"
// README, "How the iGPU path is fast", item 1: int8 GEMMs with activations
// quantized per 32-block).  One v_mfma_i32_32x32x32_i8 covers exactly one
// block for a 32 x 32 output tile, so its int32 results are the exact block
// dots s.  The per-block scale product Dx[m] * Dw[n] of the same tile comes
// from a rank-1 v_mfma_f32_32x32x8_f16 (one non-zero k: fp16 x fp16 is exact
// in fp32), so it lands in the same register layout as s and the VALU only
// converts s and fuses it in:
//   group accumulator  a = fma(float(s), Dx * Dw, a)  over the 8 blocks of a
//                          256-value group (the first block multiplies),
//   output             y = ((a_0 + a_1) + a_2) + ...   over the groups.
// The order depends on k only, so each row is bit-identical for any m and
// any row order.  Two VALU operations per output and block remain; with
// packed fp32 unavailable they, not the MFMA, bound this kernel.
//
// Tiling: a 256-thread workgroup owns a 128 x 128 output tile; each wave a
// 64 x 64 quarter (2 x 2 MFMA tiles).  Operands are read straight from global
// memory in the MFMA register layout: activation rows are row-major int8, and
// the packed weight layout already places 32 rows x 16 values of one block
// half contiguously (one 16-byte load per lane).  The k order inside one
// MFMA is the same for both operands (lane half h holds values 16h..16h+15 of
// the block), which is all an exact integer dot needs.
#include "device.hpp"
#include "launch.hpp"

namespace q8k {

constexpr int GT_M = 128;
constexpr int GT_N = 128;

typedef _Float16 v4h __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));

// Operand of the rank-1 scale MFMA: lanes 0..31 carry their fp16 scale in
// k = 0, every other element is zero.
__device__ __forceinline__ v4h rank1_operand(uint32_t h16, bool low_half) {
    v4h v = {(_Float16)0.0f, (_Float16)0.0f, (_Float16)0.0f, (_Float16)0.0f};
    if (low_half) v[0] = __builtin_bit_cast(_Float16, (uint16_t)h16);
    return v;
}

__global__ __launch_bounds__(256, 2) void gemm_kernel(const int8_t *__restrict__ xq, const uint16_t *__restrict__ xs,
                                                      int64_t M, const uint8_t *__restrict__ w, int64_t N, int64_t K,
                                                      float *__restrict__ y, int64_t ld_y) {
    const int lane = threadIdx.x & 63, wave = wave_id();
    const int wm = wave & 1, wn = wave >> 1;
    const int half = lane >> 5, l32 = lane & 31;
    const bool low = half == 0;
    const int64_t m_wave = (int64_t)blockIdx.y * GT_M + wm * 64;
    const int64_t n_wave = (int64_t)blockIdx.x * GT_N + wn * 64;
    if (n_wave >= N) return;  // N % 64 == 0: a wave is either fully in range or idle
    const int64_t G = K / GROUP_K;
    const int64_t nb = K / QK;
    const int64_t T = n_wave / TILE_ROWS;

    // activation rows this lane feeds to the MFMAs (clamped into range; rows
    // past M compute values that are never stored)
    const int8_t *arow[2];
    const uint16_t *srow[2];
#pragma unroll
    for (int i = 0; i < 2; i++) {
        int64_t r = m_wave + i * 32 + l32;
        r = r < M ? r : M - 1;
        arow[i] = xq + r * K + half * 16;
        srow[i] = xs + r * nb;
    }

    float acc[2][2][16];
    for (int64_t g = 0; g < G; g++) {
        const uint8_t *rec = w + (T * G + g) * RECORD_BYTES;
        uint4 xsc[2], wsc[2];
#pragma unroll
        for (int i = 0; i < 2; i++) xsc[i] = *reinterpret_cast<const uint4 *>(srow[i] + g * GROUP_BLOCKS);
#pragma unroll
        for (int j = 0; j < 2; j++) wsc[j] = *reinterpret_cast<const uint4 *>(rec + RECORD_Q_BYTES + (j * 32 + l32) * 16);
        float ga[2][2][16];
#pragma unroll
        for (int bb = 0; bb < GROUP_BLOCKS; bb++) {
            v4i a[2], b[2];
            v4h as[2], bs[2];
#pragma unroll
            for (int i = 0; i < 2; i++) {
                a[i] = *reinterpret_cast<const v4i *>(arow[i] + g * GROUP_K + bb * QK);
                as[i] = rank1_operand((word_of(xsc[i], bb >> 1) >> (16 * (bb & 1))) & 0xffffu, low);
            }
#pragma unroll
            for (int j = 0; j < 2; j++) {
                b[j] = *reinterpret_cast<const v4i *>(rec + bb * 2048 + half * 1024 + (j * 32 + l32) * 16);
                bs[j] = rank1_operand((word_of(wsc[j], bb >> 1) >> (16 * (bb & 1))) & 0xffffu, low);
            }
#pragma unroll
            for (int i = 0; i < 2; i++)
#pragma unroll
                for (int j = 0; j < 2; j++) {
                    const v16i zi = {0};
                    const v16f zf = {0};
                    const v16i s = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[i], b[j], zi, 0, 0, 0);
                    const v16f sp = __builtin_amdgcn_mfma_f32_32x32x8f16(as[i], bs[j], zf, 0, 0, 0);
#pragma unroll
                    for (int r = 0; r < 16; r++)
                        ga[i][j][r] = bb == 0 ? (float)s[r] * sp[r] : __builtin_fmaf((float)s[r], sp[r], ga[i][j][r]);
                }
        }
#pragma unroll
        for (int i = 0; i < 2; i++)
#pragma unroll
            for (int j = 0; j < 2; j++)
#pragma unroll
                for (int r = 0; r < 16; r++) acc[i][j][r] = g == 0 ? ga[i][j][r] : acc[i][j][r] + ga[i][j][r];
    }
    // lane holds column l32 of each 32 x 32 tile and rows 8q + 4*half + p
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
        for (int r = 0; r < 16; r++) {
            const int64_t row = m_wave + i * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
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
