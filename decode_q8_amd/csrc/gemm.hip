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
// Tiling: a 512-thread workgroup owns a 128 x 128 output tile (two packed
// 64-row weight tiles); each of its 8 waves a 32 x 64 strip (1 x 2 MFMA
// tiles), which keeps a wave's accumulators small enough for 4 waves per
// SIMD.  The
// k loop runs in stages of 4 blocks (128 values): the workgroup copies the
// stage's activation rows, the two weight tiles' 4 block records (each 8 KB
// contiguous in the packed layout) and both sets of scales into LDS, double
// buffered, so the global loads of stage s + 1 are in flight while stage s
// is computed.  The k order inside one MFMA is the same for both operands
// (lane half h holds values 16h..16h+15 of the block), which is all an exact
// integer dot needs.
#include "device.hpp"
#include "launch.hpp"

namespace q8k {

constexpr int GT_M = 128;
constexpr int GT_N = 128;
constexpr int SB = 4;                            // blocks per stage
constexpr int A_ROW = SB * QK + 16;              // 144: padded LDS row of the activation stage
constexpr int A_BYTES = GT_M * A_ROW;            // 18432
constexpr int B_TILE = SB * 2048;                // 8192: one weight tile's 4 block records
constexpr int B_BYTES = 2 * B_TILE;              // 16384
constexpr int S_BYTES = SB * GT_M * 2;           // 1024: fp16 scales [block][row]
constexpr int STAGE_BYTES = A_BYTES + B_BYTES + 2 * S_BYTES;  // 36864

typedef _Float16 v4h __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int THREADS = 512;

// Operand of the rank-1 scale MFMA: lanes 0..31 carry their fp16 scale in
// k = 0, every other element is zero.
__device__ __forceinline__ v4h rank1_operand(uint16_t h16, bool low_half) {
    v4h v = {(_Float16)0.0f, (_Float16)0.0f, (_Float16)0.0f, (_Float16)0.0f};
    if (low_half) v[0] = __builtin_bit_cast(_Float16, h16);
    return v;
}

// One stage's global loads: two 16-byte activation chunks, one 16-byte chunk
// of each weight tile's records and 8 bytes of scales per thread.
__device__ __forceinline__ void load_stage(uint4 &a0, uint4 &a1, uint4 &b0, uint4 &b1, uint2 &sc, const int8_t *xq,
                                           const uint16_t *xs, int64_t M, int64_t m_tile, const uint8_t *rec0,
                                           const uint8_t *rec1, int64_t K, int64_t nb, int64_t blk0, int bb0,
                                           int tid) {
    // activation rows tid / 8 and 64 + tid / 8, 16-byte chunk tid % 8
    int64_t ra0 = m_tile + (tid >> 3), ra1 = ra0 + 64;
    ra0 = ra0 < M ? ra0 : M - 1;
    ra1 = ra1 < M ? ra1 : M - 1;
    a0 = *reinterpret_cast<const uint4 *>(xq + ra0 * K + blk0 * QK + (tid & 7) * 16);
    a1 = *reinterpret_cast<const uint4 *>(xq + ra1 * K + blk0 * QK + (tid & 7) * 16);
    // each weight tile's 4 block records are 8 KB contiguous: chunk tid of each
    b0 = *reinterpret_cast<const uint4 *>(rec0 + bb0 * 2048 + tid * 16);
    b1 = *reinterpret_cast<const uint4 *>(rec1 + bb0 * 2048 + tid * 16);  // rec1 == rec0 when tile 2 is absent
    // scales: threads 0..127 one activation row each, 128..255 one weight row each
    int64_t rs = m_tile + (tid & 127);
    rs = rs < M ? rs : M - 1;
    const uint8_t *rec = (tid & 64) ? rec1 : rec0;
    const uint8_t *sp = tid < GT_M ? reinterpret_cast<const uint8_t *>(xs + rs * nb + blk0)
                                   : rec + RECORD_Q_BYTES + (tid & 63) * 16 + bb0 * 2;
    sc = *reinterpret_cast<const uint2 *>(sp);
}

__device__ __forceinline__ void store_stage(const uint4 &a0, const uint4 &a1, const uint4 &b0, const uint4 &b1,
                                            const uint2 &sc, uint8_t *lds, int tid) {
    uint8_t *A = lds, *B = lds + A_BYTES;
    *reinterpret_cast<uint4 *>(A + (tid >> 3) * A_ROW + (tid & 7) * 16) = a0;
    *reinterpret_cast<uint4 *>(A + (64 + (tid >> 3)) * A_ROW + (tid & 7) * 16) = a1;
    *reinterpret_cast<uint4 *>(B + tid * 16) = b0;
    *reinterpret_cast<uint4 *>(B + B_TILE + tid * 16) = b1;
    if (tid >= 2 * GT_M) return;
    uint16_t *S = reinterpret_cast<uint16_t *>(lds + A_BYTES + B_BYTES) + (tid < GT_M ? 0 : SB * GT_M);
    const int row = tid & 127;
    S[0 * GT_M + row] = (uint16_t)(sc.x & 0xffffu);
    S[1 * GT_M + row] = (uint16_t)(sc.x >> 16);
    S[2 * GT_M + row] = (uint16_t)(sc.y & 0xffffu);
    S[3 * GT_M + row] = (uint16_t)(sc.y >> 16);
}

__global__ __launch_bounds__(512) void gemm_kernel(const int8_t *__restrict__ xq, const uint16_t *__restrict__ xs,
                                                      int64_t M, const uint8_t *__restrict__ w, int64_t N, int64_t K,
                                                      float *__restrict__ y, int64_t ld_y) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[2 * STAGE_BYTES];  // 72 KB: gfx950 has 160 KB per CU
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = wave_id();
    const int wm = wave & 3, wn = wave >> 2;  // 32-row strip wm of packed tile wn
    const int half = lane >> 5, l32 = lane & 31;
    const bool low = half == 0;
    const int64_t m_tile = (int64_t)blockIdx.y * GT_M;
    const int64_t T0 = (int64_t)blockIdx.x * 2;  // packed weight tiles T0 and T0 + 1
    const int64_t tiles = N / TILE_ROWS;
    const bool has1 = T0 + 1 < tiles;
    const int64_t G = K / GROUP_K;
    const int64_t nb = K / QK;
    const int64_t stages = G * (GROUP_BLOCKS / SB);

    uint4 a0, a1, b0, b1;
    uint2 sc;
    {
        const uint8_t *rec0 = w + (T0 * G) * RECORD_BYTES;
        const uint8_t *rec1 = has1 ? w + ((T0 + 1) * G) * RECORD_BYTES : rec0;
        load_stage(a0, a1, b0, b1, sc, xq, xs, M, m_tile, rec0, rec1, K, nb, 0, 0, tid);
        store_stage(a0, a1, b0, b1, sc, lds, tid);
    }
    __syncthreads();

    float acc[2][16], ga[2][16];
    for (int64_t s = 0; s < stages; s++) {
        if (s + 1 < stages) {
            const int64_t g1 = (s + 1) / 2;
            const int bb1 = (int)((s + 1) & 1) * SB;
            const uint8_t *rec0 = w + (T0 * G + g1) * RECORD_BYTES;
            const uint8_t *rec1 = has1 ? w + ((T0 + 1) * G + g1) * RECORD_BYTES : rec0;
            load_stage(a0, a1, b0, b1, sc, xq, xs, M, m_tile, rec0, rec1, K, nb, (s + 1) * SB, bb1, tid);
        }
        const uint8_t *buf = lds + (s & 1) * STAGE_BYTES;
        const uint8_t *A = buf;
        const uint8_t *B = buf + A_BYTES + wn * B_TILE;
        const uint16_t *SX = reinterpret_cast<const uint16_t *>(buf + A_BYTES + B_BYTES);
        const uint16_t *SW = SX + SB * GT_M;
        const bool first_half = (s & 1) == 0;
#pragma unroll
        for (int bb = 0; bb < SB; bb++) {
            const int row = wm * 32 + l32;
            const v4i a = *reinterpret_cast<const v4i *>(A + row * A_ROW + bb * QK + half * 16);
            const v4h as = rank1_operand(SX[bb * GT_M + row], low);
            v4i b[2];
            v4h bs[2];
#pragma unroll
            for (int j = 0; j < 2; j++) {
                b[j] = *reinterpret_cast<const v4i *>(B + bb * 2048 + half * 1024 + (j * 32 + l32) * 16);
                bs[j] = rank1_operand(SW[bb * GT_M + wn * 64 + j * 32 + l32], low);
            }
            const bool group_start = first_half && bb == 0;
#pragma unroll
            for (int j = 0; j < 2; j++) {
                const v16i zi = {0};
                const v16f zf = {0};
                const v16i sv = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b[j], zi, 0, 0, 0);
                const v16f sp = __builtin_amdgcn_mfma_f32_32x32x8f16(as, bs[j], zf, 0, 0, 0);
#pragma unroll
                for (int r = 0; r < 16; r++)
                    ga[j][r] = group_start ? (float)sv[r] * sp[r] : __builtin_fmaf((float)sv[r], sp[r], ga[j][r]);
            }
        }
        if (!first_half) {  // group g = s / 2 complete
#pragma unroll
            for (int j = 0; j < 2; j++)
#pragma unroll
                for (int r = 0; r < 16; r++) acc[j][r] = s == 1 ? ga[j][r] : acc[j][r] + ga[j][r];
        }
        if (s + 1 < stages) store_stage(a0, a1, b0, b1, sc, lds + ((s + 1) & 1) * STAGE_BYTES, tid);
        __syncthreads();
    }
    if (wn == 1 && !has1) return;
    const int64_t n_wave = (T0 + wn) * TILE_ROWS;
    // lane holds column l32 of each 32 x 32 tile and rows 8q + 4*half + p
#pragma unroll
    for (int r = 0; r < 16; r++) {
        const int64_t row = m_tile + wm * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
        if (row >= M) continue;
#pragma unroll
        for (int j = 0; j < 2; j++) y[row * ld_y + n_wave + j * 32 + l32] = acc[j][r];
    }
}

hipError_t launch_gemm(const void *x_q, int64_t m, const void *w, int64_t n, int64_t k, float *y, int64_t ld_y,
                       hipStream_t s) {
    const int8_t *xq = (const int8_t *)x_q;
    const uint16_t *xs = (const uint16_t *)((const uint8_t *)x_q + m * k);
    const dim3 grid((unsigned)((n + GT_N - 1) / GT_N), (unsigned)((m + GT_M - 1) / GT_M));
    hipLaunchKernelGGL(gemm_kernel, grid, dim3(THREADS), 0, s, xq, xs, m, (const uint8_t *)w, n, k, y, ld_y);
    return hipGetLastError();
}

}  // namespace q8k
