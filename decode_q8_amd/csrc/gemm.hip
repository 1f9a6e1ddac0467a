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
// tiles).  The k loop runs in stages of 4 blocks (128 values).  Stages move
// from HBM straight into LDS with global_load_lds_dwordx4 / _dword (no
// register staging), NS = 4 stages deep, so three stages are in flight while
// one is computed.  Every wave issues exactly LOADS_PER_STAGE such loads per
// stage; loads return in issue order, so "stage s has landed" is a vmcnt
// threshold, followed by one barrier per stage.  The k order inside one MFMA
// is the same for both operands (lane half h holds values 16h..16h+15 of the
// block), which is all an exact integer dot needs.
//
// LDS stage layout (35 KB, NS = 4 stages = 140 KB of gfx950's 160 KB):
//   A   16 KB  activation rows: row r's 16-byte chunk c at r*128 + (c ^ (r & 7))*16
//              (the XOR swizzle keeps the MFMA operand reads bank-conflict free)
//   B   16 KB  the two weight tiles' 4 block records, as packed (8 KB each)
//   SX   1 KB  activation scales [row][4 blocks]
//   SW   1 KB  weight scales [tile][row][4 blocks]
//   Z    1 KB  zeros, read by the lanes that carry no scale in the rank-1 MFMA
#include "device.hpp"
#include "launch.hpp"

namespace q8k {

constexpr int GT_M = 128;
constexpr int GT_N = 128;
constexpr int SB = 4;                        // blocks per stage
constexpr int NS = 4;                        // stages resident in LDS
constexpr int A_BYTES = GT_M * SB * QK;      // 16384
constexpr int B_TILE = SB * 2048;            // 8192: one weight tile's 4 block records
constexpr int B_BYTES = 2 * B_TILE;          // 16384
constexpr int S_BYTES = GT_M * SB * 2;       // 1024
constexpr int SX_OFF = A_BYTES + B_BYTES;
constexpr int SW_OFF = SX_OFF + S_BYTES;
constexpr int Z_OFF = SW_OFF + S_BYTES;
constexpr int STAGE_BYTES = Z_OFF + S_BYTES;  // 35840
constexpr int THREADS = 512;
constexpr int LOADS_PER_STAGE = 5;  // per wave: 2 activation, 2 weight, 1 scale

typedef _Float16 v4h __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef uint32_t v2u __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void *lds_ptr;

// Operand of the rank-1 scale MFMA: lanes 0..31 carry their fp16 scale in
// k = 0, every other element is zero.  Lanes 32..63 read their "scale" from
// the zero region, so the operand is built without a select.
__device__ __forceinline__ v4h rank1_operand(const uint8_t *p) {
    const v2u v = {(uint32_t)*reinterpret_cast<const uint16_t *>(p), 0u};
    return __builtin_bit_cast(v4h, v);
}

// Issue this wave's LOADS_PER_STAGE direct-to-LDS loads of stage s (blocks
// 4s..4s+3).  Each load writes 64 lanes x size bytes contiguously from the
// wave-uniform LDS address; the lane decides which global bytes it fetches.
__device__ __forceinline__ void issue_stage(uint8_t *buf, const int8_t *xq, const uint16_t *xs, int64_t M,
                                            int64_t m_tile, const uint8_t *w0, const uint8_t *w1, int64_t K,
                                            int64_t nb, int64_t s, int wave, int lane) {
    const int64_t blk0 = s * SB;
    const int64_t grp = s >> 1;
    const int bb0 = (int)(s & 1) * SB;
    const uint8_t *rec0 = w0 + grp * RECORD_BYTES;
    const uint8_t *rec1 = w1 + grp * RECORD_BYTES;
    // activations: 16 loads of 8 rows x 128 bytes, waves w and w + 8
#pragma unroll
    for (int u = 0; u < 2; u++) {
        const int i = wave + 8 * u;
        const int r = 8 * i + (lane >> 3);
        const int c = (lane & 7) ^ (lane >> 3);  // (r & 7) == lane >> 3
        int64_t row = m_tile + r;
        row = row < M ? row : M - 1;
        __builtin_amdgcn_global_load_lds(xq + row * K + blk0 * QK + c * 16, (lds_ptr)(buf + i * 1024), 16, 0, 0);
    }
    // weights: each tile's 4 block records are 8 KB contiguous; 8 loads per tile
#pragma unroll
    for (int u = 0; u < 2; u++) {
        const int q = wave + 8 * u;
        const uint8_t *rec = q < 8 ? rec0 : rec1;
        __builtin_amdgcn_global_load_lds(rec + bb0 * 2048 + (q & 7) * 1024 + lane * 16,
                                         (lds_ptr)(buf + A_BYTES + q * 1024), 16, 0, 0);
    }
    // scales, 4 bytes (two blocks) per lane: waves 0..3 activation rows, 4..7 weight rows
    const int d = (wave & 3) * 64 + lane;
    const int pair = d & 1;
    const void *src;
    if (wave < 4) {
        int64_t row = m_tile + (d >> 1);
        row = row < M ? row : M - 1;
        src = xs + row * nb + blk0 + 2 * pair;
    } else {
        const uint8_t *rec = d < 128 ? rec0 : rec1;
        src = rec + RECORD_Q_BYTES + ((d >> 1) & 63) * 16 + bb0 * 2 + pair * 4;
    }
    __builtin_amdgcn_global_load_lds(src, (lds_ptr)(buf + SX_OFF + wave * 256), 4, 0, 0);
}

// Wait until this wave's loads of the stage about to be computed have landed
// (pending = how many later stages it has issued since), then barrier, so
// every wave's loads have landed and every wave is done with the stage
// before it.
__device__ __forceinline__ void stage_barrier(int pending) {
    if (pending >= 2)
        asm volatile("s_waitcnt vmcnt(10) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    else if (pending == 1)
        asm volatile("s_waitcnt vmcnt(5) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    else
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
static_assert(NS == 4 && LOADS_PER_STAGE == 5, "stage_barrier's vmcnt thresholds assume 4 stages of 5 loads");

struct Lane {
    int a_off[SB];  // activation chunk offsets of this lane's row, per block
    int b_off;      // weight chunk offset in the wave's tile
    int sx_off, sw_off;
};

// One 256-value group = stages 2g and 2g + 1, resident in buffers 2P and 2P + 1.
template <int P>
__device__ __forceinline__ void group(float (&acc)[2][16], uint8_t *lds, const Lane &ln, const int8_t *xq,
                                      const uint16_t *xs, int64_t M, int64_t m_tile, const uint8_t *w0,
                                      const uint8_t *w1, int64_t K, int64_t nb, int64_t g, int64_t S, int wave,
                                      int lane) {
    float ga[2][16];
#pragma unroll
    for (int h = 0; h < 2; h++) {
        const int64_t s = 2 * g + h;
        const int64_t last = s + NS - 2 < S - 1 ? s + NS - 2 : S - 1;  // latest stage issued so far
        stage_barrier((int)(last - s));
        if (s + NS - 1 < S)
            issue_stage(lds + ((2 * P + h + NS - 1) % NS) * STAGE_BYTES, xq, xs, M, m_tile, w0, w1, K, nb,
                        s + NS - 1, wave, lane);
        const uint8_t *buf = lds + (2 * P + h) * STAGE_BYTES;
#pragma unroll
        for (int bb = 0; bb < SB; bb++) {
            const v4i a = *reinterpret_cast<const v4i *>(buf + ln.a_off[bb]);
            const v4h as = rank1_operand(buf + ln.sx_off + bb * 2);
            v4i b[2];
            v4h bs[2];
#pragma unroll
            for (int j = 0; j < 2; j++) {
                b[j] = *reinterpret_cast<const v4i *>(buf + A_BYTES + ln.b_off + bb * 2048 + j * 512);
                bs[j] = rank1_operand(buf + ln.sw_off + j * 256 + bb * 2);
            }
#pragma unroll
            for (int j = 0; j < 2; j++) {
                const v16i zi = {0};
                const v16f zf = {0};
                const v16i sv = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b[j], zi, 0, 0, 0);
                const v16f sp = __builtin_amdgcn_mfma_f32_32x32x8f16(as, bs[j], zf, 0, 0, 0);
#pragma unroll
                for (int r = 0; r < 16; r++)
                    ga[j][r] = (h == 0 && bb == 0) ? (float)sv[r] * sp[r]
                                                   : __builtin_fmaf((float)sv[r], sp[r], ga[j][r]);
            }
            // pin the block's results here, so the epilogue is not sunk past the
            // next stage's barrier with every MFMA result of the stage live
#pragma unroll
            for (int j = 0; j < 2; j++)
#pragma unroll
                for (int r = 0; r < 16; r++) asm volatile("" : "+v"(ga[j][r]));
        }
    }
#pragma unroll
    for (int j = 0; j < 2; j++)
#pragma unroll
        for (int r = 0; r < 16; r++) acc[j][r] += ga[j][r];
}

__global__ __launch_bounds__(512) void gemm_kernel(const int8_t *__restrict__ xq, const uint16_t *__restrict__ xs,
                                                      int64_t M, const uint8_t *__restrict__ w, int64_t N, int64_t K,
                                                      float *__restrict__ y, int64_t ld_y) {
    __shared__ __attribute__((aligned(1024))) uint8_t lds[NS * STAGE_BYTES];  // 140 KB of gfx950's 160 KB
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = wave_id();
    const int wm = wave & 3, wn = wave >> 2;  // 32-row strip wm of packed tile wn
    const int half = lane >> 5, l32 = lane & 31;
    const int64_t m_tile = (int64_t)blockIdx.y * GT_M;
    const int64_t T0 = (int64_t)blockIdx.x * 2;  // packed weight tiles T0 and T0 + 1
    const int64_t tiles = N / TILE_ROWS;
    const bool has1 = T0 + 1 < tiles;
    const int64_t G = K / GROUP_K;
    const int64_t S = 2 * G;  // stages
    const int64_t nb = K / QK;
    const uint8_t *w0 = w + (T0 * G) * RECORD_BYTES;
    const uint8_t *w1 = has1 ? w + ((T0 + 1) * G) * RECORD_BYTES : w0;  // tile 2 absent: reload tile 1

    if (tid < NS * S_BYTES / 16) {  // every buffer's zero region, written once
        const int b = tid / (S_BYTES / 16), c = tid % (S_BYTES / 16);
        *reinterpret_cast<uint4 *>(lds + b * STAGE_BYTES + Z_OFF + c * 16) = make_uint4(0u, 0u, 0u, 0u);
    }
    __syncthreads();
    for (int s = 0; s < NS - 1; s++)
        if (s < S) issue_stage(lds + s * STAGE_BYTES, xq, xs, M, m_tile, w0, w1, K, nb, s, wave, lane);

    Lane ln;
    const int row = wm * 32 + l32;
#pragma unroll
    for (int bb = 0; bb < SB; bb++) ln.a_off[bb] = row * 128 + (((2 * bb + half) ^ (row & 7)) * 16);
    ln.b_off = wn * B_TILE + half * 1024 + l32 * 16;
    ln.sx_off = (half == 0 ? SX_OFF : Z_OFF) + row * 8;
    ln.sw_off = (half == 0 ? SW_OFF : Z_OFF) + (wn * 64 + l32) * 8;

    float acc[2][16];
#pragma unroll
    for (int j = 0; j < 2; j++)
#pragma unroll
        for (int r = 0; r < 16; r++) acc[j][r] = -0.0f;  // -0 + x == x for every x
    for (int64_t g = 0; g < G; g += 2) {
        group<0>(acc, lds, ln, xq, xs, M, m_tile, w0, w1, K, nb, g, S, wave, lane);
        if (g + 1 < G) group<1>(acc, lds, ln, xq, xs, M, m_tile, w0, w1, K, nb, g + 1, S, wave, lane);
    }
    if (wn == 1 && !has1) return;
    const int64_t n_wave = (T0 + wn) * TILE_ROWS;
    // lane holds column l32 of each 32 x 32 tile and rows 8q + 4*half + p
#pragma unroll
    for (int r = 0; r < 16; r++) {
        const int64_t orow = m_tile + wm * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
        if (orow >= M) continue;
#pragma unroll
        for (int j = 0; j < 2; j++) y[orow * ld_y + n_wave + j * 32 + l32] = acc[j][r];
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
