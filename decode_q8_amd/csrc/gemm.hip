// Prefill GEMM (m > 8) for gfx950 on int8 MFMA.
//
// The Q8_0 block dot is a dense int8 contraction per 32-value block ("ferro"
// README, "How the iGPU path is fast", item 1: int8 GEMMs with activations
// quantized per 32-block).  One v_mfma_i32_32x32x32_i8 covers exactly one
// block for a 32 x 32 output tile, so its int32 results are the exact block
// dots s.  The per-block scale product Dx[m] * Dw[n] of the same tile comes
// from a rank-1 f16 MFMA (one non-zero k: fp16 x fp16 is exact in fp32), so
// it lands in the same register layout as s and the VALU only converts s and
// fuses it in:
//   group accumulator  a = fma(float(s), Dx * Dw, a)  over the 8 blocks of a
//                          256-value group (the first block multiplies),
//   output             y = ((a_0 + a_1) + a_2) + ...   over the groups.
// The order depends on k only, so each row is bit-identical for any m and
// any row order.  Two VALU operations per output and block remain, on top of
// the staging of the operands through LDS.
//
// Tiling: each wave owns a 32 x 64 output strip (1 x 2 MFMA tiles); a
// workgroup of WM x WN = 4 x 2 waves owns a 128 x 128 tile when the problem
// has at least 256 such tiles; smaller problems run gemm_strip_kernel below
// (32 x 64 strips, k split across 8 waves).  The k loop runs in stages of 4
// blocks (128 values).  Stages move
// from HBM straight into LDS with global_load_lds_dwordx4 / _dword (no
// register staging), NS = 4 stages deep, so three stages are in flight while
// one is computed.  Every wave issues exactly LOADS_PER_STAGE such loads per
// stage; loads return in issue order, so "stage s has landed" is a vmcnt
// threshold, followed by one barrier per stage.  The k order inside one MFMA
// is the same for both operands (lane half h holds values 16h..16h+15 of the
// block), which is all an exact integer dot needs.
//
// LDS stage layout (128 x 128: 34 KB, NS = 4 stages = 136 KB of gfx950's
// 160 KB):
//   A   activation rows: row r's 16-byte chunk c at r*128 + (c ^ (r & 7))*16
//       (the XOR swizzle keeps the MFMA operand reads bank-conflict free)
//   B   the weight tiles' 4 block records, as packed (8 KB per tile)
//   SX  activation scales [row][4 blocks]
//   SW  weight scales [tile][row][4 blocks]
#include "device.hpp"
#include "launch.hpp"

namespace q8k {

constexpr int SB = 4;   // blocks per stage
constexpr int NS = 4;   // stages resident in LDS

// Workgroup shape: WM x WN waves, each a 32 x 64 output strip (1 x 2 MFMA
// tiles), so the workgroup tile is (32 WM) x (64 WN).
template <int WM, int WN>
struct Tile {
    static constexpr int WAVES = WM * WN;
    static constexpr int THREADS = 64 * WAVES;
    static constexpr int ROWS = 32 * WM;                  // output rows per workgroup
    static constexpr int COLS = 64 * WN;                  // output columns (packed tiles x 64)
    static constexpr int A_BYTES = ROWS * SB * QK;         // activation rows, 128 bytes each
    static constexpr int B_BYTES = WN * SB * 2048;         // WN weight tiles' 4 block records
    static constexpr int SX_BYTES = ROWS * SB * 2;
    static constexpr int SW_BYTES = COLS * SB * 2;
    static constexpr int SX_OFF = A_BYTES + B_BYTES;
    static constexpr int SW_OFF = SX_OFF + SX_BYTES;
    static constexpr int STAGE_BYTES = SW_OFF + SW_BYTES;
    // direct-to-LDS loads per stage: 1 KB activation / weight loads, 256-byte scale loads
    static constexpr int NA = A_BYTES / 1024, NB = B_BYTES / 1024, NSX = SX_BYTES / 256, NSW = SW_BYTES / 256;
    static constexpr int LOADS = NA + NB + NSX + NSW;
    static constexpr int PER_WAVE = (LOADS + WAVES - 1) / WAVES;  // a wave short of work repeats its last load
    static_assert(PER_WAVE * (NS - 2) <= 63, "vmcnt threshold out of range");
};

typedef _Float16 v4h __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v32f __attribute__((ext_vector_type(32)));
typedef uint32_t v2u __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void *lds_ptr;

// Operand of the rank-1 scale MFMA: the lane's fp16 scale in k = 0, zeros in
// k = 1..3.  One v_mfma_f32_32x32x4_2b_f16 then yields the scale products
// Dx * Dw of both 32 x 32 tiles of a wave (block 0 of the instruction: lanes
// 0..31, tile 0; block 1: lanes 32..63, tile 1), each in the register layout of
// the i8 MFMA's output.
__device__ __forceinline__ v4h rank1_operand(const uint8_t *p) {
    const v2u v = {(uint32_t)*reinterpret_cast<const uint16_t *>(p), 0u};
    return __builtin_bit_cast(v4h, v);
}

// This wave's PER_WAVE direct-to-LDS loads of a stage (load i of a stage goes
// to wave i % WAVES).  Each load writes 64 lanes x size bytes contiguously
// from a wave-uniform LDS offset; the lane decides which global bytes it
// fetches.  Every address is this lane's stage-0 address plus a wave-uniform
// offset of the stage, (s >> 1) * p + (s & 1) * q (two stages per 256-value
// group; the weight records of group s / 2 are RECORD_BYTES apart), so a
// stage costs one 64-bit add per load instead of the address arithmetic.
template <int WM, int WN>
struct StageLoads {
    using T = Tile<WM, WN>;
    const uint8_t *g[T::PER_WAVE];  // this lane's global address in stage 0
    int lds[T::PER_WAVE];           // offset in the stage buffer (wave-uniform)
    int p[T::PER_WAVE], q[T::PER_WAVE];
    bool wide[T::PER_WAVE];         // 16-byte loads (operands), else 4-byte (scales)

    // Stage 0 of the workgroup at output rows m_tile.. and packed tiles from
    // w_tiles (tile_stride bytes apart; 0: one tile, reloaded).  Activation
    // rows past M read row M - 1 (their outputs are not stored).
    __device__ __forceinline__ void init(const int8_t *xq, const uint16_t *xs, int64_t M, int64_t m_tile,
                                         const uint8_t *w_tiles, int64_t tile_stride, int64_t K, int64_t nb, int wave,
                                         int lane) {
#pragma unroll
        for (int u = 0; u < T::PER_WAVE; u++) {
            int i = wave + T::WAVES * u;
            i = i < T::LOADS ? i : T::LOADS - 1;  // a wave short of work repeats the last load
            if (i < T::NA) {  // activations: 8 rows x 128 bytes, row r's chunk c at position c ^ (r & 7)
                const int r = 8 * i + (lane >> 3);
                const int c = (lane & 7) ^ (lane >> 3);
                int64_t row = m_tile + r;
                row = row < M ? row : M - 1;
                g[u] = reinterpret_cast<const uint8_t *>(xq + row * K + c * 16);
                lds[u] = i * 1024;
                p[u] = 2 * SB * QK;
                q[u] = SB * QK;
                wide[u] = true;
            } else if (i < T::NA + T::NB) {  // weights: a tile's 4 block records are 8 KB contiguous
                const int e = i - T::NA;
                g[u] = w_tiles + (e >> 3) * tile_stride + (e & 7) * 1024 + lane * 16;
                lds[u] = T::A_BYTES + e * 1024;
                p[u] = RECORD_BYTES;
                q[u] = SB * 2048;
                wide[u] = true;
            } else if (i < T::NA + T::NB + T::NSX) {  // activation scales [row][4], 4 bytes per lane
                const int e = i - T::NA - T::NB;
                const int d = e * 64 + lane;
                int64_t row = m_tile + (d >> 1);
                row = row < M ? row : M - 1;
                g[u] = reinterpret_cast<const uint8_t *>(xs + row * nb + 2 * (d & 1));
                lds[u] = T::SX_OFF + e * 256;
                p[u] = 2 * SB * 2;
                q[u] = SB * 2;
                wide[u] = false;
            } else {  // weight scales [tile][row][4], 4 bytes per lane
                const int e = i - T::NA - T::NB - T::NSX;
                const int d = e * 64 + lane;
                g[u] = w_tiles + (d >> 7) * tile_stride + RECORD_Q_BYTES + ((d >> 1) & 63) * 16 + (d & 1) * 4;
                lds[u] = T::SW_OFF + e * 256;
                p[u] = RECORD_BYTES;
                q[u] = SB * 2;
                wide[u] = false;
            }
        }
    }

    __device__ __forceinline__ void issue(uint8_t *buf, int64_t s) const {
        const int half = (int)(s >> 1), odd = (int)(s & 1);
#pragma unroll
        for (int u = 0; u < T::PER_WAVE; u++) {
            const uint8_t *src = g[u] + ((int64_t)half * p[u] + odd * q[u]);
            if (wide[u])
                __builtin_amdgcn_global_load_lds(src, (lds_ptr)(buf + lds[u]), 16, 0, 0);
            else
                __builtin_amdgcn_global_load_lds(src, (lds_ptr)(buf + lds[u]), 4, 0, 0);
        }
    }
};

// Wait until this wave's loads of the stage about to be computed have landed
// (pending = how many later stages it has issued since), then barrier, so
// every wave's loads have landed and every wave is done with the stage
// before it.
template <int L>
__device__ __forceinline__ void stage_barrier(int pending) {
    static_assert(NS == 4, "thresholds below assume at most two later stages in flight");
    if (pending >= 2)
        asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(2 * L) : "memory");
    else if (pending == 1)
        asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(L) : "memory");
    else
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

struct Lane {
    int a_off[SB];  // activation chunk offsets of this lane's row, per block
    int b_off;      // weight chunk offset in the wave's tile
    int sx_off, sw_off;
};


// Read block bb's operands from the stage buffer and issue its MFMAs: the
// exact int32 block dots (one i8 MFMA per 32 x 32 tile) and the rank-1 scale
// products Dx * Dw in the same register layout.
template <typename T>
__device__ __forceinline__ void mfma_block(v16i (&sv)[2], v16f (&sp)[2], const uint8_t *buf, const Lane &ln, int bb) {
    const v4i av = *reinterpret_cast<const v4i *>(buf + ln.a_off[bb]);
    const v4h as = rank1_operand(buf + ln.sx_off + bb * 2);
    const v4h bs = rank1_operand(buf + ln.sw_off + bb * 2);
    v4i b[2];
#pragma unroll
    for (int j = 0; j < 2; j++) b[j] = *reinterpret_cast<const v4i *>(buf + T::A_BYTES + ln.b_off + bb * 2048 + j * 512);
    const v16i zi = {0};
    const v32f zf = {0};
#pragma unroll
    for (int j = 0; j < 2; j++) sv[j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(av, b[j], zi, 0, 0, 0);
    const v32f pp = __builtin_amdgcn_mfma_f32_32x32x4f16(as, bs, zf, 0, 0, 0);
    sp[0] = __builtin_shufflevector(pp, pp, 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15);
    sp[1] = __builtin_shufflevector(pp, pp, 16, 17, 18, 19, 20, 21, 22, 23, 24, 25, 26, 27, 28, 29, 30, 31);
}

// One 256-value group = stages 2g and 2g + 1, resident in buffers 2P and 2P + 1.
template <int WM, int WN, int P>
__device__ __forceinline__ void group(float (&acc)[2][16], uint8_t *lds, const Lane &ln, const StageLoads<WM, WN> &sl,
                                      int64_t S, int64_t g) {
    using T = Tile<WM, WN>;
    float ga[2][16];
#pragma unroll
    for (int h = 0; h < 2; h++) {
        const int64_t s = 2 * g + h;
        const int64_t last = s + NS - 2 < S - 1 ? s + NS - 2 : S - 1;  // latest stage issued so far
        stage_barrier<T::PER_WAVE>((int)(last - s));
        if (s + NS - 1 < S) sl.issue(lds + ((2 * P + h + NS - 1) % NS) * T::STAGE_BYTES, s + NS - 1);
        const uint8_t *buf = lds + (2 * P + h) * T::STAGE_BYTES;
        // Software pipeline over the stage's blocks: the MFMAs of block bb + 1
        // are issued before the VALU epilogue of block bb, so the matrix core
        // works while the VALU converts and accumulates the previous result.
        v16i sv[2][2];
        v16f sp[2][2];
        mfma_block<T>(sv[0], sp[0], buf, ln, 0);
#pragma unroll
        for (int bb = 0; bb < SB; bb++) {
            if (bb + 1 < SB) mfma_block<T>(sv[(bb + 1) & 1], sp[(bb + 1) & 1], buf, ln, bb + 1);
#pragma unroll
            for (int j = 0; j < 2; j++)
#pragma unroll
                for (int r = 0; r < 16; r++)
                    ga[j][r] = (h == 0 && bb == 0)
                                   ? (float)sv[bb & 1][j][r] * sp[bb & 1][j][r]
                                   : __builtin_fmaf((float)sv[bb & 1][j][r], sp[bb & 1][j][r], ga[j][r]);
            // pin the block's results here, so the epilogue is not sunk past the
            // next stage's barrier with every MFMA result of the stage live
#pragma unroll
            for (int j = 0; j < 2; j++)
#pragma unroll
                for (int r = 0; r < 16; r++) asm volatile("" : "+v"(ga[j][r]));
            // interleave: operand reads, then each MFMA followed by a slice of the
            // epilogue, so the VALU runs while the matrix core is busy
            __builtin_amdgcn_sched_group_barrier(0x100, 5, 0);  // LDS reads
            __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);  // VALU
#pragma unroll
            for (int i = 0; i < 3; i++) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
                __builtin_amdgcn_sched_group_barrier(0x002, 19, 0);  // VALU
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    }
#pragma unroll
    for (int j = 0; j < 2; j++)
#pragma unroll
        for (int r = 0; r < 16; r++) acc[j][r] += ga[j][r];
}

// Output tile of this workgroup, XCD-aware.  A launch's workgroups go to the
// 8 XCDs round-robin by linear id, and each XCD has its own L2.  The tiles are
// put in a grouped order -- XCD_GROUP_M row blocks at a time, all column
// blocks of the group, the row blocks fastest -- and XCD x takes the x-th
// eighth of that order, so the workgroups one XCD runs at the same time
// cover a compact block of rows and columns and share their operand stages in
// its L2 (with the plain order, one XCD would hold every row block of a few
// column blocks and stream all of A through its L2).  Grids whose tile count
// is not a multiple of 8 keep the plain order.  Only speed depends on this.
constexpr int XCDS = 8;
constexpr int XCD_GROUP_M = 4;

__device__ __forceinline__ void xcd_tile(int &tm, int &tn) {
    const int tiles_n = gridDim.x, tiles_m = gridDim.y;
    const int total = tiles_n * tiles_m;
    const int id = blockIdx.x + tiles_n * blockIdx.y;
    if (total % XCDS) {
        tn = blockIdx.x;
        tm = blockIdx.y;
        return;
    }
    const int t = (id % XCDS) * (total / XCDS) + id / XCDS;  // position in the grouped order
    const int per_group = XCD_GROUP_M * tiles_n;
    const int first_m = (t / per_group) * XCD_GROUP_M;
    const int gm = tiles_m - first_m < XCD_GROUP_M ? tiles_m - first_m : XCD_GROUP_M;
    const int r = t % per_group;
    tm = first_m + r % gm;
    tn = r / gm;
}

template <int WM, int WN>
__global__ __launch_bounds__(64 * WM * WN) void gemm_kernel(const int8_t *__restrict__ xq,
                                                             const uint16_t *__restrict__ xs, int64_t M,
                                                             const uint8_t *__restrict__ w, int64_t N, int64_t K,
                                                             float *__restrict__ y, int64_t ld_y) {
    using T = Tile<WM, WN>;
    __shared__ __attribute__((aligned(1024))) uint8_t lds[NS * T::STAGE_BYTES];
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = wave_id();
    const int wm = wave % WM, wn = wave / WM;  // 32-row strip wm of packed tile wn
    const int half = lane >> 5, l32 = lane & 31;
    const int64_t tiles = N / TILE_ROWS;
    int tm, tn;  // the workgroup's output tile (row block, column block)
    xcd_tile(tm, tn);
    const int64_t T0 = (int64_t)tn * WN;  // the workgroup's first packed weight tile
    const int64_t G = K / GROUP_K, S = 2 * G;
    const int64_t m_tile = (int64_t)tm * T::ROWS;
    const bool ragged = T0 + WN > tiles;
    StageLoads<WM, WN> sl;
    // tiles past the last one (N not a multiple of the workgroup's columns) reload the last tile
    sl.init(xq, xs, M, m_tile, w + (T0 * G) * RECORD_BYTES, ragged ? 0 : G * RECORD_BYTES, K, K / QK, wave, lane);
    for (int s = 0; s < NS - 1; s++)
        if (s < S) sl.issue(lds + s * T::STAGE_BYTES, s);

    Lane ln;
    const int row = wm * 32 + l32;
#pragma unroll
    for (int bb = 0; bb < SB; bb++) ln.a_off[bb] = row * 128 + (((2 * bb + half) ^ (row & 7)) * 16);
    ln.b_off = wn * SB * 2048 + half * 1024 + l32 * 16;
    ln.sx_off = T::SX_OFF + row * 8;
    ln.sw_off = T::SW_OFF + (wn * 64 + half * 32 + l32) * 8;

    float acc[2][16];
#pragma unroll
    for (int j = 0; j < 2; j++)
#pragma unroll
        for (int r = 0; r < 16; r++) acc[j][r] = -0.0f;  // -0 + x == x for every x
    for (int64_t g = 0; g < G; g += 2) {
        group<WM, WN, 0>(acc, lds, ln, sl, S, g);
        if (g + 1 < G) group<WM, WN, 1>(acc, lds, ln, sl, S, g + 1);
    }
    if (ragged && T0 + wn >= tiles) return;
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

template <int WM, int WN>
static hipError_t launch_tiles(const int8_t *xq, const uint16_t *xs, int64_t m, const uint8_t *w, int64_t n,
                               int64_t k, float *y, int64_t ld_y, hipStream_t s) {
    using T = Tile<WM, WN>;
    const dim3 grid((unsigned)((n + T::COLS - 1) / T::COLS), (unsigned)((m + T::ROWS - 1) / T::ROWS));
    hipLaunchKernelGGL((gemm_kernel<WM, WN>), grid, dim3(T::THREADS), 0, s, xq, xs, m, w, n, k, y, ld_y);
    return hipGetLastError();
}

// Small problems: one workgroup of 8 waves owns a 32 x 64 output strip (32
// rows, one packed weight tile) and splits k across its waves instead.  The k
// loop runs in batches of up to 8 groups, one per wave: each wave loads its
// group's operands straight into registers (26 16-byte loads per lane, all in
// flight together), forms the group accumulator a_g exactly as the tiled
// kernel does (same MFMAs, same convert / multiply / fma sequence), and parks
// it in LDS; after a barrier the 512 threads fold the batch's a_g into their
// outputs' running sums in group order, so every output sees the same
// sequence of fp32 operations as in the tiled kernel and rows stay
// bit-identical whichever kernel m selects.  Many small strips with all waves
// busy replace few large tiles with one wave per SIMD.
constexpr int STRIP_WAVES = 8;

__global__ __launch_bounds__(512) void gemm_strip_kernel(const int8_t *__restrict__ xq,
                                                         const uint16_t *__restrict__ xs, int64_t M,
                                                         const uint8_t *__restrict__ w, int64_t N, int64_t K,
                                                         float *__restrict__ y, int64_t ld_y) {
    __shared__ float park[STRIP_WAVES][2 * 16 * 64];  // [wave][(j * 16 + r) * 64 + lane]: 64 KB
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = wave_id();
    const int half = lane >> 5, l32 = lane & 31;
    const int64_t m0 = (int64_t)blockIdx.y * 32;
    const int64_t T = blockIdx.x;
    const int G = (int)(K >> 8), nb = (int)(K >> 5);
    int64_t row = m0 + l32;
    row = row < M ? row : M - 1;
    const int8_t *xrow = xq + row * K + half * 16;
    const uint16_t *xsrow = xs + row * nb;
    const uint8_t *wt = w + T * (int64_t)G * RECORD_BYTES;
    float acc[4];
#pragma unroll
    for (int i = 0; i < 4; i++) acc[i] = -0.0f;  // -0 + x == x for every x
    for (int g0 = 0; g0 < G; g0 += STRIP_WAVES) {
        const int g = g0 + wave;
        if (g < G) {
            const uint8_t *rec = wt + (int64_t)g * RECORD_BYTES;
            // scales first: loads complete in order, so block 0 can start while the rest arrive
            const uint4 sx = *reinterpret_cast<const uint4 *>(xsrow + g * GROUP_BLOCKS);  // the row's 8 scales
            const uint4 sw = *reinterpret_cast<const uint4 *>(rec + RECORD_Q_BYTES + (half * 32 + l32) * 16);
            __builtin_amdgcn_sched_barrier(0);
            v4i a[GROUP_BLOCKS], b[GROUP_BLOCKS][2];
#pragma unroll
            for (int bb = 0; bb < GROUP_BLOCKS; bb++) {
                a[bb] = *reinterpret_cast<const v4i *>(xrow + (g * GROUP_BLOCKS + bb) * QK);
#pragma unroll
                for (int j = 0; j < 2; j++)
                    b[bb][j] = *reinterpret_cast<const v4i *>(rec + bb * 2048 + half * 1024 + (j * 32 + l32) * 16);
                __builtin_amdgcn_sched_barrier(0);
            }
            // all of the group's loads are in flight before the first MFMA
            float ga[2][16];
#pragma unroll
            for (int bb = 0; bb < GROUP_BLOCKS; bb++) {
                const v2u xa = {(word_of(sx, bb >> 1) >> (16 * (bb & 1))) & 0xffffu, 0u};
                const v2u wa = {(word_of(sw, bb >> 1) >> (16 * (bb & 1))) & 0xffffu, 0u};
                const v16i zi = {0};
                const v32f zf = {0};
                v16i sv[2];
#pragma unroll
                for (int j = 0; j < 2; j++) sv[j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[bb], b[bb][j], zi, 0, 0, 0);
                const v32f pp = __builtin_amdgcn_mfma_f32_32x32x4f16(__builtin_bit_cast(v4h, xa),
                                                                     __builtin_bit_cast(v4h, wa), zf, 0, 0, 0);
#pragma unroll
                for (int j = 0; j < 2; j++)
#pragma unroll
                    for (int r = 0; r < 16; r++)
                        ga[j][r] = bb == 0 ? (float)sv[j][r] * pp[16 * j + r]
                                           : __builtin_fmaf((float)sv[j][r], pp[16 * j + r], ga[j][r]);
            }
#pragma unroll
            for (int j = 0; j < 2; j++)
#pragma unroll
                for (int r = 0; r < 16; r++) park[wave][(j * 16 + r) * 64 + lane] = ga[j][r];
        }
        __syncthreads();
        const int gn = G - g0 < STRIP_WAVES ? G - g0 : STRIP_WAVES;
        for (int q = 0; q < gn; q++)
#pragma unroll
            for (int i = 0; i < 4; i++) acc[i] += park[q][tid + 512 * i];
        __syncthreads();
    }
    // thread tid holds outputs o = tid + 512 i, o = (j * 16 + r) * 64 + lane of the MFMA layout:
    // column j * 32 + (lane & 31), row 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3)
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const int o = tid + 512 * i;
        const int ol = o & 63, r = (o >> 6) & 15, j = o >> 10;
        const int64_t orow = m0 + 8 * (r >> 2) + 4 * (ol >> 5) + (r & 3);
        if (orow < M) y[orow * ld_y + T * TILE_ROWS + j * 32 + (ol & 31)] = acc[i];
    }
}

// Kernel by problem size: 128 x 128 tiles when there are at least 256 of them
// (one per CU), else 32 x 64 strips with k split across the waves.  Each
// output's arithmetic is the same in both, so rows stay bit-identical across m.
static bool gemm_tiled(int64_t m, int64_t n) { return ((m + 127) / 128) * ((n + 127) / 128) >= 256; }

hipError_t launch_gemm(const void *x_q, int64_t m, const void *w, int64_t n, int64_t k, float *y, int64_t ld_y,
                       hipStream_t s) {
    const int8_t *xq = (const int8_t *)x_q;
    const uint16_t *xs = (const uint16_t *)((const uint8_t *)x_q + m * k);
    const uint8_t *wb = (const uint8_t *)w;
    if (gemm_tiled(m, n)) return launch_tiles<4, 2>(xq, xs, m, wb, n, k, y, ld_y, s);
    const dim3 grid((unsigned)(n / TILE_ROWS), (unsigned)((m + 31) / 32));
    hipLaunchKernelGGL(gemm_strip_kernel, grid, dim3(512), 0, s, xq, xs, m, wb, n, k, y, ld_y);
    return hipGetLastError();
}

}  // namespace q8k
