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
// workgroup of 4 x 2 waves owns a 128 x 128 tile when the problem has at
// least 256 such tiles; smaller problems run gemm_strip_kernel below (32 x 64
// strips, k split across 8 waves).  The 128 x 128 kernel's k loop is the
// generated inline-asm block of gemm_loop.inc (explicit registers and
// schedule): stages of 4 blocks (128 values) move from HBM straight into LDS
// with global_load_lds_dwordx4 / _dword (no register staging), four stages
// resident; every wave issues the same 5 loads per stage, so "stage s has
// landed" is a vmcnt threshold, followed by one barrier per stage; operand
// reads and MFMAs run one block ahead of the epilogue.  The k order inside
// one MFMA is the same for both operands (lane half h holds values
// 16h..16h+15 of the block), which is all an exact integer dot needs.
//
// LDS stage layout (128 x 128: 34 KB, NS = 4 stages = 136 KB of gfx950's
// 160 KB):
//   A   activation rows: row r's 16-byte chunk c at r*128 + (c ^ (r & 7))*16
//       (the XOR swizzle keeps the MFMA operand reads bank-conflict free)
//   B   the weight tiles' 4 block records, as packed (8 KB per tile)
//   SX  activation scales [row][4 blocks]
//   SW  weight scales [tile][row][4 blocks]
#include "device.hpp"
#include "gemm_loop.inc"
#include "gemm_strip.inc"
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

// The main loop is the generated inline-asm block of gemm_loop.inc (explicit
// registers and schedule; its header comment gives the register map and the
// pipeline).  This function computes the lane's LDS read addresses, the
// stage-0 load offsets and destinations, runs the loop and stores the tile.
__global__ __launch_bounds__(512) void gemm_kernel(const int8_t *__restrict__ xq, const uint16_t *__restrict__ xs,
                                                    int64_t M, const uint8_t *__restrict__ w, int64_t N, int64_t K,
                                                    float *__restrict__ y, int64_t ld_y) {
    using T = Tile<4, 2>;
    static_assert(T::STAGE_BYTES == 34816 && T::A_BYTES == 16384 && T::PER_WAVE == 5 && T::WAVES == 8,
                  "gemm_loop.inc is generated for this stage layout");
    static_assert(T::NA == 16 && T::NB == 16 && T::NSX == 4 && T::NSW == 4, "load split of gemm_loop.inc");
    __shared__ __attribute__((aligned(1024))) uint8_t lds[NS * T::STAGE_BYTES];
    const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t *)lds;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = wave_id();
    const int wm = wave % 4, wn = wave / 4;  // 32-row strip wm of packed tile wn
    const int half = lane >> 5, l32 = lane & 31;
    const int64_t tiles = N / TILE_ROWS;
    int tm, tn;  // the workgroup's output tile (row block, column block)
    xcd_tile(tm, tn);
    const int64_t T0 = (int64_t)tn * 2;  // the workgroup's first packed weight tile
    const int64_t G = K / GROUP_K, nb = K / QK;
    const int64_t m_tile = (int64_t)tm * T::ROWS;
    const bool ragged = T0 + 2 > tiles;
    // tiles past the last one (N not a multiple of 128) reload the last tile
    const uint8_t *w_tiles = w + (T0 * G) * RECORD_BYTES;
    const uint32_t tile_stride = ragged ? 0u : (uint32_t)(G * RECORD_BYTES);

    // Stage-0 loads of this wave (load i of a stage goes to wave i % 8): 1 KB
    // activation loads i = wave, wave + 8 (8 rows x 128 bytes, row r's 16-byte
    // chunk c stored at position c ^ (r & 7)), weight loads i = 16 + wave,
    // 24 + wave (a tile's 4 block records are 8 KB contiguous), and one
    // 256-byte scale load (activation scales [row][4] for waves 0-3, weight
    // scales [tile][row][4] for waves 4-7).  Offsets are from the row block's
    // first activation row / scale row and from the first weight tile;
    // activation rows past M read row M - 1 (their outputs are not stored).
    v4i gl;       // loads 2, 3 (weights), 4 (scales), unused
    uint32_t g01[2];
    uint32_t ldst[5];
#pragma unroll
    for (int u = 0; u < 2; u++) {
        const int i = wave + 8 * u;
        const int r = 8 * i + (lane >> 3), c = (lane & 7) ^ (lane >> 3);
        const int64_t row = m_tile + r < M ? r : M - 1 - m_tile;
        g01[u] = (uint32_t)(row * K + c * 16);
        ldst[u] = lds0 + i * 1024;
    }
#pragma unroll
    for (int u = 0; u < 2; u++) {
        const int e = wave + 8 * u;
        gl[u] = (int)((uint32_t)(e >> 3) * tile_stride + (e & 7) * 1024 + lane * 16);
        ldst[2 + u] = lds0 + T::A_BYTES + e * 1024;
    }
    const uint8_t *sbase;
    uint32_t sinc;  // scale base step from an odd stage to the next (even) one
    if (wave < 4) {
        const int d = wave * 64 + lane;
        const int64_t row = m_tile + (d >> 1) < M ? (d >> 1) : M - 1 - m_tile;
        gl[2] = (int)(row * nb * 2 + (d & 1) * 4);
        ldst[4] = lds0 + T::SX_OFF + wave * 256;
        sbase = reinterpret_cast<const uint8_t *>(xs + m_tile * nb);
        sinc = 8;
    } else {
        const int d = (wave - 4) * 64 + lane;
        gl[2] = (int)((uint32_t)(d >> 7) * tile_stride + RECORD_Q_BYTES + ((d >> 1) & 63) * 16 + (d & 1) * 4);
        ldst[4] = lds0 + T::SW_OFF + (wave - 4) * 256;
        sbase = w_tiles;
        sinc = RECORD_BYTES - 8;
    }
    gl[3] = 0;

    // LDS read addresses of this lane, for stage buffers 0 / 1 (immediate
    // offset 0 or one stage) and 2 / 3 (the same + two stages)
    const int row = wm * 32 + l32;
    v16i ad;
#pragma unroll
    for (int bb = 0; bb < SB; bb++) {
        ad[bb] = (int)(lds0 + row * 128 + (((2 * bb + half) ^ (row & 7)) * 16));
        ad[4 + bb] = ad[bb] + 2 * T::STAGE_BYTES;
    }
    ad[8] = (int)(lds0 + T::A_BYTES + wn * SB * 2048 + half * 1024 + l32 * 16);
    ad[9] = ad[8] + 2 * T::STAGE_BYTES;
    ad[10] = (int)(lds0 + T::SX_OFF + row * 8);
    ad[11] = ad[10] + 2 * T::STAGE_BYTES;
    ad[12] = (int)(lds0 + T::SW_OFF + (wn * 64 + half * 32 + l32) * 8);
    ad[13] = ad[12] + 2 * T::STAGE_BYTES;
    ad[14] = (int)g01[0];
    ad[15] = (int)g01[1];

    typedef uint32_t v8u __attribute__((ext_vector_type(8)));
    v8u sc = {sinc, ldst[0], ldst[1], ldst[2], ldst[3], ldst[4], (uint32_t)(2 * G), (uint32_t)G};
    uint64_t abase = (uint64_t)(xq + m_tile * K), bbase = (uint64_t)w_tiles, sb = (uint64_t)sbase;
    v32f acc, ga;
#pragma unroll
    for (int r = 0; r < 32; r++) acc[r] = ga[r] = -0.0f;  // -0 + x == x for every x
    // m0 is written by the loop (LDS destinations of the stage loads); clang
    // warns that a clobbered reserved register is not preserved, which is the intent
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
    asm volatile(Q8_GEMM_LOOP_ASM
                 : "+{v[0:31]}"(acc), "+{v[32:63]}"(ga), "+{s[40:41]}"(abase), "+{s[42:43]}"(bbase),
                   "+{s[44:45]}"(sb), "+{s[48:55]}"(sc)
                 : "{v[226:241]}"(ad), "{v[242:245]}"(gl)
                 : Q8_GEMM_LOOP_CLOBBERS, "memory", "m0", "scc", "s57");
#pragma clang diagnostic pop

    if (ragged && T0 + wn >= tiles) return;
    const int64_t n_wave = (T0 + wn) * TILE_ROWS;
    // lane holds column l32 of each 32 x 32 tile and rows 8q + 4*half + p
#pragma unroll
    for (int r = 0; r < 16; r++) {
        const int64_t orow = m_tile + wm * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
        if (orow >= M) continue;
        // written once: the non-temporal hint keeps the output from displacing
        // operand stages that other tiles still read through L2 (+1.2% over
        // the nine prefill shapes)
#pragma unroll
        for (int j = 0; j < 2; j++) __builtin_nontemporal_store(acc[16 * j + r], &y[orow * ld_y + n_wave + j * 32 + l32]);
    }
}

static hipError_t launch_tiles(const int8_t *xq, const uint16_t *xs, int64_t m, const uint8_t *w, int64_t n,
                               int64_t k, float *y, int64_t ld_y, hipStream_t s) {
    using T = Tile<4, 2>;
    const dim3 grid((unsigned)((n + T::COLS - 1) / T::COLS), (unsigned)((m + T::ROWS - 1) / T::ROWS));
    hipLaunchKernelGGL(gemm_kernel, grid, dim3(T::THREADS), 0, s, xq, xs, m, w, n, k, y, ld_y);
    return hipGetLastError();
}

// Small problems: one workgroup owns a 32 x 64 output strip (32 rows, one
// packed weight tile) and splits k across its W waves (4, or 8 when the grid
// would leave SIMDs without a wave): wave w takes groups w, w + W, ...; each
// wave forms its group's sums exactly as the tiled kernel does (same MFMAs,
// same convert / multiply / fma sequence) and parks them in LDS; after a
// barrier the workgroup's threads fold each batch of group sums into their
// outputs' running sums in group order, so every output sees the same
// sequence of fp32 operations as in the tiled kernel and rows stay
// bit-identical whichever kernel m selects.  The k loop is the generated
// inline-asm block of gemm_strip.inc (operands straight into registers, the
// wave's next group loading while it computes the current one; its header
// comment gives the register map).
template <int W>
__global__ __launch_bounds__(64 * W) void gemm_strip_kernel(const int8_t *__restrict__ xq,
                                                             const uint16_t *__restrict__ xs, int64_t M,
                                                             const uint8_t *__restrict__ w, int64_t N, int64_t K,
                                                             float *__restrict__ y, int64_t ld_y) {
    static_assert(W == 4 || W == 8, "gemm_strip.inc has the 4- and 8-wave loops");
    constexpr int PER = 32 / W;  // outputs per thread
    // park[buffer][wave][(j * 16 + r) * 64 + lane]: 2 x W x 8 KB
    __shared__ __attribute__((aligned(16))) float park[2 * W * 2048];
    const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) float *)park;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = wave_id();
    const int half = lane >> 5, l32 = lane & 31;
    const int64_t m0 = (int64_t)blockIdx.y * 32;
    const int64_t T = blockIdx.x;
    const int G = (int)(K >> 8), nb = (int)(K >> 5);
    int64_t row = m0 + l32;
    row = row < M ? row : M - 1;  // rows past M read row M - 1 (their outputs are not stored)
    const uint8_t *wt = w + T * (int64_t)G * RECORD_BYTES;

    typedef int v8i __attribute__((ext_vector_type(8)));
    v8i off;  // v222-229 of the loop: lane offsets and LDS addresses
    off[0] = (int)(row * K + half * 16);
    off[1] = (int)(row * nb * 2);
    off[2] = half * 1024 + l32 * 16;
    off[3] = RECORD_Q_BYTES + lane * 16;
    off[4] = (int)(lds0 + wave * 8192 + lane * 4);
    off[5] = (int)(lds0 + tid * 4);
    off[6] = off[4] + W * 8192;
    off[7] = off[5] + W * 8192;
    typedef uint32_t v4u __attribute__((ext_vector_type(4)));
    v4u ctl = {(uint32_t)wave, (uint32_t)G, 0u, 0u};
    v4u steps = {256u * W, (uint32_t)RECORD_BYTES * W, 16u * W, 0u};
    uint64_t abase = (uint64_t)(xq + wave * 256), wbase = (uint64_t)(wt + (int64_t)wave * RECORD_BYTES),
             xbase = (uint64_t)(reinterpret_cast<const uint8_t *>(xs) + wave * 16);
    typedef float v8f __attribute__((ext_vector_type(8)));
    v8f acc;
#pragma unroll
    for (int i = 0; i < 8; i++) acc[i] = -0.0f;  // -0 + x == x for every x
    if constexpr (W == 4) {
        asm volatile(Q8_GEMM_STRIP_ASM_W4
                     : "+{v[214:221]}"(acc), "+{s[40:41]}"(abase), "+{s[42:43]}"(wbase), "+{s[44:45]}"(xbase),
                       "+{s[48:51]}"(ctl)
                     : "{v[222:229]}"(off), "{s[52:55]}"(steps)
                     : Q8_GEMM_STRIP_CLOBBERS, "s46", "s47", "memory", "scc");
    } else {
        asm volatile(Q8_GEMM_STRIP_ASM_W8
                     : "+{v[214:221]}"(acc), "+{s[40:41]}"(abase), "+{s[42:43]}"(wbase), "+{s[44:45]}"(xbase),
                       "+{s[48:51]}"(ctl)
                     : "{v[222:229]}"(off), "{s[52:55]}"(steps)
                     : Q8_GEMM_STRIP_CLOBBERS, "s46", "s47", "memory", "scc");
    }
    // thread tid holds outputs o = tid + 64 W i, o = (j * 16 + r) * 64 + lane of the MFMA layout:
    // column j * 32 + (lane & 31), row 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3)
#pragma unroll
    for (int i = 0; i < PER; i++) {
        const int o = tid + 64 * W * i;
        const int ol = o & 63, r = (o >> 6) & 15, j = o >> 10;
        const int64_t orow = m0 + 8 * (r >> 2) + 4 * (ol >> 5) + (r & 3);
        if (orow < M) __builtin_nontemporal_store(acc[i], &y[orow * ld_y + T * TILE_ROWS + j * 32 + (ol & 31)]);
    }
}

// The 8-wave strip kernel when the 4-wave grid would have fewer waves than
// the 1024 SIMDs of the GPU (the split over more waves then costs no
// occupancy); else the 4-wave one (two workgroups per CU).
constexpr int64_t STRIP_W8_BELOW_WAVES = 1024;

// Kernel by problem size: 128 x 128 tiles when there are at least 256 of them
// (one per CU), else 32 x 64 strips with k split across the waves.  Each
// output's arithmetic is the same in both, so rows stay bit-identical across m.
static bool gemm_tiled(int64_t m, int64_t n) { return ((m + 127) / 128) * ((n + 127) / 128) >= 256; }

hipError_t launch_gemm(const void *x_q, int64_t m, const void *w, int64_t n, int64_t k, float *y, int64_t ld_y,
                       hipStream_t s) {
    const int8_t *xq = (const int8_t *)x_q;
    const uint16_t *xs = (const uint16_t *)((const uint8_t *)x_q + m * k);
    const uint8_t *wb = (const uint8_t *)w;
    if (gemm_tiled(m, n)) return launch_tiles(xq, xs, m, wb, n, k, y, ld_y, s);
    const dim3 grid((unsigned)(n / TILE_ROWS), (unsigned)((m + 31) / 32));
    if ((int64_t)grid.x * grid.y * 4 < STRIP_W8_BELOW_WAVES)
        hipLaunchKernelGGL(gemm_strip_kernel<8>, grid, dim3(512), 0, s, xq, xs, m, wb, n, k, y, ld_y);
    else
        hipLaunchKernelGGL(gemm_strip_kernel<4>, grid, dim3(256), 0, s, xq, xs, m, wb, n, k, y, ld_y);
    return hipGetLastError();
}

}  // namespace q8k
