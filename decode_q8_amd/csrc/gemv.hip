// Decode GEMV (m <= 8) and routed-expert GEMV for gfx950.
//
// Per output row the arithmetic is the Q8_0 block dot of the pages ("ferro"
// README, "How the iGPU path is fast", item 1): s = exact int32 sum of 32
// int8 products (v_dot4c_i32_i8, 8 per block), t = fp32(s * (Dw * Dx)), and
// the terms are summed in one fixed order that depends on k only: a tree over
// the 8 blocks of each 256-value group, the group sums left to right within
// each 2048-value segment, then the segment sums left to right.
//
// Work split (gfx950 first, not the pages' N100/AVX-512 designs):
//  - lane = output row: a wave owns a 64-row tile, so no cross-lane
//    reduction exists and the row's arithmetic cannot depend on how many
//    activation rows share the launch (the batch-invariance contract of the
//    "ferro" README, "Exactness contract");
//  - packed weights: every 16-byte load of a wave reads 1 KB contiguous
//    (64 rows x 16 values); a row's 8 scales arrive in one 16-byte load;
//  - activations are wave-uniform: the compiler reads them with scalar loads
//    into SGPRs, which feed v_dot4c directly (no LDS traffic);
//  - a workgroup of up to 8 waves shares a tile's groups and chains them in
//    LDS; narrow matrices with long rows spread a tile over one workgroup per
//    segment and hand the segment sums over through the workspace.  The
//    order of additions is the same for every split, so the bits are too.
#include "device.hpp"
#include "launch.hpp"

namespace q8k {

// One lane's bytes of one group of one row: chunks [2*bb + h] hold the 16
// values of block bb, half h; chunk 16 holds the 8 fp16 scales.
struct GroupRegs {
    uint4 c[17];
};

template <int LAYOUT>
__device__ __forceinline__ void load_group(GroupRegs &g, const uint8_t *p) {
    if (LAYOUT == 1) {  // packed: p = record + lane * 16
#pragma unroll
        for (int i = 0; i < 16; i++) g.c[i] = *reinterpret_cast<const uint4 *>(p + i * 1024);
        g.c[16] = *reinterpret_cast<const uint4 *>(p + RECORD_Q_BYTES);
    } else {  // rows: p = this row's 272 bytes of the group (8 blocks of 34 bytes)
#pragma unroll
        for (int i = 0; i < 17; i++) g.c[i] = *reinterpret_cast<const uint4 *>(p + i * 16);
    }
}

// Row-contiguous bytes [d0 q0..q31][d1 q0..q31]... -> the packed register form.
// Even blocks start on a dword boundary (scale in the low half); odd blocks
// start 2 bytes into a dword (scale in the high half, values dword aligned).
__device__ __forceinline__ void rows_to_packed(GroupRegs &g) {
    uint32_t w[68];
#pragma unroll
    for (int i = 0; i < 17; i++) {
        w[4 * i] = g.c[i].x; w[4 * i + 1] = g.c[i].y; w[4 * i + 2] = g.c[i].z; w[4 * i + 3] = g.c[i].w;
    }
    uint32_t q[64], sc[8];
#pragma unroll
    for (int bb = 0; bb < 8; bb++) {
        const int wi = 17 * (bb >> 1) + ((bb & 1) ? 8 : 0);
        if ((bb & 1) == 0) {
            sc[bb] = w[wi] & 0xffffu;
#pragma unroll
            for (int c = 0; c < 8; c++) q[8 * bb + c] = __builtin_amdgcn_alignbyte(w[wi + c + 1], w[wi + c], 2);
        } else {
            sc[bb] = w[wi] >> 16;
#pragma unroll
            for (int c = 0; c < 8; c++) q[8 * bb + c] = w[wi + 1 + c];
        }
    }
#pragma unroll
    for (int i = 0; i < 16; i++) g.c[i] = make_uint4(q[4 * i], q[4 * i + 1], q[4 * i + 2], q[4 * i + 3]);
    g.c[16] = make_uint4(sc[0] | (sc[1] << 16), sc[2] | (sc[3] << 16), sc[4] | (sc[5] << 16), sc[6] | (sc[7] << 16));
}

__device__ __forceinline__ uint32_t half_of(const uint4 &v, int bb) {
    return (word_of(v, bb >> 1) >> (16 * (bb & 1))) & 0xffffu;
}

typedef __attribute__((address_space(4))) int const_i32;

// Group sums u[m] for M activation rows.  xg[m] / sg[m] point at the group's
// 256 int8 values / 8 fp16 scales of row m (wave-uniform).
template <int M>
__device__ __forceinline__ void group_sums(const GroupRegs &g, const int8_t *const (&xg)[M],
                                           const uint16_t *const (&sg)[M], float (&u)[M]) {
    float dw[8];
#pragma unroll
    for (int bb = 0; bb < 8; bb++) dw[bb] = half_bits_to_float(half_of(g.c[16], bb));
#pragma unroll
    for (int m = 0; m < M; m++) {
        // Activations are read-only and wave-uniform: constant-address-space
        // loads become scalar loads into SGPRs, which v_dot4c reads directly.
        const const_i32 *xi = (const const_i32 *)(xg[m]);
        const const_i32 *xsp = (const const_i32 *)(sg[m]);
        const uint4 xsv = make_uint4((uint32_t)xsp[0], (uint32_t)xsp[1], (uint32_t)xsp[2], (uint32_t)xsp[3]);
        float t[8];
#pragma unroll
        for (int bb = 0; bb < 8; bb++) {
            int s = 0;
#pragma unroll
            for (int h = 0; h < 2; h++)
#pragma unroll
                for (int c = 0; c < 4; c++)
                    s = __builtin_amdgcn_sdot4((int)word_of(g.c[2 * bb + h], c), xi[8 * bb + 4 * h + c], s, false);
            const float dx = half_bits_to_float(half_of(xsv, bb));
            t[bb] = (float)s * (dw[bb] * dx);  // Dw * Dx exact: one rounding
        }
        u[m] = tree8(t);
    }
}

// Group sums with the activation quantization fused in: xv[m] holds lane l's
// values 4l..4l+3 of the group's 256 fp32 values of row m (loaded by the
// caller ahead of the weights, so the quantization does not wait for them).
// Lane l quantizes values 4l..4l+3 (block
// l / 8) with exactly the arithmetic of the standalone quantizer (amax over
// the block by an exact max butterfly, d = amax / 127, q = round-half-away of
// x / d, stored scale fp16(d)), so the codes and scales are bit-identical to
// q8_quantize_rows.  The packed codes and scales are then broadcast from their
// lane to the whole wave (v_readlane) as v_dot4c's scalar operand.
template <int M>
__device__ __forceinline__ void group_sums_f32(const GroupRegs &g, const float4 (&xv)[M], float (&u)[M]) {
    float dw[8];
#pragma unroll
    for (int bb = 0; bb < 8; bb++) dw[bb] = half_bits_to_float(half_of(g.c[16], bb));
#pragma unroll
    for (int m = 0; m < M; m++) {
        const float4 v = xv[m];
        float amax = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
        amax = fmaxf(amax, __shfl_xor(amax, 1));
        amax = fmaxf(amax, __shfl_xor(amax, 2));
        amax = fmaxf(amax, __shfl_xor(amax, 4));
        const float d = amax / 127.0f;
        int q0 = 0, q1 = 0, q2 = 0, q3 = 0;
        if (d != 0.0f) {
            q0 = (int)roundf(v.x / d);
            q1 = (int)roundf(v.y / d);
            q2 = (int)roundf(v.z / d);
            q3 = (int)roundf(v.w / d);
        }
        const int qd = (int)(((uint32_t)q0 & 0xffu) | (((uint32_t)q1 & 0xffu) << 8) | (((uint32_t)q2 & 0xffu) << 16) |
                             ((uint32_t)q3 << 24));
        const float dxl = half_bits_to_float(float_to_half_bits(d));
        float t[8];
#pragma unroll
        for (int bb = 0; bb < 8; bb++) {
            int s = 0;
#pragma unroll
            for (int h = 0; h < 2; h++)
#pragma unroll
                for (int c = 0; c < 4; c++)
                    s = __builtin_amdgcn_sdot4((int)word_of(g.c[2 * bb + h], c),
                                               __builtin_amdgcn_readlane(qd, 8 * bb + 4 * h + c), s, false);
            const float dx = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, dxl), 8 * bb));
            t[bb] = (float)s * (dw[bb] * dx);
        }
        u[m] = tree8(t);
    }
}

// Walk groups g0, g0 + step, ... (< g1) of one lane's row.  TO_LDS = true:
// store each group sum u_g at lds[((g - g0) * M + m) * 64 + lane] (the caller
// points lds at group g0's slot; slots of M x 64 floats hold consecutive
// groups); the workgroup chains them later.  TO_LDS = false (step 1, g0 = 0): the wave owns
// groups [0, G) of its row and chains in registers in the canonical two-level
// order.  wbase/gstride: address of group 0 of this lane and the step between
// groups in memory.
template <int M, int LAYOUT, bool TO_LDS, typename ACT, bool ONE = false>
__device__ __forceinline__ void row_groups(const uint8_t *wbase, int64_t gstride, int g0, int g1, int step,
                                           const ACT *const (&xrow)[M], const uint16_t *const (&srow)[M],
                                           float (&acc)[M], float *lds, int lane) {
    if (g0 >= g1) return;
    // ONE: the caller guarantees at most one group (g0 + step >= g1), so no
    // second register buffer is allocated (17 VGPRs x 4 fewer per lane, more
    // waves per SIMD to keep loads in flight).
    GroupRegs cur;
    GroupRegs nxt;
    float seg[M];
    // fp32 activations: each group's x values are loaded before its weights
    // (loads complete in order, so the quantization can start early)
    constexpr bool F32 = sizeof(ACT) == 4;
    float4 xv[M], xn[M];
    if constexpr (F32) {
#pragma unroll
        for (int m = 0; m < M; m++) xv[m] = *reinterpret_cast<const float4 *>(xrow[m] + g0 * GROUP_K + 4 * lane);
    }
    load_group<LAYOUT>(cur, wbase + g0 * gstride);
    for (int g = g0; g < g1; g += step) {
        if (!ONE && g + step < g1) {
            if constexpr (F32) {
#pragma unroll
                for (int m = 0; m < M; m++)
                    xn[m] = *reinterpret_cast<const float4 *>(xrow[m] + (g + step) * GROUP_K + 4 * lane);
            }
            load_group<LAYOUT>(nxt, wbase + (g + step) * gstride);
        }
        if (LAYOUT == 0) rows_to_packed(cur);
        float u[M];
        if constexpr (!F32) {
            const ACT *xg[M];
            const uint16_t *sg[M];
#pragma unroll
            for (int m = 0; m < M; m++) {
                xg[m] = xrow[m] + g * GROUP_K;
                sg[m] = srow[m] + g * GROUP_BLOCKS;
            }
            group_sums<M>(cur, xg, sg, u);
        } else {
            group_sums_f32<M>(cur, xv, u);
        }
        if (TO_LDS) {
#pragma unroll
            for (int m = 0; m < M; m++) lds[((g - g0) * M + m) * TILE_ROWS + lane] = u[m];
        } else {
            const bool seg_first = (g % SEG_GROUPS) == 0;
            const bool seg_last = (g % SEG_GROUPS) == SEG_GROUPS - 1 || g == g1 - 1;
#pragma unroll
            for (int m = 0; m < M; m++) {
                seg[m] = seg_first ? u[m] : seg[m] + u[m];
                if (seg_last) acc[m] = (g < SEG_GROUPS) ? seg[m] : acc[m] + seg[m];
            }
        }
        if (ONE) break;
        cur = nxt;
        if constexpr (F32) {
#pragma unroll
            for (int m = 0; m < M; m++) xv[m] = xn[m];
        }
    }
}

// The GEMV.  A tile's groups are split into segments of 8 (2048 values); a
// workgroup covers segs_per_wg consecutive segments of one tile, its W waves
// take those groups round-robin (wave w: groups w, w + W, ...) and leave every
// group sum in LDS.  After a barrier each (row, m) is chained in the canonical order:
//   S_j = ((u_8j + u_8j+1) + ...) + u_8j+7   within segment j,
//   y   = ((S_0 + S_1) + S_2) + ...          over the segments.
// When one workgroup covers the whole tile it writes y.  Otherwise (narrow
// matrices with long rows, where one workgroup per tile would leave most CUs
// idle) each workgroup hands its segment sums to the workspace and counts in
// at its tile's counter; the workgroup that arrives last chains all segment
// sums and writes y, then clears the counter (so counters that start at zero
// stay zero).  Cross-workgroup visibility without cache-wide fences: segment
// sums are written and read back with read-modify-write atomics (exchange in;
// exchange with 0 out -- an idempotent RMW would be lowered to a plain atomic
// load, which can hit a stale line of a non-coherent L2), performed at the
// device-coherent point like the counter; every thread waits for its
// exchanges before the barrier that precedes the counter increment, and the
// last workgroup reads only after that increment returned the final count.
// Workspace: uint32 counters [tiles] (256-byte aligned), then fp32 segment sums
// [S][M][n].
template <int M, int LAYOUT, typename ACT, bool ONE>
__global__ __launch_bounds__(512) void gemv_kernel(const ACT *__restrict__ xq, int64_t ld_x,
                                                   const uint16_t *__restrict__ xs, const uint8_t *__restrict__ w,
                                                   int64_t n, int64_t k, float *__restrict__ y, int64_t ld_y,
                                                   int segs_per_wg, uint32_t *__restrict__ ctr,
                                                   float *__restrict__ part) {
    extern __shared__ float lds_u[];  // [groups of this workgroup][M][64]
    __shared__ int last_wg;
    // Grid: x = workgroup within the tile, y = tile.  Everything below is
    // 32-bit and division-free, so the first weight load issues after a few
    // scalar instructions (64-bit divisions here cost hundreds).
    const int lane = threadIdx.x & 63;
    const int wv = wave_id();
    const int W = blockDim.x >> 6;
    const int wgs_per_tile = gridDim.x;
    const int wi = blockIdx.x;
    const int64_t T = blockIdx.y;
    const int G = (int)(k >> 8);                        // k is a multiple of 256
    const int S = (G + SEG_GROUPS - 1) / SEG_GROUPS;    // constant divisor: a shift
    const int s0 = wi * segs_per_wg, s1 = min(s0 + segs_per_wg, S);
    const int ga = s0 * SEG_GROUPS, gb = min(s1 * SEG_GROUPS, G);
    const int64_t row = T * TILE_ROWS + lane;
    const int64_t row_c = row < n ? row : n - 1;

    const ACT *xrow[M];
    const uint16_t *srow[M];
#pragma unroll
    for (int m = 0; m < M; m++) {
        xrow[m] = xq + m * ld_x;
        srow[m] = xs + m * (k / QK);
    }
    const uint8_t *wbase = LAYOUT == 1 ? w + T * G * RECORD_BYTES + lane * 16 : w + row_c * (k / QK) * BLOCK_BYTES;
    const int64_t gstride = LAYOUT == 1 ? RECORD_BYTES : ROW_GROUP_BYTES;
    float unused[M];
    // wave wv takes the workgroup's groups ga + wv, ga + wv + W, ...; each sum lands in its group's LDS slot
    row_groups<M, LAYOUT, true, ACT, ONE>(wbase, gstride, ga + wv, gb, W, xrow, srow, unused,
                                          lds_u + wv * M * TILE_ROWS, lane);
    __syncthreads();

    const int t = threadIdx.x;  // the plan gives at least M waves: one thread per (m, row)
    const bool chain_thread = t < M * TILE_ROWS;
    const int cm = t >> 6, cr = t & 63;
    const int64_t out_row = T * TILE_ROWS + cr;
    const bool out_ok = chain_thread && out_row < n;
    float acc = 0.0f;
    if (chain_thread) {
        for (int64_t sj = s0; sj < s1; sj++) {
            const int64_t gs = sj * SEG_GROUPS, ge = (gs + SEG_GROUPS) < G ? (gs + SEG_GROUPS) : G;
            float sv = lds_u[((gs - ga) * M + cm) * TILE_ROWS + cr];
            for (int64_t g = gs + 1; g < ge; g++) sv += lds_u[((g - ga) * M + cm) * TILE_ROWS + cr];
            if (wgs_per_tile == 1) {
                acc = sj == 0 ? sv : acc + sv;
            } else if (out_ok) {
                __hip_atomic_exchange((uint32_t *)&part[(sj * M + cm) * n + out_row], __builtin_bit_cast(uint32_t, sv),
                                      __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
    }
    if (wgs_per_tile == 1) {
        if (out_ok) y[cm * ld_y + out_row] = acc;
        return;
    }
    __builtin_amdgcn_s_waitcnt(0);  // this thread's exchanges have completed
    __syncthreads();
    if (t == 0) {
        const uint32_t old = __hip_atomic_fetch_add(&ctr[T], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        last_wg = old == (uint32_t)(wgs_per_tile - 1);
    }
    __syncthreads();
    if (!last_wg) return;
    if (out_ok) {
        for (int64_t b0 = 0; b0 < S; b0 += 8) {
            float v[8];  // eight exchanges in flight, then the in-order chain
#pragma unroll
            for (int j = 0; j < 8; j++)
                v[j] = b0 + j < S ? __builtin_bit_cast(float, __hip_atomic_exchange(
                                                                  (uint32_t *)&part[((b0 + j) * M + cm) * n + out_row],
                                                                  0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
                                  : 0.0f;
#pragma unroll
            for (int j = 0; j < 8; j++)
                if (b0 + j < S) acc = (b0 + j == 0) ? v[j] : acc + v[j];
        }
        y[cm * ld_y + out_row] = acc;
    }
    if (t == 0) __hip_atomic_exchange(&ctr[T], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

constexpr int GEMV_MAX_WAVES = 8;
constexpr int64_t GEMV_LDS_LIMIT = 64 * 1024;

// Execution plan of a GEMV.  Only speed depends on it; every plan produces
// the same bits.  Up to 8 waves per workgroup (one or more groups each);
// tiles of narrow matrices are spread over one workgroup per segment so that
// at least ~256 workgroups run; the group sums a workgroup keeps in LDS must
// fit in 64 KB.
GemvPlan gemv_plan(int64_t m, int64_t n, int64_t k) {
    GemvPlan p;
    p.tiles = (n + TILE_ROWS - 1) / TILE_ROWS;
    p.groups = k / GROUP_K;
    const int64_t S = (p.groups + SEG_GROUPS - 1) / SEG_GROUPS;
    int64_t wgs = 1;
    if (p.tiles < 256) wgs = (256 + p.tiles - 1) / p.tiles;
    if (wgs > S) wgs = S;
    for (;;) {  // LDS bound: groups per workgroup x m x 64 rows x 4 bytes
        const int64_t sp = (S + wgs - 1) / wgs;
        const int64_t gpw = sp * SEG_GROUPS < p.groups ? sp * SEG_GROUPS : p.groups;
        if (gpw * m * TILE_ROWS * (int64_t)sizeof(float) <= GEMV_LDS_LIMIT || wgs >= S) break;
        wgs++;
    }
    const int64_t sp = (S + wgs - 1) / wgs;
    wgs = (S + sp - 1) / sp;  // no workgroup without a segment
    const int64_t gpw = sp * SEG_GROUPS < p.groups ? sp * SEG_GROUPS : p.groups;
    p.wgs_per_tile = (int)wgs;
    p.segs_per_wg = (int)sp;
    // one chain thread per (row, activation row) after the barrier: at least m waves
    int64_t waves = gpw < GEMV_MAX_WAVES ? gpw : GEMV_MAX_WAVES;
    if (waves < m) waves = m;
    p.waves = (int)waves;
    p.lds = (size_t)(gpw * m * TILE_ROWS) * sizeof(float);
    p.workspace = 0;
    if (wgs > 1) p.workspace = (size_t)((p.tiles * 4 + 255) / 256 * 256) + (size_t)(S * m * n) * sizeof(float);
    return p;
}

size_t gemv_workspace_bytes(int64_t m, int64_t n, int64_t k) { return gemv_plan(m, n, k).workspace; }

template <int LAYOUT, typename ACT>
static void launch_gemv_m(int64_t m, const GemvPlan &p, hipStream_t s, const ACT *x, int64_t ld_x,
                          const uint16_t *xs, const uint8_t *w, int64_t n, int64_t k, float *y, int64_t ld_y,
                          void *ws) {
    uint32_t *ctr = (uint32_t *)ws;
    float *part = ws ? (float *)((uint8_t *)ws + (p.tiles * 4 + 255) / 256 * 256) : nullptr;
    const dim3 grid((unsigned)p.wgs_per_tile, (unsigned)p.tiles), block((unsigned)(64 * p.waves));
    // one group per wave whenever the workgroup's groups do not exceed its waves
    const int64_t gpw = (int64_t)p.segs_per_wg * SEG_GROUPS < p.groups ? (int64_t)p.segs_per_wg * SEG_GROUPS : p.groups;
    const bool one = gpw <= p.waves;
#define Q8_GEMV_CASE(MM)                                                                                          \
    case MM:                                                                                                      \
        if (one)                                                                                                  \
            hipLaunchKernelGGL((gemv_kernel<MM, LAYOUT, ACT, true>), grid, block, p.lds, s, x, ld_x, xs, w, n, k, \
                               y, ld_y, p.segs_per_wg, ctr, part);                                                \
        else                                                                                                      \
            hipLaunchKernelGGL((gemv_kernel<MM, LAYOUT, ACT, false>), grid, block, p.lds, s, x, ld_x, xs, w, n,   \
                               k, y, ld_y, p.segs_per_wg, ctr, part);                                             \
        break;
    switch (m) {
        Q8_GEMV_CASE(1) Q8_GEMV_CASE(2) Q8_GEMV_CASE(3) Q8_GEMV_CASE(4)
        Q8_GEMV_CASE(5) Q8_GEMV_CASE(6) Q8_GEMV_CASE(7) Q8_GEMV_CASE(8)
        default: break;
    }
#undef Q8_GEMV_CASE
}

template <typename ACT>
static hipError_t launch_gemv_any(const ACT *x, int64_t ld_x, const uint16_t *xs, int64_t m, const void *w,
                                  int layout, int64_t n, int64_t k, float *y, int64_t ld_y, void *ws, hipStream_t s) {
    const GemvPlan p = gemv_plan(m, n, k);
    if (layout == 1)
        launch_gemv_m<1, ACT>(m, p, s, x, ld_x, xs, (const uint8_t *)w, n, k, y, ld_y, ws);
    else
        launch_gemv_m<0, ACT>(m, p, s, x, ld_x, xs, (const uint8_t *)w, n, k, y, ld_y, ws);
    return hipGetLastError();
}

hipError_t launch_gemv(const void *x_q, int64_t m, const void *w, int layout, int64_t n, int64_t k, float *y,
                       int64_t ld_y, void *workspace, hipStream_t s) {
    const int8_t *xq = (const int8_t *)x_q;
    const uint16_t *xs = (const uint16_t *)((const uint8_t *)x_q + m * k);
    return launch_gemv_any<int8_t>(xq, k, xs, m, w, layout, n, k, y, ld_y, workspace, s);
}

hipError_t launch_gemv_f32(const float *x, int64_t ld_x, int64_t m, const void *w, int layout, int64_t n, int64_t k,
                           float *y, int64_t ld_y, void *workspace, hipStream_t s) {
    return launch_gemv_any<float>(x, ld_x, nullptr, m, w, layout, n, k, y, ld_y, workspace, s);
}

// ---------------------------------------------------------------------------
// Routed experts.
//
// Workspace (int32 words): [0] status, [1] number of active experts,
// [16, 16+E) active expert ids (ascending), [16+E, 16+2E+1) offsets of each
// active expert's pairs, then the pair list (pairs of one expert in
// increasing pair index p = t * topk + j).
// ---------------------------------------------------------------------------

constexpr int GROUP_THREADS = 1024;
constexpr int ID_CHUNK = 4096;

__device__ __forceinline__ int block_exclusive_scan(int v, int *sh) {
    // Hillis-Steele inclusive scan over GROUP_THREADS values, then shift.
    const int tid = threadIdx.x;
    sh[tid] = v;
    __syncthreads();
    for (int off = 1; off < GROUP_THREADS; off <<= 1) {
        const int add = tid >= off ? sh[tid - off] : 0;
        __syncthreads();
        sh[tid] += add;
        __syncthreads();
    }
    const int incl = sh[tid];
    __syncthreads();
    return incl - v;
}

__global__ __launch_bounds__(GROUP_THREADS) void group_pairs_kernel(const int32_t *__restrict__ ids, int64_t pairs,
                                                                   int64_t n_experts, int32_t *__restrict__ ws) {
    __shared__ int32_t chunk[ID_CHUNK];
    __shared__ int scan_sh[GROUP_THREADS];
    __shared__ int bad_sh;
    const int tid = threadIdx.x;
    const int E = (int)n_experts;
    int32_t *active = ws + 16;
    int32_t *offs = active + E;
    int32_t *list = offs + E + 1;
    if (tid == 0) bad_sh = 0;
    int cnt = 0;
    bool bad = false;
    for (int64_t base = 0; base < pairs; base += ID_CHUNK) {
        const int len = (int)((pairs - base) < ID_CHUNK ? (pairs - base) : ID_CHUNK);
        __syncthreads();
        for (int i = tid; i < len; i += GROUP_THREADS) {
            const int32_t v = ids[base + i];
            chunk[i] = v;
            bad |= (v < 0 || v >= E);
        }
        __syncthreads();
        if (tid < E)
            for (int j = 0; j < len; j++) cnt += (chunk[j] == tid);
    }
    if (bad) atomicOr(&bad_sh, 1);
    const int is_active = (tid < E && cnt > 0) ? 1 : 0;
    const int slot = block_exclusive_scan(is_active, scan_sh);
    const int off = block_exclusive_scan(is_active ? cnt : 0, scan_sh);
    if (is_active) {
        active[slot] = tid;
        offs[slot] = off;
    }
    if (tid == GROUP_THREADS - 1) {
        const int n_active = slot + is_active;
        ws[1] = n_active;
        offs[n_active] = off + (is_active ? cnt : 0);
    }
    __syncthreads();
    if (tid == 0) ws[0] = bad_sh ? 1 : 0;
    // scatter each active expert's pairs in increasing p
    int pos = off;
    for (int64_t base = 0; base < pairs; base += ID_CHUNK) {
        const int len = (int)((pairs - base) < ID_CHUNK ? (pairs - base) : ID_CHUNK);
        __syncthreads();
        for (int i = tid; i < len; i += GROUP_THREADS) chunk[i] = ids[base + i];
        __syncthreads();
        if (is_active)
            for (int j = 0; j < len; j++)
                if (chunk[j] == tid) list[pos++] = (int32_t)(base + j);
    }
}

template <int M>
__device__ __forceinline__ void expert_pass(const int8_t *xq, const uint16_t *xs, int64_t k, int x_per_pair, int topk,
                                            const int32_t *plist, const uint8_t *wbase, int64_t G, int64_t row,
                                            int64_t n, float *y) {
    const int8_t *xrow[M];
    const uint16_t *srow[M];
    int32_t p[M];
#pragma unroll
    for (int i = 0; i < M; i++) {
        p[i] = plist[i];  // < 65536 pairs: 32-bit division
        const int64_t xr = x_per_pair ? (int64_t)p[i] : (int64_t)((uint32_t)p[i] / (uint32_t)topk);
        xrow[i] = xq + xr * k;
        srow[i] = xs + xr * (k / QK);
    }
    float acc[M];
    row_groups<M, 1, false>(wbase, RECORD_BYTES, 0, (int)G, 1, xrow, srow, acc, nullptr, 0);
#pragma unroll
    for (int i = 0; i < M; i++) y[(int64_t)p[i] * n + row] = acc[i];
}

__global__ __launch_bounds__(256) void grouped_gemv_kernel(const int8_t *__restrict__ xq,
                                                           const uint16_t *__restrict__ xs, int64_t k, int x_per_pair,
                                                           int topk, const uint8_t *__restrict__ w,
                                                           int64_t expert_stride, int64_t n, int64_t n_experts,
                                                           float *__restrict__ y, const int32_t *__restrict__ ws) {
    // Grid: x = 4 consecutive tiles (one per wave), y = active-expert slot.
    const int lane = threadIdx.x & 63;
    const int64_t tiles = n / TILE_ROWS;
    const int64_t T = (int64_t)blockIdx.x * 4 + wave_id();
    const int64_t slot = blockIdx.y;
    const int n_active = ws[1];
    if (slot >= n_active || T >= tiles) return;
    const int32_t *active = ws + 16;
    const int32_t *offs = active + n_experts;
    const int32_t *list = offs + n_experts + 1;
    const int64_t e = active[slot];
    const int beg = offs[slot], cnt = offs[slot + 1] - beg;
    const int64_t G = k >> 8;  // k is a multiple of 256
    const uint8_t *wbase = w + e * expert_stride + T * G * RECORD_BYTES + lane * 16;
    const int64_t row = T * TILE_ROWS + lane;
    for (int start = 0; start < cnt; start += 8) {
        const int mp = (cnt - start) < 8 ? (cnt - start) : 8;
        const int32_t *pl = list + beg + start;
        switch (mp) {
            case 1: expert_pass<1>(xq, xs, k, x_per_pair, topk, pl, wbase, G, row, n, y); break;
            case 2: expert_pass<2>(xq, xs, k, x_per_pair, topk, pl, wbase, G, row, n, y); break;
            case 3: expert_pass<3>(xq, xs, k, x_per_pair, topk, pl, wbase, G, row, n, y); break;
            case 4: expert_pass<4>(xq, xs, k, x_per_pair, topk, pl, wbase, G, row, n, y); break;
            case 5: expert_pass<5>(xq, xs, k, x_per_pair, topk, pl, wbase, G, row, n, y); break;
            case 6: expert_pass<6>(xq, xs, k, x_per_pair, topk, pl, wbase, G, row, n, y); break;
            case 7: expert_pass<7>(xq, xs, k, x_per_pair, topk, pl, wbase, G, row, n, y); break;
            default: expert_pass<8>(xq, xs, k, x_per_pair, topk, pl, wbase, G, row, n, y); break;
        }
    }
}

size_t grouped_workspace_bytes(int64_t tokens, int topk, int64_t n_experts) {
    return (size_t)(16 + 2 * n_experts + 1 + tokens * topk) * sizeof(int32_t);
}

hipError_t launch_grouped(const void *x_q, int64_t x_rows, int x_per_pair, const int32_t *ids, int64_t tokens,
                          int topk, const void *w, int64_t n_experts, int64_t expert_stride, int64_t n, int64_t k,
                          float *y, void *workspace, hipStream_t s) {
    const int64_t pairs = tokens * topk;
    int32_t *ws = (int32_t *)workspace;
    hipLaunchKernelGGL(group_pairs_kernel, dim3(1), dim3(GROUP_THREADS), 0, s, ids, pairs, n_experts, ws);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t max_slots = n_experts < pairs ? n_experts : pairs;
    const int64_t tiles = n / TILE_ROWS;
    const int8_t *xq = (const int8_t *)x_q;
    const uint16_t *xs = (const uint16_t *)((const uint8_t *)x_q + x_rows * k);
    hipLaunchKernelGGL(grouped_gemv_kernel, dim3((unsigned)((tiles + 3) / 4), (unsigned)max_slots), dim3(256), 0, s,
                       xq, xs, k, x_per_pair, topk, (const uint8_t *)w, expert_stride, n, n_experts, y,
                       (const int32_t *)ws);
    return hipGetLastError();
}

}  // namespace q8k
