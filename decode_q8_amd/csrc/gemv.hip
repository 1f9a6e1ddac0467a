// Decode GEMV (m <= 8) and routed-expert GEMV for gfx950.
//
// Per output row the arithmetic is the Q8_0 block dot of the pages ("ferro"
// README, "How the iGPU path is fast", item 1): s = exact int32 sum of 32
// int8 products (v_dot4c_i32_i8, 8 per block), t = fp32(s * (Dw * Dx)), and
// the terms are summed in one fixed order that depends on k only: a tree over
// the 8 blocks of each 256-value group, then the group sums left to right.
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
//  - narrow matrices (fewer than 1024 row tiles) run one group per wave and a
//    second pass chains the group sums in order, which yields the same bits
//    as one wave walking all groups.
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

// Walk groups [g0, g1) of one lane's row and chain the group sums.
// wbase/gstride: address of group 0 of this lane and the step between groups.
template <int M, int LAYOUT>
__device__ __forceinline__ void row_chain(const uint8_t *wbase, int64_t gstride, int64_t g0, int64_t g1,
                                          const int8_t *const (&xrow)[M], const uint16_t *const (&srow)[M],
                                          float (&acc)[M]) {
    GroupRegs cur, nxt;
    load_group<LAYOUT>(cur, wbase + g0 * gstride);
    for (int64_t g = g0; g < g1; g++) {
        if (g + 1 < g1) load_group<LAYOUT>(nxt, wbase + (g + 1) * gstride);
        if (LAYOUT == 0) rows_to_packed(cur);
        const int8_t *xg[M];
        const uint16_t *sg[M];
#pragma unroll
        for (int m = 0; m < M; m++) {
            xg[m] = xrow[m] + g * GROUP_K;
            sg[m] = srow[m] + g * GROUP_BLOCKS;
        }
        float u[M];
        group_sums<M>(cur, xg, sg, u);
#pragma unroll
        for (int m = 0; m < M; m++) acc[m] = (g == g0) ? u[m] : acc[m] + u[m];
        cur = nxt;
    }
}

template <int M, int LAYOUT>
__global__ __launch_bounds__(256) void gemv_kernel(const int8_t *__restrict__ xq, const uint16_t *__restrict__ xs,
                                                   const uint8_t *__restrict__ w, int64_t n, int64_t k,
                                                   float *__restrict__ y, int64_t ld_y, float *__restrict__ part,
                                                   int split) {
    const int lane = threadIdx.x & 63;
    const int64_t unit = (int64_t)blockIdx.x * 4 + wave_id();
    const int64_t G = k / GROUP_K;
    const int64_t tiles = (n + TILE_ROWS - 1) / TILE_ROWS;
    int64_t T, g0, g1;
    if (split) {
        if (unit >= tiles * G) return;
        T = unit / G;
        g0 = unit - T * G;
        g1 = g0 + 1;
    } else {
        if (unit >= tiles) return;
        T = unit;
        g0 = 0;
        g1 = G;
    }
    const int64_t row = T * TILE_ROWS + lane;
    const bool row_ok = row < n;
    const int64_t row_c = row_ok ? row : n - 1;

    const int8_t *xrow[M];
    const uint16_t *srow[M];
#pragma unroll
    for (int m = 0; m < M; m++) {
        xrow[m] = xq + m * k;
        srow[m] = xs + m * (k / QK);
    }
    const uint8_t *wbase;
    int64_t gstride;
    if (LAYOUT == 1) {
        wbase = w + T * G * RECORD_BYTES + lane * 16;
        gstride = RECORD_BYTES;
    } else {
        wbase = w + row_c * (k / QK) * BLOCK_BYTES;
        gstride = ROW_GROUP_BYTES;
    }
    float acc[M];
    row_chain<M, LAYOUT>(wbase, gstride, g0, g1, xrow, srow, acc);
    if (!row_ok) return;
    if (split) {
#pragma unroll
        for (int m = 0; m < M; m++) part[(g0 * M + m) * n + row] = acc[m];
    } else {
#pragma unroll
        for (int m = 0; m < M; m++) y[m * ld_y + row] = acc[m];
    }
}

// Second pass of a split GEMV: y = ((u_0 + u_1) + u_2) + ... per output.
__global__ __launch_bounds__(256) void chain_kernel(const float *__restrict__ part, int64_t m, int64_t n, int64_t G,
                                                    float *__restrict__ y, int64_t ld_y) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= m * n) return;
    const int64_t mi = idx / n, ni = idx - mi * n;
    float acc = part[mi * n + ni];
    for (int64_t g = 1; g < G; g++) acc += part[(g * m + mi) * n + ni];
    y[mi * ld_y + ni] = acc;
}

GemvPlan gemv_plan(int64_t n, int64_t k) {
    GemvPlan p;
    p.tiles = (n + TILE_ROWS - 1) / TILE_ROWS;
    p.groups = k / GROUP_K;
    p.split = p.tiles < 1024 && p.groups > 1;
    return p;
}

size_t gemv_workspace_bytes(int64_t m, int64_t n, int64_t k) {
    const GemvPlan p = gemv_plan(n, k);
    if (!p.split) return 0;
    return (size_t)(p.groups * m * n) * sizeof(float);
}

template <int LAYOUT>
static void launch_gemv_m(int64_t m, dim3 grid, hipStream_t s, const int8_t *xq, const uint16_t *xs,
                          const uint8_t *w, int64_t n, int64_t k, float *y, int64_t ld_y, float *part, int split) {
#define Q8_GEMV_CASE(MM)                                                                                      \
    case MM:                                                                                                  \
        hipLaunchKernelGGL((gemv_kernel<MM, LAYOUT>), grid, dim3(256), 0, s, xq, xs, w, n, k, y, ld_y, part, \
                           split);                                                                            \
        break;
    switch (m) {
        Q8_GEMV_CASE(1) Q8_GEMV_CASE(2) Q8_GEMV_CASE(3) Q8_GEMV_CASE(4)
        Q8_GEMV_CASE(5) Q8_GEMV_CASE(6) Q8_GEMV_CASE(7) Q8_GEMV_CASE(8)
        default: break;
    }
#undef Q8_GEMV_CASE
}

hipError_t launch_gemv(const void *x_q, int64_t m, const void *w, int layout, int64_t n, int64_t k, float *y,
                       int64_t ld_y, void *workspace, hipStream_t s) {
    const GemvPlan p = gemv_plan(n, k);
    const int8_t *xq = (const int8_t *)x_q;
    const uint16_t *xs = (const uint16_t *)((const uint8_t *)x_q + m * k);
    const int64_t units = p.split ? p.tiles * p.groups : p.tiles;
    const dim3 grid((unsigned)((units + 3) / 4));
    float *part = (float *)workspace;
    if (layout == 1)
        launch_gemv_m<1>(m, grid, s, xq, xs, (const uint8_t *)w, n, k, y, ld_y, part, p.split ? 1 : 0);
    else
        launch_gemv_m<0>(m, grid, s, xq, xs, (const uint8_t *)w, n, k, y, ld_y, part, p.split ? 1 : 0);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !p.split) return e;
    const int64_t outs = m * n;
    hipLaunchKernelGGL(chain_kernel, dim3((unsigned)((outs + 255) / 256)), dim3(256), 0, s, part, m, n, p.groups,
                       y, ld_y);
    return hipGetLastError();
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
        p[i] = plist[i];
        const int64_t xr = x_per_pair ? (int64_t)p[i] : (int64_t)p[i] / topk;
        xrow[i] = xq + xr * k;
        srow[i] = xs + xr * (k / QK);
    }
    float acc[M];
    row_chain<M, 1>(wbase, RECORD_BYTES, 0, G, xrow, srow, acc);
#pragma unroll
    for (int i = 0; i < M; i++) y[(int64_t)p[i] * n + row] = acc[i];
}

__global__ __launch_bounds__(256) void grouped_gemv_kernel(const int8_t *__restrict__ xq,
                                                           const uint16_t *__restrict__ xs, int64_t k, int x_per_pair,
                                                           int topk, const uint8_t *__restrict__ w,
                                                           int64_t expert_stride, int64_t n, int64_t n_experts,
                                                           float *__restrict__ y, const int32_t *__restrict__ ws) {
    const int lane = threadIdx.x & 63;
    const int64_t unit = (int64_t)blockIdx.x * 4 + wave_id();
    const int64_t tiles = n / TILE_ROWS;
    const int64_t slot = unit / tiles, T = unit - slot * tiles;
    const int n_active = ws[1];
    if (slot >= n_active) return;
    const int32_t *active = ws + 16;
    const int32_t *offs = active + n_experts;
    const int32_t *list = offs + n_experts + 1;
    const int64_t e = active[slot];
    const int beg = offs[slot], cnt = offs[slot + 1] - beg;
    const int64_t G = k / GROUP_K;
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
    const int64_t units = max_slots * (n / TILE_ROWS);
    const int8_t *xq = (const int8_t *)x_q;
    const uint16_t *xs = (const uint16_t *)((const uint8_t *)x_q + x_rows * k);
    hipLaunchKernelGGL(grouped_gemv_kernel, dim3((unsigned)((units + 3) / 4)), dim3(256), 0, s, xq, xs, k, x_per_pair,
                       topk, (const uint8_t *)w, expert_stride, n, n_experts, y, (const int32_t *)ws);
    return hipGetLastError();
}

}  // namespace q8k
