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
#include "gemv_core.hpp"
#include "launch.hpp"

namespace q8k {

// The per-matrix GEMV kernel: grid x = workgroup within the tile, y = tile.
// Everything in the index math is 32-bit and division-free, so the first
// weight load issues after a few scalar instructions (64-bit divisions here
// cost hundreds).
template <int M, int LAYOUT, typename ACT, bool ONE>
__global__ __launch_bounds__(512) void gemv_kernel(const ACT *__restrict__ xq, int64_t ld_x,
                                                   const uint16_t *__restrict__ xs, const uint8_t *__restrict__ w,
                                                   int64_t n, int64_t k, float *__restrict__ y, int64_t ld_y,
                                                   int segs_per_wg, uint32_t *__restrict__ ctr,
                                                   float *__restrict__ part) {
    extern __shared__ float lds_u[];  // [groups of this workgroup][M][64]
    __shared__ int last_wg;
    tile_unit<M, LAYOUT, ACT, ONE, GEMV_MF_MIN_ROWS>(xq, ld_x, xs, w, n, k, y, ld_y, (int64_t)blockIdx.y, (int)blockIdx.x,
                                   (int)gridDim.x, segs_per_wg, ctr, part, lds_u, &last_wg, false, NoWait());
}


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

// Exclusive prefix sum over the GROUP_THREADS threads of the workgroup: a
// shuffle scan inside each wave, the wave totals scanned by wave 0, two
// barriers in all.
__device__ __forceinline__ int block_exclusive_scan(int v, int *wave_tot) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int incl = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int t = __shfl_up(incl, off);
        if (lane >= off) incl += t;
    }
    if (lane == 63) wave_tot[wave] = incl;
    __syncthreads();
    if (wave == 0) {
        int w = lane < GROUP_THREADS / 64 ? wave_tot[lane] : 0;
#pragma unroll
        for (int off = 1; off < GROUP_THREADS / 64; off <<= 1) {
            const int t = __shfl_up(w, off);
            if (lane >= off) w += t;
        }
        if (lane < GROUP_THREADS / 64) wave_tot[lane] = w;  // inclusive over waves
    }
    __syncthreads();
    return (wave ? wave_tot[wave - 1] : 0) + incl - v;
}

// Occurrences of `id` in chunk[0, len): four ids per LDS read, unrolled so
// that several reads are in flight.
__device__ __forceinline__ int count_in_chunk(const int32_t *chunk, int len, int id) {
    int cnt = 0;
    const int4 *c4 = reinterpret_cast<const int4 *>(chunk);
    const int n4 = len >> 2;
#pragma unroll 8
    for (int j = 0; j < n4; j++) {
        const int4 v = c4[j];
        cnt += (v.x == id) + (v.y == id) + (v.z == id) + (v.w == id);
    }
    for (int j = n4 << 2; j < len; j++) cnt += (chunk[j] == id);
    return cnt;
}

__global__ __launch_bounds__(GROUP_THREADS) void group_pairs_kernel(const int32_t *__restrict__ ids, int64_t pairs,
                                                                   int64_t n_experts, int32_t *__restrict__ ws) {
    __shared__ __align__(16) int32_t chunk[ID_CHUNK];
    __shared__ int scan_sh[GROUP_THREADS / 64];
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
        if (tid < E) cnt += count_in_chunk(chunk, len, tid);
    }
    if (bad) atomicOr(&bad_sh, 1);
    // one scan of (active flag, pair count): the flag in bits 17 and up (at
    // most 1024 experts), the count below (at most 65536 pairs)
    const int is_active = (tid < E && cnt > 0) ? 1 : 0;
    const int packed = (is_active << 17) | (is_active ? cnt : 0);
    const int excl = block_exclusive_scan(packed, scan_sh);
    const int slot = excl >> 17, off = excl & 0x1ffff;
    if (is_active) {
        active[slot] = tid;
        offs[slot] = off;
    }
    if (tid == GROUP_THREADS - 1) {
        const int incl = excl + packed;
        ws[1] = incl >> 17;
        offs[incl >> 17] = incl & 0x1ffff;
    }
    __syncthreads();
    if (tid == 0) ws[0] = bad_sh ? 1 : 0;
    // scatter each active expert's pairs in increasing p
    int pos = off;
    for (int64_t base = 0; base < pairs; base += ID_CHUNK) {
        const int len = (int)((pairs - base) < ID_CHUNK ? (pairs - base) : ID_CHUNK);
        if (pairs > ID_CHUNK) {  // a single chunk is still in LDS from the count
            __syncthreads();
            for (int i = tid; i < len; i += GROUP_THREADS) chunk[i] = ids[base + i];
            __syncthreads();
        }
        if (is_active) {
            const int4 *c4 = reinterpret_cast<const int4 *>(chunk);
            const int n4 = len >> 2;
#pragma unroll 8
            for (int j = 0; j < n4; j++) {
                const int4 v = c4[j];
                const int32_t p0 = (int32_t)(base + 4 * j);
                if (v.x == tid) list[pos++] = p0;
                if (v.y == tid) list[pos++] = p0 + 1;
                if (v.z == tid) list[pos++] = p0 + 2;
                if (v.w == tid) list[pos++] = p0 + 3;
            }
            for (int j = n4 << 2; j < len; j++)
                if (chunk[j] == tid) list[pos++] = (int32_t)(base + j);
        }
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
    row_groups<M, 1, false, int8_t, false>(wbase, RECORD_BYTES, 0, (int)G, 1, xrow, srow, acc, nullptr, 0, NoWait());
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
