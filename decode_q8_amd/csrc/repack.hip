// Weight repack for gfx950: row-contiguous Q8_0 -> packed 64-row x 8-block
// records.  A pure byte permutation that keeps the size (the packed record of
// the "Ember packed Q8 decode" post holds exactly the bytes of the blocks it
// covers; here one record covers 64 rows x 8 blocks = 17,408 bytes so that a
// 64-lane wave reads 1 KB contiguous per 16-byte load).
//
// One workgroup per record: 1,088 coalesced 16-byte loads of the 64 source
// row segments (272 bytes each, 16-byte aligned because k % 256 == 0) into LDS,
// then 1,088 coalesced 16-byte stores of the reordered record.  A 272-byte
// segment is not a whole number of 128-byte cache lines, so consecutive
// records of a tile share their boundary lines.  Workgroups go to the 8 XCDs
// round-robin by id, each with its own L2, so records are taken XCD-aware:
// XCD x gets the x-th eighth of the records, consecutive records on one XCD
// at about the same time, and a shared line is fetched from memory once
// instead of once per XCD (only speed and memory traffic depend on this).
#include "device.hpp"
#include "launch.hpp"

namespace q8k {

constexpr int XCDS = 8;

__global__ __launch_bounds__(256) void repack_kernel(const uint8_t *__restrict__ src, int64_t k,
                                                     uint8_t *__restrict__ dst) {
    __shared__ uint4 lds[RECORD_BYTES / 16];  // 64 rows x 17 chunks
    const int64_t groups = k / GROUP_K;
    const int64_t records = gridDim.x;
    const int64_t rec = records % XCDS ? (int64_t)blockIdx.x
                                       : (int64_t)(blockIdx.x % XCDS) * (records / XCDS) + blockIdx.x / XCDS;
    const int64_t T = rec / groups, G = rec - T * groups;
    const int64_t row_bytes = (k / QK) * BLOCK_BYTES;

    for (int c = threadIdx.x; c < RECORD_BYTES / 16; c += blockDim.x) {
        const int r = c / 17, i = c - r * 17;
        lds[c] = load_nt(src + (T * TILE_ROWS + r) * row_bytes + G * ROW_GROUP_BYTES + i * 16);  // read once: 112 -> 96 us
    }
    __syncthreads();
    const uint8_t *l8 = reinterpret_cast<const uint8_t *>(lds);
    uint8_t *out = dst + rec * RECORD_BYTES;
    for (int o = threadIdx.x; o < RECORD_BYTES / 16; o += blockDim.x) {
        uint32_t w[4];
        if (o < RECORD_Q_BYTES / 16) {
            // values of row r, block bb, half h (16 bytes), 2-byte aligned in LDS
            const int bb = o >> 7, h = (o >> 6) & 1, r = o & 63;
            const uint16_t *p = reinterpret_cast<const uint16_t *>(l8 + r * ROW_GROUP_BYTES + bb * BLOCK_BYTES + 2 + 16 * h);
#pragma unroll
            for (int j = 0; j < 4; j++) w[j] = (uint32_t)p[2 * j] | ((uint32_t)p[2 * j + 1] << 16);
        } else {
            // the 8 scales of row r
            const int r = o - RECORD_Q_BYTES / 16;
            const uint8_t *p = l8 + r * ROW_GROUP_BYTES;
#pragma unroll
            for (int j = 0; j < 4; j++) {
                const uint32_t lo = *reinterpret_cast<const uint16_t *>(p + (2 * j) * BLOCK_BYTES);
                const uint32_t hi = *reinterpret_cast<const uint16_t *>(p + (2 * j + 1) * BLOCK_BYTES);
                w[j] = lo | (hi << 16);
            }
        }
        *reinterpret_cast<uint4 *>(out + o * 16) = make_uint4(w[0], w[1], w[2], w[3]);
    }
}

hipError_t launch_repack(const void *w_rows, int64_t n, int64_t k, void *w_packed, hipStream_t s) {
    const int64_t records = (n / TILE_ROWS) * (k / GROUP_K);
    hipLaunchKernelGGL(repack_kernel, dim3((unsigned)records), dim3(256), 0, s, (const uint8_t *)w_rows, k,
                       (uint8_t *)w_packed);
    return hipGetLastError();
}

}  // namespace q8k
