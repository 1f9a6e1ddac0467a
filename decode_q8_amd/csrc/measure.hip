// A plain streaming read of one buffer: the bandwidth ceiling that the
// weight-streaming kernels are measured against (the "ferro" README, "Using
// LFM2.5 language models", reports decode as a fraction of what a pure
// streaming-read kernel reaches on the same device).
//
// Every 16-byte chunk is read exactly once.  Each wave reads one contiguous
// span of READ_SPAN chunks (32 KB): READ_UNROLL loads in flight per lane, a
// wave access being 64 consecutive chunks (1 KB), so the open DRAM pages are
// read through before the wave moves on (a grid-stride order over the whole
// buffer, which scatters concurrent accesses over many pages, streamed 1 GiB
// ~20% slower).  The loaded words are XOR-folded (one VALU op per word, far
// below the load rate) so that no load can be dropped; each workgroup folds
// its waves' results and XORs them into *sink with one atomic.  One wave per
// span, so a 1 GiB read is 32,768 waves, many more than the GPU holds at once.
// Measured shapes (waves per workgroup 4/8/16, spans of 16-64 KB) stay within
// about 5% of each other at 36 MB, 279 MB and 1 GiB, none best at every size;
// this one is within 1% of the best at 1 GiB.  The loads carry the non-temporal hint, as the
// weight loads of the GEMVs do: ~5% faster at 1 GiB (6.28 against 5.98 TB/s
// by graph replay), so the ceiling is the faster form.
#include <hip/hip_runtime.h>

#include "device.hpp"
#include "launch.hpp"

namespace q8k {

constexpr int READ_THREADS = 512;
constexpr int READ_UNROLL = 16;
constexpr int READ_ITERS = 2;
constexpr int64_t READ_SPAN = (int64_t)READ_ITERS * READ_UNROLL * 64;  // chunks per wave
constexpr int64_t READ_WG_SPAN = READ_SPAN * (READ_THREADS / 64);     // chunks per workgroup

__global__ __launch_bounds__(READ_THREADS) void stream_read_kernel(const uint4 *__restrict__ p, int64_t chunks,
                                                                   uint32_t *sink) {
    const int lane = threadIdx.x & 63;
    const int64_t base = (int64_t)blockIdx.x * READ_WG_SPAN + (int64_t)(threadIdx.x >> 6) * READ_SPAN + lane;
    uint32_t x = 0, y = 0, z = 0, w = 0;
    for (int it = 0; it < READ_ITERS; it++) {
        uint4 v[READ_UNROLL];
#pragma unroll
        for (int u = 0; u < READ_UNROLL; u++) {
            const int64_t i = base + (int64_t)(it * READ_UNROLL + u) * 64;
            v[u] = i < chunks ? load_nt(p + i) : make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int u = 0; u < READ_UNROLL; u++) {
            x ^= v[u].x;
            y ^= v[u].y;
            z ^= v[u].z;
            w ^= v[u].w;
        }
    }
    uint32_t f = (x ^ y) ^ (z ^ w);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) f ^= (uint32_t)__shfl_xor((int)f, o, 64);
    __shared__ uint32_t part[READ_THREADS / 64];
    if (lane == 0) part[threadIdx.x >> 6] = f;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t t = 0;
#pragma unroll
        for (int j = 0; j < READ_THREADS / 64; j++) t ^= part[j];
        __hip_atomic_fetch_xor(sink, t, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

hipError_t launch_stream_read(const void *buf, size_t bytes, uint32_t *sink, hipStream_t s) {
    const int64_t chunks = (int64_t)(bytes / 16);
    const int64_t wgs = (chunks + READ_WG_SPAN - 1) / READ_WG_SPAN;
    if (wgs > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)wgs), dim3(READ_THREADS), 0, s,
                       static_cast<const uint4 *>(buf), chunks, sink);
    return hipGetLastError();
}

}  // namespace q8k
