// A sequence of fused-quantization GEMVs in one persistent launch (a decode
// step's matrices, each consuming the activation of the step before it).
//
// Every GEMV is computed exactly as the per-matrix kernel computes it (the
// same tile_unit, so the outputs are bit-identical); what changes is how the
// work is scheduled.  A fixed grid of workgroups that all fit on the GPU at
// once walks the steps in order.  Step p's work units (a 64-row tile, or one
// workgroup's share of a split tile) go to the workgroups round-robin,
// starting where step p - 1's units ended, so consecutive small steps land on
// different workgroups.  A workgroup issues the weight loads of its next unit
// as soon as it is free, then waits until every unit of step p - 1 has been
// counted done before it reads step p's activations: the weights of the next
// matrix stream in while the previous one finishes, which a launch per matrix
// cannot do (the weights do not depend on the activations; the activations
// do depend on the step before, which the wait models).
//
// Step completion is counted in the workspace with device-scope atomics
// (performed at the device-coherent point) once a unit is done: directly in
// the step's counter when the step has at most SEQ_SUB_MIN_UNITS units, else
// first in one of SEQ_NSUB sub-counters (unit u in sub-counter u mod SEQ_NSUB)
// whose last unit then counts the sub-counter in -- hundreds of units
// incrementing one address queue up behind each other, a few do not.  Every
// counter sits in a 128-byte line of its own and is returned to zero by the
// unit that completes it.  The unit that completes a step raises the step's
// flag in FLAG_LINES separate lines with system-scope stores (in each line
// every step's flag sits alone in a 128-byte slot, so the polls of one step
// and the raising of the next never meet on a cache line), and a waiting
// workgroup polls "its" line (workgroup index mod FLAG_LINES: with workgroups
// dealt to the XCDs in turn, two lines per XCD and 32 pollers per line) with
// system-scope loads: both bypass the per-XCD L2s, which
// are not coherent with each other, and spreading the pollers over lines
// keeps hundreds of them from queueing on one address (measured: polling the
// counter itself with read-modify-writes made the step 2x slower).  The poll
// is bounded: a wait that does not end within the limit (only possible if the
// grid did not fit on the GPU) records Q8_ERR_LAUNCH in the workspace status
// word and proceeds, so the launch always ends.  The call's outputs are then
// undefined (a successor may chain handed-over segment sums that are not all
// written yet) and a late unit may leave a flag raised, so the caller must
// zero the workspace again.  The unit that completes the last step returns
// every flag to zero; by then no workgroup is waiting any more, since each
// wait precedes a unit that the last step transitively depends on.
//
// A step whose tiles are split over several workgroups (long rows, few tiles)
// and that has a successor hands its segment sums over instead of chaining
// them itself: its workgroups only leave the sums in the workspace (no
// per-tile counter, no last-workgroup chain), and the successor's units, which
// wait for the step anyway, chain them and write its outputs (unit u takes
// tiles u, u + units, ...) while their own activation loads are in flight.
// Every output is still the same chain of the same segment sums, so it stays
// bit-identical to its own launch; the step's outputs are complete when its
// successor is.
#include <atomic>

#include "device.hpp"
#include "gemv_core.hpp"
#include "launch.hpp"

namespace q8k {

constexpr uint32_t SEQ_SPIN_LIMIT = 1u << 18;  // polls of roughly 1 us each
constexpr int SEQ_SUB_MIN_UNITS = 64;  // more units than this: two-level counting
// Prefetch stagger per wave, in 10 ns ticks of s_memrealtime: 0.65 us with
// one activation row, 1.5 us with more.  Measured per row count (decode step,
// same-box sweeps): m = 1 at 0.25 / 0.35 / 0.5 / 0.55 / 0.6 / 0.65 / 0.7 /
// 0.75 / 1.0 us took 302 / 304 / 288 / 287 / 285.2 / 285.0 / 288 / 292 / 296
// us; m = 2 and 4 were 3-4% slower at 0.75 us than at 1.5, m = 8 unchanged.
template <int M>
constexpr uint32_t seq_pace_ticks() { return M == 1 ? 65u : 150u; }

// Whether a workgroup paces the weight loads of its unit of step p (its
// previous unit was of step prev_p, -1 for none): when the unit is needed two
// or more steps after the previous one, and with one activation row also for
// the workgroup's first unit past step 0 (every workgroup fetches its first
// unit at once at the start: 300.6 -> 299.4 us per decode step; with 4 rows
// it cost 3%).
template <int M>
__device__ __forceinline__ bool paced(int prev_p, int p) {
    return prev_p >= 0 ? p > prev_p + 1 : (M == 1 && p > 0);
}
constexpr int FLAG_LINES = SEQ_FLAG_LINES;
constexpr int FLAG_LINE_BYTES = SEQ_FLAG_LINE_BYTES;
constexpr int CTR_LINE = SEQ_CTR_LINE;
constexpr int CTR_PER_STEP = SEQ_CTR_PER_STEP;
static_assert(SEQ_MAX_STEPS * SEQ_FLAG_SLOT_BYTES <= FLAG_LINE_BYTES, "a flag line holds every step's flag");
static_assert((SEQ_NSUB & (SEQ_NSUB - 1)) == 0 && SEQ_NSUB <= SEQ_SUB_MIN_UNITS, "every sub-counter has units");

struct SeqStep {
    const float *x;
    const uint8_t *w;
    float *y;
    int32_t ld_x, ld_y, n, k;
    uint32_t ws_off;  // this step's tile counters and segment sums at ws + 256 * ws_off (0: none)
    uint16_t wgs;     // workgroups per tile
    uint16_t segs;    // segments per workgroup
};
static_assert(sizeof(SeqStep) == 48, "kernel-argument layout");

// Workspace layout: see SeqPlan (plan.cpp).
struct SeqArgs {
    uint8_t *ws;
    int32_t count, nwg;
    int32_t flag_off;
    SeqStep step[SEQ_MAX_STEPS];
};

__device__ __forceinline__ uint32_t *step_counter(uint8_t *ws, int p, int c) {
    return reinterpret_cast<uint32_t *>(ws + 256 + CTR_LINE * (CTR_PER_STEP * p + c));
}

__device__ __forceinline__ uint32_t *step_flag(const SeqArgs &a, int line, int p) {
    return reinterpret_cast<uint32_t *>(a.ws + a.flag_off + FLAG_LINE_BYTES * line + SEQ_FLAG_SLOT_BYTES * p);
}

__device__ __forceinline__ uint32_t atomic_inc_old(uint32_t *c) {
    return __hip_atomic_fetch_add(c, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void atomic_clear(uint32_t *c) {
    __hip_atomic_exchange(c, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Counts unit u of a step of `units` units in; true for the unit that
// completes the step (one thread calls this).
__device__ __forceinline__ bool count_unit(uint8_t *ws, int p, int u, int units) {
    uint32_t *top = step_counter(ws, p, 0);
    if (units > SEQ_SUB_MIN_UNITS) {
        const int c = u & (SEQ_NSUB - 1);
        uint32_t *sub = step_counter(ws, p, 1 + c);
        if (atomic_inc_old(sub) != (uint32_t)((units - 1 - c) / SEQ_NSUB)) return false;
        atomic_clear(sub);
        if (atomic_inc_old(top) != (uint32_t)(SEQ_NSUB - 1)) return false;
    } else if (atomic_inc_old(top) != (uint32_t)(units - 1)) {
        return false;
    }
    atomic_clear(top);
    return true;
}

// Thread-level wait until *flag != 0 (bounded; see the file comment).
__device__ __forceinline__ void wait_flag(uint32_t *flag, int32_t *status) {
    for (uint32_t i = 0; i < SEQ_SPIN_LIMIT; i++) {
        if (__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM) != 0u) return;
        __builtin_amdgcn_s_sleep(1);
    }
    __hip_atomic_exchange(status, 6 /* Q8_ERR_LAUNCH */, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ bool hands_over(const SeqArgs &a, int p) { return a.step[p].wgs > 1 && p + 1 < a.count; }

__device__ __forceinline__ uint32_t *split_counters(const SeqArgs &a, int p) {
    return reinterpret_cast<uint32_t *>(a.ws + 256 * (size_t)a.step[p].ws_off);
}

__device__ __forceinline__ float *split_sums(const SeqArgs &a, int p) {
    const int tiles = a.step[p].n >> 6;
    return reinterpret_cast<float *>(reinterpret_cast<uint8_t *>(split_counters(a, p)) + (tiles * 4 + 255) / 256 * 256);
}

// Unit u (of `units`) of step p chains its share of step p - 1's handed-over
// sums: tiles u, u + units, ...
template <int M>
__device__ __forceinline__ void finish_previous(const SeqArgs &a, int p, int u, int units) {
    if (p > 0 && hands_over(a, p - 1)) {
        const SeqStep &q = a.step[p - 1];
        finish_split<M>(split_sums(a, p - 1), q.y, q.ld_y, q.n, ((q.k >> 8) + SEG_GROUPS - 1) / SEG_GROUPS, u, units);
    }
}

// The per-unit hooks of tile_unit in the sequence: wait for the previous
// step (first unit of this step on this workgroup only); then, for one
// activation row, chain this unit's share of the previous step's handed-over
// sums while the activation loads are in flight.  With more rows the weights
// and activations held at that point leave no registers for it, and the
// sequence kernel does it after the unit instead.
template <int M>
struct SeqHooks {
    const SeqArgs &a;
    int p, wg, u, units;
    bool ready;
    bool pace;  // stagger this unit's weight loads over the waves (see paced())
    uint64_t t0;  // s_memrealtime when the workgroup took up the unit
    int32_t *status;
    __device__ void before() const {
        if (pace) {  // wave w issues its weight loads w * seq_pace_ticks<M>() after the unit was taken up
            const uint64_t until = t0 + (uint64_t)seq_pace_ticks<M>() * (threadIdx.x >> 6);
            for (int i = 0; i < 4096 && __builtin_amdgcn_s_memrealtime() < until; i++) __builtin_amdgcn_s_sleep(2);
        }
    }
    __device__ void operator()() const {
        if (!ready) {
            if (threadIdx.x == 0) wait_flag(step_flag(a, wg % FLAG_LINES, p - 1), status);
            __syncthreads();
        }
    }
    __device__ void after() const {
        if constexpr (M == 1) finish_previous<M>(a, p, u, units);
    }
};

// ONE (at most one group per wave), lane form (m below SEQ_MF_MIN_ROWS): at
// most 128 VGPRs, so that two 512-thread workgroups fit on a CU.  The MFMA
// form (m >= SEQ_MF_MIN_ROWS) keeps up to 256 VGPRs and one workgroup per CU:
// capped at 128 it spilled ~190 bytes per lane, and the reloads on each
// step's critical path cost more than the halved grid (m = 8: 906 -> 698 us
// per decode step).
template <int M, bool ONE>
__global__ __launch_bounds__(SEQ_THREADS) __attribute__((amdgpu_waves_per_eu(ONE && M < SEQ_MF_MIN_ROWS ? 4 : 1, 8))) void
gemv_sequence_kernel(const SeqArgs a) {
    extern __shared__ float lds_u[];  // [groups of a unit][M][64]
    __shared__ int last_wg;
    const int wg = blockIdx.x, nwg = a.nwg;
    int32_t *status = reinterpret_cast<int32_t *>(a.ws);
    int prev_p = -1;     // step of this workgroup's previous unit
    int start = 0;       // workgroup of step p's first unit: (units of all earlier steps) mod nwg
    for (int p = 0; p < a.count; p++) {
        const SeqStep &st = a.step[p];
        const int tiles = st.n >> 6;
        const int units = tiles * st.wgs;
        uint32_t *ctr = st.ws_off ? split_counters(a, p) : nullptr;
        float *part = ctr ? split_sums(a, p) : nullptr;
        const bool handover = hands_over(a, p);
        // this workgroup's units of step p: u = first, first + nwg, ... (32-bit arithmetic throughout)
        const int first = wg >= start ? wg - start : wg - start + nwg;
        bool ready = p == 0;
        for (int u = first; u < units; u += nwg) {
            const int T = u / st.wgs, wi = u - T * st.wgs;
            asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");  // previous unit's LDS reads done
            tile_unit<M, 1, float, ONE, SEQ_MF_MIN_ROWS>(st.x, st.ld_x, nullptr, st.w, st.n, st.k, st.y, st.ld_y, T, wi,
                                                        st.wgs,
                                        st.segs, ctr, part, lds_u, &last_wg, handover,
                                        SeqHooks<M>{a, p, wg, u, units, ready, paced<M>(prev_p, p),
                                                    __builtin_amdgcn_s_memrealtime(), status});
            prev_p = p;
            if constexpr (M > 1) finish_previous<M>(a, p, u, units);
            ready = true;
            // every wave of the unit is done (its LDS work complete, handed-over
            // sums and chained outputs of the previous step written at the
            // coherent point or stored); its own output stores may still be in
            // flight: nothing in the launch reads them
            asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
            if (threadIdx.x < 64) {  // wave 0: count the unit in; the last one raises the step's flags
                int last = 0;
                if (threadIdx.x == 0) last = count_unit(a.ws, p, u, units);
                last = __builtin_amdgcn_readfirstlane(last);
                if (last && threadIdx.x < FLAG_LINES)
                    __hip_atomic_store(step_flag(a, threadIdx.x, p), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
                if (last && p == a.count - 1) {  // the whole sequence is done: clear the flags
                    for (int i = threadIdx.x; i < FLAG_LINES * a.count; i += 64)
                        __hip_atomic_store(step_flag(a, i / a.count, i % a.count), 0u, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_SYSTEM);
                }
            }
        }
        start = (start + units % nwg) % nwg;
    }
}

// Host side ---------------------------------------------------------------

struct SeqLayout {
    bool one;
    size_t lds, workspace;
    SeqArgs args;
};

static bool seq_layout(const SeqHostStep *steps, int count, int64_t m, SeqLayout &L) {
    SeqPlan P;
    seq_plan(steps, count, m, P);
    L.one = P.one;
    L.lds = P.lds;
    L.workspace = P.workspace;
    L.args.count = count;
    L.args.flag_off = P.flag_off;
    for (int i = 0; i < count; i++) {
        const SeqHostStep &h = steps[i];
        SeqStep &s = L.args.step[i];
        s.x = h.x;
        s.w = (const uint8_t *)h.w;
        s.y = h.y;
        s.ld_x = (int32_t)h.ld_x;
        s.ld_y = (int32_t)h.ld_y;
        s.n = (int32_t)h.n;
        s.k = (int32_t)h.k;
        s.wgs = P.wgs[i];
        s.segs = P.segs[i];
        s.ws_off = P.ws_off[i];
    }
    return true;
}

// Resident workgroups per CU of each kernel variant, per device and dynamic
// LDS size (whole KB, at most 64), and the CU count per device: discovered on
// the first launch that needs them and kept, so later calls on the token path
// query nothing about the device.
constexpr int SEQ_MAX_DEVICES = 64;
constexpr int SEQ_LDS_KB_MAX = 64;
static std::atomic<int16_t> g_seq_per_cu[SEQ_MAX_DEVICES][8][2][SEQ_LDS_KB_MAX + 1];  // 0: not yet known
static std::atomic<int32_t> g_seq_cus[SEQ_MAX_DEVICES];

template <int M, bool ONE>
static hipError_t launch_seq(SeqLayout &L, void *ws, hipStream_t s) {
    // The grid is as many workgroups as the GPU holds at once: the waits need
    // every workgroup resident.
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const int lds_kb = (int)((L.lds + 1023) / 1024);
    if (dev < 0 || dev >= SEQ_MAX_DEVICES || lds_kb > SEQ_LDS_KB_MAX) return hipErrorInvalidConfiguration;
    std::atomic<int16_t> &slot = g_seq_per_cu[dev][M - 1][ONE ? 1 : 0][lds_kb];
    int per_cu = slot.load(std::memory_order_relaxed);
    if (per_cu == 0) {
        note_device_query();
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, gemv_sequence_kernel<M, ONE>, SEQ_THREADS,
                                                         (size_t)lds_kb * 1024);
        if (e != hipSuccess) return e;
        if (per_cu < 1) return hipErrorInvalidConfiguration;
        slot.store((int16_t)per_cu, std::memory_order_relaxed);
    }
    int cus = g_seq_cus[dev].load(std::memory_order_relaxed);
    if (cus == 0) {
        note_device_query();
        e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return e;
        if (cus < 1) return hipErrorInvalidConfiguration;
        g_seq_cus[dev].store(cus, std::memory_order_relaxed);
    }
    L.args.ws = (uint8_t *)ws;
    L.args.nwg = per_cu * cus;
    hipLaunchKernelGGL((gemv_sequence_kernel<M, ONE>), dim3((unsigned)L.args.nwg), dim3(SEQ_THREADS), L.lds, s,
                       L.args);
    return hipGetLastError();
}

static hipError_t launch_layout(SeqLayout &L, int64_t m, void *ws, hipStream_t s) {
#define Q8_SEQ_CASE(MM) \
    case MM:            \
        return L.one ? launch_seq<MM, true>(L, ws, s) : launch_seq<MM, false>(L, ws, s);
    switch (m) {
        Q8_SEQ_CASE(1) Q8_SEQ_CASE(2) Q8_SEQ_CASE(3) Q8_SEQ_CASE(4)
        Q8_SEQ_CASE(5) Q8_SEQ_CASE(6) Q8_SEQ_CASE(7) Q8_SEQ_CASE(8)
        default: return hipErrorInvalidValue;
    }
#undef Q8_SEQ_CASE
}

hipError_t launch_gemv_sequence(const SeqHostStep *steps, int count, int64_t m, void *ws, hipStream_t s) {
    SeqLayout L;
    seq_layout(steps, count, m, L);
    return launch_layout(L, m, ws, s);
}

// ---------------------------------------------------------------------------
// The allocation-free variant: the workspace is this library's own device
// array, one per GPU, held until the process ends.  Host code never passes
// the array's name to a kernel (on the host it is only a stand-in for the
// symbol): its device address is looked up once per device with
// hipGetSymbolAddress and kept, and that address is what the kernels get.
// Calls on one GPU share the array, so calls that overlap in time on one GPU
// race; the part a call uses is zeroed at the start of every call (by a fill
// kernel, so the call can be captured in a graph).
// ---------------------------------------------------------------------------

static __device__ __align__(256) uint8_t scratch[SEQ_SCRATCH_BYTES];

static std::atomic<void *> g_scratch_ptr[SEQ_MAX_DEVICES];

// Device address of this GPU's scratch array (the current device), looked up
// on the first call on that device.
static hipError_t scratch_address(void **ptr) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= SEQ_MAX_DEVICES) return hipErrorInvalidDevice;
    void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        note_device_query();
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
    *ptr = p;
    return hipSuccess;
}

// Zero `words` 16-byte words from p (a grid-stride fill).
__global__ __launch_bounds__(256) void zero_fill_kernel(uint4 *__restrict__ p, int64_t words) {
    const uint4 z = {0u, 0u, 0u, 0u};
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < words; i += (int64_t)gridDim.x * 256) p[i] = z;
}

// *out = the sequence's status word (one thread).
__global__ void copy_status_kernel(const int32_t *__restrict__ ws, int32_t *__restrict__ out) { *out = ws[0]; }

hipError_t launch_gemv_sequence_scratch(const SeqHostStep *steps, int count, int64_t m, int32_t *status,
                                        hipStream_t s) {
    SeqLayout L;
    seq_layout(steps, count, m, L);
    if (L.workspace > SEQ_SCRATCH_BYTES) return hipErrorInvalidValue;  // the caller checked this already
    void *ws = nullptr;
    hipError_t e = scratch_address(&ws);
    if (e != hipSuccess) return e;
    const int64_t words = (int64_t)((L.workspace + 15) / 16);
    const int64_t blocks = (words + 255) / 256 < 1024 ? (words + 255) / 256 : 1024;
    hipLaunchKernelGGL(zero_fill_kernel, dim3((unsigned)blocks), dim3(256), 0, s, (uint4 *)ws, words);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    e = launch_layout(L, m, ws, s);
    if (e != hipSuccess || !status) return e;
    hipLaunchKernelGGL(copy_status_kernel, dim3(1), dim3(1), 0, s, (const int32_t *)ws, status);
    return hipGetLastError();
}

}  // namespace q8k
