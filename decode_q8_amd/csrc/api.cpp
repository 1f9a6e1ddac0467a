// C ABI of libq8: argument validation, device check and dispatch.
//
// Every check that can be made from the arguments alone runs before the
// first HIP call, so a caller learns about a bad request even without a GPU.
// The device check then confirms the current device is gfx950 (cached per
// device); other hardware is rejected rather than served by a fallback.
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <string.h>

#include <atomic>

#include "../../include/q8.h"
#include "launch.hpp"

#ifndef Q8_BUILD_DIGEST
#define Q8_BUILD_DIGEST "unknown"
#endif

static_assert(Q8_SEQUENCE_MAX_STEPS == q8k::SEQ_MAX_STEPS, "sequence length limit");
static_assert(Q8_SEQUENCE_SCRATCH_BYTES == q8k::SEQ_SCRATCH_BYTES, "sequence scratch size");
static_assert(Q8_ROUTE_MAX_EXPERTS == q8k::ROUTE_MAX_EXPERTS && Q8_ROUTE_MAX_TOPK == q8k::ROUTE_MAX_TOPK,
              "router limits");
static_assert(Q8_ATTENTION_MAX_LEN == q8k::ATT_MAX_LEN, "attention context limit");

namespace q8k {
static std::atomic<uint32_t> g_device_queries{0};
void note_device_query() { g_device_queries.fetch_add(1, std::memory_order_relaxed); }
}  // namespace q8k

namespace {

constexpr int kMaxDevices = 64;
std::atomic<int8_t> g_arch_ok[kMaxDevices];  // 0 unknown, 1 gfx950, -1 other

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// Do [a, a + na) and [b, b + nb) share a byte?  (NULL never overlaps.)
bool overlap(const void *a, size_t na, const void *b, size_t nb) {
    if (!a || !b) return false;
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + nb && y < x + na;
}

int check_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return Q8_ERR_DEVICE;
    if (dev < kMaxDevices) {
        const int8_t known = g_arch_ok[dev].load(std::memory_order_relaxed);
        if (known == 1) return Q8_OK;
        if (known == -1) return Q8_ERR_DEVICE;
    }
    hipDeviceProp_t prop;
    q8k::note_device_query();
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return Q8_ERR_DEVICE;
    const bool ok = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    if (dev < kMaxDevices) g_arch_ok[dev].store(ok ? 1 : -1, std::memory_order_relaxed);
    return ok ? Q8_OK : Q8_ERR_DEVICE;
}

int launched(hipError_t e) { return e == hipSuccess ? Q8_OK : Q8_ERR_LAUNCH; }

}  // namespace

extern "C" {

uint32_t q8_abi_version(void) { return Q8_ABI_VERSION; }

const char *q8_build_digest(void) { return Q8_BUILD_DIGEST; }

uint32_t q8_device_queries(void) { return q8k::g_device_queries.load(std::memory_order_relaxed); }

const char *q8_status_str(int status) {
    switch (status) {
        case Q8_OK: return "Q8_OK";
        case Q8_ERR_ARG: return "Q8_ERR_ARG: invalid argument";
        case Q8_ERR_SHAPE: return "Q8_ERR_SHAPE: unsupported shape";
        case Q8_ERR_ALIGN: return "Q8_ERR_ALIGN: misaligned pointer or stride";
        case Q8_ERR_WORKSPACE: return "Q8_ERR_WORKSPACE: workspace missing or too small";
        case Q8_ERR_DEVICE: return "Q8_ERR_DEVICE: no gfx950 device";
        case Q8_ERR_LAUNCH: return "Q8_ERR_LAUNCH: kernel launch failed";
        default: return "Q8_ERR_UNKNOWN";
    }
}

size_t q8_quantized_bytes(int64_t rows, int64_t k) {
    if (rows < 0 || k < 0 || k % Q8_BLOCK) return 0;
    return (size_t)rows * (size_t)(k / Q8_BLOCK) * Q8_BLOCK_BYTES;
}

int q8_quantize_rows(const float *x, int64_t ld_x, int64_t rows, int64_t k, int layout, void *q_out,
                     hipStream_t stream) {
    if (!x || !q_out || rows < 0 || k <= 0 || ld_x < k) return Q8_ERR_ARG;
    if (layout != Q8_LAYOUT_ROWS && layout != Q8_LAYOUT_ACT) return Q8_ERR_ARG;
    if (k % Q8_BLOCK) return Q8_ERR_SHAPE;
    if (!aligned16(x) || !aligned16(q_out) || ld_x % 4) return Q8_ERR_ALIGN;
    if (rows == 0) return Q8_OK;
    const int dev = check_device();
    if (dev != Q8_OK) return dev;
    return launched(q8k::launch_quantize(x, ld_x, rows, k, layout, q_out, stream));
}

int q8_repack_weights(const void *w_rows, int64_t n, int64_t k, void *w_packed, hipStream_t stream) {
    if (!w_rows || !w_packed || n <= 0 || k <= 0) return Q8_ERR_ARG;
    if (n % Q8_TILE_ROWS || k % (Q8_BLOCK * Q8_TILE_BLOCKS)) return Q8_ERR_SHAPE;
    if (!aligned16(w_rows) || !aligned16(w_packed)) return Q8_ERR_ALIGN;
    const int dev = check_device();
    if (dev != Q8_OK) return dev;
    return launched(q8k::launch_repack(w_rows, n, k, w_packed, stream));
}

size_t q8_matmul_workspace_bytes(int64_t m, int64_t n, int64_t k) {
    if (m <= 0 || n <= 0 || k <= 0 || k % (Q8_BLOCK * Q8_TILE_BLOCKS)) return 0;
    if (m > Q8_GEMV_MAX_ROWS) return 0;
    return q8k::gemv_workspace_bytes(m, n, k);
}

int q8_matmul(const void *x_q, int64_t m, const void *w, int layout, int64_t n, int64_t k, float *y, int64_t ld_y,
              void *workspace, size_t workspace_bytes, hipStream_t stream) {
    if (!x_q || !w || !y || m <= 0 || n <= 0 || k <= 0 || ld_y < n) return Q8_ERR_ARG;
    if (layout != Q8_LAYOUT_ROWS && layout != Q8_LAYOUT_PACKED) return Q8_ERR_ARG;
    if (k % (Q8_BLOCK * Q8_TILE_BLOCKS)) return Q8_ERR_SHAPE;
    if (layout == Q8_LAYOUT_PACKED && n % Q8_TILE_ROWS) return Q8_ERR_SHAPE;
    if (m > Q8_GEMV_MAX_ROWS && layout != Q8_LAYOUT_PACKED) return Q8_ERR_SHAPE;
    if (!aligned16(x_q) || !aligned16(w) || !aligned16(y)) return Q8_ERR_ALIGN;
    const size_t need = q8_matmul_workspace_bytes(m, n, k);
    if (need > 0) {
        if (!workspace || workspace_bytes < need) return Q8_ERR_WORKSPACE;
        if (!aligned16(workspace)) return Q8_ERR_ALIGN;
    }
    const int dev = check_device();
    if (dev != Q8_OK) return dev;
    if (m <= Q8_GEMV_MAX_ROWS)
        return launched(q8k::launch_gemv(x_q, m, w, layout, n, k, y, ld_y, workspace, stream));
    return launched(q8k::launch_gemm(x_q, m, w, n, k, y, ld_y, stream));
}

int q8_quantize_matmul(const float *x, int64_t ld_x, int64_t m, const void *w, int layout, int64_t n, int64_t k,
                       float *y, int64_t ld_y, void *workspace, size_t workspace_bytes, hipStream_t stream) {
    if (!x || !w || !y || m <= 0 || n <= 0 || k <= 0 || ld_x < k || ld_y < n) return Q8_ERR_ARG;
    if (layout != Q8_LAYOUT_ROWS && layout != Q8_LAYOUT_PACKED) return Q8_ERR_ARG;
    if (m > Q8_GEMV_MAX_ROWS || k % (Q8_BLOCK * Q8_TILE_BLOCKS)) return Q8_ERR_SHAPE;
    if (layout == Q8_LAYOUT_PACKED && n % Q8_TILE_ROWS) return Q8_ERR_SHAPE;
    if (!aligned16(x) || !aligned16(w) || !aligned16(y) || ld_x % 4) return Q8_ERR_ALIGN;
    const size_t need = q8_matmul_workspace_bytes(m, n, k);
    if (need > 0) {
        if (!workspace || workspace_bytes < need) return Q8_ERR_WORKSPACE;
        if (!aligned16(workspace)) return Q8_ERR_ALIGN;
    }
    const int dev = check_device();
    if (dev != Q8_OK) return dev;
    return launched(q8k::launch_gemv_f32(x, ld_x, m, w, layout, n, k, y, ld_y, workspace, stream));
}

namespace {

// Validates a sequence and converts it to the launcher's form; returns a status.
int sequence_steps(const q8_gemv_step *steps, int count, int64_t m, q8k::SeqHostStep *out) {
    if (!steps || count <= 0 || m <= 0) return Q8_ERR_ARG;
    if (count > Q8_SEQUENCE_MAX_STEPS || m > Q8_GEMV_MAX_ROWS) return Q8_ERR_SHAPE;
    for (int i = 0; i < count; i++) {
        const q8_gemv_step &s = steps[i];
        if (!s.x || !s.w || !s.y || s.n <= 0 || s.k <= 0 || s.ld_x < s.k || s.ld_y < s.n) return Q8_ERR_ARG;
        if (s.n % Q8_TILE_ROWS || s.k % (Q8_BLOCK * Q8_TILE_BLOCKS)) return Q8_ERR_SHAPE;
        if (s.n > INT32_MAX || s.k > INT32_MAX || s.ld_x > INT32_MAX || s.ld_y > INT32_MAX) return Q8_ERR_SHAPE;
        if (!aligned16(s.x) || !aligned16(s.w) || !aligned16(s.y) || s.ld_x % 4) return Q8_ERR_ALIGN;
        out[i] = q8k::SeqHostStep{s.x, s.w, s.y, s.ld_x, s.ld_y, s.n, s.k};
    }
    return Q8_OK;
}

// Every x must be ready before the call: no y may overlap any x (the
// chaining y_i == x_(i+1) included), the y's must be disjoint, and the
// workspace (if any) must overlap neither.
int sequence_aliasing(const q8k::SeqHostStep *hs, int count, int64_t m, const void *workspace, size_t need) {
    for (int i = 0; i < count; i++) {
        const size_t yb = (size_t)((m - 1) * hs[i].ld_y + hs[i].n) * 4;
        if (overlap(workspace, need, hs[i].y, yb)) return Q8_ERR_ARG;
        if (overlap(workspace, need, hs[i].x, (size_t)((m - 1) * hs[i].ld_x + hs[i].k) * 4)) return Q8_ERR_ARG;
        for (int j = 0; j < count; j++) {
            if (overlap(hs[i].y, yb, hs[j].x, (size_t)((m - 1) * hs[j].ld_x + hs[j].k) * 4)) return Q8_ERR_ARG;
            if (j != i && overlap(hs[i].y, yb, hs[j].y, (size_t)((m - 1) * hs[j].ld_y + hs[j].n) * 4))
                return Q8_ERR_ARG;
        }
    }
    return Q8_OK;
}

}  // namespace

size_t q8_sequence_workspace_bytes(const q8_gemv_step *steps, int count, int64_t m) {
    q8k::SeqHostStep hs[Q8_SEQUENCE_MAX_STEPS];
    if (sequence_steps(steps, count, m, hs) != Q8_OK) return 0;
    return q8k::gemv_sequence_workspace_bytes(hs, count, m);
}

int q8_quantize_matmul_sequence(const q8_gemv_step *steps, int count, int64_t m, void *workspace,
                                size_t workspace_bytes, hipStream_t stream) {
    q8k::SeqHostStep hs[Q8_SEQUENCE_MAX_STEPS];
    const int st = sequence_steps(steps, count, m, hs);
    if (st != Q8_OK) return st;
    const size_t need = q8k::gemv_sequence_workspace_bytes(hs, count, m);
    if (!workspace || workspace_bytes < need) return Q8_ERR_WORKSPACE;
    if (!aligned16(workspace)) return Q8_ERR_ALIGN;
    const int alias = sequence_aliasing(hs, count, m, workspace, need);
    if (alias != Q8_OK) return alias;
    const int dev = check_device();
    if (dev != Q8_OK) return dev;
    return launched(q8k::launch_gemv_sequence(hs, count, m, workspace, stream));
}

int q8_quantize_matmul_sequence_noalloc(const q8_gemv_step *steps, int count, int64_t m, int32_t *status,
                                        hipStream_t stream) {
    q8k::SeqHostStep hs[Q8_SEQUENCE_MAX_STEPS];
    const int st = sequence_steps(steps, count, m, hs);
    if (st != Q8_OK) return st;
    if (q8k::gemv_sequence_workspace_bytes(hs, count, m) > (size_t)Q8_SEQUENCE_SCRATCH_BYTES) return Q8_ERR_WORKSPACE;
    if ((uintptr_t)status & 3u) return Q8_ERR_ALIGN;
    const int alias = sequence_aliasing(hs, count, m, nullptr, 0);
    if (alias != Q8_OK) return alias;
    for (int i = 0; i < count; i++)
        if (overlap(status, 4, hs[i].y, (size_t)((m - 1) * hs[i].ld_y + hs[i].n) * 4) ||
            overlap(status, 4, hs[i].x, (size_t)((m - 1) * hs[i].ld_x + hs[i].k) * 4))
            return Q8_ERR_ARG;
    const int dev = check_device();
    if (dev != Q8_OK) return dev;
    return launched(q8k::launch_gemv_sequence_scratch(hs, count, m, status, stream));
}

int q8_rmsnorm_quantize(const float *x, const float *residual_in, float *residual_out, const float *weight,
                        int64_t rows, int64_t k, float eps, void *q_out, hipStream_t stream) {
    if (!x || !weight || !q_out || rows < 0 || k <= 0) return Q8_ERR_ARG;
    if (!(eps >= 0.0f) || eps > 3.4e38f) return Q8_ERR_ARG;  // rejects NaN, negatives and infinity
    if (k % Q8_BLOCK || k > q8k::NORM_MAX_K || rows > INT32_MAX) return Q8_ERR_SHAPE;
    if (!aligned16(x) || !aligned16(weight) || !aligned16(q_out) || !aligned16(residual_in) ||
        !aligned16(residual_out))
        return Q8_ERR_ALIGN;
    if (rows == 0) return Q8_OK;
    // aliasing: residual_out may coincide exactly with x or residual_in; no other overlap
    const size_t fb = (size_t)rows * (size_t)k * 4, qb = q8_quantized_bytes(rows, k);
    if (overlap(q_out, qb, x, fb) || overlap(q_out, qb, residual_in, fb) || overlap(q_out, qb, residual_out, fb) ||
        overlap(q_out, qb, weight, (size_t)k * 4))
        return Q8_ERR_ARG;
    if (residual_out && residual_out != x && overlap(residual_out, fb, x, fb)) return Q8_ERR_ARG;
    if (residual_out && residual_out != residual_in && overlap(residual_out, fb, residual_in, fb)) return Q8_ERR_ARG;
    if (residual_out && overlap(residual_out, fb, weight, (size_t)k * 4)) return Q8_ERR_ARG;
    const int dev = check_device();
    if (dev != Q8_OK) return dev;
    return launched(q8k::launch_rmsnorm_quantize(x, residual_in, residual_out, weight, rows, k, eps, q_out, stream));
}

int q8_moe_route(const float *logits, int64_t tokens, int64_t n_experts, int topk, int normalize, int32_t *ids,
                 float *weights, hipStream_t stream) {
    if (!logits || !ids || !weights || tokens < 0 || n_experts <= 0 || topk < 1) return Q8_ERR_ARG;
    if (topk > n_experts || n_experts > Q8_ROUTE_MAX_EXPERTS || topk > Q8_ROUTE_MAX_TOPK || tokens > INT32_MAX)
        return Q8_ERR_SHAPE;
    if (((uintptr_t)logits & 3u) || ((uintptr_t)ids & 3u) || ((uintptr_t)weights & 3u)) return Q8_ERR_ALIGN;
    if (tokens == 0) return Q8_OK;
    const size_t pb = (size_t)tokens * (size_t)topk * 4;
    if (overlap(ids, pb, weights, pb) || overlap(ids, pb, logits, (size_t)tokens * (size_t)n_experts * 4) ||
        overlap(weights, pb, logits, (size_t)tokens * (size_t)n_experts * 4))
        return Q8_ERR_ARG;
    const int dev = check_device();
    if (dev != Q8_OK) return dev;
    return launched(q8k::launch_moe_route(logits, tokens, n_experts, topk, normalize ? 1 : 0, ids, weights, stream));
}

int q8_swiglu_quantize(const float *gate, int64_t ld_gate, const float *up, int64_t ld_up, int64_t rows, int64_t n,
                       void *q_out, hipStream_t stream) {
    if (!gate || !up || !q_out || rows < 0 || n <= 0 || ld_gate < n || ld_up < n) return Q8_ERR_ARG;
    if (n % Q8_BLOCK) return Q8_ERR_SHAPE;
    if (!aligned16(gate) || !aligned16(up) || !aligned16(q_out) || ld_gate % 4 || ld_up % 4) return Q8_ERR_ALIGN;
    if (rows == 0) return Q8_OK;
    const size_t qb = q8_quantized_bytes(rows, n);
    if (overlap(q_out, qb, gate, (size_t)((rows - 1) * ld_gate + n) * 4) ||
        overlap(q_out, qb, up, (size_t)((rows - 1) * ld_up + n) * 4))
        return Q8_ERR_ARG;
    const int dev = check_device();
    if (dev != Q8_OK) return dev;
    return launched(q8k::launch_swiglu_quantize(gate, ld_gate, up, ld_up, rows, n, q_out, stream));
}

int q8_moe_combine(const float *y, int64_t ld_y, const float *weights, int64_t tokens, int topk, int64_t n, float *out,
                   int64_t ld_out, hipStream_t stream) {
    if (!y || !weights || !out || tokens < 0 || topk < 1 || n <= 0 || ld_y < n || ld_out < n) return Q8_ERR_ARG;
    if (n % 4) return Q8_ERR_SHAPE;
    if (!aligned16(y) || !aligned16(out) || ((uintptr_t)weights & 3u) || ld_y % 4 || ld_out % 4) return Q8_ERR_ALIGN;
    if (tokens == 0) return Q8_OK;
    if (overlap(out, (size_t)((tokens - 1) * ld_out + n) * 4, y, (size_t)((tokens * topk - 1) * ld_y + n) * 4) ||
        overlap(out, (size_t)((tokens - 1) * ld_out + n) * 4, weights, (size_t)tokens * (size_t)topk * 4))
        return Q8_ERR_ARG;
    const int dev = check_device();
    if (dev != Q8_OK) return dev;
    return launched(q8k::launch_moe_combine(y, ld_y, weights, tokens, topk, n, out, ld_out, stream));
}

int q8_kv_write(const float *qkv, int64_t tokens, int n_heads, int n_kv, int head_dim, const int32_t *positions,
                int64_t max_pos, const float *cos_tab, const float *sin_tab, const float *q_gain, const float *k_gain,
                float eps, const int32_t *slots, int64_t n_slots, float *q_out, int8_t *k_cache, float *k_scale,
                int8_t *v_cache, float *v_scale, int32_t *status, hipStream_t stream) {
    if (!qkv || !positions || !cos_tab || !sin_tab || !slots || !q_out || !k_cache || !k_scale || !v_cache ||
        !v_scale || tokens < 0 || n_heads <= 0 || n_kv <= 0 || max_pos <= 0 || n_slots <= 0)
        return Q8_ERR_ARG;
    if ((q_gain || k_gain) && (!(eps >= 0.0f) || eps > 3.4e38f)) return Q8_ERR_ARG;
    if (n_heads % n_kv || (head_dim != 64 && head_dim != 128 && head_dim != 256)) return Q8_ERR_SHAPE;
    if (tokens > INT32_MAX || max_pos > INT32_MAX || (int64_t)tokens * (n_heads + 2 * n_kv) * head_dim > INT64_MAX / 8)
        return Q8_ERR_SHAPE;
    if (!aligned16(qkv) || !aligned16(cos_tab) || !aligned16(sin_tab) || !aligned16(q_gain) || !aligned16(k_gain) ||
        !aligned16(q_out) || !aligned16(k_cache) || !aligned16(v_cache) || ((uintptr_t)k_scale & 3u) ||
        ((uintptr_t)v_scale & 3u) || ((uintptr_t)positions & 3u) || ((uintptr_t)slots & 3u) ||
        ((uintptr_t)status & 3u))
        return Q8_ERR_ALIGN;
    if (tokens == 0) return Q8_OK;
    if (overlap(q_out, (size_t)tokens * n_heads * head_dim * 4, qkv,
                (size_t)tokens * (n_heads + 2 * n_kv) * head_dim * 4))
        return Q8_ERR_ARG;
    const int dev = check_device();
    if (dev != Q8_OK) return dev;
    return launched(q8k::launch_kv_write(qkv, tokens, n_heads, n_kv, head_dim, positions, max_pos, cos_tab, sin_tab,
                                         q_gain, k_gain, eps, slots, n_slots, q_out, k_cache, k_scale, v_cache,
                                         v_scale, status, stream));
}

static bool attention_shape_ok(int64_t seqs, int n_heads, int n_kv, int head_dim, int64_t max_len) {
    if (seqs < 0 || n_heads <= 0 || n_kv <= 0 || max_len <= 0 || n_heads % n_kv) return false;
    const int G = n_heads / n_kv;
    return (head_dim == 64 || head_dim == 128) && (G == 1 || G == 2 || G == 4 || G == 8) && max_len <= Q8_ATTENTION_MAX_LEN &&
           seqs <= 65535 && n_kv <= 65535;
}

size_t q8_attention_workspace_bytes(int64_t seqs, int n_heads, int n_kv, int head_dim, int64_t max_len) {
    if (!attention_shape_ok(seqs, n_heads, n_kv, head_dim, max_len)) return 0;
    return q8k::attention_workspace_bytes(seqs, n_heads, n_kv, head_dim, max_len);
}

int q8_attention_decode(const float *q, int64_t seqs, int n_heads, int n_kv, int head_dim, const int8_t *k_cache,
                        const float *k_scale, const int8_t *v_cache, const float *v_scale, int64_t n_slots,
                        const int32_t *base, const int32_t *len, int64_t max_len, float scale, float *out,
                        void *workspace, size_t workspace_bytes, hipStream_t stream) {
    if (!q || !k_cache || !k_scale || !v_cache || !v_scale || !base || !len || !out || seqs < 0 || n_heads <= 0 ||
        n_kv <= 0 || n_slots <= 0 || max_len <= 0)
        return Q8_ERR_ARG;
    if (!(scale == scale) || scale > 3.4e38f || scale < -3.4e38f) return Q8_ERR_ARG;
    if (!attention_shape_ok(seqs, n_heads, n_kv, head_dim, max_len)) return Q8_ERR_SHAPE;
    if (!aligned16(q) || !aligned16(out) || !aligned16(k_cache) || !aligned16(v_cache) || ((uintptr_t)k_scale & 3u) ||
        ((uintptr_t)v_scale & 3u) || ((uintptr_t)base & 3u) || ((uintptr_t)len & 3u))
        return Q8_ERR_ALIGN;
    if (seqs == 0) return Q8_OK;
    const size_t need = q8k::attention_workspace_bytes(seqs, n_heads, n_kv, head_dim, max_len);
    if (!workspace || workspace_bytes < need) return Q8_ERR_WORKSPACE;
    if (!aligned16(workspace)) return Q8_ERR_ALIGN;
    if (overlap(out, (size_t)seqs * n_heads * head_dim * 4, q, (size_t)seqs * n_heads * head_dim * 4) ||
        overlap(workspace, need, out, (size_t)seqs * n_heads * head_dim * 4))
        return Q8_ERR_ARG;
    const int dev = check_device();
    if (dev != Q8_OK) return dev;
    return launched(q8k::launch_attention_decode(q, seqs, n_heads, n_kv, head_dim, k_cache, k_scale, v_cache, v_scale,
                                                 n_slots, base, len, max_len, scale, out, workspace, stream));
}

size_t q8_grouped_workspace_bytes(int64_t tokens, int topk, int64_t n_experts, int64_t n, int64_t k) {
    (void)n;
    (void)k;
    if (tokens <= 0 || topk <= 0 || n_experts <= 0) return 0;
    return q8k::grouped_workspace_bytes(tokens, topk, n_experts);
}

int q8_grouped_matmul(const void *x_q, int64_t x_rows, int x_per_pair, const int32_t *topk_ids, int64_t tokens,
                      int topk, const void *w_experts, int64_t n_experts, int64_t expert_stride_bytes, int64_t n,
                      int64_t k, float *y, void *workspace, size_t workspace_bytes, hipStream_t stream) {
    if (!x_q || !topk_ids || !w_experts || !y || tokens <= 0 || topk <= 0 || n_experts <= 0 || n <= 0 || k <= 0)
        return Q8_ERR_ARG;
    if (x_per_pair != 0 && x_per_pair != 1) return Q8_ERR_ARG;
    if (x_rows != (x_per_pair ? tokens * topk : tokens)) return Q8_ERR_ARG;
    if (n % Q8_TILE_ROWS || k % (Q8_BLOCK * Q8_TILE_BLOCKS)) return Q8_ERR_SHAPE;
    if (topk > n_experts || n_experts > 1024 || tokens * topk > 65536) return Q8_ERR_SHAPE;
    if (expert_stride_bytes < (int64_t)q8_quantized_bytes(n, k) || expert_stride_bytes % 16) return Q8_ERR_SHAPE;
    if (!aligned16(x_q) || !aligned16(w_experts) || !aligned16(y) || ((uintptr_t)topk_ids & 3u)) return Q8_ERR_ALIGN;
    const size_t need = q8_grouped_workspace_bytes(tokens, topk, n_experts, n, k);
    if (!workspace || workspace_bytes < need) return Q8_ERR_WORKSPACE;
    if (!aligned16(workspace)) return Q8_ERR_ALIGN;
    const int dev = check_device();
    if (dev != Q8_OK) return dev;
    return launched(q8k::launch_grouped(x_q, x_rows, x_per_pair, topk_ids, tokens, topk, w_experts, n_experts,
                                        expert_stride_bytes, n, k, y, workspace, stream));
}

int q8_stream_read(const void *buf, size_t bytes, uint32_t *sink, hipStream_t stream) {
    if (!buf || !sink) return Q8_ERR_ARG;
    if (bytes % 16) return Q8_ERR_SHAPE;
    if (!aligned16(buf) || ((uintptr_t)sink & 3u)) return Q8_ERR_ALIGN;
    if (bytes == 0) return Q8_OK;
    if (overlap(sink, 4, buf, bytes)) return Q8_ERR_ARG;
    const int dev = check_device();
    if (dev != Q8_OK) return dev;
    return launched(q8k::launch_stream_read(buf, bytes, sink, stream));
}

}  // extern "C"
