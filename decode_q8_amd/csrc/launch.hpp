// Internal launchers between the C ABI (api.cpp) and the kernel sources.
// Arguments are already validated; each returns the hipError_t of its launch.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

#include "layout.hpp"

namespace q8k {

// Counts the library's queries of device properties (architecture, CU count,
// occupancy).  Each is made once per device and kernel variant and then
// cached, so the count stops growing after the first calls.
void note_device_query();

hipError_t launch_quantize(const float *x, int64_t ld_x, int64_t rows, int64_t k, int layout, void *out,
                           hipStream_t s);

hipError_t launch_repack(const void *w_rows, int64_t n, int64_t k, void *w_packed, hipStream_t s);

// Execution plan of a GEMV (only speed depends on it, never the bits).
struct GemvPlan {
    int64_t tiles;     // 64-row tiles
    int64_t groups;    // 256-value groups along k
    int wgs_per_tile;  // workgroups sharing one tile (one or more segments each)
    int segs_per_wg;   // 2048-value segments per workgroup
    int waves;         // waves per workgroup
    size_t lds;        // dynamic LDS bytes per workgroup
    size_t workspace;  // bytes: tile counters + segment sums when wgs_per_tile > 1
};
// mf_min_rows: the threshold of the kernel that runs the plan (it decides
// whether the MFMA form's LDS scratch is reserved).
GemvPlan gemv_plan(int64_t m, int64_t n, int64_t k, int mf_min_rows = GEMV_MF_MIN_ROWS);
size_t gemv_workspace_bytes(int64_t m, int64_t n, int64_t k);

hipError_t launch_gemv(const void *x_q, int64_t m, const void *w, int layout, int64_t n, int64_t k, float *y,
                       int64_t ld_y, void *workspace, hipStream_t s);

// GEMV from fp32 activations, quantized inside the kernel (m <= 8).
hipError_t launch_gemv_f32(const float *x, int64_t ld_x, int64_t m, const void *w, int layout, int64_t n, int64_t k,
                           float *y, int64_t ld_y, void *workspace, hipStream_t s);

// A sequence of fused-quantization GEMVs in one persistent launch (packed
// weights, m <= 8 rows each, step p + 1 reading its activations only after
// step p is complete).
constexpr int SEQ_MAX_STEPS = 72;
struct SeqHostStep {
    const float *x;
    const void *w;
    float *y;
    int64_t ld_x, ld_y, n, k;
};
// Host plan of a sequence launch: kernel variant, dynamic LDS, workspace size
// and layout (flag lines, each split step's counters and sums), and each
// step's split of its tiles over workgroups.
struct SeqPlan {
    bool one;          // every unit has at most one group per wave
    size_t lds;        // dynamic LDS bytes per workgroup
    size_t workspace;  // bytes
    int32_t flag_off;  // byte offset of the flag lines
    uint32_t ws_off[SEQ_MAX_STEPS];  // split step's counters and sums at 256 * ws_off (0: none)
    uint16_t wgs[SEQ_MAX_STEPS];     // workgroups per tile
    uint16_t segs[SEQ_MAX_STEPS];    // segments per workgroup
};
void seq_plan(const SeqHostStep *steps, int count, int64_t m, SeqPlan &plan);
size_t gemv_sequence_workspace_bytes(const SeqHostStep *steps, int count, int64_t m);
hipError_t launch_gemv_sequence(const SeqHostStep *steps, int count, int64_t m, void *workspace, hipStream_t s);
// The same with the library's own per-GPU scratch array as the workspace
// (zeroed at the start of the call); copies the status word to *status when
// status is not NULL.
hipError_t launch_gemv_sequence_scratch(const SeqHostStep *steps, int count, int64_t m, int32_t *status,
                                        hipStream_t s);

// Residual add + RMSNorm + quantization to Q8_LAYOUT_ACT (k <= 16384).
constexpr int64_t NORM_MAX_K = 16384;
hipError_t launch_rmsnorm_quantize(const float *x, const float *res_in, float *res_out, const float *w,
                                   int64_t rows, int64_t k, float eps, void *q_out, hipStream_t s);

// Around the routed experts: router, SwiGLU + quantization, weighted combine.
constexpr int ROUTE_MAX_EXPERTS = 1024;
constexpr int ROUTE_MAX_TOPK = 32;
hipError_t launch_moe_route(const float *logits, int64_t tokens, int64_t n_experts, int topk, int normalize,
                            int32_t *ids, float *weights, hipStream_t s);
hipError_t launch_swiglu_quantize(const float *gate, int64_t ld_gate, const float *up, int64_t ld_up, int64_t rows,
                                  int64_t n, void *q_out, hipStream_t s);
hipError_t launch_moe_combine(const float *y, int64_t ld_y, const float *w, int64_t tokens, int topk, int64_t n,
                              float *out, int64_t ld_out, hipStream_t s);

// Q8 KV cache: fused norm + rope + cache write; decode attention.
hipError_t launch_kv_write(const float *qkv, int64_t tokens, int n_heads, int n_kv, int head_dim,
                           const int32_t *positions, int64_t max_pos, const float *cos_tab, const float *sin_tab,
                           const float *q_gain, const float *k_gain, float eps, const int32_t *slots, int64_t n_slots,
                           float *q_out, int8_t *k_cache, float *k_scale, int8_t *v_cache, float *v_scale,
                           int32_t *status, hipStream_t s);
constexpr int64_t ATT_MAX_LEN = 65536;  // cached positions per sequence
size_t attention_workspace_bytes(int64_t seqs, int n_heads, int n_kv, int head_dim, int64_t max_len);
hipError_t launch_attention_decode(const float *q, int64_t seqs, int n_heads, int n_kv, int head_dim,
                                   const int8_t *k_cache, const float *k_scale, const int8_t *v_cache,
                                   const float *v_scale, int64_t n_slots, const int32_t *base, const int32_t *len,
                                   int64_t max_len, float scale, float *out, void *ws, hipStream_t s);

hipError_t launch_gemm(const void *x_q, int64_t m, const void *w, int64_t n, int64_t k, float *y, int64_t ld_y,
                       hipStream_t s);

size_t grouped_workspace_bytes(int64_t tokens, int topk, int64_t n_experts);
hipError_t launch_grouped(const void *x_q, int64_t x_rows, int x_per_pair, const int32_t *ids, int64_t tokens,
                          int topk, const void *w, int64_t n_experts, int64_t expert_stride, int64_t n, int64_t k,
                          float *y, void *workspace, hipStream_t s);

// Measurement only: a plain streaming read of `bytes` (a multiple of 16)
// that XORs the XOR of all its 32-bit words into *sink.
hipError_t launch_stream_read(const void *buf, size_t bytes, uint32_t *sink, hipStream_t s);

}  // namespace q8k
