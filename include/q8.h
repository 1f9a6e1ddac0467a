/*
 * q8.h: C ABI of libq8, the MI355X (gfx950) Q8_0 block-quantized matmul.
 *
 * What is computed (the method of the pages this library implements):
 *  - Q8_0 block: 32 values stored as one fp16 scale followed by 32 int8, 34
 *    bytes ("Ember packed Q8 decode" post, row-contiguous source diagram).
 *  - Quantization of weights and activations alike: per 32-value block,
 *    d = amax / 127 (fp32), q = nearest integer to x / d with ties away from
 *    zero, stored scale = fp16(d) ("ferro" README, "How the iGPU path is
 *    fast", item 1: activations quantized per 32-block; "Using LFM2.5":
 *    weights converted to Q8_0 at load).
 *  - Block dot: s = exact int32 sum of the 32 products, term
 *    t = fp32(s * (Dw * Dx)) (Dw * Dx is exact in fp32, so one rounding).
 *  - Output: the terms of a row summed in fp32 in one fixed order that
 *    depends on k only: groups of 8 consecutive blocks (256 values) are summed
 *    as the tree ((t0+t1)+(t2+t3))+((t4+t5)+(t6+t7)); the group sums of each
 *    segment of 8 consecutive groups (2048 values) are added left to right;
 *    the segment sums are added left to right.  Every entry point that produces
 *    GEMV outputs (m <= 8, and every routed pair) uses exactly this order, so
 *    a row's output is bit-identical alone, in any batch of up to 8 rows, in
 *    any row order, in either weight layout, for any n, and in the routed
 *    expert path (the batch-invariance contract of the "ferro" README,
 *    "Exactness contract").  The prefill GEMM (m > 8) accumulates each group
 *    with fused multiply-adds instead; its rows are bit-identical for any m
 *    and row order, but need not equal the GEMV bitwise ("ferro" README,
 *    "Exactness contract": decode rows and prefill rows take different
 *    kernels).  Any correct fp32 order lies within
 *    |y - exact| <= 1e-5 * sum_b |t_b| of the exact sum.
 *
 * Conventions:
 *  - Every data pointer is a device pointer that the caller allocates and
 *    owns; the library allocates no memory and keeps no state except a
 *    per-device architecture check.
 *  - Every call is asynchronous on the caller's stream (0 = the null
 *    stream).  The returned status covers host-side validation and the
 *    launch only.  Validation happens before any HIP call, so argument
 *    errors are reported without a GPU.
 *  - Pointers must be 16-byte aligned; sizes are in elements unless named
 *    *_bytes.  Unsupported requests fail with a status; there is no
 *    fallback path ("Ferrule" README, "Core features" and "System vision":
 *    missing capabilities and other hardware fail explicitly).
 *  - Calls are stateless and may run concurrently on different streams as
 *    long as their output and workspace buffers do not overlap.
 *
 * Layouts (byte formats):
 *  Q8_LAYOUT_ROWS   row-contiguous Q8_0: rows x (k/32) blocks of
 *                   [fp16 d][32 x int8], 34 bytes each.
 *  Q8_LAYOUT_PACKED weights for gfx950: records of 64 rows x 8 blocks,
 *                   17,408 bytes (= 512 blocks x 34 = 32 x 544: the same
 *                   bytes, reordered; "Ember packed Q8 decode" post: a packed
 *                   record holds exactly the bytes of the blocks it covers).
 *                   Record (T, G) starts at byte (T * (k/256) + G) * 17408;
 *                   inside it, the int8 value of row 64T + r, column
 *                   256G + 32bb + 16h + j is at bb*2048 + h*1024 + r*16 + j
 *                   (so one 16-byte load per lane, 64 lanes = 64 rows, reads
 *                   1 KB contiguous), and the fp16 scale of (row r, block bb)
 *                   is at 16384 + r*16 + bb*2 (one 16-byte load per lane gives
 *                   a row's 8 scales).  Needs n % 64 == 0 and k % 256 == 0.
 *  Q8_LAYOUT_ACT    quantized activations: int8 [rows][k] followed by fp16
 *                   [rows][k/32]; rows * k/32 * 34 bytes in all.
 */
#ifndef DECODE_Q8_AMD_Q8_H
#define DECODE_Q8_AMD_Q8_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define Q8_ABI_VERSION 5u  /* 2: q8_gemv_step and the sequence entry points; 3: q8_rmsnorm_quantize, the
                              MoE router, SwiGLU and combine, and the Q8 KV cache entry points;
                              4: q8_stream_read; 5: q8_device_queries, q8_build_digest,
                              q8_quantize_matmul_sequence_noalloc */
#define Q8_BLOCK 32          /* values per block */
#define Q8_BLOCK_BYTES 34    /* fp16 scale + 32 int8 */
#define Q8_TILE_ROWS 64      /* rows per packed record */
#define Q8_TILE_BLOCKS 8     /* blocks per packed record and per summation group */
#define Q8_RECORD_BYTES 17408
#define Q8_GEMV_MAX_ROWS 8   /* m <= 8 takes the GEMV */

typedef enum {
    Q8_OK = 0,
    Q8_ERR_ARG = 1,       /* null pointer, size <= 0, unknown enum, ld too small  */
    Q8_ERR_SHAPE = 2,     /* k % 32 (quantize), k % 256, n % 64 (packed), ...     */
    Q8_ERR_ALIGN = 3,     /* pointer not 16-byte aligned, fp32 row stride % 4      */
    Q8_ERR_WORKSPACE = 4, /* workspace missing or smaller than required            */
    Q8_ERR_DEVICE = 5,    /* no HIP device, or the current device is not gfx950   */
    Q8_ERR_LAUNCH = 6     /* the kernel launch failed                              */
} q8_status;

typedef enum { Q8_LAYOUT_ROWS = 0, Q8_LAYOUT_PACKED = 1, Q8_LAYOUT_ACT = 2 } q8_layout;

/* Version of this ABI (Q8_ABI_VERSION). */
uint32_t q8_abi_version(void);

/* Number of device-property queries (architecture, CU count, kernel
 * occupancy) the library has made in this process.  Each is made once per
 * device and kernel variant, at its first use, and cached; a caller can check
 * that repeated calls on the token path query nothing ("Ferrule" README,
 * "Core features": the token hot path performs no architecture discovery). */
uint32_t q8_device_queries(void);

/* sha256 (hex) of the sources and compile flags this library was built from
 * (static string, never NULL); the Python binding compares it with the tree
 * it is loaded from and refuses a stale build. */
const char *q8_build_digest(void);

/* Static, human-readable name of a status code (never NULL). */
const char *q8_status_str(int status);

/* Bytes of rows x k values in any of the three layouts: rows * k/32 * 34.
 * Returns 0 if k % 32 != 0 or a size is negative. */
size_t q8_quantized_bytes(int64_t rows, int64_t k);

/* Quantize fp32 rows.
 *  x       device, rows x k fp32, row stride ld_x elements (ld_x >= k,
 *          ld_x % 4 == 0), 16-byte aligned.  Not modified.
 *  layout  Q8_LAYOUT_ROWS (weights, GGUF-style blocks) or Q8_LAYOUT_ACT
 *          (activations for q8_matmul / q8_grouped_matmul).
 *  q_out   device, q8_quantized_bytes(rows, k) bytes, 16-byte aligned; must
 *          not overlap x.
 *  k % 32 == 0; rows == 0 is a no-op.  Quantized values and scales are
 *  bit-identical to the definition above (one wavefront-reduction per block).
 *  Errors: Q8_ERR_ARG, Q8_ERR_SHAPE, Q8_ERR_ALIGN, Q8_ERR_DEVICE, Q8_ERR_LAUNCH. */
int q8_quantize_rows(const float *x, int64_t ld_x, int64_t rows, int64_t k, int layout, void *q_out,
                     hipStream_t stream);

/* Reorder row-contiguous Q8_0 weights (Q8_LAYOUT_ROWS, n x k) into
 * Q8_LAYOUT_PACKED.  A pure byte permutation: the output has the same size,
 * q8_quantized_bytes(n, k).  Needs n % 64 == 0, k % 256 == 0; buffers must
 * not overlap ("Ember packed Q8 decode" post: packing at prepare time).
 *  Errors: Q8_ERR_ARG, Q8_ERR_SHAPE, Q8_ERR_ALIGN, Q8_ERR_DEVICE, Q8_ERR_LAUNCH. */
int q8_repack_weights(const void *w_rows, int64_t n, int64_t k, void *w_packed, hipStream_t stream);

/* Workspace bytes q8_matmul / q8_quantize_matmul need for this shape (0 when
 * none).  Depends on (m, n, k) only.  Narrow matrices with long rows (fewer
 * than 256 row tiles of 64 and k > 2048) spread each tile's 2048-value
 * segments over several workgroups; they need a workspace holding one uint32
 * counter per tile (first 256-byte-aligned part) and the per-segment partial
 * sums.  The counters must be zero before the first
 * call that uses a workspace (allocate it zero-filled); every completed call
 * leaves them zero again, so one workspace serves any sequence of calls on one
 * stream, including replays of a captured graph.  Calls that run concurrently
 * need separate workspaces. */
size_t q8_matmul_workspace_bytes(int64_t m, int64_t n, int64_t k);

/* y[i][j] = sum over blocks of x_q row i against weight row j (the Q8_0
 * block dot product, "ferro" README, "How the iGPU path is fast", item 1).
 *  x_q     device, Q8_LAYOUT_ACT, m rows of k.
 *  w       device, n x k weights in Q8_LAYOUT_PACKED (n % 64 == 0) or
 *          Q8_LAYOUT_ROWS (any n; only for m <= 8).
 *  y       device fp32, m x n with row stride ld_y >= n (elements).
 *  workspace, workspace_bytes: device scratch of at least
 *          q8_matmul_workspace_bytes(m, n, k) (may be NULL when that is 0),
 *          counters zero as described above; must not overlap y.
 *  Routing is by m alone: m <= 8 runs the GEMV, m > 8 the MFMA GEMM.
 *  k % 256 == 0.
 *  Errors: Q8_ERR_ARG, Q8_ERR_SHAPE, Q8_ERR_ALIGN, Q8_ERR_WORKSPACE,
 *  Q8_ERR_DEVICE, Q8_ERR_LAUNCH. */
int q8_matmul(const void *x_q, int64_t m, const void *w, int layout, int64_t n, int64_t k, float *y,
              int64_t ld_y, void *workspace, size_t workspace_bytes, hipStream_t stream);

/* Decode GEMV straight from fp32 activations: each of the m <= 8 rows of x is
 * quantized inside the GEMV kernel with exactly the arithmetic of
 * q8_quantize_rows (bit-identical codes and scales), then multiplied as
 * q8_matmul does; the output is bit-identical to q8_quantize_rows(...,
 * Q8_LAYOUT_ACT, ...) followed by q8_matmul.  One launch instead of two
 * ("ferro" README, "How the iGPU path is fast", item 3: producers emit the
 * next GEMM's int8 input directly).  Each 64-row tile quantizes the
 * activation groups it reads, so the codes are never written to memory.
 *  x       device fp32, m x k, row stride ld_x (ld_x >= k, ld_x % 4 == 0),
 *          16-byte aligned.
 *  w, layout, n, k, y, ld_y, workspace: as for q8_matmul (1 <= m <= 8).
 *  Errors: Q8_ERR_ARG, Q8_ERR_SHAPE, Q8_ERR_ALIGN, Q8_ERR_WORKSPACE,
 *  Q8_ERR_DEVICE, Q8_ERR_LAUNCH. */
int q8_quantize_matmul(const float *x, int64_t ld_x, int64_t m, const void *w, int layout, int64_t n, int64_t k,
                       float *y, int64_t ld_y, void *workspace, size_t workspace_bytes, hipStream_t stream);

/* One GEMV of a sequence: y = q8_quantize_matmul(x, ld_x, m, w,
 * Q8_LAYOUT_PACKED, n, k, y, ld_y) with the sequence's m. */
typedef struct {
    const float *x; /* device fp32, m x k, row stride ld_x (ld_x >= k, ld_x % 4 == 0), 16-byte aligned */
    const void *w;  /* device, n x k weights in Q8_LAYOUT_PACKED, 16-byte aligned */
    float *y;       /* device fp32, m x n, row stride ld_y >= n, 16-byte aligned */
    int64_t ld_x, ld_y, n, k;
} q8_gemv_step;

#define Q8_SEQUENCE_MAX_STEPS 72

/* Workspace bytes q8_quantize_matmul_sequence needs for these steps (0 if the
 * arguments are invalid).  Depends on the shapes and m only. */
size_t q8_sequence_workspace_bytes(const q8_gemv_step *steps, int count, int64_t m);

/* A chain of decode GEMVs in one persistent launch (launch amortization of a
 * decode step: one launch instead of one per matrix; the "ferro" README,
 * "Using LFM2.5", attributes the decode time beyond weight streaming to some
 * 70 small-kernel launches per token).  Step i's output is bit-identical to q8_quantize_matmul on step i
 * alone.  Steps run in order: step i + 1 reads its activations only after
 * every output of step i is complete (the dependency of consecutive layers;
 * its weight loads may start earlier, since weights do not depend on
 * activations).  A step's x must be ready before the call: no step's y may
 * overlap any step's x, and the y's must not overlap each other.
 *  steps     host array of count descriptors (read during the call only),
 *            1 <= count <= Q8_SEQUENCE_MAX_STEPS, each with n % 64 == 0 and
 *            k % 256 == 0; 1 <= m <= 8 for all steps.
 *  workspace device, >= q8_sequence_workspace_bytes(steps, count, m) bytes,
 *            zero-filled before its first use; every completed call leaves
 *            it zero, so one workspace serves any sequence of calls on one
 *            stream (graph replays included).  Calls that run concurrently
 *            need separate workspaces.  Its int32 word at byte 0 is the
 *            call's status: 0, or Q8_ERR_LAUNCH if one of the internal waits
 *            timed out (possible only when other work occupies the GPU so
 *            that not all of the call's workgroups are resident at once).
 *            After a non-zero status the outputs of that call are undefined
 *            and the workspace must be zero-filled again before reuse.
 *  Aliasing: no y may overlap any step's x (so step i + 1 cannot read step
 *  i's y in place: copy it, or give each step its own input), the y's must
 *  be disjoint, and the workspace must overlap no x or y; violations return
 *  Q8_ERR_ARG.
 *  Errors: Q8_ERR_ARG, Q8_ERR_SHAPE, Q8_ERR_ALIGN, Q8_ERR_WORKSPACE,
 *  Q8_ERR_DEVICE, Q8_ERR_LAUNCH. */
int q8_quantize_matmul_sequence(const q8_gemv_step *steps, int count, int64_t m, void *workspace,
                                size_t workspace_bytes, hipStream_t stream);

#define Q8_SEQUENCE_SCRATCH_BYTES (8ll << 20)  /* the allocation-free variant's workspace per GPU */

/* q8_quantize_matmul_sequence without a caller workspace, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation): the workspace is the library's
 * own device array of Q8_SEQUENCE_SCRATCH_BYTES per GPU, held until the
 * process ends; no call allocates or frees memory.  Outputs are bit-identical
 * to q8_quantize_matmul_sequence with the same steps.
 *  steps, count, m  as for q8_quantize_matmul_sequence, and the same aliasing
 *            rules; q8_sequence_workspace_bytes(steps, count, m) must not
 *            exceed Q8_SEQUENCE_SCRATCH_BYTES (else Q8_ERR_WORKSPACE, before
 *            any HIP call).  The Llama-3.2-1B-shaped decode step needs about
 *            1.0 MB at m = 1 and 4.6 MB at m = 8.
 *  status    device int32 or NULL: receives the call's status word (0, or
 *            Q8_ERR_LAUNCH if an internal wait timed out, which leaves the
 *            outputs undefined) when the call completes.  4-byte aligned,
 *            outside every x and y.
 * The part of the array a call uses is zeroed at the start of every call (by
 * a kernel, so the call can be captured in a graph).  Every call on one GPU
 * uses that GPU's one array: calls that overlap in time on one GPU (other
 * streams, other threads) race and must be serialized by the caller.
 *  Errors: Q8_ERR_ARG, Q8_ERR_SHAPE, Q8_ERR_ALIGN, Q8_ERR_WORKSPACE,
 *  Q8_ERR_DEVICE, Q8_ERR_LAUNCH. */
int q8_quantize_matmul_sequence_noalloc(const q8_gemv_step *steps, int count, int64_t m, int32_t *status,
                                        hipStream_t stream);

/* Fused producer of a GEMM input: residual add + RMSNorm + quantization of
 * each row to Q8_LAYOUT_ACT in one pass ("ferro" README, "How the iGPU path
 * is fast", item 3: residual add, norm and int8 quantization fused, the
 * producer emitting the next matmul's int8 input).  The pages name the fusion
 * but not the norm; this is Llama's RMSNorm, per row:
 *   h_j = fp32(residual_in_j + x_j)   (h_j = x_j when residual_in is NULL)
 *   ss  = sum_j (double)h_j^2 (each square exact in fp64), the exact sum
 *         rounded to fp64; the library sums the squares in fp64 in one fixed
 *         order (512 partials over 4-value chunks, then a halving tree),
 *         which is within k * 2^-52 (relative) of that exactly rounded sum
 *   r   = fp32(1 / sqrt(ss / k + eps)), each fp64 operation correctly rounded
 *   r   = fp32(1 / sqrt(ss / k + eps)), each fp64 operation correctly rounded
 *   n_j = fp32(fp32(h_j * r) * weight_j)
 * then n is quantized per 32-value block exactly as q8_quantize_rows does.
 * Codes, scales and h are deterministic (bit-identical for any rows count);
 * they equal the exactly rounded definition's unless 1 / sqrt(ss / k + eps)
 * lies within that fp64 margin of an fp32 rounding boundary.
 *  x            device fp32 [rows][k] (row stride k), 16-byte aligned.
 *  residual_in  device fp32 [rows][k] or NULL (a norm without residual add).
 *  residual_out device fp32 [rows][k] receiving h, or NULL; may be the same
 *               buffer as x or residual_in (in-place update of the residual
 *               stream), otherwise must not overlap them.
 *  weight       device fp32 [k], the norm's per-channel gain.
 *  eps          >= 0 and finite.
 *  q_out        device, q8_quantized_bytes(rows, k) bytes (Q8_LAYOUT_ACT, the
 *               input of q8_matmul); must not overlap the other buffers.
 *  k % 32 == 0, k <= 16384; 0 <= rows <= 2^31 - 1 (rows == 0: no launch).
 *  Errors: Q8_ERR_ARG, Q8_ERR_SHAPE, Q8_ERR_ALIGN, Q8_ERR_DEVICE,
 *  Q8_ERR_LAUNCH. */
int q8_rmsnorm_quantize(const float *x, const float *residual_in, float *residual_out, const float *weight,
                        int64_t rows, int64_t k, float eps, void *q_out, hipStream_t stream);

/* Workspace bytes q8_grouped_matmul needs. */
size_t q8_grouped_workspace_bytes(int64_t tokens, int topk, int64_t n_experts, int64_t n, int64_t k);

/* Routed-expert matmul (the expert GEMVs of a mixture-of-experts layer;
 * "Ferrule" README, routed-expert roofline: each selected expert's weights
 * are streamed once per pass).  For token t and slot j (pair p = t*topk + j):
 *   y[p][:] = GEMV of activation row (x_per_pair ? p : t) with expert
 *             topk_ids[t][j]'s weights,
 * bit-identical to q8_matmul with m = 1 on that row and that expert.
 * Pairs are grouped by expert on the device (stable in p), each active
 * expert's weights are streamed once per 8 pairs.
 *  x_q        device, Q8_LAYOUT_ACT with x_rows rows of k
 *             (x_rows == tokens, or tokens*topk when x_per_pair).
 *  topk_ids   device int32 [tokens][topk].
 *  w_experts  device, expert e in Q8_LAYOUT_PACKED (n x k) at byte
 *             e * expert_stride_bytes (expert_stride_bytes >=
 *             q8_quantized_bytes(n, k), multiple of 16).
 *  y          device fp32 [tokens*topk][n].
 *  workspace  device, >= q8_grouped_workspace_bytes(...); its first 4 bytes
 *             receive an int32 status after the call completes: 0, or
 *             Q8_ERR_ARG if some id was outside [0, n_experts) (those pairs'
 *             outputs are left unwritten).
 *  n % 64 == 0, k % 256 == 0, tokens*topk <= 65536, topk <= n_experts <= 1024.
 *  Errors: Q8_ERR_ARG, Q8_ERR_SHAPE, Q8_ERR_ALIGN, Q8_ERR_WORKSPACE,
 *  Q8_ERR_DEVICE, Q8_ERR_LAUNCH. */
int q8_grouped_matmul(const void *x_q, int64_t x_rows, int x_per_pair, const int32_t *topk_ids, int64_t tokens,
                      int topk, const void *w_experts, int64_t n_experts, int64_t expert_stride_bytes, int64_t n,
                      int64_t k, float *y, void *workspace, size_t workspace_bytes, hipStream_t stream);

/* ---- The steps either side of the routed-expert GEMVs ("Ferrule" README:
 * device routing; the real router decides expert ids and weights; a sparse-MoE
 * execution path).  A mixture-of-experts layer on a token batch is
 *   q8_moe_route -> q8_grouped_matmul (gate||up, x_per_pair = 0)
 *   -> q8_swiglu_quantize -> q8_grouped_matmul (down, x_per_pair = 1)
 *   -> q8_moe_combine.
 * The pages give no formulas; these are Mixtral/DeepSeek/OLMoE-style readings.
 * Wherever a result is an integer or is reproduced bit for bit (expert ids,
 * weights, SwiGLU codes), e^x (x <= 0) is one fixed fp64 algorithm of
 * correctly rounded basic operations:
 *   k = rint(x * fp64(1/ln 2)), r = (x - k*C1) - k*C2 (C1 = ln 2 truncated to
 *   a multiple of 2^-32, C2 = fp64(ln 2 - C1)), p = Horner sum of r^i / i!
 *   for i = 13..0 with coefficients fp64(1/i!), one multiply and one add per
 *   step; e^x = ldexp(p, k); x < -745.5 gives +0. */

#define Q8_ROUTE_MAX_EXPERTS 1024
#define Q8_ROUTE_MAX_TOPK 32

/* Router: top-k experts per token and their weights.
 *  logits   device fp32 [tokens][n_experts] (finite values; NaN is outside
 *           the contract), 4-byte aligned.
 *  ids      device int32 [tokens][topk]: the k largest logits, ties to the
 *           lower expert id, slots in descending logit order.
 *  weights  device fp32 [tokens][topk]: with m the largest logit and
 *           e_i = exp((double)l_i - m):
 *             normalize != 0: w_j = fp32(e_j / D), D = sum of the selected
 *               e (softmax over the selected experts);
 *             normalize == 0: D = sum over all experts (softmax over all
 *               experts, selected ones kept).
 *           D is defined as the exact sum rounded to fp64.  The library adds
 *           the selected e in slot order, and all experts as 64 partials
 *           (experts l, l + 64, ... ascending) folded P_l += P_{l+s},
 *           s = 32..1: within a few fp64 ulps of the exact sum, so w_j equals
 *           the definition's unless e_j / D lies that close to an fp32
 *           rounding boundary.
 *  1 <= topk <= min(n_experts, 32), n_experts <= 1024, tokens >= 0.
 *  Errors: Q8_ERR_ARG, Q8_ERR_SHAPE, Q8_ERR_ALIGN, Q8_ERR_DEVICE, Q8_ERR_LAUNCH. */
int q8_moe_route(const float *logits, int64_t tokens, int64_t n_experts, int topk, int normalize, int32_t *ids,
                 float *weights, hipStream_t stream);

/* SwiGLU between the gate/up and the down GEMVs, quantized for the down GEMV:
 *   s = g / (1 + e^-g) evaluated in fp64 as (e = exp(-|g|))
 *       g >= 0 ? g / (1 + e) : (g * e) / (1 + e),
 *   h = fp32(s * (double)u), quantized per 32-value block as
 *   q8_quantize_rows does, into Q8_LAYOUT_ACT.
 *  gate, up  device fp32 [rows][n], row strides ld_gate, ld_up (>= n, % 4),
 *            16-byte aligned (gate and up may be the two halves of one
 *            fused gate||up output row).
 *  q_out     device, q8_quantized_bytes(rows, n), 16-byte aligned, no overlap.
 *  n % 32 == 0; rows == 0 is a no-op.
 *  Errors: Q8_ERR_ARG, Q8_ERR_SHAPE, Q8_ERR_ALIGN, Q8_ERR_DEVICE, Q8_ERR_LAUNCH. */
int q8_swiglu_quantize(const float *gate, int64_t ld_gate, const float *up, int64_t ld_up, int64_t rows, int64_t n,
                       void *q_out, hipStream_t stream);

/* Weighted combine of the routed outputs:
 *   out[t][c] = sum_j weights[t][j] * y[t*topk + j][c]
 * in fp32, j ascending, each product and each sum rounded (so within
 * 2 * topk * 2^-24 * sum_j |w y| of the exact value).
 *  y        device fp32 [tokens*topk][n], row stride ld_y.
 *  weights  device fp32 [tokens][topk].
 *  out      device fp32 [tokens][n], row stride ld_out; must not overlap y.
 *  n % 4 == 0, ld_y and ld_out >= n and % 4 == 0, y and out 16-byte aligned.
 *  Errors: Q8_ERR_ARG, Q8_ERR_SHAPE, Q8_ERR_ALIGN, Q8_ERR_DEVICE, Q8_ERR_LAUNCH. */
int q8_moe_combine(const float *y, int64_t ld_y, const float *weights, int64_t tokens, int topk, int64_t n, float *out,
                   int64_t ld_out, hipStream_t stream);

/* ---- Q8 KV cache ("ferro" README, "KV cache": K/V rows stored as int8 with
 * one fp32 scale per 32 values, quantized in the fused norm + rope +
 * cache-write kernel, dequantized inside attention).  Cache layout, head-major
 * so that one head's positions are contiguous:
 *   k_cache, v_cache  int8 [n_kv][n_slots][head_dim]
 *   k_scale, v_scale  fp32 [n_kv][n_slots][head_dim / 32]
 * A block of 32 values x is stored as d = fp32(amax / 127) (kept in fp32) and
 * q = round(x / d) (ties away from zero; d = 0 gives q = 0). */

/* Fused per-head norm + rotary embedding + KV cache write for `tokens` rows
 * of a fused QKV projection.
 *  qkv        device fp32 [tokens][(n_heads + 2 n_kv) head_dim]: n_heads
 *             query heads, then n_kv key heads, then n_kv value heads.
 *  positions  device int32 [tokens], each in [0, max_pos).
 *  cos_tab, sin_tab  device fp32 [max_pos][head_dim / 2] (model constants).
 *  q_gain, k_gain    device fp32 [head_dim] or NULL: per-head RMSNorm of the
 *             query / key heads before the rotation (ss = sum of the exact
 *             fp64 squares x^2 rounded to fp64 -- the library adds them as
 *             head_dim/4 partials of 4 consecutive values folded
 *             p_c += p_{c+s} for s = head_dim/8 .. 1, within a few fp64 ulps
 *             of that; r = fp32(1 / sqrt(ss / head_dim + eps));
 *             x = fp32(fp32(x * r) * gain)).
 *  rotation   half-split: for i < head_dim/2 with c, s = tables[pos][i]:
 *             x_i <- fp32(fp32(x_i c) - fp32(x_{i+h} s)),
 *             x_{i+h} <- fp32(fp32(x_{i+h} c) + fp32(x_i s)),  h = head_dim/2.
 *  slots      device int32 [tokens], each in [0, n_slots): the cache slot of
 *             every head of that token.
 *  q_out      device fp32 [tokens][n_heads][head_dim]: normalized, rotated q.
 *  status     device int32 or NULL: set to Q8_ERR_ARG (never cleared) if a
 *             position or slot is out of range; that token is not written.
 *  head_dim in {64, 128, 256}; n_heads % n_kv == 0; all fp32 and int8 arrays
 *  16-byte aligned except the scales (4-byte).  tokens == 0 is a no-op.
 *  Errors: Q8_ERR_ARG, Q8_ERR_SHAPE, Q8_ERR_ALIGN, Q8_ERR_DEVICE, Q8_ERR_LAUNCH. */
int q8_kv_write(const float *qkv, int64_t tokens, int n_heads, int n_kv, int head_dim, const int32_t *positions,
                int64_t max_pos, const float *cos_tab, const float *sin_tab, const float *q_gain, const float *k_gain,
                float eps, const int32_t *slots, int64_t n_slots, float *q_out, int8_t *k_cache, float *k_scale,
                int8_t *v_cache, float *v_scale, int32_t *status, hipStream_t stream);

#define Q8_ATTENTION_MAX_LEN 65536  /* cached positions per sequence */

/* Workspace bytes of q8_attention_decode (0 if the arguments are invalid). */
size_t q8_attention_workspace_bytes(int64_t seqs, int n_heads, int n_kv, int head_dim, int64_t max_len);

/* Decode attention over the Q8 KV cache: one query row per sequence.  For
 * query head h (kv head h / (n_heads / n_kv)) of sequence s, the keys and
 * values of positions j < len[s] sit at slot base[s] + j:
 *   s_j = scale * q . k_j,  out = sum_j e^(s_j - max) v_j / sum_j e^(s_j - max)
 * with k, v dequantized (code * block scale).  Cached positions are taken in
 * fixed chunks of 256, so a sequence's result depends only on its own data
 * (bit-identical whatever the other sequences of the batch).
 *  q          device fp32 [seqs][n_heads][head_dim] (q8_kv_write's q_out).
 *  base, len  device int32 [seqs]: 1 <= len <= max_len, base >= 0,
 *             base + len <= n_slots; a sequence violating this gets NaN
 *             outputs and the status word set.
 *  out        device fp32 [seqs][n_heads][head_dim].
 *  workspace  device, >= q8_attention_workspace_bytes(...), 16-byte aligned;
 *             its first int32 is the call's status (0, or Q8_ERR_ARG).
 *  head_dim in {64, 128}; n_heads / n_kv in {1, 2, 4, 8};
 *  max_len <= Q8_ATTENTION_MAX_LEN; seqs and n_kv <= 65535.
 *  Errors: Q8_ERR_ARG, Q8_ERR_SHAPE, Q8_ERR_ALIGN, Q8_ERR_WORKSPACE,
 *  Q8_ERR_DEVICE, Q8_ERR_LAUNCH. */
int q8_attention_decode(const float *q, int64_t seqs, int n_heads, int n_kv, int head_dim, const int8_t *k_cache,
                        const float *k_scale, const int8_t *v_cache, const float *v_scale, int64_t n_slots,
                        const int32_t *base, const int32_t *len, int64_t max_len, float scale, float *out,
                        void *workspace, size_t workspace_bytes, hipStream_t stream);

/* ---- Measurement: the streaming-read ceiling ("ferro" README, "Using LFM2.5
 * language models": decode weight streaming is reported as a fraction of what
 * a pure streaming-read kernel reaches on the same device). ---- */

/* Reads every byte of buf once, in coalesced 16-byte loads, and XORs the XOR
 * of all its 32-bit words into *sink (so *sink = 0 before the call leaves the
 * buffer's XOR checksum there).  Its only purpose is to time the device's
 * streaming-read bandwidth; it computes nothing the matmuls use.
 *  buf   device, 16-byte aligned, bytes a multiple of 16 (0: no-op).
 *  sink  device uint32, 4-byte aligned, outside buf.
 *  Errors: Q8_ERR_ARG, Q8_ERR_SHAPE, Q8_ERR_ALIGN, Q8_ERR_DEVICE, Q8_ERR_LAUNCH. */
int q8_stream_read(const void *buf, size_t bytes, uint32_t *sink, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif
