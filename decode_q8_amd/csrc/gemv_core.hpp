// Device code of the GEMV shared by the per-matrix kernel (gemv.hip) and the
// persistent sequence kernel (gemv_seq.hip): one lane's group of weights, the
// group sums (int8 or fp32 activations), the walk over a row's groups and one
// workgroup's share of a 64-row tile with its fixed-order chain.
#pragma once

#include "device.hpp"

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
        for (int i = 0; i < 16; i++) g.c[i] = load_nt(p + i * 1024);
        g.c[16] = load_nt(p + RECORD_Q_BYTES);
    } else {  // rows: p = this row's 272 bytes of the group (8 blocks of 34 bytes)
        // plain loads: a lane reads each 128-byte line in eight 16-byte loads,
        // and with the non-temporal hint the line is given up between them
        // (measured: the decode step's GEMVs took twice as long)
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

// Round half away from zero of an fp32 q with |q| < 2^23: q + copysign(0.5 -
// 2^-25, q), truncated.  Equal to (int)roundf(q) for every such q (checked
// exhaustively on the host for |q| <= 128): the offset just below one half
// keeps 0.5 - 2^-25 itself from rounding up to 1, and at an exact half the
// sum n + 1 - 2^-25 still rounds (to nearest even) to n + 1.
__device__ __forceinline__ int round_half_away(float q) { return (int)(q + __builtin_copysignf(0x1.fffffep-2f, q)); }

// Lane l's block scale d = amax / 127 (amax over the block of the 8 aligned
// lanes l & ~7, by an exact max butterfly) and its four codes x / d, rounded
// half away from zero (0 when d == 0), packed low byte first.  When every
// lane's amax lies in [2^-89, 2^96] (a wave-uniform test):
//  - d is amax * y with y = RN(1/127), corrected once by its exact fma
//    residual: with the correctly rounded reciprocal, one correction gives the
//    correctly rounded quotient (Markstein's theorem; checked on the host for
//    every fp32 significand);
//  - the four quotients x / d share one reciprocal of d refined by a
//    Newton-Raphson step, each corrected twice by its exact fma residual:
//    exactly the operations of the compiler's correctly rounded fp32 division
//    without its range-scaling steps, and for d in [2^-96, 2^89] those steps
//    change nothing whenever the quotient can round to a nonzero code (they act
//    only on a zero or very small numerator or a subnormal quotient, where both
//    paths give code 0).
// So d and the codes equal amax / 127 and (int)roundf(x / d).  Otherwise the
// whole wave takes the IEEE divisions.
// quantize_rows4 does this for M activation rows at once (row m's values in
// v[m]) with one range test over all of them, so the rows' dependency chains
// have no branch between them and interleave; any row out of range sends all
// M rows to the IEEE divisions, which give the same codes and scales where
// the fast path applies.
template <int M>
__device__ __forceinline__ void quantize_rows4(const float4 (&v)[M], uint32_t (&q_out)[M], float (&d_out)[M]) {
    float amax[M];
    bool out_of_range = false;
#pragma unroll
    for (int m = 0; m < M; m++) {
        amax[m] = max_over_8_lanes(fmaxf(fmaxf(fabsf(v[m].x), fabsf(v[m].y)), fmaxf(fabsf(v[m].z), fabsf(v[m].w))));
        out_of_range |= !(amax[m] >= 0x1p-89f && amax[m] <= 0x1p96f);
    }
    int q[M][4];
    if (__builtin_amdgcn_ballot_w64(out_of_range) == 0) {
        constexpr float y = 1.0f / 127.0f;
#pragma unroll
        for (int m = 0; m < M; m++) {
            const float qd = amax[m] * y;
            const float d = fmaf(fmaf(-127.0f, qd, amax[m]), y, qd);
            const float r0 = __builtin_amdgcn_rcpf(d);
            const float r = fmaf(fmaf(-d, r0, 1.0f), r0, r0);
            auto quot = [d, r](float x) {
                const float qa = x * r;
                const float qb = fmaf(fmaf(-d, qa, x), r, qa);
                return fmaf(fmaf(-d, qb, x), r, qb);
            };
            q[m][0] = round_half_away(quot(v[m].x));
            q[m][1] = round_half_away(quot(v[m].y));
            q[m][2] = round_half_away(quot(v[m].z));
            q[m][3] = round_half_away(quot(v[m].w));
            d_out[m] = d;
        }
    } else {
#pragma unroll
        for (int m = 0; m < M; m++) {
            const float d = amax[m] / 127.0f;
            q[m][0] = q[m][1] = q[m][2] = q[m][3] = 0;
            if (d != 0.0f) {
                q[m][0] = (int)roundf(v[m].x / d);
                q[m][1] = (int)roundf(v[m].y / d);
                q[m][2] = (int)roundf(v[m].z / d);
                q[m][3] = (int)roundf(v[m].w / d);
            }
            d_out[m] = d;
        }
    }
#pragma unroll
    for (int m = 0; m < M; m++)  // low bytes of q0, q1 into bytes 0, 1 and of q2, q3 into bytes 2, 3 (v_perm_b32)
        q_out[m] = __builtin_amdgcn_perm((uint32_t)q[m][1], (uint32_t)q[m][0], 0x0c0c0400u) |
                   __builtin_amdgcn_perm((uint32_t)q[m][3], (uint32_t)q[m][2], 0x04000c0cu);
}

// The wave's 64 packed code dwords (dword l in lane l) copied into every
// 16-lane row: x16[i] holds dwords 16 i .. 16 i + 15 in lanes 16 r .. 16 r +
// 15 of each row r, so an operand with DPP row_newbcast:j reads dword 16 i +
// j in all 64 lanes.  One 32-lane swap gives [r0 r1 r0 r1] and [r2 r3 r2 r3]
// (rows of 16 dwords), a 16-lane swap of each with itself the four copies.
// Needs every lane active.
__device__ __forceinline__ void replicate_rows(uint32_t qd, uint32_t (&x16)[4]) {
    const auto h = __builtin_amdgcn_permlane32_swap(qd, qd, false, false);
    const auto lo = __builtin_amdgcn_permlane16_swap(h[0], h[0], false, false);
    const auto hi = __builtin_amdgcn_permlane16_swap(h[1], h[1], false, false);
    x16[0] = lo[0];
    x16[1] = lo[1];
    x16[2] = hi[0];
    x16[3] = hi[1];
}

// The block terms t0 = fp32(s0) * (Dw0 * Dx0) and t1 of blocks 2i and 2i + 1:
// s0, s1 are their int8 dots with the activation codes in x = x16[i]
// (dwords 0..7 of each row are block 2i, 8..15 block 2i + 1; weight chunks
// a0, a1 and b0, b1), each code dword broadcast by DPP straight into
// v_dot4c, the two chains interleaved; Dx comes by DPP from dx8, which holds
// block j's activation scale in lane j of every row.  The compiler does not
// see inside the asm, so it keeps its own wait states: the two moves give a
// DPP read of x 2 after its last VALU write, and the two multiplies plus a
// convert put 3 between each dot chain's last write and the convert that
// reads it (a dot result read too early by another VALU instruction is stale
// on this chip family).
__device__ __forceinline__ void block_pair_terms(float &t0, float &t1, uint32_t x, float dx8, float dw0, float dw1,
                                                 int i, const uint4 &a0, const uint4 &a1, const uint4 &b0,
                                                 const uint4 &b1) {
    int s0, s1;
    float p0, p1;
#define Q8_PAIR_ASM(BC0, BC1)                                                                           \
    asm("v_mov_b32 %2, 0\n\t"                                                                          \
        "v_mov_b32 %3, 0\n\t"                                                                          \
        "v_dot4c_i32_i8_dpp %2, %6, %10 row_newbcast:0 row_mask:0xf bank_mask:0xf\n\t"                 \
        "v_dot4c_i32_i8_dpp %3, %6, %18 row_newbcast:8 row_mask:0xf bank_mask:0xf\n\t"                 \
        "v_dot4c_i32_i8_dpp %2, %6, %11 row_newbcast:1 row_mask:0xf bank_mask:0xf\n\t"                 \
        "v_dot4c_i32_i8_dpp %3, %6, %19 row_newbcast:9 row_mask:0xf bank_mask:0xf\n\t"                 \
        "v_dot4c_i32_i8_dpp %2, %6, %12 row_newbcast:2 row_mask:0xf bank_mask:0xf\n\t"                 \
        "v_dot4c_i32_i8_dpp %3, %6, %20 row_newbcast:10 row_mask:0xf bank_mask:0xf\n\t"                \
        "v_dot4c_i32_i8_dpp %2, %6, %13 row_newbcast:3 row_mask:0xf bank_mask:0xf\n\t"                 \
        "v_dot4c_i32_i8_dpp %3, %6, %21 row_newbcast:11 row_mask:0xf bank_mask:0xf\n\t"                \
        "v_dot4c_i32_i8_dpp %2, %6, %14 row_newbcast:4 row_mask:0xf bank_mask:0xf\n\t"                 \
        "v_dot4c_i32_i8_dpp %3, %6, %22 row_newbcast:12 row_mask:0xf bank_mask:0xf\n\t"                \
        "v_dot4c_i32_i8_dpp %2, %6, %15 row_newbcast:5 row_mask:0xf bank_mask:0xf\n\t"                 \
        "v_dot4c_i32_i8_dpp %3, %6, %23 row_newbcast:13 row_mask:0xf bank_mask:0xf\n\t"                \
        "v_dot4c_i32_i8_dpp %2, %6, %16 row_newbcast:6 row_mask:0xf bank_mask:0xf\n\t"                 \
        "v_dot4c_i32_i8_dpp %3, %6, %24 row_newbcast:14 row_mask:0xf bank_mask:0xf\n\t"                \
        "v_dot4c_i32_i8_dpp %2, %6, %17 row_newbcast:7 row_mask:0xf bank_mask:0xf\n\t"                 \
        "v_dot4c_i32_i8_dpp %3, %6, %25 row_newbcast:15 row_mask:0xf bank_mask:0xf\n\t"                \
        "v_mul_f32_dpp %4, %7, %8 row_newbcast:" #BC0 " row_mask:0xf bank_mask:0xf\n\t"                 \
        "v_mul_f32_dpp %5, %7, %9 row_newbcast:" #BC1 " row_mask:0xf bank_mask:0xf\n\t"                 \
        "v_cvt_f32_i32 %0, %2\n\t"                                                                     \
        "v_cvt_f32_i32 %1, %3\n\t"                                                                     \
        "v_mul_f32 %0, %0, %4\n\t"                                                                     \
        "v_mul_f32 %1, %1, %5"                                                                         \
        : "=&v"(t0), "=&v"(t1), "=&v"(s0), "=&v"(s1), "=&v"(p0), "=&v"(p1)                             \
        : "v"(x), "v"(dx8), "v"(dw0), "v"(dw1), "v"(a0.x), "v"(a0.y), "v"(a0.z), "v"(a0.w), "v"(a1.x),  \
          "v"(a1.y), "v"(a1.z), "v"(a1.w), "v"(b0.x), "v"(b0.y), "v"(b0.z), "v"(b0.w), "v"(b1.x),       \
          "v"(b1.y), "v"(b1.z), "v"(b1.w))
    switch (i) {
        case 0: Q8_PAIR_ASM(0, 1); break;
        case 1: Q8_PAIR_ASM(2, 3); break;
        case 2: Q8_PAIR_ASM(4, 5); break;
        default: Q8_PAIR_ASM(6, 7); break;
    }
#undef Q8_PAIR_ASM
}

// Group sums with the activation quantization fused in: xv[m] holds lane l's
// values 4l..4l+3 of the group's 256 fp32 values of row m (loaded by the
// caller ahead of the weights, so the quantization does not wait for them).
// Lane l quantizes values 4l..4l+3 (block l / 8) with exactly the arithmetic
// of the standalone quantizer (bit-identical codes and scales, see
// quantize_rows4).  The packed codes are copied into every 16-lane row and fed to
// v_dot4c by DPP broadcast, and so are the blocks' activation scales to the
// multiplies of the block terms.
constexpr int JOINT_QUANT_MAX_ROWS = 3;

template <int M>
__device__ __forceinline__ void group_sums_f32(const GroupRegs &g, const float4 (&xv)[M], float (&u)[M]) {
    float dw[8];
#pragma unroll
    for (int bb = 0; bb < 8; bb++) dw[bb] = half_bits_to_float(half_of(g.c[16], bb));
    // the rows' quantizations together (their chains interleave) where the
    // registers allow it (m = 2 / 3 decode step 334 -> 330 / 378.5 -> 371 us);
    // with 4 rows under the lane form's 128-register cap that spilled more and
    // was slower (457 -> 470 us), so there each row is quantized right before
    // its dots
    constexpr int MQ = M <= JOINT_QUANT_MAX_ROWS ? M : 1;
    uint32_t qm[M];
    float dm[M];
    if constexpr (MQ == M) quantize_rows4<M>(xv, qm, dm);
#pragma unroll
    for (int m = 0; m < M; m++) {
        if constexpr (MQ != M) {
            const float4 v1[1] = {xv[m]};
            uint32_t q1[1];
            float d1[1];
            quantize_rows4<1>(v1, q1, d1);
            qm[m] = q1[0];
            dm[m] = d1[0];
        }
        uint32_t x16[4];
        replicate_rows(qm[m], x16);
        const float dxl = half_bits_to_float(float_to_half_bits(dm[m]));
        // lane j of every row gets block (j & 7)'s scale, held by lane 8 (j & 7)
        const float dx8 = __builtin_bit_cast(
            float, __builtin_amdgcn_ds_bpermute(32 * (int)(threadIdx.x & 7), __builtin_bit_cast(int, dxl)));
        float t[8];
#pragma unroll
        for (int i = 0; i < 4; i++)
            block_pair_terms(t[2 * i], t[2 * i + 1], x16[i], dx8, dw[2 * i], dw[2 * i + 1], i, g.c[4 * i],
                             g.c[4 * i + 1], g.c[4 * i + 2], g.c[4 * i + 3]);
        u[m] = tree8(t);
    }
}

// Walk groups g0, g0 + step, ... (< g1) of one lane's row.  TO_LDS = true:
// store each group sum u_g at lds[((g - g0) * M + m) * 64 + lane] (the caller
// points lds at group g0's slot; slots of M x 64 floats hold consecutive
// groups); the workgroup chains them later.  TO_LDS = false (step 1, g0 = 0):
// the wave owns groups [0, G) of its row and chains in registers in the
// canonical two-level order.  wbase/gstride: address of group 0 of this lane
// and the step between groups in memory.
// hooks.before() runs before the first group's weight loads are issued;
// hooks() runs after they are issued and before any activation is read;
// hooks.after() runs once the first activation loads are issued (work that may
// overlap them).  Every wave calls all three, also a wave without a group, so
// hooks() may contain a workgroup barrier.
template <int M, int LAYOUT, bool TO_LDS, typename ACT, bool ONE, typename Wait>
__device__ __forceinline__ void row_groups(const uint8_t *wbase, int64_t gstride, int g0, int g1, int step,
                                           const ACT *const (&xrow)[M], const uint16_t *const (&srow)[M],
                                           float (&acc)[M], float *lds, int lane, Wait &&hooks) {
    // ONE: the caller guarantees at most one group (g0 + step >= g1), so no
    // second register buffer is allocated (17 VGPRs x 4 fewer per lane, more
    // waves per SIMD to keep loads in flight).
    GroupRegs cur;
    GroupRegs nxt;
    float seg[M];
    constexpr bool F32 = sizeof(ACT) == 4;
    float4 xv[M], xn[M];
    const bool any = g0 < g1;
    hooks.before();
    if (any) load_group<LAYOUT>(cur, wbase + g0 * gstride);
    hooks();
    if constexpr (F32) {
        if (any) {
#pragma unroll
            for (int m = 0; m < M; m++) xv[m] = *reinterpret_cast<const float4 *>(xrow[m] + g0 * GROUP_K + 4 * lane);
        }
    }
    hooks.after();
    if (!any) return;
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

// ---------------------------------------------------------------------------
// MFMA form of a group, for 2..8 activation rows and packed weights.  The
// block dots of all M activation rows with the tile's 64 weight rows come from
// v_mfma_i32_32x32x32_i8 (one instruction = one block for 32 weight rows; the
// activation rows sit on the instruction's other 32-row side, padded), so the
// VALU no longer broadcasts every activation code to every lane.  Each output
// keeps exactly the arithmetic of the lane-per-row form -- s exact, t =
// fp32(s) * (Dw * Dx) with Dw * Dx exact, the tree over the group's 8 blocks
// -- so its bits do not depend on which form computed it (rows stay
// bit-identical to m = 1).
// Register form: lane l holds, for block bb and weight-row half th, the 16
// values 16 * (l / 32) .. + 15 of block bb of weight row 32 * th + l % 32 (the
// instruction's B operand), and the scale chunks of rows l % 32 and
// 32 + l % 32.  Output: lane l holds weight row 32 * th + l % 32 for the
// activation rows 4 * (l / 32) + p, p = 0..3 (instruction registers 0..3).
// ---------------------------------------------------------------------------
struct GroupRegsMF {
    uint4 c[18];
};

__device__ __forceinline__ void load_group_mf(GroupRegsMF &g, const uint8_t *rec, int lane) {
    const uint8_t *p = rec + (lane >> 5) * 1024 + (lane & 31) * 16;
#pragma unroll
    for (int bb = 0; bb < GROUP_BLOCKS; bb++)
#pragma unroll
        for (int th = 0; th < 2; th++) g.c[2 * bb + th] = load_nt(p + bb * 2048 + th * 512);
#pragma unroll
    for (int th = 0; th < 2; th++)
        g.c[16 + th] = load_nt(rec + RECORD_Q_BYTES + (32 * th + (lane & 31)) * 16);
}

// Per-wave LDS scratch of the MFMA form: the M rows' packed codes as the lanes
// quantized them ([m][64] dwords) and the activation scales ([block][8]
// floats, Dx of row m at [bb * 8 + m]).
template <int M>
struct MfScratch {
    static constexpr int DWORDS = M * 64 + GROUP_BLOCKS * 8;
};

// u[th][p] = the group sum of weight row 32 * th + lane % 32 with activation
// row 4 * (lane / 32) + p (meaningful for rows < M).  src.a(bb) gives the A
// operand of block bb (16 activation codes of row lane % 32, values
// 16 * (lane / 32) ..) and src.dx(bb, d) the activation scales of rows
// 4 * (lane / 32) + p; they are fetched block by block so that few registers
// are live.  The tree over the group's blocks is built as the blocks arrive,
// with the association of tree8.
template <int M, typename Src>
__device__ __forceinline__ void group_sums_mf(const GroupRegsMF &g, const Src &src, float (&u)[2][4]) {
    // Block by block: the block's A operand and activation scales are fetched
    // one block ahead, its two MFMAs (weight rows 0..31 and 32..63) issued
    // together, and the epilogue pinned in place, so that few registers are
    // live (left alone, the compiler issues all 16 MFMAs first and keeps every
    // result register).  Only the activation rows a lane half can hold are
    // computed: rows 4 * (lane / 32) + p, p < min(M, 4).
    constexpr int P = M < 4 ? M : 4;
    const v16i zi = {0};
    float x0[2][P], p01[2][P], x2[2][P], q03[2][P], x4[2][P], p45[2][P], x6[2][P];
    v4i a_cur = src.a(0), a_nxt = a_cur;
    float dx_cur[4], dx_nxt[4];
    src.dx(0, dx_cur);
#pragma unroll
    for (int bb = 0; bb < GROUP_BLOCKS; bb++) {
        if (bb + 1 < GROUP_BLOCKS) {
            a_nxt = src.a(bb + 1);
            src.dx(bb + 1, dx_nxt);
        }
        v16i sv[2];
#pragma unroll
        for (int th = 0; th < 2; th++)
            sv[th] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a_cur, __builtin_bit_cast(v4i, g.c[2 * bb + th]), zi, 0, 0, 0);
#pragma unroll
        for (int th = 0; th < 2; th++) {
            const float dw = half_bits_to_float(half_of(g.c[16 + th], bb));
#pragma unroll
            for (int p = 0; p < P; p++) {
                const float t = (float)sv[th][p] * (dw * dx_cur[p]);  // Dw * Dx exact: one rounding
                float *pin;
                switch (bb) {  // ((t0 + t1) + (t2 + t3)) + ((t4 + t5) + (t6 + t7))
                    case 0: x0[th][p] = t; pin = &x0[th][p]; break;
                    case 1: p01[th][p] = x0[th][p] + t; pin = &p01[th][p]; break;
                    case 2: x2[th][p] = t; pin = &x2[th][p]; break;
                    case 3: q03[th][p] = p01[th][p] + (x2[th][p] + t); pin = &q03[th][p]; break;
                    case 4: x4[th][p] = t; pin = &x4[th][p]; break;
                    case 5: p45[th][p] = x4[th][p] + t; pin = &p45[th][p]; break;
                    case 6: x6[th][p] = t; pin = &x6[th][p]; break;
                    default: u[th][p] = q03[th][p] + (p45[th][p] + (x6[th][p] + t)); pin = &u[th][p]; break;
                }
                asm volatile("" : "+v"(*pin) :: "memory");
            }
        }
        a_cur = a_nxt;
#pragma unroll
        for (int p = 0; p < 4; p++) dx_cur[p] = dx_nxt[p];
    }
}

// Operands of the fp32 path: the wave's scratch, filled by quantize_group.
template <int M>
struct ScratchOperands {
    const uint32_t *scr;
    int lane;
    __device__ __forceinline__ v4i a(int bb) const {
        const int mm = (lane & 31) < M ? (lane & 31) : M - 1;
        return *reinterpret_cast<const v4i *>(scr + mm * 64 + 8 * bb + 4 * (lane >> 5));
    }
    __device__ __forceinline__ void dx(int bb, float (&d)[4]) const {
        const float4 d4 = *reinterpret_cast<const float4 *>(scr + M * 64 + bb * 8 + 4 * (lane >> 5));
        d[0] = d4.x;
        d[1] = d4.y;
        d[2] = d4.z;
        d[3] = d4.w;
    }
};

// The lanes' quantization of a group of M fp32 activation rows (xv[m]: lane
// l's values 4l..4l+3, exactly the arithmetic of group_sums_f32) into the
// wave's scratch: packed codes of row m at [m * 64 + l], the fp32 value of
// each block's stored fp16 scale at [M * 64 + bb * 8 + m].
template <int M>
__device__ __forceinline__ void quantize_group(const float4 (&xv)[M], uint32_t *scr, int lane) {
    // every lane has read the previous group's operands before they are overwritten
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    float *sdx = reinterpret_cast<float *>(scr + M * 64);
    uint32_t qm[M];
    float dm[M];
    quantize_rows4<M>(xv, qm, dm);
#pragma unroll
    for (int m = 0; m < M; m++) {
        scr[m * 64 + lane] = qm[m];
        if ((lane & 7) == 0) sdx[(lane >> 3) * 8 + m] = half_bits_to_float(float_to_half_bits(dm[m]));
    }
    // the wave's own LDS writes complete before its lanes read each other's
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}

// Operands of the int8 path (Q8_LAYOUT_ACT already quantized): codes of row
// min(lane % 32, M - 1) straight from memory; the scale chunks of rows
// 4 * (lane / 32) + p (clamped to M - 1) loaded once per group.
template <int M>
struct ActOperands {
    const int8_t *xr;  // this lane's activation row at the group, + 16 * (lane / 32)
    uint4 sc[4];
    __device__ __forceinline__ void init(const int8_t *x0, int64_t ld_x, const uint16_t *s0, int64_t nb, int g,
                                         int lane) {
        const int mm = (lane & 31) < M ? (lane & 31) : M - 1;
        xr = x0 + mm * ld_x + g * GROUP_K + 16 * (lane >> 5);
#pragma unroll
        for (int p = 0; p < 4; p++) {
            int r = 4 * (lane >> 5) + p;
            r = r < M ? r : M - 1;
            sc[p] = *reinterpret_cast<const uint4 *>(s0 + r * nb + g * GROUP_BLOCKS);
        }
    }
    __device__ __forceinline__ v4i a(int bb) const { return *reinterpret_cast<const v4i *>(xr + bb * QK); }
    __device__ __forceinline__ void dx(int bb, float (&d)[4]) const {
#pragma unroll
        for (int p = 0; p < 4; p++) d[p] = half_bits_to_float(half_of(sc[p], bb));
    }
};

// row_groups for the MFMA form (packed weights, group sums to LDS): groups
// g0, g0 + step, ... (< g1) of the tile whose record 0 is at rec0; each
// group's sums go to lds[((g - g0) * M + m) * 64 + row].  xf (fp32 rows, ACT =
// float) or xq / xs (int8 rows and scales) give the activations; scr is the
// wave's MfScratch.  Hooks as in row_groups.
template <int M, typename ACT, bool ONE, typename Wait>
__device__ __forceinline__ void row_groups_mf(const uint8_t *rec0, int g0, int g1, int step, const ACT *x0,
                                              int64_t ld_x, const uint16_t *xs0, int64_t nb, float *lds,
                                              uint32_t *scr, int lane, Wait &&hooks) {
    constexpr bool F32 = sizeof(ACT) == 4;
    GroupRegsMF cur, nxt;
    float4 xv[M], xn[M];
    const bool any = g0 < g1;
    hooks.before();
    if (any) load_group_mf(cur, rec0 + (int64_t)g0 * RECORD_BYTES, lane);
    hooks();
    if constexpr (F32) {
        if (any) {
#pragma unroll
            for (int m = 0; m < M; m++)
                xv[m] = *reinterpret_cast<const float4 *>(x0 + m * ld_x + g0 * GROUP_K + 4 * lane);
        }
    }
    hooks.after();
    if (!any) return;
    for (int g = g0; g < g1; g += step) {
        if (!ONE && g + step < g1) {
            if constexpr (F32) {
#pragma unroll
                for (int m = 0; m < M; m++)
                    xn[m] = *reinterpret_cast<const float4 *>(x0 + m * ld_x + (g + step) * GROUP_K + 4 * lane);
            }
            load_group_mf(nxt, rec0 + (int64_t)(g + step) * RECORD_BYTES, lane);
        }
        float u[2][4];
        if constexpr (F32) {
            quantize_group<M>(xv, scr, lane);
            group_sums_mf<M>(cur, ScratchOperands<M>{scr, lane}, u);
        } else {
            ActOperands<M> src;
            src.init((const int8_t *)x0, ld_x, xs0, nb, g, lane);
            group_sums_mf<M>(cur, src, u);
        }
#pragma unroll
        for (int th = 0; th < 2; th++)
#pragma unroll
            for (int p = 0; p < (M < 4 ? M : 4); p++) {
                const int m = 4 * (lane >> 5) + p;
                if (m < M) lds[((g - g0) * M + m) * TILE_ROWS + 32 * th + (lane & 31)] = u[th][p];
            }
        if (ONE) break;
        cur = nxt;
        if constexpr (F32) {
#pragma unroll
            for (int m = 0; m < M; m++) xv[m] = xn[m];
        }
    }
}

struct NoWait {
    __device__ void before() const {}
    __device__ void operator()() const {}
    __device__ void after() const {}
};

// One workgroup's share of one 64-row tile: segments [wi * segs_per_wg, ...)
// of tile T.  A tile's groups are split into segments of 8 (2048 values); the
// workgroup's W waves take its groups round-robin (wave w: groups w, w + W,
// ...) and leave every group sum in LDS.  After a barrier each (row, m) is
// chained in the canonical order:
//   S_j = ((u_8j + u_8j+1) + ...) + u_8j+7   within segment j,
//   y   = ((S_0 + S_1) + S_2) + ...          over the segments.
// When one workgroup covers the whole tile (wgs_per_tile == 1) it writes y.
// Otherwise (narrow matrices with long rows, where one workgroup per tile
// would leave most CUs idle) each workgroup hands its segment sums to the
// workspace and counts in at its tile's counter; the workgroup that arrives
// last chains all segment sums and writes y, then clears the counter (so
// counters that start at zero stay zero).  Cross-workgroup visibility without
// cache-wide fences: segment sums are written and read back with
// read-modify-write atomics (exchange in; exchange with 0 out -- an idempotent
// RMW would be lowered to a plain atomic load, which can hit a stale line of a
// non-coherent L2), performed at the device-coherent point like the counter;
// every thread waits for its exchanges before the barrier that precedes the
// counter increment, and the last workgroup reads only after that increment
// returned the final count.  handover = true skips the counter: the
// workgroup only leaves its segment sums (complete when it returns) for a
// later finish_split (the sequence kernel's next step chains them).  Every
// thread of the workgroup calls this (it contains barriers); lds_u holds
// [groups of the workgroup][M][64] floats, followed by the waves' MFMA-form
// scratch when M >= MF_MIN (packed weights take the MFMA form from MF_MIN
// activation rows on: the choice changes speed only, never bits).  Workspace: uint32 counters [tiles]
// (256-byte aligned), then fp32 segment sums [S][M][n].
template <int M, int LAYOUT, typename ACT, bool ONE, int MF_MIN, typename Wait>
__device__ __forceinline__ void tile_unit(const ACT *__restrict__ xq, int64_t ld_x, const uint16_t *__restrict__ xs,
                                          const uint8_t *__restrict__ w, int64_t n, int64_t k, float *__restrict__ y,
                                          int64_t ld_y, int64_t T, int wi, int wgs_per_tile, int segs_per_wg,
                                          uint32_t *__restrict__ ctr, float *__restrict__ part, float *lds_u,
                                          int *last_wg, bool handover, Wait &&hooks) {
    // fetched now and kept in registers: in the sequence they come from the
    // kernel-argument array, and a late scalar load would sit right before
    // the output store
    asm volatile("" : "+s"(y), "+s"(ld_y));
    typedef __attribute__((address_space(1))) float global_float;
    global_float *const yg = (global_float *)y;  // global stores (a flat store would also count as an LDS access)
    const int lane = threadIdx.x & 63;
    const int wv = wave_id();
    const int W = blockDim.x >> 6;
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
    // wave wv takes the workgroup's groups ga + wv, ga + wv + W, ...; each sum lands in its group's LDS slot
    if constexpr (M >= MF_MIN && LAYOUT == 1) {
        // MFMA form; the waves' scratch follows the group slots (the plan's
        // LDS holds min(segs_per_wg * 8, G) slots of M x 64 floats)
        const int slots = segs_per_wg * SEG_GROUPS < G ? segs_per_wg * SEG_GROUPS : G;
        uint32_t *scr = reinterpret_cast<uint32_t *>(lds_u + slots * M * TILE_ROWS) + wv * MfScratch<M>::DWORDS;
        row_groups_mf<M, ACT, ONE>(w + T * G * RECORD_BYTES, ga + wv, gb, W, xq, ld_x, xs, k / QK,
                                   lds_u + wv * M * TILE_ROWS, scr, lane, hooks);
    } else {
        float unused[M];
        row_groups<M, LAYOUT, true, ACT, ONE>(wbase, gstride, ga + wv, gb, W, xrow, srow, unused,
                                              lds_u + wv * M * TILE_ROWS, lane, hooks);
    }
    __syncthreads();

    const int t = threadIdx.x;  // the plan gives at least M waves: one thread per (m, row)
    const bool chain_thread = t < M * TILE_ROWS;
    const int cm = t >> 6, cr = t & 63;
    const int64_t out_row = T * TILE_ROWS + cr;
    const bool out_ok = chain_thread && out_row < n;
    float acc = 0.0f;
    if (chain_thread) {
        for (int sj = s0; sj < s1; sj++) {
            const int gs = sj * SEG_GROUPS, cnt = min(G - gs, SEG_GROUPS);  // groups in the segment, >= 1
            const float *src = lds_u + ((gs - ga) * M + cm) * TILE_ROWS + cr;
            float v[SEG_GROUPS];  // the segment's group sums, all LDS reads in flight at once
            float sv;
            if (cnt == SEG_GROUPS) {  // a whole segment: no per-group tests
#pragma unroll
                for (int j = 0; j < SEG_GROUPS; j++) v[j] = src[j * M * TILE_ROWS];
                sv = v[0];
#pragma unroll
                for (int j = 1; j < SEG_GROUPS; j++) sv += v[j];
            } else {
#pragma unroll
                for (int j = 0; j < SEG_GROUPS; j++) v[j] = j < cnt ? src[j * M * TILE_ROWS] : 0.0f;
                sv = v[0];
#pragma unroll
                for (int j = 1; j < SEG_GROUPS; j++)
                    if (j < cnt) sv += v[j];
            }
            if (wgs_per_tile == 1) {
                acc = sj == 0 ? sv : acc + sv;
            } else if (out_ok) {
                __hip_atomic_exchange((uint32_t *)&part[((int64_t)sj * M + cm) * n + out_row], __builtin_bit_cast(uint32_t, sv),
                                      __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
    }
    if (wgs_per_tile == 1) {
        if (out_ok) yg[cm * ld_y + out_row] = acc;
        return;
    }
    __builtin_amdgcn_s_waitcnt(0);  // this thread's exchanges have completed
    if (handover) return;
    __syncthreads();
    if (t == 0) {
        const uint32_t old = __hip_atomic_fetch_add(&ctr[T], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        *last_wg = old == (uint32_t)(wgs_per_tile - 1);
    }
    __syncthreads();
    if (!*last_wg) return;
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
        yg[cm * ld_y + out_row] = acc;
    }
    if (t == 0) __hip_atomic_exchange(&ctr[T], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}


// Chains the handed-over segment sums of tiles T = first, first + stride, ...
// (< tiles) of a split GEMV and writes their outputs: output (m, row) is
// ((S_0 + S_1) + S_2) + ..., exactly the chain of tile_unit's last
// workgroup.  The sums are read with exchanges (returning them to zero) at
// the device-coherent point where the handing-over workgroups left them.
// Any number of threads may call this; each takes whole outputs.
template <int M>
__device__ __forceinline__ void finish_split(float *__restrict__ part, float *__restrict__ y, int64_t ld_y, int n,
                                             int S, int first, int stride) {
    const int tiles = n / TILE_ROWS;
    for (int T = first; T < tiles; T += stride) {
        for (int i = threadIdx.x; i < M * TILE_ROWS; i += blockDim.x) {
            const int cm = i / TILE_ROWS, row = T * TILE_ROWS + i % TILE_ROWS;
            float acc = 0.0f;
            uint32_t *pp = (uint32_t *)&part[(int64_t)cm * n + row];
            const int64_t seg_stride = (int64_t)M * n;  // between consecutive segments' sums
            for (int b0 = 0; b0 < S; b0 += 4) {
                float v[4];  // four exchanges in flight (registers are scarce here), then the in-order chain
#pragma unroll
                for (int j = 0; j < 4; j++)
                    v[j] = b0 + j < S ? __builtin_bit_cast(float, __hip_atomic_exchange(pp + (b0 + j) * seg_stride, 0u,
                                                                                      __ATOMIC_RELAXED,
                                                                                      __HIP_MEMORY_SCOPE_AGENT))
                                      : 0.0f;
#pragma unroll
                for (int j = 0; j < 4; j++)
                    if (b0 + j < S) acc = (b0 + j == 0) ? v[j] : acc + v[j];
            }
            y[cm * ld_y + row] = acc;
        }
    }
}

}  // namespace q8k
