// Q8 KV cache ("ferro" README, "KV cache": K/V rows stored as int8 with one
// fp32 scale per 32 values, quantized in the fused norm + rope + cache-write
// kernel and dequantized inside attention).
//
// kv_write_kernel: for each token and head of a fused QKV row, HD/4 lanes hold
// the head (4 values each).  Optional per-head RMSNorm (fp64 sum of squares:
// one partial per lane over its 4 values in order, then a halving fold over
// the lanes), rotary embedding in the half-split layout from caller tables
// (the partner value i +- HD/2 is HD/8 lanes away), then K and V heads are
// quantized per 32 values (8 lanes, 3-step butterfly for the amax) with the
// scale kept in fp32, into a head-major cache [kv head][slot][HD].
//
// attn_partial_kernel / attn_combine_kernel: decode attention (one query row
// per sequence) in fixed chunks of 256 cached positions, so the arithmetic of
// a sequence depends only on its own length.  A workgroup takes one chunk of
// one (sequence, kv head) for the G query heads sharing that kv head: each of
// its 4 waves scores 64 keys (lane = key: the key row is dequantized once and
// dotted with the G queries read as scalars), takes its own softmax in the
// exp2 domain, then turns its lanes to dimensions and accumulates p * v over
// its keys from a wave-local LDS tile; only then do the 4 waves meet, and
// their sums are rescaled to the chunk maximum and added in order.  The
// combine kernel rescales the chunks' (max, sum, weighted sum) and divides,
// chunks in order.
#include <math.h>

#include "device.hpp"
#include "launch.hpp"

namespace q8k {

typedef __attribute__((address_space(3))) void *lds_ptr;

// ---------------------------------------------------------------------------
// Fused norm + rope + cache write
// ---------------------------------------------------------------------------

template <int HD>
__global__ __launch_bounds__(256) void kv_write_kernel(const float *__restrict__ qkv, int32_t tokens, int32_t n_heads,
                                                       int32_t n_kv, const int32_t *__restrict__ positions,
                                                       int32_t max_pos, const float *__restrict__ cos_tab,
                                                       const float *__restrict__ sin_tab,
                                                       const float *__restrict__ q_gain,
                                                       const float *__restrict__ k_gain, float eps,
                                                       const int32_t *__restrict__ slots, int64_t n_slots,
                                                       float *__restrict__ q_out, int8_t *__restrict__ k_cache,
                                                       float *__restrict__ k_scale, int8_t *__restrict__ v_cache,
                                                       float *__restrict__ v_scale, int32_t *__restrict__ status) {
    constexpr int LPH = HD / 4;  // lanes per head (16, 32 or 64: heads never straddle waves)
    constexpr int NB = HD / 32;
    const int heads = n_heads + 2 * n_kv;
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t grp = gid / LPH;
    const int l = (int)(gid % LPH);
    bool valid = grp < (int64_t)tokens * heads;
    const int t = valid ? (int)(grp / heads) : 0;
    const int h = valid ? (int)(grp % heads) : 0;
    const int kind = h < n_heads ? 0 : (h < n_heads + n_kv ? 1 : 2);  // q, k, v
    int pos = 0;
    int64_t slot = 0;
    if (valid) {
        pos = positions[t];
        slot = slots[t];
        if (pos < 0 || pos >= max_pos || slot < 0 || slot >= n_slots) {
            if (status && l == 0) __hip_atomic_store(status, 1 /* Q8_ERR_ARG */, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT);
            valid = false;
        }
    }
    float x[4] = {0.f, 0.f, 0.f, 0.f};
    if (valid) {
        const float4 v = *reinterpret_cast<const float4 *>(qkv + ((int64_t)t * heads + h) * HD + 4 * l);
        x[0] = v.x;
        x[1] = v.y;
        x[2] = v.z;
        x[3] = v.w;
    }
    // per-head RMSNorm (every lane joins the shuffles; applied where a gain is given)
    const float *gain = kind == 0 ? q_gain : (kind == 1 ? k_gain : nullptr);
    double p = (double)x[0] * (double)x[0];
    p += (double)x[1] * (double)x[1];
    p += (double)x[2] * (double)x[2];
    p += (double)x[3] * (double)x[3];
#pragma unroll
    for (int s = LPH / 2; s >= 1; s >>= 1) p += __shfl_down(p, s, LPH);
    const double ss = __shfl(p, 0, LPH);
    if (valid && gain) {
        const float r = (float)(1.0 / sqrt(ss / (double)HD + (double)eps));
        const float4 g = *reinterpret_cast<const float4 *>(gain + 4 * l);
        const float gg[4] = {g.x, g.y, g.z, g.w};
#pragma unroll
        for (int e = 0; e < 4; e++) {
            const float xr = x[e] * r;
            x[e] = xr * gg[e];
        }
    }
    // rotary embedding of q and k: lane l < LPH/2 holds x_i, its partner x_{i+HD/2}
    float y[4];
#pragma unroll
    for (int e = 0; e < 4; e++) y[e] = __shfl_xor(x[e], LPH / 2, LPH);
    if (valid && kind != 2) {
        const bool lo = l < LPH / 2;
        const int i0 = 4 * (lo ? l : l - LPH / 2);
        const float4 c4 = *reinterpret_cast<const float4 *>(cos_tab + (int64_t)pos * (HD / 2) + i0);
        const float4 s4 = *reinterpret_cast<const float4 *>(sin_tab + (int64_t)pos * (HD / 2) + i0);
        const float cc[4] = {c4.x, c4.y, c4.z, c4.w}, sn[4] = {s4.x, s4.y, s4.z, s4.w};
#pragma unroll
        for (int e = 0; e < 4; e++) {
            if (lo) {  // x_i = a, partner b = x_{i+h}
                const float ac = x[e] * cc[e], bs = y[e] * sn[e];
                x[e] = ac - bs;
            } else {   // x_{i+h} = b, partner a = x_i
                const float bc = x[e] * cc[e], as = y[e] * sn[e];
                x[e] = bc + as;
            }
        }
    }
    // quantize K and V per 32 values (8 lanes), scale kept in fp32
    float amax = fmaxf(fmaxf(fabsf(x[0]), fabsf(x[1])), fmaxf(fabsf(x[2]), fabsf(x[3])));
    amax = fmaxf(amax, __shfl_xor(amax, 1));
    amax = fmaxf(amax, __shfl_xor(amax, 2));
    amax = fmaxf(amax, __shfl_xor(amax, 4));
    if (!valid) return;
    if (kind == 0) {
        *reinterpret_cast<float4 *>(q_out + ((int64_t)t * n_heads + h) * HD + 4 * l) =
            make_float4(x[0], x[1], x[2], x[3]);
        return;
    }
    const float d = amax / 127.0f;
    uint32_t packed = 0u;
#pragma unroll
    for (int e = 0; e < 4; e++) {
        int qv = 0;
        if (d != 0.0f) qv = (int)roundf(x[e] / d);
        packed |= ((uint32_t)qv & 0xffu) << (8 * e);
    }
    const int kvh = kind == 1 ? h - n_heads : h - n_heads - n_kv;
    const int64_t row = (int64_t)kvh * n_slots + slot;
    int8_t *cache = kind == 1 ? k_cache : v_cache;
    float *scale = kind == 1 ? k_scale : v_scale;
    *reinterpret_cast<uint32_t *>(cache + row * HD + 4 * l) = packed;
    if ((l & 7) == 0) scale[row * NB + (l >> 3)] = d;
}

// ---------------------------------------------------------------------------
// Decode attention
// ---------------------------------------------------------------------------


// Wave-wide max / sum through DPP lane moves (quad swaps, half-row and row
// mirrors, row broadcasts 15 and 31; lane 63 ends with the result, read back
// as a scalar): a fixed order of operations, and no LDS round trips.
template <bool SUM>
__device__ __forceinline__ float wave_reduce_f32(float x) {
#define Q8_DPPF(ctrl, rows)                                                                                        \
    {                                                                                                              \
        const float y = __builtin_bit_cast(                                                                        \
            float, __builtin_amdgcn_update_dpp(SUM ? 0 : __builtin_bit_cast(int, -INFINITY),                        \
                                               __builtin_bit_cast(int, x), ctrl, rows, 0xf, false));               \
        x = SUM ? x + y : fmaxf(x, y);                                                                             \
    }
    Q8_DPPF(0xb1, 0xf);   // quad_perm [1, 0, 3, 2]
    Q8_DPPF(0x4e, 0xf);   // quad_perm [2, 3, 0, 1]
    Q8_DPPF(0x141, 0xf);  // row_half_mirror
    Q8_DPPF(0x140, 0xf);  // row_mirror
    Q8_DPPF(0x142, 0xa);  // row_bcast:15 into rows 1 and 3
    Q8_DPPF(0x143, 0xc);  // row_bcast:31 into rows 2 and 3
#undef Q8_DPPF
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 63));
}

__device__ __forceinline__ float wave_max_f32(float x) { return wave_reduce_f32<false>(x); }
__device__ __forceinline__ float wave_sum_f32(float x) { return wave_reduce_f32<true>(x); }

__device__ __forceinline__ float byte_f32(uint32_t w, int i) {
    return (float)((int32_t)(w << (24 - 8 * i)) >> 24);  // sign-extended int8 -> exact fp32
}

// A sequence's cached range is usable: 1 <= len <= max_len, inside the cache.
__device__ __forceinline__ bool seq_ok(int32_t b, int32_t L, int32_t max_len, int64_t n_slots) {
    return L >= 1 && L <= max_len && b >= 0 && (int64_t)b + L <= n_slots;
}

// Partial results per (sequence, kv head, chunk): for each of the G heads the
// chunk maximum (log2 domain), the chunk sum of p and the HD weighted sums.
template <int HD, int G>
__global__ __launch_bounds__(256) void attn_partial_kernel(const float *__restrict__ q, int32_t n_heads,
                                                           int32_t n_kv, const int8_t *__restrict__ k_cache,
                                                           const float *__restrict__ k_scale,
                                                           const int8_t *__restrict__ v_cache,
                                                           const float *__restrict__ v_scale, int64_t n_slots,
                                                           const int32_t *__restrict__ base,
                                                           const int32_t *__restrict__ len, int32_t max_len,
                                                           float scale_log2, float *__restrict__ part,
                                                           int32_t *__restrict__ status) {
    constexpr int NB = HD / 32;
    constexpr int W16 = HD / 16;  // 16-byte words per cached row
    constexpr int DPL = HD / 64;  // dimensions per lane in the weighted sum
    // per wave one tile: its 64 keys' K rows (XOR-swizzled 16-byte chunks),
    // then, once the lanes hold their K rows, its V rows, then its G x HD
    // weighted sums (G <= 16); likewise one array for the block scales
    // ([block][key]: K's, then V's); and the softmax weights [key][G].  Sharing
    // the tiles keeps a workgroup at 22 KB of LDS for HD = 64 (7 workgroups
    // per CU instead of 4 with separate K and V tiles).
    __shared__ __align__(16) int8_t kv[4][64 * HD];
    static_assert(G * HD * 4 <= 64 * HD, "the weighted sums fit in the wave's tile");
    __shared__ float ksv[4][NB][64];
    __shared__ float pls[4][64][G];
    __shared__ float redm[4][G], reds[4][G];
    const int sp = blockIdx.x, kvh = blockIdx.y, s = blockIdx.z;
    const int splits = gridDim.x;
    if ((sp | kvh | s) == 0 && threadIdx.x == 0)  // the status word of this call starts clear
        __hip_atomic_store(status, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int32_t L = len[s], b0 = base[s];
    if (!seq_ok(b0, L, max_len, n_slots)) return;  // the combine kernel reports it
    const int c0 = sp * ATT_CHUNK;
    if (c0 >= L) return;  // the whole workgroup: this chunk is past the sequence
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;

    // the G query rows: the same for every lane, read with scalar loads
    const float *qg = q + ((int64_t)s * n_heads + (int64_t)kvh * G) * HD;

    // this wave's keys: rows r0 .. r0 + nv - 1 of the head's cache (nv >= 1 for
    // wave 0; a wave past the end loads row r0 - 1 .. and masks everything)
    const int kw = c0 + 64 * w;                        // first key of the wave
    const int nv = min(max(L - kw, 0), 64);            // valid keys
    const int64_t r0 = (int64_t)kvh * n_slots + b0 + (nv > 0 ? kw : L - 1);
    const int last = nv > 0 ? nv - 1 : 0;
    const bool valid = lane < nv;
    // coalesced direct-to-LDS loads: each instruction moves 1 KB of whole rows
    // (rows past the valid ones repeat the last valid row: in bounds, masked).
    // All four carry the non-temporal hint (the cache is read once per call):
    // a decode step's attention 498 -> 461 us; on the code loads alone 466.
    // K and its scales first; V and its scales are issued once the lanes hold
    // their K rows, so they arrive while the scores are computed.
#pragma unroll
    for (int t = 0; t < W16; t++) {
        const int p16 = 64 * t + lane;                 // 16-byte position in the tile
        const int r = p16 / W16, slot = p16 % W16;
        const int chunk = slot ^ (r & (W16 - 1));      // the K row chunk stored at this slot
        __builtin_amdgcn_global_load_lds(k_cache + (r0 + min(r, last)) * HD + chunk * 16,
                                         (lds_ptr)(&kv[w][0] + 1024 * t), 16, 0, CPOL_NT);
    }
#pragma unroll
    for (int b = 0; b < NB; b++)
        __builtin_amdgcn_global_load_lds(k_scale + (r0 + min(lane, last)) * NB + b, (lds_ptr)(&ksv[w][b][0]), 4, 0, CPOL_NT);
    // the wave's own K loads have landed in LDS (nothing else touches its tiles)
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __builtin_amdgcn_wave_barrier();
    uint4 kr[W16];
    float ks[NB];
#pragma unroll
    for (int i = 0; i < W16; i++)
        kr[i] = *reinterpret_cast<const uint4 *>(&kv[w][0] + lane * HD + 16 * (i ^ (lane & (W16 - 1))));
#pragma unroll
    for (int b = 0; b < NB; b++) ks[b] = ksv[w][b][lane];
    // the K rows and scales are in registers before V overwrites them
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int t = 0; t < W16; t++) {
        const int p16 = 64 * t + lane;
        const int r = p16 / W16, slot = p16 % W16;
        __builtin_amdgcn_global_load_lds(v_cache + (r0 + min(r, last)) * HD + slot * 16,
                                         (lds_ptr)(&kv[w][0] + 1024 * t), 16, 0, CPOL_NT);
    }
#pragma unroll
    for (int b = 0; b < NB; b++)
        __builtin_amdgcn_global_load_lds(v_scale + (r0 + min(lane, last)) * NB + b, (lds_ptr)(&ksv[w][b][0]), 4, 0, CPOL_NT);

    // scores of this lane's key for the G heads, per 32-value block then scaled
    float sc[G];
#pragma unroll
    for (int g = 0; g < G; g++) sc[g] = 0.0f;
#pragma unroll
    for (int b = 0; b < NB; b++) {
        float kf[32];  // this block's 32 key values, converted once for the G heads
#pragma unroll
        for (int i = 0; i < 32; i++) {
            const uint4 &u = kr[b * 2 + i / 16];
            const uint32_t word = (i & 15) < 4 ? u.x : (i & 15) < 8 ? u.y : (i & 15) < 12 ? u.z : u.w;
            kf[i] = byte_f32(word, i & 3);
        }
#pragma unroll
        for (int g = 0; g < G; g++) {
            float a[4] = {0.0f, 0.0f, 0.0f, 0.0f};  // four independent chains (value i in chain i % 4)
#pragma unroll
            for (int i = 0; i < 32; i += 4) {
                const float4 qv = *reinterpret_cast<const float4 *>(qg + g * HD + 32 * b + i);
                a[0] = __builtin_fmaf(qv.x, kf[i], a[0]);
                a[1] = __builtin_fmaf(qv.y, kf[i + 1], a[1]);
                a[2] = __builtin_fmaf(qv.z, kf[i + 2], a[2]);
                a[3] = __builtin_fmaf(qv.w, kf[i + 3], a[3]);
            }
            sc[g] = __builtin_fmaf((a[0] + a[1]) + (a[2] + a[3]), ks[b], sc[g]);
        }
    }
#pragma unroll
    for (int g = 0; g < G; g++) sc[g] = valid ? sc[g] * scale_log2 : -INFINITY;

    // this wave's softmax over its 64 keys (exp2 domain); waves run on
    // independently until the one barrier that combines them
    float(*pl_w)[G] = pls[w];
    float mw[G], lw[G], p[G];
#pragma unroll
    for (int g = 0; g < G; g++) {
        mw[g] = wave_max_f32(sc[g]);
        p[g] = valid ? __builtin_amdgcn_exp2f(sc[g] - mw[g]) : 0.0f;
        pl_w[lane][g] = p[g];
        lw[g] = wave_sum_f32(p[g]);
    }
    // the wave reads back its own V rows from LDS: keep the writes above the
    // reads, and wait for the V loads
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __builtin_amdgcn_wave_barrier();

    // weighted sum of V over this wave's 64 keys: lanes are dimensions now
    // two independent chains over the keys (even and odd), added at the end
    float acc[DPL][G], acc2[DPL][G];
#pragma unroll
    for (int e = 0; e < DPL; e++)
#pragma unroll
        for (int g = 0; g < G; g++) acc[e][g] = acc2[e][g] = 0.0f;
#pragma unroll 2
    for (int jj = 0; jj < 64; jj += 2) {
        float pj[2][G];
#pragma unroll
        for (int k = 0; k < 2; k++)
#pragma unroll
            for (int g = 0; g < G; g++) pj[k][g] = pl_w[jj + k][g];
#pragma unroll
        for (int e = 0; e < DPL; e++) {
            const int d = lane + 64 * e;
            const float v0 = (float)kv[w][jj * HD + d] * ksv[w][d >> 5][jj];
            const float v1 = (float)kv[w][(jj + 1) * HD + d] * ksv[w][d >> 5][jj + 1];
#pragma unroll
            for (int g = 0; g < G; g++) {
                acc[e][g] = __builtin_fmaf(pj[0][g], v0, acc[e][g]);
                acc2[e][g] = __builtin_fmaf(pj[1][g], v1, acc2[e][g]);
            }
        }
    }
#pragma unroll
    for (int e = 0; e < DPL; e++)
#pragma unroll
        for (int g = 0; g < G; g++) acc[e][g] += acc2[e][g];
    // the wave's sums go where its V tile was (read by no one else, and its
    // own reads of it are done: LDS operations of a wave complete in order)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_wave_barrier();
    float(*accw_w)[HD] = reinterpret_cast<float(*)[HD]>(&kv[w][0]);
#pragma unroll
    for (int e = 0; e < DPL; e++)
#pragma unroll
        for (int g = 0; g < G; g++) accw_w[g][lane + 64 * e] = acc[e][g];
    if (lane < G) {
        // lane g publishes head g's (max, sum); the values are wave-uniform
        float m = mw[0], l = lw[0];
#pragma unroll
        for (int g = 1; g < G; g++)
            if (lane == g) {
                m = mw[g];
                l = lw[g];
            }
        redm[w][lane] = m;
        reds[w][lane] = l;
    }
    __syncthreads();

    // the workgroup's chunk: rescale the 4 waves to the chunk maximum, in order
    float *o = part + (((int64_t)s * n_kv + kvh) * splits + sp) * (G * (HD + 2));
    for (int i = tid; i < G * HD; i += 256) {
        const int g = i / HD, d = i % HD;
        const float m = fmaxf(fmaxf(redm[0][g], redm[1][g]), fmaxf(redm[2][g], redm[3][g]));
        float a = 0.0f;
#pragma unroll
        for (int ww = 0; ww < 4; ww++) {
            const float f = redm[ww][g] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(redm[ww][g] - m);
            a = __builtin_fmaf(f, reinterpret_cast<const float(*)[HD]>(&kv[ww][0])[g][d], a);
        }
        o[g * (HD + 2) + 2 + d] = a;
    }
    if (tid < G) {
        const int g = tid;
        const float m = fmaxf(fmaxf(redm[0][g], redm[1][g]), fmaxf(redm[2][g], redm[3][g]));
        float l = 0.0f;
#pragma unroll
        for (int ww = 0; ww < 4; ww++) {
            const float f = redm[ww][g] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(redm[ww][g] - m);
            l = __builtin_fmaf(f, reds[ww][g], l);
        }
        o[g * (HD + 2)] = m;
        o[g * (HD + 2) + 1] = l;
    }
}

constexpr int ATT_MAX_SPLITS = 256;
static_assert(ATT_MAX_SPLITS * ATT_CHUNK == ATT_MAX_LEN, "the combine kernel holds every chunk of a sequence");

template <int HD, int G>
__global__ __launch_bounds__(64) void attn_combine_kernel(int32_t n_heads, int32_t n_kv, int64_t n_slots,
                                                          const int32_t *__restrict__ base,
                                                          const int32_t *__restrict__ len, int32_t max_len,
                                                          int32_t splits, const float *__restrict__ part,
                                                          float *__restrict__ out, int32_t *__restrict__ status) {
    constexpr int DPL = HD / 64;
    __shared__ float ml[ATT_MAX_SPLITS][2];  // each chunk's (max, sum)
    const int h = blockIdx.x, s = blockIdx.y, lane = threadIdx.x;
    const int kvh = h / G, g = h % G;
    const int32_t L = len[s];
    float *o = out + ((int64_t)s * n_heads + h) * HD;
    if (!seq_ok(base[s], L, max_len, n_slots)) {
        if (lane == 0) __hip_atomic_store(status, 1 /* Q8_ERR_ARG */, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
        for (int e = 0; e < DPL; e++) o[lane + 64 * e] = __builtin_nanf("");
        return;
    }
    const int nsp = (L + ATT_CHUNK - 1) / ATT_CHUNK;
    const float *pb = part + ((int64_t)s * n_kv + kvh) * splits * (G * (HD + 2)) + g * (HD + 2);
    // every chunk's (max, sum) at once, one chunk per lane
    for (int c = lane; c < nsp; c += 64) {
        ml[c][0] = pb[(int64_t)c * G * (HD + 2)];
        ml[c][1] = pb[(int64_t)c * G * (HD + 2) + 1];
    }
    __syncthreads();
    float M = -INFINITY;
    for (int c = 0; c < nsp; c++) M = fmaxf(M, ml[c][0]);
    float den = 0.0f, num[DPL];
#pragma unroll
    for (int e = 0; e < DPL; e++) num[e] = 0.0f;
    // chunks in order; the weighted-sum loads of 8 chunks are issued together
    for (int c0 = 0; c0 < nsp; c0 += 8) {
        float v[8][DPL];
#pragma unroll
        for (int i = 0; i < 8; i++)
#pragma unroll
            for (int e = 0; e < DPL; e++)
                v[i][e] = c0 + i < nsp ? pb[(int64_t)(c0 + i) * G * (HD + 2) + 2 + lane + 64 * e] : 0.0f;
#pragma unroll
        for (int i = 0; i < 8; i++) {
            if (c0 + i < nsp) {
                const float f = __builtin_amdgcn_exp2f(ml[c0 + i][0] - M);
                den = __builtin_fmaf(f, ml[c0 + i][1], den);
#pragma unroll
                for (int e = 0; e < DPL; e++) num[e] = __builtin_fmaf(f, v[i][e], num[e]);
            }
        }
    }
#pragma unroll
    for (int e = 0; e < DPL; e++) o[lane + 64 * e] = num[e] / den;
}

// Host side ---------------------------------------------------------------

hipError_t launch_kv_write(const float *qkv, int64_t tokens, int n_heads, int n_kv, int head_dim,
                           const int32_t *positions, int64_t max_pos, const float *cos_tab, const float *sin_tab,
                           const float *q_gain, const float *k_gain, float eps, const int32_t *slots, int64_t n_slots,
                           float *q_out, int8_t *k_cache, float *k_scale, int8_t *v_cache, float *v_scale,
                           int32_t *status, hipStream_t s) {
    const int64_t threads = tokens * (n_heads + 2 * n_kv) * (head_dim / 4);
    if (threads == 0) return hipSuccess;
    const dim3 grid((unsigned)((threads + 255) / 256));
#define Q8_KVW(HD)                                                                                                 \
    hipLaunchKernelGGL(kv_write_kernel<HD>, grid, dim3(256), 0, s, qkv, (int32_t)tokens, n_heads, n_kv, positions, \
                       (int32_t)max_pos, cos_tab, sin_tab, q_gain, k_gain, eps, slots, n_slots, q_out, k_cache,   \
                       k_scale, v_cache, v_scale, status)
    switch (head_dim) {
        case 64: Q8_KVW(64); break;
        case 128: Q8_KVW(128); break;
        case 256: Q8_KVW(256); break;
        default: return hipErrorInvalidValue;
    }
#undef Q8_KVW
    return hipGetLastError();
}

template <int HD, int G>
static hipError_t launch_attn(const float *q, int64_t seqs, int n_heads, int n_kv, const int8_t *k_cache,
                              const float *k_scale, const int8_t *v_cache, const float *v_scale, int64_t n_slots,
                              const int32_t *base, const int32_t *len, int64_t max_len, float scale, float *out,
                              void *ws, hipStream_t s) {
    const int32_t splits = (int32_t)((max_len + ATT_CHUNK - 1) / ATT_CHUNK);
    int32_t *status = (int32_t *)ws;
    float *part = (float *)((uint8_t *)ws + 256);
    const float scale_log2 = scale * 1.4426950408889634f;
    hipLaunchKernelGGL((attn_partial_kernel<HD, G>), dim3((unsigned)splits, (unsigned)n_kv, (unsigned)seqs), dim3(256),
                       0, s, q, n_heads, n_kv, k_cache, k_scale, v_cache, v_scale, n_slots, base, len,
                       (int32_t)max_len, scale_log2, part, status);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((attn_combine_kernel<HD, G>), dim3((unsigned)n_heads, (unsigned)seqs), dim3(64), 0, s, n_heads,
                       n_kv, n_slots, base, len, (int32_t)max_len, splits, part, out, status);
    return hipGetLastError();
}

hipError_t launch_attention_decode(const float *q, int64_t seqs, int n_heads, int n_kv, int head_dim,
                                   const int8_t *k_cache, const float *k_scale, const int8_t *v_cache,
                                   const float *v_scale, int64_t n_slots, const int32_t *base, const int32_t *len,
                                   int64_t max_len, float scale, float *out, void *ws, hipStream_t s) {
    if (seqs == 0) return hipSuccess;
    const int G = n_heads / n_kv;
#define Q8_ATT(HD, GG) \
    if (head_dim == HD && G == GG) \
        return launch_attn<HD, GG>(q, seqs, n_heads, n_kv, k_cache, k_scale, v_cache, v_scale, n_slots, base, len, \
                                   max_len, scale, out, ws, s);
    Q8_ATT(64, 1) Q8_ATT(64, 2) Q8_ATT(64, 4) Q8_ATT(64, 8)
    Q8_ATT(128, 1) Q8_ATT(128, 2) Q8_ATT(128, 4) Q8_ATT(128, 8)
#undef Q8_ATT
    return hipErrorInvalidValue;
}

}  // namespace q8k
