// Host-side planning of libq8's launches: work decomposition and workspace
// layouts.  Plain C++ (no device code), shared by the launchers and the
// argument checks of the C ABI.
#include "launch.hpp"
#include "layout.hpp"

namespace q8k {

// Execution plan of a GEMV.  Only speed depends on it; every plan produces
// the same bits.  Up to 8 waves per workgroup (one or more groups each);
// tiles of narrow matrices are spread over one workgroup per segment so that
// at least ~256 workgroups run; the group sums a workgroup keeps in LDS must
// fit in 64 KB.
GemvPlan gemv_plan(int64_t m, int64_t n, int64_t k, int mf_min_rows) {
    GemvPlan p;
    p.tiles = (n + TILE_ROWS - 1) / TILE_ROWS;
    p.groups = k / GROUP_K;
    const int64_t S = (p.groups + SEG_GROUPS - 1) / SEG_GROUPS;
    int64_t wgs = 1;
    if (p.tiles < 256) wgs = (256 + p.tiles - 1) / p.tiles;
    if (wgs > S) wgs = S;
    for (;;) {  // LDS bound: groups per workgroup x m x 64 rows x 4 bytes
        const int64_t sp = (S + wgs - 1) / wgs;
        const int64_t gpw = sp * SEG_GROUPS < p.groups ? sp * SEG_GROUPS : p.groups;
        if (gpw * m * TILE_ROWS * (int64_t)sizeof(float) <= GEMV_LDS_LIMIT || wgs >= S) break;
        wgs++;
    }
    const int64_t sp = (S + wgs - 1) / wgs;
    wgs = (S + sp - 1) / sp;  // no workgroup without a segment
    const int64_t gpw = sp * SEG_GROUPS < p.groups ? sp * SEG_GROUPS : p.groups;
    p.wgs_per_tile = (int)wgs;
    p.segs_per_wg = (int)sp;
    // one chain thread per (row, activation row) after the barrier: at least m waves
    int64_t waves = gpw < GEMV_MAX_WAVES ? gpw : GEMV_MAX_WAVES;
    if (waves < m) waves = m;
    p.waves = (int)waves;
    p.lds = (size_t)(gpw * m * TILE_ROWS) * sizeof(float);
    // the MFMA form (packed weights, m >= mf_min_rows): each of up to 8 waves
    // keeps the group's m rows of packed codes (m x 64 dwords) and 8 x 8
    // activation scales after the group slots
    if (m >= mf_min_rows && m >= 2)
        p.lds += (size_t)GEMV_MAX_WAVES * (m * 64 + GROUP_BLOCKS * 8) * sizeof(uint32_t);
    p.workspace = 0;
    if (wgs > 1) p.workspace = (size_t)((p.tiles * 4 + 255) / 256 * 256) + (size_t)(S * m * n) * sizeof(float);
    return p;
}

size_t gemv_workspace_bytes(int64_t m, int64_t n, int64_t k) { return gemv_plan(m, n, k).workspace; }

size_t grouped_workspace_bytes(int64_t tokens, int topk, int64_t n_experts) {
    return (size_t)(16 + 2 * n_experts + 1 + tokens * topk) * sizeof(int32_t);
}

size_t attention_workspace_bytes(int64_t seqs, int n_heads, int n_kv, int head_dim, int64_t max_len) {
    const int64_t splits = (max_len + ATT_CHUNK - 1) / ATT_CHUNK;
    return 256 + (size_t)seqs * n_kv * splits * (n_heads / n_kv) * (head_dim + 2) * 4;
}

// The sequence workspace: status line and SEQ_CTR_PER_STEP counters per step,
// then the flag lines (4 KB aligned), then each split step's tile counters
// and segment sums (256-byte aligned, addressed in units of 256 bytes).
void seq_plan(const SeqHostStep *steps, int count, int64_t m, SeqPlan &P) {
    P.one = true;
    P.lds = 0;
    const size_t ctr_end = 256 + (size_t)SEQ_CTR_LINE * SEQ_CTR_PER_STEP * count;
    const size_t flag_off = (ctr_end + 4095) / 4096 * 4096;
    size_t off = flag_off + (size_t)SEQ_FLAG_LINES * SEQ_FLAG_LINE_BYTES;
    P.flag_off = (int32_t)flag_off;
    for (int i = 0; i < count; i++) {
        const GemvPlan p = gemv_plan(m, steps[i].n, steps[i].k, SEQ_MF_MIN_ROWS);
        const int64_t gpw = (int64_t)p.segs_per_wg * SEG_GROUPS < p.groups ? (int64_t)p.segs_per_wg * SEG_GROUPS
                                                                           : p.groups;
        if (gpw > SEQ_THREADS / 64) P.one = false;
        if (p.lds > P.lds) P.lds = p.lds;
        P.wgs[i] = (uint16_t)p.wgs_per_tile;
        P.segs[i] = (uint16_t)p.segs_per_wg;
        P.ws_off[i] = 0;
        if (p.workspace) {
            P.ws_off[i] = (uint32_t)(off / 256);
            off += (p.workspace + 255) / 256 * 256;
        }
    }
    P.workspace = off;
}

size_t gemv_sequence_workspace_bytes(const SeqHostStep *steps, int count, int64_t m) {
    SeqPlan P;
    seq_plan(steps, count, m, P);
    return P.workspace;
}

}  // namespace q8k
