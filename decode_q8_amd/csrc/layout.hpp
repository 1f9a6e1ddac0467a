// Sizes of the byte formats and of the work decomposition, shared by the
// kernels and the host-side planning (plain constants: this header compiles
// with any C++17 host compiler as well as hipcc).
#pragma once

#include <stdint.h>

namespace q8k {

// Q8_0 blocks and the packed layout
constexpr int QK = 32;            // values per block
constexpr int BLOCK_BYTES = 34;   // fp16 scale + 32 int8
constexpr int TILE_ROWS = 64;     // rows per packed record = lanes per wave
constexpr int GROUP_BLOCKS = 8;   // blocks per packed record and per summation group
constexpr int GROUP_K = GROUP_BLOCKS * QK;              // 256 values
constexpr int RECORD_BYTES = TILE_ROWS * GROUP_BLOCKS * BLOCK_BYTES;  // 17408
constexpr int RECORD_Q_BYTES = TILE_ROWS * GROUP_K;     // 16384
constexpr int ROW_GROUP_BYTES = GROUP_BLOCKS * BLOCK_BYTES;           // 272
constexpr int SEG_GROUPS = 8;     // groups per summation segment (2048 values)

// GEMV plan: up to 8 waves per workgroup; the group sums a workgroup keeps in
// LDS must fit in 64 KB
constexpr int GEMV_MAX_WAVES = 8;
constexpr int64_t GEMV_LDS_LIMIT = 64 * 1024;
// Activation rows from which a GEMV on packed weights takes the MFMA form
// (the int8 block dots of all rows from one MFMA per block and 32 weight
// rows) instead of a lane per weight row with the activation codes broadcast
// by DPP: from 7 rows in the per-matrix kernel and from 5 in the sequence
// kernel, where the MFMA form runs with up to 256 registers (one workgroup per
// CU) and the lane form with 128 (two per CU, spilling more with every row).
// Measured (decode step at m = 4 / 5: lane form 515 / 684 us, MFMA form
// 596 / 614 us; one launch per matrix, the lane form is ahead up to m = 6);
// only speed depends on it.  Each kernel's plan reserves the MFMA form's LDS
// scratch from its own threshold.
constexpr int GEMV_MF_MIN_ROWS = 7;
constexpr int SEQ_MF_MIN_ROWS = 5;

// Sequence workspace: [0, 4) status word; from byte 256 SEQ_CTR_PER_STEP
// counters of SEQ_CTR_LINE bytes per step (the step's counter, then its
// sub-counters); SEQ_FLAG_LINES flag lines of SEQ_FLAG_LINE_BYTES from a
// 4 KB-aligned offset; then the split steps' tile counters and segment sums.
// A flag line holds one int32 flag per step, each alone in its own
// SEQ_FLAG_SLOT_BYTES cache line: with the flags of consecutive steps packed
// into one line, the polls of one step and the raising of the next met on it
// (300.0 -> 291.7 us per decode step once spread).
constexpr int SEQ_FLAG_LINES = 16;
constexpr int SEQ_FLAG_SLOT_BYTES = 128;
constexpr int SEQ_FLAG_LINE_BYTES = 72 * SEQ_FLAG_SLOT_BYTES;  // every step of the longest sequence
constexpr int SEQ_NSUB = 32;               // sub-counters of a step with many units (16: +1 us per decode step)
constexpr int SEQ_CTR_LINE = 128;          // bytes per counter
constexpr int SEQ_CTR_PER_STEP = SEQ_NSUB + 1;
constexpr int SEQ_THREADS = 512;
// The allocation-free sequence entry point's own workspace, per GPU (holds
// the Llama-3.2-1B-shaped decode step's workspace up to m = 8, ~4.6 MB).
constexpr int64_t SEQ_SCRATCH_BYTES = 8ll << 20;

// Decode attention: cached positions per workgroup
constexpr int ATT_CHUNK = 256;

}  // namespace q8k
