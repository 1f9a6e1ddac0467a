"""Writes gemm_loop.inc: the main loop of the 128 x 128 prefill GEMM kernel as
one inline-asm block with explicit registers (run: python gemm_loop_gen.py).

Why asm: per 32 x 32 output tile and 32-value block the kernel needs one i8
MFMA (the exact block dots s), half of a rank-1 f16 MFMA (the scale products
Dx * Dw) and two VALU operations per output (convert, fused multiply-add).  On
gfx950 matrix-core and VALU time on one SIMD largely add up rather than
overlap, so the loop is only fast when nothing else is in the way: operand
reads issued a block ahead without waiting, MFMAs issued a block ahead of
their epilogue, the epilogue's three operands in different VGPR banks, and
one barrier per stage, reached by both waves of a SIMD at about the same
time (wave priorities below).  The compiler's schedule of the same loop waited on
every LDS read and consumed MFMA results right after issuing them.

The arithmetic per output is the kernel's documented order: per 256-value
group g, ga = s_0 * p_0, then ga = fma(s_b, p_b, ga) for b = 1..7 (s_b the
block dot converted to fp32, p_b = Dx_b * Dw_b exact in fp32); then
acc = acc + ga, group after group, from acc = -0.

Register map (VGPRs):
  v0-31     acc, 32 outputs of the lane: tile j register r at v(16 j + r)
  v32-63    ga, group sums; output 16 j + r at v(32 + 4 q + (i + 1) % 4),
            16 j + r = 4 q + i (one VGPR bank away from acc, s and p)
  v64-95    S0: block dots of the even block of a pair (tile 0 v64-79,
            tile 1 v80-95); v96-127 S1 (odd block)
  v130-161  P0: scale products (2b MFMA: block 0 = tile 0, block 1 = tile 1);
            v162-193 P1
  v194-209  OP0: A v194-197, B tile 0 v198-201, B tile 1 v202-205,
            Dx v206 (v207 = 0), Dw v208 (v209 = 0); v210-225 OP1
  v226-229  LDS address of the lane's A chunk of block bb = 0..3 (buffers 0, 1)
  v230-233  the same + 2 stage buffers (buffers 2, 3)
  v234/235  LDS address of the lane's B chunk, buffers 0-1 / 2-3
  v236/237  Dx, v238/239 Dw, same split
  v240-244  byte offsets of this lane's five stage loads from their bases
            (v226-241 and v242-245 are passed in as two vectors)
SGPRs: s[40:41] A base, s[42:43] B base, s[44:45] scale base (activation
scales for waves 0-3, weight scales for waves 4-7), s48 scale-base step from
an odd to an even stage, s49-53 the five loads' LDS destinations in buffer 0,
s54 stages not yet loaded, s55 groups left (s48-55 passed in as one vector;
tuples of more than two SGPRs start at a multiple of 4); s57 whether the stage
load being spread over slots is a real one (clobbered).

Stage loads: every wave issues 5 direct-to-LDS loads per 128-value stage (2
activation, 2 weight, 1 scale), four stages deep.  Stage s + 1 is waited for
(vmcnt) and barriered in slot 2 of stage s; right after that barrier every
wave has finished reading stage s, so stage s + 4 is loaded into its buffer,
its five loads spread over slots 2 and 3 of stage s and slots 0 and 1 of
stage s + 1 (issuing all 40 KB of a workgroup's loads right after the barrier
measured 2-3% slower); all of them are issued before the wait for stage s + 2,
so the loads outstanding after stage s + 1's are always stages s + 2 and s + 3.
Once no real stage is left to load, the wait becomes vmcnt(0) (everything
issued has landed) and nothing more is loaded.

Slots: slot (i, b) of stage i issues the MFMAs of the next block, the LDS
reads of the block after it and the epilogue of block (i, b), in that order.
Results are consumed at least 80 instructions after their MFMA issued (the
rank-1 MFMA needs 18 wait states before a VALU read, the i8 MFMA 10), operand
registers are rewritten one slot after their MFMA read them, result
registers one slot after their epilogue.
"""
import os

STAGE_BYTES = 34816
A_BYTES = 16384
NBUF = 4
BUF_OFF = [0, STAGE_BYTES, 0, STAGE_BYTES]  # immediate part; buffers 2, 3 use the "hi" address VGPRs

ACC, GA = 0, 32
S = (64, 96)
P = (130, 162)
OP = (194, 210)
VA_LO, VA_HI = 226, 230
VB = (234, 235)
VX = (236, 237)
VW = (238, 239)
VG = 240  # 240..244
S_ABASE, S_BBASE, S_SBASE, S_SINC, S_LDS, S_LEFT, S_GLEFT = 40, 42, 44, 48, 49, 54, 55
S_ISSUING = 57  # 1 while the stage load started in slot 2 still has parts to issue

PRIO_AFTER_BARRIER = {2: 3, 3: 2, 0: 1, 1: 0}  # slot b -> wave priority (the barrier is in slot 2)

INC_A = 128            # activation rows: 128 bytes per stage
INC_B = (8192, 9216)   # weight records: +4 blocks within a group, then to the next record
INC_SX_EVEN = 8        # scale bases: +4 scales (8 bytes) within a group; the odd->even step is s46


def ga(r):
    return GA + 4 * (r // 4) + (r + 1) % 4


def ds_reads(buf, bb, st):
    o = OP[st]
    hi = buf >= 2
    base = BUF_OFF[buf]
    va = (VA_HI if hi else VA_LO) + bb
    vb, vx, vw = VB[hi], VX[hi], VW[hi]
    return [
        f"ds_read_b128 v[{o}:{o+3}], v{va} offset:{base}",
        f"ds_read_b128 v[{o+4}:{o+7}], v{vb} offset:{base + bb*2048}",
        f"ds_read_b128 v[{o+8}:{o+11}], v{vb} offset:{base + bb*2048 + 512}",
        f"ds_read_u16 v{o+12}, v{vx} offset:{base + bb*2}",
        f"ds_read_u16 v{o+14}, v{vw} offset:{base + bb*2}",
    ]


def mfmas(st):
    o, s, p = OP[st], S[st], P[st]
    return [
        f"v_mfma_f32_32x32x4_2b_f16 v[{p}:{p+31}], v[{o+12}:{o+13}], v[{o+14}:{o+15}], 0",
        f"v_mfma_i32_32x32x32_i8 v[{s}:{s+15}], v[{o}:{o+3}], v[{o+4}:{o+7}], 0",
        f"v_mfma_i32_32x32x32_i8 v[{s+16}:{s+31}], v[{o}:{o+3}], v[{o+8}:{o+11}], 0",
    ]


def epilogue(st, first):
    """Convert and accumulate one block's 32 outputs; the first block of a group
    folds the previous group's sums into acc and multiplies."""
    s, p = S[st], P[st]
    ops = []
    for i in range(0, 32, 2):
        ops += [f"v_cvt_f32_i32_e32 v{s+r}, v{s+r}" for r in (i, i + 1)]
        for r in (i, i + 1):
            if first:
                ops.append(f"v_add_f32_e32 v{ACC+r}, v{ACC+r}, v{ga(r)}")
                ops.append(f"v_mul_f32_e32 v{ga(r)}, v{s+r}, v{p+r}")
            else:
                ops.append(f"v_fmac_f32_e32 v{ga(r)}, v{s+r}, v{p+r}")
    return ops


def issue(buf, parity):
    """If a stage is left to load: its five loads into buffer buf, then advance
    the bases if another one follows (parity: of the stage being loaded)."""
    out = [f"s_cmp_eq_u32 s{S_LEFT}, 0", "s_cbranch_scc1 6f"]
    kinds = [("dwordx4", S_ABASE), ("dwordx4", S_ABASE), ("dwordx4", S_BBASE), ("dwordx4", S_BBASE),
             ("dword", S_SBASE)]
    for u, (size, sb) in enumerate(kinds):
        out += [f"s_add_u32 m0, s{S_LDS+u}, {buf * STAGE_BYTES}", "s_nop 0",
                f"global_load_lds_{size} v{VG+u}, s[{sb}:{sb+1}]"]
    inc_b = INC_B[parity]
    inc_s = str(INC_SX_EVEN) if parity == 0 else f"s{S_SINC}"
    out += [f"s_cmp_gt_u32 s{S_LEFT}, 1", "s_cbranch_scc0 2f",
            f"s_add_u32 s{S_ABASE}, s{S_ABASE}, {INC_A}", f"s_addc_u32 s{S_ABASE+1}, s{S_ABASE+1}, 0",
            f"s_add_u32 s{S_BBASE}, s{S_BBASE}, {inc_b}", f"s_addc_u32 s{S_BBASE+1}, s{S_BBASE+1}, 0",
            f"s_add_u32 s{S_SBASE}, s{S_SBASE}, {inc_s}", f"s_addc_u32 s{S_SBASE+1}, s{S_SBASE+1}, 0",
            "2:",
            f"s_sub_u32 s{S_LEFT}, s{S_LEFT}, 1",
            "6:"]
    return out


SPREAD = [[0, 1], [2], [3], [4]]  # the stage's five loads over four slots


def issue_part(buf, parity, part):
    """Part `part` of loading the next stage into buffer buf: the loads are
    spread over four slots (slot 2 right after the barrier, slot 3, and slots
    0 and 1 of the next stage) instead of all eight waves issuing 40 KB at
    once; the buffer is not read before the barrier three stages later.  The
    first part decides whether a stage is left to load (s57), the last one
    advances the bases."""
    kinds = [("dwordx4", S_ABASE), ("dwordx4", S_ABASE), ("dwordx4", S_BBASE), ("dwordx4", S_BBASE),
             ("dword", S_SBASE)]
    out = []
    if part == 0:
        out += [f"s_cmp_eq_u32 s{S_LEFT}, 0", f"s_cselect_b32 s{S_ISSUING}, 0, 1"]
    out += [f"s_cmp_eq_u32 s{S_ISSUING}, 0", "s_cbranch_scc1 6f"]
    for u in SPREAD[part]:
        size, sb = kinds[u]
        out += [f"s_add_u32 m0, s{S_LDS+u}, {buf * STAGE_BYTES}", "s_nop 0",
                f"global_load_lds_{size} v{VG+u}, s[{sb}:{sb+1}]"]
    if part == len(SPREAD) - 1:
        inc_b = INC_B[parity]
        inc_s = str(INC_SX_EVEN) if parity == 0 else f"s{S_SINC}"
        out += [f"s_cmp_gt_u32 s{S_LEFT}, 1", "s_cbranch_scc0 2f",
                f"s_add_u32 s{S_ABASE}, s{S_ABASE}, {INC_A}", f"s_addc_u32 s{S_ABASE+1}, s{S_ABASE+1}, 0",
                f"s_add_u32 s{S_BBASE}, s{S_BBASE}, {inc_b}", f"s_addc_u32 s{S_BBASE+1}, s{S_BBASE+1}, 0",
                f"s_add_u32 s{S_SBASE}, s{S_SBASE}, {inc_s}", f"s_addc_u32 s{S_SBASE+1}, s{S_SBASE+1}, 0",
                "2:",
                f"s_sub_u32 s{S_LEFT}, s{S_LEFT}, 1"]
    out += ["6:"]
    return out


def slot(i, b):
    """Stage i of the four-stage loop body (buffer i), block b."""
    nxt_set = (b + 1) & 1
    cur_set = b & 1
    if b < 2:
        reads = ds_reads(i, b + 2, cur_set)
    else:
        reads = ds_reads((i + 1) % NBUF, b - 2, cur_set)
    head = ["s_waitcnt lgkmcnt(0)"]
    if b == 2:
        # stage i + 1 landed for every wave (two later stages may still be in
        # flight; at the tail, fewer: wait for all), stage i read by every
        # wave: load stage i + 4 into buffer i
        head = [f"s_cmp_eq_u32 s{S_LEFT}, 0", "s_cbranch_scc1 4f",
                "s_waitcnt vmcnt(10) lgkmcnt(0)", "s_branch 5f",
                "4:", "s_waitcnt vmcnt(0) lgkmcnt(0)",
                "5:", "s_barrier"] + issue_part(i, i & 1, 0)
    elif b == 3:
        head = head + issue_part(i, i & 1, 1)
    else:  # slots 0 and 1 finish the load the previous stage started
        head = head + issue_part((i - 1) % NBUF, (i - 1) & 1, 2 + b)
    # wave priority falls as the wave moves from one barrier to the next
    # (3 right after it, 0 in the slot before the next), so of the two waves
    # sharing a SIMD the one behind wins issue and they reach the barrier
    # together instead of one waiting there while the other runs alone
    prio = f"s_setprio {PRIO_AFTER_BARRIER[b]}"
    if b == 2:
        k = head.index("s_barrier") + 1
        head = head[:k] + [prio] + head[k:]
    else:
        head = [prio] + head
    # the next block's three MFMAs first, then its operand reads, then this
    # block's epilogue (measured 2% faster than spreading the MFMAs through
    # the epilogue)
    return head + mfmas(nxt_set) + reads + epilogue(cur_set, (i & 1) == 0 and b == 0)


def loop():
    lines = [f"v_mov_b32 v{OP[st]+k}, 0" for st in (0, 1) for k in (13, 15)] + [f"s_mov_b32 s{S_ISSUING}, 0"]
    for buf in range(NBUF):
        lines += issue(buf, buf & 1)
    # stage 0 landed: 15 later loads may be in flight if 4 stages were issued (2+ groups)
    lines += [f"s_cmp_lt_u32 s{S_GLEFT}, 2", "s_cbranch_scc1 7f", "s_waitcnt vmcnt(15)", "s_branch 8f",
              "7:", "s_waitcnt vmcnt(0)", "8:", "s_barrier"]
    lines += ds_reads(0, 0, 0) + ds_reads(0, 1, 1)
    lines += ["s_waitcnt lgkmcnt(5)", "s_nop 4"] + mfmas(0) + ["s_nop 15", "s_nop 15", "s_nop 7"]
    lines += ["1:"]
    for i in range(NBUF):
        for b in range(4):
            lines += slot(i, b)
        if i & 1:  # a group ends with stage i
            lines += [f"s_sub_u32 s{S_GLEFT}, s{S_GLEFT}, 1", f"s_cmp_eq_u32 s{S_GLEFT}, 0", "s_cbranch_scc1 3f"]
    lines += ["s_branch 1b", "3:", "s_setprio 0"]
    lines += [f"v_add_f32_e32 v{ACC+r}, v{ACC+r}, v{ga(r)}" for r in range(32)]
    # every load of this wave has landed and every MFMA has finished before
    # the compiler's code may touch these registers or the workgroup ends
    lines += ["s_waitcnt vmcnt(0) lgkmcnt(0)", "s_nop 15", "s_nop 15", "s_nop 15", "s_nop 15"]
    return lines


def clobbers():
    pinned = set(range(ACC, GA + 32)) | set(range(VA_LO, VG + 5))
    return [f"v{r}" for r in range(64, 256) if r not in pinned and r < 226]


def main():
    body = "".join(f'"{l}\\n\\t"\n' for l in loop())
    clob = ", ".join(f'"{c}"' for c in clobbers())
    text = ("// Generated by gemm_loop_gen.py; do not edit.\n"
            "#define Q8_GEMM_LOOP_ASM \\\n" + " \\\n".join(body.rstrip("\n").split("\n")) + "\n"
            "#define Q8_GEMM_LOOP_CLOBBERS " + clob + "\n")
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "gemm_loop.inc")
    with open(path, "w") as f:
        f.write(text)


if __name__ == "__main__":
    main()
