"""Writes gemm_strip.inc: the k loop of the small-problem prefill GEMM kernel
(gemm_strip_kernel, one 32 x 64 output strip per workgroup, k split across its
waves) as one inline-asm block with explicit registers
(run: python gemm_strip_gen.py).

Work split: the workgroup's W waves (4 or 8: two variants are generated)
take the 256-value groups in batches,
wave w group w + W i in batch i.  For its group a wave computes the group sum
of each of its 32 x 64 outputs exactly as the 128 x 128 kernel does (per
block one i8 MFMA per 32 x 32 tile for the exact block dots s, one rank-1 f16
MFMA for the scale products p = Dx * Dw of both tiles, then ga = s_0 * p_0,
ga = fma(s_b, p_b, ga) for b = 1..7) and parks it in LDS; after a barrier the
workgroup's threads fold the batch's group sums into their outputs' running
sums in group order (acc = acc + ga_g), so every output sees the same
sequence of fp32 operations as in the 128 x 128 kernel.

Pipelining: a wave loads its group's operands straight into registers (per
block the 16-byte activation chunk and two 16-byte weight chunks, per group
16 bytes of activation scales and 16 bytes of weight scales).  While it
computes group g it issues the loads of its next group g + W block by block,
each into the registers that block of g has just released (its MFMAs have
issued), so those loads are in flight for about one group's compute.  The
MFMAs of block b + 1 issue before the epilogue of block b.  Loads return in
issue order, so "block b's operands have landed" is a vmcnt threshold that
the generator counts.  The group sums go to one of two LDS park buffers by
batch parity, so one barrier per batch suffices (a thread finishes folding
batch i before it reaches the barrier of batch i + 1, after which batch i + 2
reuses the buffer).  The scale registers alternate between two sets by group
parity (the next group's scales load while the current ones are still read).

Hazards: the generator inserts s_nop where an instruction reads a VGPR
written by an MFMA fewer wait states ago than that MFMA needs (i8 32x32x32:
12, rank-1 f16 2-block: 20) or where an MFMA reads a VGPR a VALU op wrote
fewer than 3 wait states ago.

Register map (VGPRs):
  v0-31     ga: output 16 j + r at v(4 q + (i + 1) % 4) with 16 j + r = 4 q + i
  v32-63    S: block dots (tile 0 v32-47, tile 1 v48-63); fold temporaries
  v66-97    P: scale products (2-block MFMA: block 0 = tile 0, block 1 = tile 1)
  v98-129   A: activation chunks of blocks 0..7 (4 VGPRs each)
  v130-193  B: weight chunks, block b tile j at v(130 + 8 b + 4 j)
  v194-197 / v198-201  activation / weight scales of even groups, v202-209 odd
  v210 (v211 = 0), v212 (v213 = 0)  rank-1 operands (the block's Dx, Dw)
  v214-221  acc: outputs t + 64 W i of thread t (i < 32 / W)
  v222 activation offset of the lane's row (row * K + 16 * half),
  v223 its scale offset (row * K / 16), v224 weight chunk offset
  (1024 * half + 16 * lane32), v225 weight scale offset (16384 + 16 * lane),
  v226 park address (lds + 8192 * wave + 4 * lane), v227 fold address (lds + 4 t),
  v228 / v229 the same in the second park buffer (+ 8192 W)
  (v222-229 passed in as one vector, v214-221 as another)
SGPRs: s[40:41] activation base, s[42:43] weight base, s[44:45] activation
scale base, all of the wave's next group to load; s[46:47] weight base of one
block; s48 this wave's group in the current batch, s49 groups G, s50 first
group of the current batch, s51 scratch; s[52:55] the bases' steps from one of
the wave's groups to the next (activation 256 W, weights 17408 W, scales 16 W)
(s48-51 and s52-55 passed in as vectors).
"""
import os
import re

GROUP_BLOCKS = 8
RECORD_BYTES = 17408
PARK_WAVE = 8192
W = 4  # waves per workgroup of the variant being generated (4 or 8); set by gen()

S = 32
P = 66
A = 98
B = 130
SC = ((194, 198), (202, 206))  # (activation scales, weight scales) by group parity
TA, TB = 210, 212
ACC = 214
V_XOFF, V_SXOFF, V_WOFF, V_SWOFF, V_PARK, V_FOLD, V_PARK1, V_FOLD1 = 222, 223, 224, 225, 226, 227, 228, 229
S_ABASE, S_WBASE, S_XBASE, S_BLK = 40, 42, 44, 46
S_G, S_GN, S_BATCH, S_TMP = 48, 49, 50, 51
S_ASTEP, S_WSTEP, S_XSTEP = 52, 53, 54

WAIT_AFTER = {"v_mfma_i32_32x32x32_i8": 12, "v_mfma_f32_32x32x4_2b_f16": 20}
VALU_TO_MFMA = 3


def ga(r):
    return 4 * (r // 4) + (r + 1) % 4


def s_reg(j, r):
    return S + 16 * j + r


def p_reg(j, r):
    return P + 16 * j + r


def b_reg(b, j):
    return B + 8 * b + 4 * j


def loads_next(b, par):
    """The next group's loads of block b (b == 0: its scales first) into the
    registers this group's block b has released."""
    out = []
    if b == 0:
        sx, sw = SC[1 - par]
        out += [f"global_load_dwordx4 v[{sx}:{sx+3}], v{V_SXOFF}, s[{S_XBASE}:{S_XBASE+1}]",
                f"global_load_dwordx4 v[{sw}:{sw+3}], v{V_SWOFF}, s[{S_WBASE}:{S_WBASE+1}]"]
    a = A + 4 * b
    out += [f"global_load_dwordx4 v[{a}:{a+3}], v{V_XOFF}, s[{S_ABASE}:{S_ABASE+1}] offset:{32 * b}",
            f"s_add_u32 s{S_BLK}, s{S_WBASE}, {2048 * b}", f"s_addc_u32 s{S_BLK+1}, s{S_WBASE+1}, 0"]
    for j in range(2):
        r = b_reg(b, j)
        out.append(f"global_load_dwordx4 v[{r}:{r+3}], v{V_WOFF}, s[{S_BLK}:{S_BLK+1}] offset:{512 * j}")
    return out


def first_loads(par):
    """Loads of the wave's first group (bases already at that group)."""
    out = []
    for b in range(GROUP_BLOCKS):
        out += loads_next(b, 1 - par)
    return out


def extract(b, par):
    """Rank-1 operands of block b: the block's 16-bit scales, zero-extended."""
    sx, sw = SC[par]
    word, hi = b // 2, b % 2
    if hi:
        return [f"v_lshrrev_b32_e32 v{TA}, 16, v{sx + word}", f"v_lshrrev_b32_e32 v{TB}, 16, v{sw + word}"]
    return [f"v_and_b32_e32 v{TA}, 0xffff, v{sx + word}", f"v_and_b32_e32 v{TB}, 0xffff, v{sw + word}"]


def mfma_tile(b, j):
    a = A + 4 * b
    r = b_reg(b, j)
    s = s_reg(j, 0)
    return f"v_mfma_i32_32x32x32_i8 v[{s}:{s+15}], v[{a}:{a+3}], v[{r}:{r+3}], 0"


def mfma_scale():
    return f"v_mfma_f32_32x32x4_2b_f16 v[{P}:{P+31}], v[{TA}:{TA+1}], v[{TB}:{TB+1}], 0"


def epilogue(j, first):
    out = [f"v_cvt_f32_i32_e32 v{s_reg(j, r)}, v{s_reg(j, r)}" for r in range(16)]
    for r in range(16):
        if first:
            out.append(f"v_mul_f32_e32 v{ga(16 * j + r)}, v{s_reg(j, r)}, v{p_reg(j, r)}")
        else:
            out.append(f"v_fmac_f32_e32 v{ga(16 * j + r)}, v{s_reg(j, r)}, v{p_reg(j, r)}")
    return out


def group(par, with_next, buf):
    """One group of the wave: operands of blocks 0..7 are in registers or in
    flight (issued in group order: scales, block 0, ..., block 7); with_next:
    the next group's loads are issued as blocks are released.  Ends with the
    group sums parked in buffer buf."""
    out = ["s_waitcnt vmcnt(21)"] + extract(0, par) + [mfma_tile(0, 0), mfma_tile(0, 1), mfma_scale()]
    for b in range(GROUP_BLOCKS):
        if with_next:
            out += loads_next(b, par)
        out += epilogue(0, b == 0)
        if b + 1 < GROUP_BLOCKS:
            # block b + 1 landed: loads issued after it are the earlier group's
            # blocks b + 2..7 (3 each) and, with_next, this group's so far
            later = 3 * (GROUP_BLOCKS - 2 - b) + ((2 + 3 * (b + 1)) if with_next else 0)
            out += [f"s_waitcnt vmcnt({later})"] + extract(b + 1, par) + [mfma_tile(b + 1, 0)]
        out += epilogue(1, b == 0)
        if b + 1 < GROUP_BLOCKS:
            out += [mfma_tile(b + 1, 1), mfma_scale()]
    for j in range(2):
        for r in range(16):
            out.append(f"ds_write_b32 v{(V_PARK, V_PARK1)[buf]}, v{ga(16 * j + r)} offset:{(16 * j + r) * 256}")
    if with_next:
        out += [f"s_add_u32 s{S_ABASE}, s{S_ABASE}, s{S_ASTEP}", f"s_addc_u32 s{S_ABASE+1}, s{S_ABASE+1}, 0",
                f"s_add_u32 s{S_WBASE}, s{S_WBASE}, s{S_WSTEP}", f"s_addc_u32 s{S_WBASE+1}, s{S_WBASE+1}, 0",
                f"s_add_u32 s{S_XBASE}, s{S_XBASE}, s{S_XSTEP}", f"s_addc_u32 s{S_XBASE+1}, s{S_XBASE+1}, 0"]
    return out


def fold(buf):
    """Every thread: acc_i += park[buf][q][t + 64 W i] for the batch's groups q
    in order (q < G - first group of the batch)."""
    per = 32 // W  # outputs per thread
    out = ["s_waitcnt lgkmcnt(0)", "s_barrier"]
    for q in range(W):
        out += [f"s_add_u32 s{S_TMP}, s{S_BATCH}, {q}", f"s_cmp_ge_u32 s{S_TMP}, s{S_GN}", "s_cbranch_scc1 9f"]
        out += [f"ds_read_b32 v{S + i}, v{(V_FOLD, V_FOLD1)[buf]} offset:{q * PARK_WAVE + i * 256 * W}"
                for i in range(per)]
        out += ["s_waitcnt lgkmcnt(0)"]
        out += [f"v_add_f32_e32 v{ACC + i}, v{ACC + i}, v{S + i}" for i in range(per)]
    out += ["9:"]
    return out


def batch(par):
    """One batch: the wave's group (if any), then the fold; buffer and scale
    set by batch parity."""
    out = [f"s_cmp_ge_u32 s{S_G}, s{S_GN}", "s_cbranch_scc1 8f",
           f"s_add_u32 s{S_TMP}, s{S_G}, {W}", f"s_cmp_ge_u32 s{S_TMP}, s{S_GN}", "s_cbranch_scc1 7f"]
    out += group(par, True, par)
    out += ["s_branch 8f", "7:"]
    out += group(par, False, par)
    out += ["8:"]
    out += fold(par)
    out += [f"s_add_u32 s{S_G}, s{S_G}, {W}", f"s_add_u32 s{S_BATCH}, s{S_BATCH}, {W}"]
    return out


def add_nops(lines):
    """Insert s_nop where a read follows an MFMA write (or an MFMA read
    follows a VALU write) too closely; labels and s_nop count as written."""
    out = []
    mfma_w = {}  # vgpr -> (position, wait needed)
    valu_w = {}  # vgpr -> position
    pos = 0

    def regs(text):
        rs = set()
        for a, b in re.findall(r"v\[(\d+):(\d+)\]", text):
            rs.update(range(int(a), int(b) + 1))
        for a in re.findall(r"\bv(\d+)\b", text):
            rs.add(int(a))
        return rs

    for l in lines:
        if l.endswith(":") or l.startswith("s_branch") or l.startswith("s_cbranch"):
            # control flow: be conservative across labels (assume nothing retired)
            out.append(l)
            continue
        op = l.split()[0]
        parts = l.split(None, 1)
        operands = parts[1] if len(parts) > 1 else ""
        if op.startswith(("v_", "ds_", "global_")):
            if op.startswith("global_load") or op.startswith("ds_read"):
                dst, srcs = set(), regs(operands.split(",", 1)[1]) if "," in operands else set()
                dst = regs(operands.split(",", 1)[0])
            elif op.startswith("ds_write"):
                dst, srcs = set(), regs(operands)
            else:
                d, _, s = operands.partition(",")
                dst, srcs = regs(d), regs(s)
                if op.startswith("v_fmac"):
                    srcs |= dst
            need = 0
            for r in srcs:
                if r in mfma_w:
                    p0, w = mfma_w[r]
                    need = max(need, w - (pos - p0))
                if op.startswith("v_mfma") and r in valu_w:
                    need = max(need, VALU_TO_MFMA - (pos - valu_w[r]))
            while need > 0:
                n = min(need, 16)
                out.append(f"s_nop {n - 1}")
                pos += n
                need -= n
            out.append(l)
            if op.startswith("v_mfma"):
                for r in dst:
                    mfma_w[r] = (pos, WAIT_AFTER[op])
                    valu_w.pop(r, None)
            elif op.startswith("v_"):
                for r in dst:
                    valu_w[r] = pos
                    mfma_w.pop(r, None)
            else:
                for r in dst:
                    mfma_w.pop(r, None)
            pos += 1
        else:
            m = re.match(r"s_nop (\d+)", l)
            pos += int(m.group(1)) + 1 if m else 1
            out.append(l)
    return out


def loop():
    lines = [f"v_mov_b32 v{TA + 1}, 0", f"v_mov_b32 v{TB + 1}, 0"]
    # the wave's first group (if it has one), bases then advanced to its next
    lines += [f"s_cmp_ge_u32 s{S_G}, s{S_GN}", "s_cbranch_scc1 6f"] + first_loads(0)
    lines += [f"s_add_u32 s{S_ABASE}, s{S_ABASE}, s{S_ASTEP}", f"s_addc_u32 s{S_ABASE+1}, s{S_ABASE+1}, 0",
              f"s_add_u32 s{S_WBASE}, s{S_WBASE}, s{S_WSTEP}", f"s_addc_u32 s{S_WBASE+1}, s{S_WBASE+1}, 0",
              f"s_add_u32 s{S_XBASE}, s{S_XBASE}, s{S_XSTEP}", f"s_addc_u32 s{S_XBASE+1}, s{S_XBASE+1}, 0", "6:"]
    lines += ["1:"]
    lines += batch(0)
    lines += [f"s_cmp_ge_u32 s{S_BATCH}, s{S_GN}", "s_cbranch_scc1 3f"]
    lines += batch(1)
    lines += [f"s_cmp_ge_u32 s{S_BATCH}, s{S_GN}", "s_cbranch_scc1 3f", "s_branch 1b", "3:"]
    lines += ["s_waitcnt vmcnt(0) lgkmcnt(0)", "s_nop 15", "s_nop 15"]
    return add_nops(lines)


def clobbers():
    pinned = set(range(ACC, ACC + 8)) | set(range(V_XOFF, V_FOLD1 + 1))
    return [f"v{r}" for r in range(0, 214) if r not in pinned]


def gen(waves):
    global W
    W = waves
    return "".join(f'"{l}\\n\\t"\n' for l in loop())


def main():
    text = "// Generated by gemm_strip_gen.py; do not edit.\n"
    for waves in (4, 8):
        body = gen(waves)
        text += f"#define Q8_GEMM_STRIP_ASM_W{waves} \\\n" + " \\\n".join(body.rstrip("\n").split("\n")) + "\n"
    text += "#define Q8_GEMM_STRIP_CLOBBERS " + ", ".join(f'"{c}"' for c in clobbers()) + "\n"
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "gemm_strip.inc")
    with open(path, "w") as f:
        f.write(text)


if __name__ == "__main__":
    main()
