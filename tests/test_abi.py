"""The C ABI without a GPU: the library loads, exports every entry point that
include/q8.h declares, and rejects bad requests on the host before any HIP
call (the pages' boundary style: unsupported requests fail explicitly at the
API boundary, "Ferrule" README, "Core features").  Nothing here launches a
kernel."""
import ctypes
import os
import re

import pytest

from decode_q8_amd import q8

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "q8.h")

# Fake but 16-byte aligned device addresses: every call below fails validation
# before it could touch them.
A = 0x7F0000000000
B = 0x7F0000100000
C = 0x7F0000200000
D = 0x7F0000300000


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^[A-Za-z_][\w\s\*]*?\b(q8_\w+)\s*\(", text, flags=re.M)))


def test_exports_every_declared_symbol():
    names = _declared()
    assert len(names) == 23, names
    assert sorted(q8.SIGNATURES) == names
    L = ctypes.CDLL(q8.LIB_PATH)
    for n in names:
        assert hasattr(L, n), n


def test_version_and_strings():
    m = re.search(r"#define Q8_ABI_VERSION (\d+)u", open(HEADER).read())
    assert int(m.group(1)) == q8.Q8_ABI_VERSION == q8.q8_abi_version() == 5
    for s in range(7):
        assert q8.status_str(s).startswith("Q8_")
    assert q8.status_str(99) == "Q8_ERR_UNKNOWN"


def test_sizes():
    assert q8.q8_quantized_bytes(1, 2048) == 2176
    assert q8.q8_quantized_bytes(2048, 2048) == 4456448
    assert q8.q8_quantized_bytes(128256, 2048) == 128256 * 64 * 34
    assert q8.q8_quantized_bytes(3, 33) == 0
    assert q8.q8_quantized_bytes(-1, 32) == 0
    # narrow GEMVs with long rows spread a tile over one workgroup per
    # 2048-value segment: tile counters (256-byte aligned) + segment sums
    assert q8.q8_matmul_workspace_bytes(1, 2048, 8192) == 256 + 4 * 1 * 2048 * 4
    assert q8.q8_matmul_workspace_bytes(8, 2048, 7168) == 256 + 4 * 8 * 2048 * 4
    assert q8.q8_matmul_workspace_bytes(8, 2048, 2048) == 0          # one segment: no hand-off
    assert q8.q8_matmul_workspace_bytes(1, 64000, 256) == 0          # a single group: no split
    assert q8.q8_matmul_workspace_bytes(1, 128256, 2048) == 0        # wide: whole rows per wave
    assert q8.q8_matmul_workspace_bytes(188, 2048, 2048) == 0
    assert q8.q8_grouped_workspace_bytes(16, 8, 256, 2048, 7168) >= 4 * (16 + 2 * 256 + 1 + 128)


def _raw(name, *args):
    return getattr(q8.lib(), name)(*args)


def test_quantize_validation():
    f = "q8_quantize_rows"
    assert _raw(f, None, 64, 1, 64, 2, B, None) == q8.Q8_ERR_ARG
    assert _raw(f, A, 64, 1, 64, 2, None, None) == q8.Q8_ERR_ARG
    assert _raw(f, A, 32, 1, 64, 2, B, None) == q8.Q8_ERR_ARG       # ld_x < k
    assert _raw(f, A, 64, 1, 64, 1, B, None) == q8.Q8_ERR_ARG       # PACKED is not a quantizer output
    assert _raw(f, A, 64, 1, 0, 2, B, None) == q8.Q8_ERR_ARG
    assert _raw(f, A, 64, -1, 64, 2, B, None) == q8.Q8_ERR_ARG
    assert _raw(f, A, 64, 1, 48, 2, B, None) == q8.Q8_ERR_SHAPE     # k % 32
    assert _raw(f, A + 4, 64, 1, 64, 2, B, None) == q8.Q8_ERR_ALIGN
    assert _raw(f, A, 66, 1, 64, 2, B, None) == q8.Q8_ERR_ALIGN     # ld_x % 4
    assert _raw(f, A, 64, 0, 64, 2, B, None) == q8.Q8_OK            # no rows: no-op, no launch


def test_repack_validation():
    f = "q8_repack_weights"
    assert _raw(f, None, 64, 256, B, None) == q8.Q8_ERR_ARG
    assert _raw(f, A, 0, 256, B, None) == q8.Q8_ERR_ARG
    assert _raw(f, A, 32, 256, B, None) == q8.Q8_ERR_SHAPE          # n % 64
    assert _raw(f, A, 64, 224, B, None) == q8.Q8_ERR_SHAPE          # k % 256
    assert _raw(f, A + 2, 64, 256, B, None) == q8.Q8_ERR_ALIGN


def test_matmul_validation():
    f = "q8_matmul"
    ok = dict(x=A, m=1, w=B, layout=1, n=2048, k=2048, y=C, ld=2048, ws=D, wsb=1 << 30)

    def call(**kw):
        a = {**ok, **kw}
        return _raw(f, a["x"], a["m"], a["w"], a["layout"], a["n"], a["k"], a["y"], a["ld"], a["ws"], a["wsb"], None)

    assert call(x=None) == q8.Q8_ERR_ARG
    assert call(m=0) == q8.Q8_ERR_ARG
    assert call(ld=2047) == q8.Q8_ERR_ARG
    assert call(layout=2) == q8.Q8_ERR_ARG
    assert call(k=2080) == q8.Q8_ERR_SHAPE                          # k % 256
    assert call(n=2000) == q8.Q8_ERR_SHAPE                          # packed needs n % 64
    assert call(m=16, layout=0) == q8.Q8_ERR_SHAPE                  # GEMM reads packed weights only
    assert call(w=B + 8) == q8.Q8_ERR_ALIGN
    assert call(y=C + 4) == q8.Q8_ERR_ALIGN
    assert call(k=8192, ws=None) == q8.Q8_ERR_WORKSPACE             # 2048 x 8192 splits by segment
    assert call(k=8192, wsb=100) == q8.Q8_ERR_WORKSPACE
    assert call(k=8192, ws=D + 4) == q8.Q8_ERR_ALIGN


def test_quantize_matmul_validation():
    f = "q8_quantize_matmul"
    ok = dict(x=A, ld=2048, m=1, w=B, layout=1, n=2048, k=2048, y=C, ldy=2048, ws=D, wsb=1 << 30)

    def call(**kw):
        a = {**ok, **kw}
        return _raw(f, a["x"], a["ld"], a["m"], a["w"], a["layout"], a["n"], a["k"], a["y"], a["ldy"], a["ws"],
                    a["wsb"], None)

    assert call(x=None) == q8.Q8_ERR_ARG
    assert call(ld=2000) == q8.Q8_ERR_ARG
    assert call(ldy=100) == q8.Q8_ERR_ARG
    assert call(layout=2) == q8.Q8_ERR_ARG
    assert call(m=9) == q8.Q8_ERR_SHAPE                             # fused path is the decode GEMV only
    assert call(k=2080, ld=2080) == q8.Q8_ERR_SHAPE
    assert call(n=100) == q8.Q8_ERR_SHAPE
    assert call(ld=2050) == q8.Q8_ERR_ALIGN
    assert call(x=A + 4) == q8.Q8_ERR_ALIGN
    assert call(k=8192, ld=8192, ws=None) == q8.Q8_ERR_WORKSPACE


def test_grouped_validation():
    f = "q8_grouped_matmul"
    ok = dict(x=A, xr=16, pp=0, ids=B, t=16, topk=8, w=C, E=256, stride=2048 * 7168 // 32 * 34, n=2048, k=7168,
              y=D, ws=D + (1 << 20), wsb=1 << 20)

    def call(**kw):
        a = {**ok, **kw}
        return _raw(f, a["x"], a["xr"], a["pp"], a["ids"], a["t"], a["topk"], a["w"], a["E"], a["stride"], a["n"],
                    a["k"], a["y"], a["ws"], a["wsb"], None)

    assert call(ids=None) == q8.Q8_ERR_ARG
    assert call(xr=128) == q8.Q8_ERR_ARG                            # rows must be tokens when not per pair
    assert call(pp=1) == q8.Q8_ERR_ARG                              # ... and tokens*topk when per pair
    assert call(pp=2) == q8.Q8_ERR_ARG
    assert call(topk=300) == q8.Q8_ERR_SHAPE
    assert call(E=2048) == q8.Q8_ERR_SHAPE
    assert call(stride=100) == q8.Q8_ERR_SHAPE
    assert call(n=2000) == q8.Q8_ERR_SHAPE
    assert call(wsb=16) == q8.Q8_ERR_WORKSPACE
    assert call(ids=B + 2) == q8.Q8_ERR_ALIGN


def _seq(steps, m, ws=D, wsb=1 << 30):
    arr, count = q8._steps(steps)
    return _raw("q8_quantize_matmul_sequence", arr, count, m, ws, wsb, None)


def test_sequence_workspace_and_validation():
    down = (A, 8192, B, 2048, 8192, C, 2048)
    o = (A, 2048, B, 2048, 2048, C, 2048)
    # status line, then 33 counters of 128 bytes per step (rounded up to 4 KB),
    # sixteen flag lines of 72 steps x 128 bytes (each step's flag in a cache
    # line of its own), then each split step's tile counters (256-byte
    # aligned) and segment sums

    def head(count):
        return (256 + 33 * 128 * count + 4095) // 4096 * 4096 + 16 * 72 * 128

    assert q8.q8_sequence_workspace_bytes([o], 1) == head(1) == 8192 + 16 * 9216
    assert q8.q8_sequence_workspace_bytes([down], 1) == head(1) + 256 + 4 * 1 * 2048 * 4
    assert q8.q8_sequence_workspace_bytes([o, down, o], 2) == head(3) + 256 + 4 * 2 * 2048 * 4
    assert q8.q8_sequence_workspace_bytes([o] * 16, 1) == head(16) == 69632 + 16 * 9216
    assert q8.q8_sequence_workspace_bytes([], 1) == 0
    assert q8.q8_sequence_workspace_bytes([o], 9) == 0
    assert _seq([], 1) == q8.Q8_ERR_ARG
    assert _seq([o], 0) == q8.Q8_ERR_ARG
    assert _seq([(None, 2048, B, 2048, 2048, C, 2048)], 1) == q8.Q8_ERR_ARG
    assert _seq([(A, 2000, B, 2048, 2048, C, 2048)], 1) == q8.Q8_ERR_ARG      # ld_x < k
    assert _seq([(A, 2048, B, 2048, 2048, C, 100)], 1) == q8.Q8_ERR_ARG       # ld_y < n
    assert _seq([o], 9) == q8.Q8_ERR_SHAPE                                     # decode rows only
    assert _seq([o] * (q8.Q8_SEQUENCE_MAX_STEPS + 1), 1) == q8.Q8_ERR_SHAPE
    assert _seq([o, (A, 2048, B, 2000, 2048, C, 2048)], 1) == q8.Q8_ERR_SHAPE  # n % 64
    assert _seq([(A, 2080, B, 2048, 2080, C, 2048)], 1) == q8.Q8_ERR_SHAPE     # k % 256
    assert _seq([(A + 4, 2048, B, 2048, 2048, C, 2048)], 1) == q8.Q8_ERR_ALIGN
    assert _seq([(A, 2050, B, 2048, 2048, C, 2048)], 1) == q8.Q8_ERR_ALIGN
    assert _seq([o], 1, ws=None) == q8.Q8_ERR_WORKSPACE
    assert _seq([down], 1, wsb=1024) == q8.Q8_ERR_WORKSPACE
    assert _seq([o], 1, ws=D + 8) == q8.Q8_ERR_ALIGN


def test_sequence_aliasing_is_rejected():
    """Every x must be ready before the call: a y over any x (the in-place
    chaining y_i == x_(i+1) among them), two y's sharing bytes, or the
    workspace over an x or y is refused before any HIP call."""
    E, F, G = 0x7F0000500000, 0x7F0000600000, 0x7F0000700000
    s0 = (A, 2048, B, 2048, 2048, C, 2048)
    s1 = (E, 2048, B, 2048, 2048, F, 2048)
    ws = q8.q8_sequence_workspace_bytes([s0, s1], 1)
    assert _seq([s0, s1], 1, ws=G, wsb=ws) == q8.Q8_ERR_DEVICE           # valid: reaches the device check
    assert _seq([s0, (C, 2048, B, 2048, 2048, F, 2048)], 1, ws=G, wsb=ws) == q8.Q8_ERR_ARG    # y_0 == x_1
    assert _seq([s0, (E, 2048, B, 2048, 2048, A, 2048)], 1, ws=G, wsb=ws) == q8.Q8_ERR_ARG    # y_1 over x_0
    assert _seq([s0, (E, 2048, B, 2048, 2048, C + 4096, 2048)], 1, ws=G, wsb=ws) == q8.Q8_ERR_ARG  # y's overlap
    assert _seq([s0, (E, 2048, B, 2048, 2048, C + 8192, 2048)], 1, ws=G, wsb=ws) == q8.Q8_ERR_DEVICE  # adjacent
    assert _seq([s0, (A + 8176, 2048, B, 2048, 2048, F, 2048)], 1, ws=G, wsb=ws) == q8.Q8_ERR_DEVICE  # x's may share
    assert _seq([s0, s1], 1, ws=E, wsb=ws) == q8.Q8_ERR_ARG              # workspace over an x
    assert _seq([s0, s1], 1, ws=F - 4096, wsb=ws) == q8.Q8_ERR_ARG       # workspace over a y
    # with m rows the extents are (m - 1) * ld + n (or k)
    s1m = (E, 4096, B, 2048, 2048, F, 4096)
    ws2 = q8.q8_sequence_workspace_bytes([s0, s1m], 2)
    assert _seq([(A, 4096, B, 2048, 2048, C, 4096), s1m], 2, ws=G, wsb=ws2) == q8.Q8_ERR_DEVICE
    assert _seq([(A, 4096, B, 2048, 2048, E + 4 * 6144, 4096), s1m], 2, ws=G, wsb=ws2) == q8.Q8_ERR_DEVICE  # adjacent
    assert _seq([(A, 4096, B, 2048, 2048, E + 4 * 6144 - 16, 4096), s1m], 2, ws=G, wsb=ws2) == q8.Q8_ERR_ARG


def test_sequence_noalloc_validation():
    """The allocation-free sequence: the same step checks, its workspace limit
    (Q8_SEQUENCE_SCRATCH_BYTES) and the status pointer are checked on the host."""
    f = "q8_quantize_matmul_sequence_noalloc"

    def call(steps, m, status=None):
        arr, count = q8._steps(steps)
        return _raw(f, arr, count, m, status, None)

    E = 0x7F0000500000
    o = (A, 2048, B, 2048, 2048, C, 2048)
    assert call([o], 1) == q8.Q8_ERR_DEVICE                                   # valid: reaches the device check
    assert call([o], 1, status=E) == q8.Q8_ERR_DEVICE
    assert call([o], 1, status=E + 2) == q8.Q8_ERR_ALIGN
    assert call([o], 1, status=C + 64) == q8.Q8_ERR_ARG                       # status inside a y
    assert call([o, (C, 2048, B, 2048, 2048, E, 2048)], 1) == q8.Q8_ERR_ARG   # y_0 == x_1
    assert call([], 1) == q8.Q8_ERR_ARG
    assert call([o], 9) == q8.Q8_ERR_SHAPE
    # 72 down-shaped steps at m = 8 need ~18.9 MB of workspace: beyond the limit
    big = [(A + i * 0x100000, 8192, B, 2048, 8192, 0x7F1000000000 + i * 0x100000, 2048) for i in range(72)]
    assert q8.q8_sequence_workspace_bytes(big, 8) > q8.Q8_SEQUENCE_SCRATCH_BYTES
    assert call(big, 8) == q8.Q8_ERR_WORKSPACE
    # the Llama-3.2-1B-shaped decode step fits at every m <= 8
    layer = [(A, 2048, B, 3072, 2048, C, 3072), (A, 2048, B, 2048, 2048, C, 2048),
             (A, 2048, B, 16384, 2048, C, 16384), (A, 8192, B, 2048, 8192, C, 2048)]
    step = layer * 16 + [(A, 2048, B, 128256, 2048, C, 128256)]
    for m in range(1, 9):
        assert q8.q8_sequence_workspace_bytes(step, m) <= q8.Q8_SEQUENCE_SCRATCH_BYTES


def test_stale_library_is_refused(monkeypatch):
    """A libq8.so built from other sources than the tree's is not loaded."""
    from decode_q8_amd import build
    assert q8.q8_build_digest() == build.source_digest()
    saved = q8._lib
    try:
        q8._lib = None
        monkeypatch.setattr(build, "source_digest", lambda: "0" * 64)
        with pytest.raises(q8.StaleLibraryError):
            q8.lib()
    finally:
        q8._lib = saved


def test_digest_covers_every_included_file():
    """Every file a kernel or host source includes from the source folder
    (the generated GEMM loops among them) is part of the build digest, so
    regenerating one makes the old library stale."""
    import re
    from decode_q8_amd import build
    names = set(os.listdir(build.CSRC))
    covered = {f for f in names if f.endswith((".hip", ".hpp", ".cpp", ".h", ".inc"))}
    for f in covered:
        for inc in re.findall(r'#include\s+"([^"]+)"', open(os.path.join(build.CSRC, f)).read()):
            if inc in names:
                assert inc in covered, (f, inc)
    assert {"gemm_loop.inc", "gemm_strip.inc"} <= covered


def test_device_queries_need_a_device():
    """Without a GPU no call gets as far as a device query."""
    before = q8.q8_device_queries()
    assert _seq([(A, 2048, B, 2048, 2048, C, 2048)], 1) == q8.Q8_ERR_DEVICE
    assert q8.q8_device_queries() == before


def test_rmsnorm_quantize_validation():
    f = "q8_rmsnorm_quantize"
    E = 0x7F0000400000
    assert _raw(f, None, B, B, C, 1, 2048, 1e-5, D, None) == q8.Q8_ERR_ARG
    assert _raw(f, A, B, B, None, 1, 2048, 1e-5, D, None) == q8.Q8_ERR_ARG
    assert _raw(f, A, B, B, C, 1, 2048, 1e-5, None, None) == q8.Q8_ERR_ARG
    assert _raw(f, A, B, B, C, -1, 2048, 1e-5, D, None) == q8.Q8_ERR_ARG
    assert _raw(f, A, B, B, C, 1, 0, 1e-5, D, None) == q8.Q8_ERR_ARG
    assert _raw(f, A, B, B, C, 1, 2048, -1e-5, D, None) == q8.Q8_ERR_ARG      # eps < 0
    assert _raw(f, A, B, B, C, 1, 2048, float("nan"), D, None) == q8.Q8_ERR_ARG
    assert _raw(f, A, B, B, C, 1, 2048, float("inf"), D, None) == q8.Q8_ERR_ARG
    assert _raw(f, A, B, B, C, 1, 2040, 1e-5, D, None) == q8.Q8_ERR_SHAPE     # k % 32
    assert _raw(f, A, B, B, C, 1, q8.Q8_NORM_MAX_K + 32, 1e-5, D, None) == q8.Q8_ERR_SHAPE
    assert _raw(f, A, B, B, C, 2 ** 31, 2048, 1e-5, D, None) == q8.Q8_ERR_SHAPE
    assert _raw(f, A + 4, B, B, C, 1, 2048, 1e-5, D, None) == q8.Q8_ERR_ALIGN
    assert _raw(f, A, B + 8, B, C, 1, 2048, 1e-5, D, None) == q8.Q8_ERR_ALIGN
    assert _raw(f, A, B, B, C, 1, 2048, 1e-5, D + 4, None) == q8.Q8_ERR_ALIGN
    # q_out overlapping an input, residual_out partially overlapping x
    assert _raw(f, A, B, B, C, 1, 2048, 1e-5, A + 4096, None) == q8.Q8_ERR_ARG
    assert _raw(f, A, B, A + 16, C, 1, 2048, 1e-5, D, None) == q8.Q8_ERR_ARG
    assert _raw(f, A, B, E, C, 1, 2048, 1e-5, C + 16, None) == q8.Q8_ERR_ARG  # q_out over the weight
    assert _raw(f, A, B, B, C, 0, 2048, 1e-5, D, None) == q8.Q8_OK            # no rows: no launch


def test_moe_route_validation():
    f = "q8_moe_route"
    assert _raw(f, None, 16, 256, 8, 1, B, C, None) == q8.Q8_ERR_ARG
    assert _raw(f, A, 16, 256, 8, 1, None, C, None) == q8.Q8_ERR_ARG
    assert _raw(f, A, 16, 256, 8, 1, B, None, None) == q8.Q8_ERR_ARG
    assert _raw(f, A, -1, 256, 8, 1, B, C, None) == q8.Q8_ERR_ARG
    assert _raw(f, A, 16, 0, 1, 1, B, C, None) == q8.Q8_ERR_ARG
    assert _raw(f, A, 16, 256, 0, 1, B, C, None) == q8.Q8_ERR_ARG
    assert _raw(f, A, 16, 4, 8, 1, B, C, None) == q8.Q8_ERR_SHAPE          # topk > n_experts
    assert _raw(f, A, 16, 2048, 8, 1, B, C, None) == q8.Q8_ERR_SHAPE       # n_experts > 1024
    assert _raw(f, A, 16, 256, 33, 1, B, C, None) == q8.Q8_ERR_SHAPE       # topk > 32
    assert _raw(f, A + 2, 16, 256, 8, 1, B, C, None) == q8.Q8_ERR_ALIGN
    assert _raw(f, A, 16, 256, 8, 1, B + 2, C, None) == q8.Q8_ERR_ALIGN
    assert _raw(f, A, 16, 256, 8, 1, B, B + 64, None) == q8.Q8_ERR_ARG     # ids and weights overlap
    assert _raw(f, A, 0, 256, 8, 1, B, C, None) == q8.Q8_OK                # no tokens: no launch


def test_swiglu_validation():
    f = "q8_swiglu_quantize"
    assert _raw(f, None, 4096, B, 4096, 128, 2048, C, None) == q8.Q8_ERR_ARG
    assert _raw(f, A, 4096, B, 4096, 128, 2048, None, None) == q8.Q8_ERR_ARG
    assert _raw(f, A, 1000, B, 4096, 128, 2048, C, None) == q8.Q8_ERR_ARG  # ld_gate < n
    assert _raw(f, A, 4096, B, 4096, -1, 2048, C, None) == q8.Q8_ERR_ARG
    assert _raw(f, A, 4096, B, 4096, 128, 2040, C, None) == q8.Q8_ERR_SHAPE  # n % 32
    assert _raw(f, A + 4, 4096, B, 4096, 128, 2048, C, None) == q8.Q8_ERR_ALIGN
    assert _raw(f, A, 4098, B, 4096, 128, 2048, C, None) == q8.Q8_ERR_ALIGN  # ld % 4
    assert _raw(f, A, 4096, A + 8192, 4096, 128, 2048, A + 4096, None) == q8.Q8_ERR_ARG  # q_out over gate
    assert _raw(f, A, 4096, B, 4096, 0, 2048, C, None) == q8.Q8_OK


def test_combine_validation():
    f = "q8_moe_combine"
    assert _raw(f, None, 7168, B, 16, 8, 7168, C, 7168, None) == q8.Q8_ERR_ARG
    assert _raw(f, A, 7168, B, 16, 0, 7168, C, 7168, None) == q8.Q8_ERR_ARG
    assert _raw(f, A, 7000, B, 16, 8, 7168, C, 7168, None) == q8.Q8_ERR_ARG   # ld_y < n
    assert _raw(f, A, 7168, B, 16, 8, 7166, C, 7168, None) == q8.Q8_ERR_SHAPE  # n % 4
    assert _raw(f, A + 4, 7168, B, 16, 8, 7168, C, 7168, None) == q8.Q8_ERR_ALIGN
    assert _raw(f, A, 7168, B + 1, 16, 8, 7168, C, 7168, None) == q8.Q8_ERR_ALIGN
    assert _raw(f, A, 7168, B, 16, 8, 7168, A + 1024, 7168, None) == q8.Q8_ERR_ARG  # out over y
    assert _raw(f, A, 7168, B, 0, 8, 7168, C, 7168, None) == q8.Q8_OK


def test_kv_write_validation():
    f = "q8_kv_write"
    E, F = 0x7F0000400000, 0x7F0000500000
    ok = [A, 16, 32, 8, 64, B, 4096, C, D, None, None, 1e-5, E, 8192, F, A + 0x10000000, B + 0x10000000,
          C + 0x10000000, D + 0x10000000, None, None]

    def call(**kw):
        args = list(ok)
        names = ["qkv", "tokens", "H", "Hk", "hd", "pos", "max_pos", "cos", "sin", "qg", "kg", "eps", "slots",
                 "n_slots", "q_out", "kc", "ks", "vc", "vs", "status", "stream"]
        for k, v in kw.items():
            args[names.index(k)] = v
        return _raw(f, *args)

    assert call(qkv=None) == q8.Q8_ERR_ARG
    assert call(pos=None) == q8.Q8_ERR_ARG
    assert call(tokens=-1) == q8.Q8_ERR_ARG
    assert call(max_pos=0) == q8.Q8_ERR_ARG
    assert call(n_slots=0) == q8.Q8_ERR_ARG
    assert call(qg=A + 0x20000000, eps=-1.0) == q8.Q8_ERR_ARG
    assert call(H=30) == q8.Q8_ERR_SHAPE                     # n_heads % n_kv
    assert call(hd=96) == q8.Q8_ERR_SHAPE
    assert call(qkv=A + 4) == q8.Q8_ERR_ALIGN
    assert call(ks=B + 0x10000002) == q8.Q8_ERR_ALIGN
    assert call(q_out=A + 1024) == q8.Q8_ERR_ARG             # q_out over qkv
    assert call(tokens=0) == q8.Q8_OK


def test_attention_validation():
    f = "q8_attention_decode"
    assert q8.q8_attention_workspace_bytes(16, 32, 8, 64, 4096) == 256 + 16 * 8 * 16 * 4 * 66 * 4
    assert q8.q8_attention_workspace_bytes(16, 32, 8, 96, 4096) == 0
    assert q8.q8_attention_workspace_bytes(16, 48, 8, 64, 4096) == 0   # group of 6
    assert q8.q8_attention_workspace_bytes(1, 8, 8, 64, 65536) > 0
    assert q8.q8_attention_workspace_bytes(1, 8, 8, 64, 65537) == 0     # beyond Q8_ATTENTION_MAX_LEN
    need = q8.q8_attention_workspace_bytes(4, 8, 2, 64, 512)
    E, F, G_, H_ = 0x7F0000400000, 0x7F0000500000, 0x7F0000600000, 0x7F0000700000
    ok = [A, 4, 8, 2, 64, B, C, D, E, 1024, F, F + 64, 512, 0.125, G_, H_, need, None]

    def call(**kw):
        args = list(ok)
        names = ["q", "seqs", "H", "Hk", "hd", "kc", "ks", "vc", "vs", "n_slots", "base", "len", "max_len", "scale",
                 "out", "ws", "wsb", "stream"]
        for k, v in kw.items():
            args[names.index(k)] = v
        return _raw(f, *args)

    assert call(q=None) == q8.Q8_ERR_ARG
    assert call(max_len=0) == q8.Q8_ERR_ARG
    assert call(scale=float("nan")) == q8.Q8_ERR_ARG
    assert call(hd=256) == q8.Q8_ERR_SHAPE
    assert call(H=6) == q8.Q8_ERR_SHAPE                      # group of 3
    assert call(q=A + 8) == q8.Q8_ERR_ALIGN
    assert call(ws=None) == q8.Q8_ERR_WORKSPACE
    assert call(wsb=need - 4) == q8.Q8_ERR_WORKSPACE
    assert call(out=A + 64) == q8.Q8_ERR_ARG                 # out over q
    assert call(seqs=0) == q8.Q8_OK


def _no_gpu():
    import torch
    return torch.cuda.device_count() == 0


@pytest.mark.skipif(not _no_gpu(), reason="checks the no-device error; would launch on a GPU host")
def test_valid_request_without_device_reports_device_error():
    assert _raw("q8_quantize_rows", A, 64, 1, 64, 2, B, None) == q8.Q8_ERR_DEVICE
    assert _raw("q8_matmul", A, 1, B, 1, 131072, 2048, C, 131072, None, 0, None) == q8.Q8_ERR_DEVICE
    assert _seq([(A, 2048, B, 2048, 2048, C, 2048)], 1) == q8.Q8_ERR_DEVICE
    assert _raw("q8_rmsnorm_quantize", A, B, B, C, 1, 2048, 1e-5, D, None) == q8.Q8_ERR_DEVICE
    assert _raw("q8_rmsnorm_quantize", A, None, A, C, 1, 2048, 1e-5, D, None) == q8.Q8_ERR_DEVICE  # in place on x
    assert _raw("q8_moe_route", A, 16, 256, 8, 1, B, C, None) == q8.Q8_ERR_DEVICE
    assert _raw("q8_swiglu_quantize", A, 4096, A + 8192, 4096, 128, 2048, C, None) == q8.Q8_ERR_DEVICE
    assert _raw("q8_moe_combine", A, 7168, B, 16, 8, 7168, 0x7F0000400000, 7168, None) == q8.Q8_ERR_DEVICE
    assert _raw("q8_kv_write", A, 16, 32, 8, 64, B, 4096, C, D, None, None, 1e-5, 0x7F0000400000, 8192,
                0x7F0000500000, A + 0x10000000, B + 0x10000000, C + 0x10000000, D + 0x10000000, None,
                None) == q8.Q8_ERR_DEVICE
    need = q8.q8_attention_workspace_bytes(4, 8, 2, 64, 512)
    assert _raw("q8_attention_decode", A, 4, 8, 2, 64, B, C, D, 0x7F0000400000, 1024, 0x7F0000500000,
                0x7F0000500040, 512, 0.125, 0x7F0000600000, 0x7F0000700000, need, None) == q8.Q8_ERR_DEVICE


def test_stream_read_validation():
    f = "q8_stream_read"
    assert _raw(f, None, 1024, B, None) == q8.Q8_ERR_ARG
    assert _raw(f, A, 1024, None, None) == q8.Q8_ERR_ARG
    assert _raw(f, A, 1000, B, None) == q8.Q8_ERR_SHAPE           # not a multiple of 16
    assert _raw(f, A + 4, 1024, B, None) == q8.Q8_ERR_ALIGN
    assert _raw(f, A, 1024, B + 2, None) == q8.Q8_ERR_ALIGN
    assert _raw(f, A, 1024, A + 512, None) == q8.Q8_ERR_ARG      # sink inside the buffer
    assert _raw(f, A, 0, B, None) == q8.Q8_OK                    # nothing to read: no-op, no launch


def test_sequence_status_word_helpers():
    """sequence_status reads the int32 at byte 0 of a sequence workspace;
    check_sequence passes on 0 and raises Q8Error (Q8_ERR_LAUNCH) on a
    timed-out wait (host tensors stand in for the device workspace)."""
    import torch
    ws = torch.zeros(256, dtype=torch.uint8)
    assert q8.sequence_status(ws) == 0
    q8.check_sequence(ws)
    ws[:4].view(torch.int32)[0] = q8.Q8_ERR_LAUNCH
    assert q8.sequence_status(ws) == q8.Q8_ERR_LAUNCH
    with pytest.raises(q8.Q8Error) as e:
        q8.check_sequence(ws)
    assert e.value.status == q8.Q8_ERR_LAUNCH
