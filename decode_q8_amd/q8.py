"""ctypes binding of libq8 (include/q8.h), one Python function per C entry point
with the same name.

Marshalling only: tensors become device pointers (``data_ptr()``), streams
become ``hipStream_t`` handles (default: torch's current stream), and a
non-zero status raises ``Q8Error``.  Every step of the computation runs in the
library's HIP kernels; there is no Python or CPU implementation behind these
functions, and importing fails loudly if the library cannot be loaded.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
# Q8_LIB names another build of the same sources (the host-only sanitizer
# build of the test suite); the digest check below applies to it as well.
LIB_PATH = os.environ.get("Q8_LIB") or os.path.join(HERE, "libq8.so")

Q8_OK, Q8_ERR_ARG, Q8_ERR_SHAPE, Q8_ERR_ALIGN, Q8_ERR_WORKSPACE, Q8_ERR_DEVICE, Q8_ERR_LAUNCH = range(7)
Q8_LAYOUT_ROWS, Q8_LAYOUT_PACKED, Q8_LAYOUT_ACT = 0, 1, 2
Q8_BLOCK = 32
Q8_BLOCK_BYTES = 34
Q8_TILE_ROWS = 64
Q8_GEMV_MAX_ROWS = 8
Q8_SEQUENCE_MAX_STEPS = 72
Q8_SEQUENCE_SCRATCH_BYTES = 8 << 20
Q8_ABI_VERSION = 5
Q8_NORM_MAX_K = 16384
Q8_ROUTE_MAX_EXPERTS = 1024
Q8_ROUTE_MAX_TOPK = 32


class q8_gemv_step(ctypes.Structure):
    """One GEMV of a sequence (the C struct q8_gemv_step)."""
    _fields_ = [("x", ctypes.c_void_p), ("w", ctypes.c_void_p), ("y", ctypes.c_void_p), ("ld_x", ctypes.c_int64),
                ("ld_y", ctypes.c_int64), ("n", ctypes.c_int64), ("k", ctypes.c_int64)]

# The C entry points declared in include/q8.h, with their ctypes signatures.
_P, _I64, _I, _SZ, _U32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t, ctypes.c_uint32
SIGNATURES = {
    "q8_abi_version": ([], _U32),
    "q8_device_queries": ([], _U32),
    "q8_build_digest": ([], ctypes.c_char_p),
    "q8_status_str": ([_I], ctypes.c_char_p),
    "q8_quantized_bytes": ([_I64, _I64], _SZ),
    "q8_quantize_rows": ([_P, _I64, _I64, _I64, _I, _P, _P], _I),
    "q8_repack_weights": ([_P, _I64, _I64, _P, _P], _I),
    "q8_matmul_workspace_bytes": ([_I64, _I64, _I64], _SZ),
    "q8_matmul": ([_P, _I64, _P, _I, _I64, _I64, _P, _I64, _P, _SZ, _P], _I),
    "q8_quantize_matmul": ([_P, _I64, _I64, _P, _I, _I64, _I64, _P, _I64, _P, _SZ, _P], _I),
    "q8_sequence_workspace_bytes": ([_P, _I, _I64], _SZ),
    "q8_quantize_matmul_sequence": ([_P, _I, _I64, _P, _SZ, _P], _I),
    "q8_quantize_matmul_sequence_noalloc": ([_P, _I, _I64, _P, _P], _I),
    "q8_rmsnorm_quantize": ([_P, _P, _P, _P, _I64, _I64, ctypes.c_float, _P, _P], _I),
    "q8_moe_route": ([_P, _I64, _I64, _I, _I, _P, _P, _P], _I),
    "q8_swiglu_quantize": ([_P, _I64, _P, _I64, _I64, _I64, _P, _P], _I),
    "q8_moe_combine": ([_P, _I64, _P, _I64, _I, _I64, _P, _I64, _P], _I),
    "q8_kv_write": ([_P, _I64, _I, _I, _I, _P, _I64, _P, _P, _P, _P, ctypes.c_float, _P, _I64, _P, _P, _P, _P, _P,
                     _P, _P], _I),
    "q8_attention_workspace_bytes": ([_I64, _I, _I, _I, _I64], _SZ),
    "q8_attention_decode": ([_P, _I64, _I, _I, _I, _P, _P, _P, _P, _I64, _P, _P, _I64, ctypes.c_float, _P, _P, _SZ,
                             _P], _I),
    "q8_grouped_workspace_bytes": ([_I64, _I, _I64, _I64, _I64], _SZ),
    "q8_grouped_matmul": ([_P, _I64, _I, _P, _I64, _I, _P, _I64, _I64, _I64, _I64, _P, _P, _SZ, _P], _I),
    "q8_stream_read": ([_P, _SZ, _P, _P], _I),
}


class Q8Error(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_str(status)}")


_lib = None


class StaleLibraryError(RuntimeError):
    """libq8.so was built from other sources than the ones in this tree."""


def lib() -> ctypes.CDLL:
    """Load libq8.so (building it first if no build exists).  A build whose
    recorded source digest differs from this tree's sources is refused: its
    kernels are not the ones the sources describe."""
    global _lib
    if _lib is None:
        from . import build as _build
        if not os.path.exists(LIB_PATH):
            _build.build()
        L = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        built, tree = L.q8_build_digest().decode(), _build.source_digest()
        if built != tree:
            raise StaleLibraryError(f"{LIB_PATH} was built from sources with digest {built}, but the tree's sources "
                                    f"have digest {tree}: rebuild it (__graft_entry__.build())")
        _lib = L
    return _lib


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(s):
    if s is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(s, int):
        return s
    return s.cuda_stream


def _check(status: int, what: str) -> int:
    if status != Q8_OK:
        raise Q8Error(status, what)
    return status


def status_str(status: int) -> str:
    return lib().q8_status_str(status).decode()


def q8_abi_version() -> int:
    return lib().q8_abi_version()


def q8_device_queries() -> int:
    return lib().q8_device_queries()


def q8_build_digest() -> str:
    return lib().q8_build_digest().decode()


def q8_status_str(status: int) -> str:
    return status_str(status)


def q8_quantized_bytes(rows: int, k: int) -> int:
    return lib().q8_quantized_bytes(rows, k)


def q8_matmul_workspace_bytes(m: int, n: int, k: int) -> int:
    return lib().q8_matmul_workspace_bytes(m, n, k)


def _steps(steps):
    """A sequence of (x, ld_x, w, n, k, y, ld_y) tuples (tensors or pointers) ->
    (ctypes array of q8_gemv_step, count)."""
    arr = (q8_gemv_step * max(1, len(steps)))()
    for i, (x, ld_x, w, n, k, y, ld_y) in enumerate(steps):
        arr[i] = q8_gemv_step(_ptr(x), _ptr(w), _ptr(y), ld_x, ld_y, n, k)
    return arr, len(steps)


def q8_sequence_workspace_bytes(steps, m: int) -> int:
    arr, count = _steps(steps)
    return lib().q8_sequence_workspace_bytes(arr, count, m)


def q8_quantize_matmul_sequence(steps, m: int, workspace, workspace_bytes: int, stream=None) -> int:
    """steps: sequence of (x, ld_x, w, n, k, y, ld_y)."""
    arr, count = _steps(steps)
    return _check(lib().q8_quantize_matmul_sequence(arr, count, m, _ptr(workspace), workspace_bytes,
                                                    _stream(stream)), "q8_quantize_matmul_sequence")


def sequence_status(workspace) -> int:
    """The status word a q8_quantize_matmul_sequence call left at byte 0 of its
    workspace (waits for the current stream): 0, or Q8_ERR_LAUNCH when one of
    the call's internal waits timed out, in which case its outputs are
    undefined and the workspace must be zero-filled again before reuse."""
    return int(workspace[:4].view(__import__("torch").int32).cpu()[0])


def check_sequence(workspace, what: str = "q8_quantize_matmul_sequence") -> None:
    """Raise Q8Error if the sequence call on this workspace reported a timeout."""
    _check(sequence_status(workspace), what)


def q8_quantize_matmul_sequence_noalloc(steps, m: int, status=None, stream=None) -> int:
    """steps: sequence of (x, ld_x, w, n, k, y, ld_y); the library's own
    per-GPU workspace; status: optional device int32 receiving the status word."""
    arr, count = _steps(steps)
    return _check(lib().q8_quantize_matmul_sequence_noalloc(arr, count, m, _ptr(status), _stream(stream)),
                  "q8_quantize_matmul_sequence_noalloc")


def q8_grouped_workspace_bytes(tokens: int, topk: int, n_experts: int, n: int, k: int) -> int:
    return lib().q8_grouped_workspace_bytes(tokens, topk, n_experts, n, k)


def q8_quantize_rows(x, ld_x: int, rows: int, k: int, layout: int, q_out, stream=None) -> int:
    return _check(lib().q8_quantize_rows(_ptr(x), ld_x, rows, k, layout, _ptr(q_out), _stream(stream)),
                  "q8_quantize_rows")


def q8_repack_weights(w_rows, n: int, k: int, w_packed, stream=None) -> int:
    return _check(lib().q8_repack_weights(_ptr(w_rows), n, k, _ptr(w_packed), _stream(stream)), "q8_repack_weights")


def q8_matmul(x_q, m: int, w, layout: int, n: int, k: int, y, ld_y: int, workspace=None, workspace_bytes: int = 0,
              stream=None) -> int:
    return _check(lib().q8_matmul(_ptr(x_q), m, _ptr(w), layout, n, k, _ptr(y), ld_y, _ptr(workspace),
                                  workspace_bytes, _stream(stream)), "q8_matmul")


def q8_quantize_matmul(x, ld_x: int, m: int, w, layout: int, n: int, k: int, y, ld_y: int, workspace=None,
                       workspace_bytes: int = 0, stream=None) -> int:
    return _check(lib().q8_quantize_matmul(_ptr(x), ld_x, m, _ptr(w), layout, n, k, _ptr(y), ld_y, _ptr(workspace),
                                           workspace_bytes, _stream(stream)), "q8_quantize_matmul")


def q8_rmsnorm_quantize(x, residual_in, residual_out, weight, rows: int, k: int, eps: float, q_out,
                        stream=None) -> int:
    return _check(lib().q8_rmsnorm_quantize(_ptr(x), _ptr(residual_in), _ptr(residual_out), _ptr(weight), rows, k,
                                            float(eps), _ptr(q_out), _stream(stream)), "q8_rmsnorm_quantize")


def q8_moe_route(logits, tokens: int, n_experts: int, topk: int, normalize: bool, ids, weights, stream=None) -> int:
    return _check(lib().q8_moe_route(_ptr(logits), tokens, n_experts, topk, int(bool(normalize)), _ptr(ids),
                                     _ptr(weights), _stream(stream)), "q8_moe_route")


def q8_swiglu_quantize(gate, ld_gate: int, up, ld_up: int, rows: int, n: int, q_out, stream=None) -> int:
    return _check(lib().q8_swiglu_quantize(_ptr(gate), ld_gate, _ptr(up), ld_up, rows, n, _ptr(q_out),
                                           _stream(stream)), "q8_swiglu_quantize")


def q8_moe_combine(y, ld_y: int, weights, tokens: int, topk: int, n: int, out, ld_out: int, stream=None) -> int:
    return _check(lib().q8_moe_combine(_ptr(y), ld_y, _ptr(weights), tokens, topk, n, _ptr(out), ld_out,
                                       _stream(stream)), "q8_moe_combine")


def q8_kv_write(qkv, tokens: int, n_heads: int, n_kv: int, head_dim: int, positions, max_pos: int, cos_tab, sin_tab,
                q_gain, k_gain, eps: float, slots, n_slots: int, q_out, k_cache, k_scale, v_cache, v_scale,
                status=None, stream=None) -> int:
    return _check(lib().q8_kv_write(_ptr(qkv), tokens, n_heads, n_kv, head_dim, _ptr(positions), max_pos,
                                    _ptr(cos_tab), _ptr(sin_tab), _ptr(q_gain), _ptr(k_gain), float(eps), _ptr(slots),
                                    n_slots, _ptr(q_out), _ptr(k_cache), _ptr(k_scale), _ptr(v_cache), _ptr(v_scale),
                                    _ptr(status), _stream(stream)), "q8_kv_write")


def q8_attention_workspace_bytes(seqs: int, n_heads: int, n_kv: int, head_dim: int, max_len: int) -> int:
    return lib().q8_attention_workspace_bytes(seqs, n_heads, n_kv, head_dim, max_len)


def q8_attention_decode(q, seqs: int, n_heads: int, n_kv: int, head_dim: int, k_cache, k_scale, v_cache, v_scale,
                        n_slots: int, base, length, max_len: int, scale: float, out, workspace, workspace_bytes: int,
                        stream=None) -> int:
    return _check(lib().q8_attention_decode(_ptr(q), seqs, n_heads, n_kv, head_dim, _ptr(k_cache), _ptr(k_scale),
                                            _ptr(v_cache), _ptr(v_scale), n_slots, _ptr(base), _ptr(length), max_len,
                                            float(scale), _ptr(out), _ptr(workspace), workspace_bytes,
                                            _stream(stream)), "q8_attention_decode")


def q8_grouped_matmul(x_q, x_rows: int, x_per_pair: int, topk_ids, tokens: int, topk: int, w_experts,
                      n_experts: int, expert_stride_bytes: int, n: int, k: int, y, workspace, workspace_bytes: int,
                      stream=None) -> int:
    return _check(lib().q8_grouped_matmul(_ptr(x_q), x_rows, int(x_per_pair), _ptr(topk_ids), tokens, topk,
                                          _ptr(w_experts), n_experts, expert_stride_bytes, n, k, _ptr(y),
                                          _ptr(workspace), workspace_bytes, _stream(stream)), "q8_grouped_matmul")


# --- torch conveniences (allocation + one call each) -------------------------

def q8_stream_read(buf, nbytes: int, sink, stream=None) -> int:
    return _check(lib().q8_stream_read(_ptr(buf), nbytes, _ptr(sink), _stream(stream)), "q8_stream_read")


def quantize(x, layout: int = Q8_LAYOUT_ACT, stream=None):
    """fp32 [rows][k] CUDA tensor (unit column stride) -> new uint8 tensor."""
    import torch
    assert x.dtype == torch.float32 and x.dim() == 2 and x.stride(1) == 1
    rows, k = x.shape
    out = torch.empty(q8_quantized_bytes(rows, k), dtype=torch.uint8, device=x.device)
    q8_quantize_rows(x, x.stride(0), rows, k, layout, out, stream)
    return out


def repack(w_rows, n: int, k: int, stream=None):
    import torch
    out = torch.empty_like(w_rows)
    q8_repack_weights(w_rows, n, k, out, stream)
    return out


def workspace(m: int, n: int, k: int, device="cuda"):
    """A zero-filled workspace for q8_matmul / q8_quantize_matmul (None when
    the shape needs none)."""
    import torch
    need = q8_matmul_workspace_bytes(m, n, k)
    return torch.zeros(need, dtype=torch.uint8, device=device) if need else None


def quantize_matmul(x, w, layout: int, n: int, ws=None, stream=None):
    """fp32 [m][k] CUDA tensor (m <= 8) -> new fp32 [m][n] tensor."""
    import torch
    assert x.dtype == torch.float32 and x.dim() == 2 and x.stride(1) == 1
    m, k = x.shape
    y = torch.empty((m, n), dtype=torch.float32, device=x.device)
    if ws is None:
        ws = workspace(m, n, k, x.device)
    q8_quantize_matmul(x, x.stride(0), m, w, layout, n, k, y, n, ws, 0 if ws is None else ws.numel(), stream)
    return y


def matmul(x_q, m: int, w, layout: int, n: int, k: int, ws=None, stream=None):
    """-> new fp32 [m][n] tensor; allocates a zeroed workspace if none is given."""
    import torch
    y = torch.empty((m, n), dtype=torch.float32, device=w.device)
    if ws is None:
        ws = workspace(m, n, k, w.device)
    q8_matmul(x_q, m, w, layout, n, k, y, n, ws, 0 if ws is None else ws.numel(), stream)
    return y


def rmsnorm_quantize(x, residual, weight, eps: float, residual_out="in_place", stream=None):
    """fp32 [rows][k] CUDA tensors -> new uint8 Q8_LAYOUT_ACT tensor of the
    normalized rows.  residual (or None) is updated in place to residual + x
    unless residual_out names another tensor (or None: not stored)."""
    import torch
    assert x.dtype == torch.float32 and x.dim() == 2 and x.is_contiguous()
    rows, k = x.shape
    if isinstance(residual_out, str):
        residual_out = residual
    out = torch.empty(q8_quantized_bytes(rows, k), dtype=torch.uint8, device=x.device)
    q8_rmsnorm_quantize(x, residual, residual_out, weight, rows, k, eps, out, stream)
    return out
