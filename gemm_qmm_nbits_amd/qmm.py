"""Thin ctypes binding of libqmm.so (include/qmm.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI.  Tensors are torch tensors on the GPU; their
data_ptr() and the current torch stream are passed through.  If the library is
missing the binding raises: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, Structure, c_double, c_float, c_int, c_int64, c_size_t, c_void_p

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libqmm.so")

QMM_F32, QMM_F16, QMM_BF16 = 0, 1, 2
QMM_ZP_NONE, QMM_ZP_PACKED, QMM_ZP_F16, QMM_ZP_UNIFORM = 0, 1, 2, 3
QMOE_FP, QMOE_INT8_ACT = 0, 1
STATUS = {0: "QMM_OK", -1: "QMM_E_NULL", -2: "QMM_E_DTYPE", -3: "QMM_E_BITS", -4: "QMM_E_BLOCK",
          -5: "QMM_E_SHAPE", -6: "QMM_E_ALIGN", -7: "QMM_E_WORKSPACE", -8: "QMM_E_MODE",
          -9: "QMM_E_DEVICE", -10: "QMM_E_PARAM"}
ENTRY_NBITS, ENTRY_CODEBOOK, ENTRY_QMOE_FC1, ENTRY_QMOE_FC2, ENTRY_QMOE_FUSED = 0, 1, 2, 3, 4


class QmmError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        name = STATUS.get(status, f"hipError {status}")
        super().__init__(f"{fn} failed: {name} ({status})")


class qmoe_weights(Structure):
    _fields_ = [("W", c_void_p), ("scales", c_void_p), ("zp", c_void_p), ("bias", c_void_p)]


class qmm_qparams(Structure):
    _fields_ = [("scale", c_float), ("zero_point", ctypes.c_int32)]


class qmm_nested_absmax(Structure):
    _fields_ = [("codes", c_void_p), ("table", c_void_p), ("scales", c_void_p), ("offset", c_float),
                ("group", c_int)]


_lib = None

_SIGS = {
    "qmm_nbits": (c_int, [c_void_p, c_int, c_int64, c_int64, c_int64, c_void_p, c_int, c_int,
                          c_void_p, c_void_p, c_int, c_float, c_void_p, c_void_p, c_int,
                          c_void_p, c_size_t, c_void_p]),
    "qmm_nbits_workspace_bytes": (c_size_t, [c_int64, c_int64, c_int64, c_int]),
    "qmm_validate_nbits": (c_int, [c_void_p, c_int, c_int64, c_int64, c_int64, c_void_p, c_int,
                                   c_int, c_void_p, c_void_p, c_int, c_void_p, c_void_p, c_int,
                                   c_void_p, c_size_t]),
    "qmm_codebook4": (c_int, [c_void_p, c_int, c_int64, c_int64, c_int64, c_void_p, c_int,
                              c_void_p, c_void_p, c_void_p, c_void_p, c_int, c_void_p, c_size_t,
                              c_void_p]),
    "qmm_codebook4_workspace_bytes": (c_size_t, [c_int64, c_int64, c_int64, c_int]),
    "qmm_validate_codebook4": (c_int, [c_void_p, c_int, c_int64, c_int64, c_int64, c_void_p, c_int,
                                       c_void_p, c_void_p, c_void_p, c_void_p, c_int, c_void_p,
                                       c_size_t]),
    "qmm_dequantize_absmax_nested": (c_int, [POINTER(qmm_nested_absmax), c_int64, c_void_p, c_void_p]),
    "qmm_codebook4_nested": (c_int, [c_void_p, c_int, c_int64, c_int64, c_int64, c_void_p, c_int,
                                     POINTER(qmm_nested_absmax), c_void_p, c_void_p, c_void_p, c_int, c_void_p,
                                     c_size_t, c_void_p]),
    "qmm_codebook4_nested_workspace_bytes": (c_size_t, [c_int64, c_int64, c_int64, c_int, c_int]),
    "qmm_fp16_uniform_value": (c_int, [c_void_p, c_int64, c_void_p, c_size_t, POINTER(c_int),
                                       POINTER(c_float), c_void_p]),
    "qmm_uniform_scratch_bytes": (c_size_t, []),
    "qmm_dequantize_nbits": (c_int, [c_void_p, c_int, c_int, c_void_p, c_void_p, c_int, c_float,
                                     c_int64, c_int64, c_void_p, c_int, c_void_p]),
    "qmm_dequantize_codebook4": (c_int, [c_void_p, c_int, c_void_p, c_void_p, c_int64, c_int64,
                                         c_void_p, c_int, c_void_p]),
    "qmoe_decode_fused": (c_int, [c_void_p, c_int64, c_int64, c_int64, c_int64, c_int, c_void_p,
                                  c_void_p, qmoe_weights, qmoe_weights, c_int, c_int, c_int,
                                  c_void_p, c_void_p, c_size_t, c_void_p]),
    "qmoe_decode_scratch_bytes": (c_size_t, [c_int64, c_int64, c_int64, c_int, c_int]),
    "qmoe_decode_status": (c_int, [c_void_p, c_size_t, c_int64, c_int64, c_int64, c_int, c_int,
                                   POINTER(c_int), c_void_p]),
    "qmoe_ragged_mm": (c_int, [c_void_p, c_int64, c_int64, c_int64, c_int64, c_void_p, qmoe_weights, c_int,
                               c_int, c_void_p, c_void_p]),
    "qmoe_decode_fused_noalloc": (c_int, [c_void_p, c_int64, c_int64, c_int64, c_int64, c_int, c_void_p,
                                          c_void_p, qmoe_weights, qmoe_weights, c_int, c_int, c_int,
                                          c_void_p, c_void_p]),
    "qmm_validate_qmoe": (c_int, [c_void_p, c_int64, c_int64, c_int64, c_int64, c_int, c_void_p,
                                  c_void_p, qmoe_weights, qmoe_weights, c_int, c_int, c_int,
                                  c_void_p, c_void_p, c_size_t]),
    "qmm_quantize_linear": (c_int, [c_void_p, c_int, c_int64, qmm_qparams, c_int, c_void_p, c_void_p]),
    "qmm_dequantize_linear": (c_int, [c_void_p, c_int64, qmm_qparams, c_int, c_void_p, c_int, c_void_p]),
    "qmm_fake_quantize": (c_int, [c_void_p, c_int, c_int64, qmm_qparams, c_int, c_void_p, c_void_p]),
    "qmm_qsigmoid": (c_int, [c_void_p, c_int64, qmm_qparams, qmm_qparams, c_int, c_void_p, c_void_p]),
    "qmm_qmul": (c_int, [c_void_p, qmm_qparams, c_void_p, qmm_qparams, c_int64, qmm_qparams, c_int,
                         c_void_p, c_void_p]),
    "qmm_qswiglu": (c_int, [c_void_p, c_void_p, c_int, c_int64, c_int, POINTER(qmm_qparams), c_void_p,
                            c_void_p]),
    "qmm_hbm_read_probe": (c_int, [c_void_p, c_int64, c_void_p, c_int, c_void_p]),
    "qmm_launch_timing_begin": (c_int, [c_int]),
    "qmm_launch_timing_end": (c_int, [c_void_p, c_int, c_void_p]),
    "qmm_set_tuning": (c_int, [c_int, c_int]),
    "qmm_num_candidates": (c_int, [c_int]),
    "qmm_nbits_gemv_matrix_core_form": (c_int, [c_int64, c_int64, c_int64, c_int, c_int]),
    "qmm_tuned_choice": (c_int, [c_int]),
    "qmm_clear_tuning": (None, []),
    "qmm_tuner_pick": (c_int, [POINTER(c_double), c_int, c_int]),
    "qmm_tuner_pick_single_launch": (c_int, [POINTER(c_double), c_int, c_int]),
    "qmm_status_string": (ctypes.c_char_p, [c_int]),
}


def lib():
    """Load libqmm.so once (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: run __graft_entry__.build() first")
        # torch ships its own HIP runtime with the same soname as ROCm's; importing
        # torch first makes libqmm.so bind to that one runtime instead of a second copy
        import torch  # noqa: F401
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name, None)
            if fn is None:  # reported by the export test; calling it raises AttributeError
                continue
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _check(fn, status):
    if status != 0:
        raise QmmError(fn, status)


# ---------------------------------------------------------------------------
# torch marshalling
# ---------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def dtype_code(t) -> int:
    torch = _torch()
    m = {torch.float32: QMM_F32, torch.float16: QMM_F16, torch.bfloat16: QMM_BF16}
    if t.dtype not in m:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return m[t.dtype]


def torch_dtype(code: int):
    torch = _torch()
    return {QMM_F32: torch.float32, QMM_F16: torch.float16, QMM_BF16: torch.bfloat16}[code]


def _ptr(t):
    return None if t is None else c_void_p(t.data_ptr())


def _stream(stream=None):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return c_void_p(s.cuda_stream)


def _contig(t, name):
    if t is not None and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def nblocks(K, block):
    return (K + block - 1) // block


def qmm_nbits(A, W, scales, K, bits, block, zp=None, zp_kind=QMM_ZP_NONE, uniform_zp=0.0,
              bias=None, out=None, out_dtype=None, workspace=None, stream=None):
    """C[M,N] = A[M,K] . dequant(W)^T (+ bias) through the C ABI."""
    torch = _torch()
    A = _contig(A, "A")
    M = A.shape[0]
    N = W.shape[0]
    ctype = dtype_code(A) if out_dtype is None else dtype_code(torch.empty(0, dtype=out_dtype))
    if out is None:
        out = torch.empty((M, N), dtype=torch_dtype(ctype), device=A.device)
    ws_bytes = lib().qmm_nbits_workspace_bytes(M, K, N, dtype_code(A))
    if ws_bytes and workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=A.device)
    st = lib().qmm_nbits(_ptr(A), dtype_code(A), M, K, N, _ptr(W), bits, block, _ptr(scales),
                         _ptr(zp), zp_kind, float(uniform_zp), _ptr(bias), _ptr(out),
                         dtype_code(out), _ptr(workspace),
                         0 if workspace is None else workspace.numel() * workspace.element_size(),
                         _stream(stream))
    _check("qmm_nbits", st)
    return out


def qmm_codebook4(A, W, absmax, codebook, K, block=64, bias=None, out=None, out_dtype=None,
                  workspace=None, stream=None):
    torch = _torch()
    A = _contig(A, "A")
    M = A.shape[0]
    N = W.shape[0]
    ctype = dtype_code(A) if out_dtype is None else dtype_code(torch.empty(0, dtype=out_dtype))
    if out is None:
        out = torch.empty((M, N), dtype=torch_dtype(ctype), device=A.device)
    ws_bytes = lib().qmm_codebook4_workspace_bytes(M, K, N, dtype_code(A))
    if ws_bytes and workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=A.device)
    st = lib().qmm_codebook4(_ptr(A), dtype_code(A), M, K, N, _ptr(W), block, _ptr(absmax),
                             _ptr(codebook), _ptr(bias), _ptr(out), dtype_code(out),
                             _ptr(workspace),
                             0 if workspace is None else workspace.numel() * workspace.element_size(),
                             _stream(stream))
    _check("qmm_codebook4", st)
    return out


def _nested(na):
    """na: dict of device tensors codes, table, scales and python offset, group."""
    return qmm_nested_absmax(na["codes"].data_ptr(), na["table"].data_ptr(), na["scales"].data_ptr(),
                             float(na["offset"]), int(na["group"]))


def qmm_dequantize_absmax_nested(na, count, stream=None):
    torch = _torch()
    out = torch.empty(count, dtype=torch.float32, device=na["codes"].device)
    desc = _nested(na)
    _check("qmm_dequantize_absmax_nested", lib().qmm_dequantize_absmax_nested(ctypes.byref(desc), count, _ptr(out),
                                                                              _stream(stream)))
    return out


def qmm_codebook4_nested(A, W, na, codebook, K, block=64, bias=None, out=None, out_dtype=None, workspace=None,
                         stream=None):
    torch = _torch()
    A = _contig(A, "A")
    M = A.shape[0]
    N = W.shape[0]
    ctype = dtype_code(A) if out_dtype is None else dtype_code(torch.empty(0, dtype=out_dtype))
    if out is None:
        out = torch.empty((M, N), dtype=torch_dtype(ctype), device=A.device)
    ws_bytes = lib().qmm_codebook4_nested_workspace_bytes(M, K, N, dtype_code(A), block)
    if ws_bytes and workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=A.device)
    desc = _nested(na)
    st = lib().qmm_codebook4_nested(_ptr(A), dtype_code(A), M, K, N, _ptr(W), block, ctypes.byref(desc),
                                    _ptr(codebook), _ptr(bias), _ptr(out), dtype_code(out), _ptr(workspace),
                                    0 if workspace is None else workspace.numel() * workspace.element_size(),
                                    _stream(stream))
    _check("qmm_codebook4_nested", st)
    return out


def qmm_fp16_uniform_value(zp, scratch=None, stream=None):
    """(is_uniform, value) of an fp16 zero-point tensor (synchronizes the stream)."""
    torch = _torch()
    if scratch is None:
        scratch = torch.empty(lib().qmm_uniform_scratch_bytes(), dtype=torch.uint8, device=zp.device)
    flag = c_int(0)
    val = c_float(0.0)
    st = lib().qmm_fp16_uniform_value(_ptr(zp), zp.numel(), _ptr(scratch), scratch.numel(),
                                      ctypes.byref(flag), ctypes.byref(val), _stream(stream))
    _check("qmm_fp16_uniform_value", st)
    return bool(flag.value), float(val.value)


def qmm_dequantize_nbits(W, scales, K, bits, block, zp=None, zp_kind=QMM_ZP_NONE, uniform_zp=0.0,
                         out_dtype=None, stream=None):
    torch = _torch()
    out_dtype = out_dtype or torch.float32
    N = W.shape[0]
    out = torch.empty((N, K), dtype=out_dtype, device=W.device)
    st = lib().qmm_dequantize_nbits(_ptr(W), bits, block, _ptr(scales), _ptr(zp), zp_kind,
                                    float(uniform_zp), N, K, _ptr(out), dtype_code(out),
                                    _stream(stream))
    _check("qmm_dequantize_nbits", st)
    return out


def qmm_dequantize_codebook4(W, absmax, codebook, K, block=64, out_dtype=None, stream=None):
    torch = _torch()
    out_dtype = out_dtype or torch.float32
    N = W.shape[0]
    out = torch.empty((N, K), dtype=out_dtype, device=W.device)
    st = lib().qmm_dequantize_codebook4(_ptr(W), block, _ptr(absmax), _ptr(codebook), N, K,
                                        _ptr(out), dtype_code(out), _stream(stream))
    _check("qmm_dequantize_codebook4", st)
    return out


def _qw(d):
    if d is None:
        return qmoe_weights(None, None, None, None)
    return qmoe_weights(d["W"].data_ptr(), d["scales"].data_ptr(),
                        None if d.get("zp") is None else d["zp"].data_ptr(),
                        None if d.get("bias") is None else d["bias"].data_ptr())


def qmoe_decode_scratch_bytes(T, H, I, k, mode=QMOE_FP):
    return lib().qmoe_decode_scratch_bytes(T, H, I, k, mode)


def qmoe_decode_fused(X, expert_ids, expert_w, fc1, fc2, H, I, E, block, mode=QMOE_FP, bits=4,
                      out=None, scratch=None, stream=None):
    """Y[T,H] fp16 = top-k MoE decode (fc1 -> SwiGLU -> fc2) through the C ABI.

    fc1 / fc2: dicts of device tensors {"W", "scales", "zp" (or None), "bias" (or None)}.
    """
    torch = _torch()
    X = _contig(X, "X")
    T = X.shape[0]
    k = expert_ids.shape[1]
    if out is None:
        out = torch.empty((T, H), dtype=torch.float16, device=X.device)
    sb = lib().qmoe_decode_scratch_bytes(T, H, I, k, mode)
    if scratch is None:
        # zeroed: the single-launch form's sync words must start at zero (calls leave them so)
        scratch = torch.zeros(max(sb, 1), dtype=torch.uint8, device=X.device)
    st = lib().qmoe_decode_fused(_ptr(X), T, H, I, E, k, _ptr(expert_ids), _ptr(expert_w), _qw(fc1),
                                 _qw(fc2), bits, block, mode, _ptr(out), _ptr(scratch),
                                 scratch.numel() * scratch.element_size(), _stream(stream))
    _check("qmoe_decode_fused", st)
    return out


def qmoe_ragged_mm(X, row_offsets, w, N, E, block, bits=4, out=None, stream=None):
    """Y[R, N] fp16: rows of X grouped by expert (row_offsets [E+1] int32 on the device),
    each row times its expert's dequantized u4 weights (w: dict W, scales, zp, bias)."""
    torch = _torch()
    X = _contig(X, "X")
    R, K = X.shape
    if out is None:
        out = torch.empty((R, N), dtype=torch.float16, device=X.device)
    st = lib().qmoe_ragged_mm(_ptr(X), R, K, N, E, _ptr(row_offsets), _qw(w), bits, block, _ptr(out),
                              _stream(stream))
    _check("qmoe_ragged_mm", st)
    return out


QMOE_NOALLOC_SCRATCH_BYTES = 8 << 20


def qmoe_decode_fused_noalloc(X, expert_ids, expert_w, fc1, fc2, H, I, E, block, out, mode=QMOE_FP, bits=4,
                              stream=None):
    """The MoE decode on the library's static scratch: no allocation in the library
    (the caller passes the output)."""
    X = _contig(X, "X")
    T = X.shape[0]
    k = expert_ids.shape[1]
    st = lib().qmoe_decode_fused_noalloc(_ptr(X), T, H, I, E, k, _ptr(expert_ids), _ptr(expert_w), _qw(fc1),
                                         _qw(fc2), bits, block, mode, _ptr(out), _stream(stream))
    _check("qmoe_decode_fused_noalloc", st)
    return out


def qmoe_decode_status(scratch, T, H, I, k, mode=QMOE_FP, stream=None) -> bool:
    """True if a single-launch decode on `scratch` gave up its wait (clears the flag)."""
    flag = c_int(0)
    st = lib().qmoe_decode_status(_ptr(scratch), scratch.numel() * scratch.element_size(), T, H, I, k,
                                  mode, ctypes.byref(flag), _stream(stream))
    _check("qmoe_decode_status", st)
    return bool(flag.value)


# ---------------------------------------------------------------------------
# activation quantization ops
# ---------------------------------------------------------------------------

def _qp(q):
    s, z = q
    return qmm_qparams(float(s), int(z))


def _code_dtype(bits):
    torch = _torch()
    return torch.uint8 if bits == 8 else torch.uint16


def quantize_linear(x, q, bits, out=None, stream=None):
    """uint8 / uint16 codes of x under the per-tensor (scale, zero_point) q."""
    torch = _torch()
    x = _contig(x, "x")
    if out is None:
        out = torch.empty(x.shape, dtype=_code_dtype(bits), device=x.device)
    _check("qmm_quantize_linear", lib().qmm_quantize_linear(_ptr(x), dtype_code(x), x.numel(), _qp(q), bits,
                                                            _ptr(out), _stream(stream)))
    return out


def dequantize_linear(codes, q, bits, out_dtype=None, out=None, stream=None):
    torch = _torch()
    codes = _contig(codes, "codes")
    if out is None:
        out = torch.empty(codes.shape, dtype=out_dtype or torch.float32, device=codes.device)
    _check("qmm_dequantize_linear", lib().qmm_dequantize_linear(_ptr(codes), codes.numel(), _qp(q), bits,
                                                                _ptr(out), dtype_code(out), _stream(stream)))
    return out


def fake_quantize(x, q, bits, out=None, stream=None):
    torch = _torch()
    x = _contig(x, "x")
    if out is None:
        out = torch.empty_like(x)
    _check("qmm_fake_quantize", lib().qmm_fake_quantize(_ptr(x), dtype_code(x), x.numel(), _qp(q), bits,
                                                        _ptr(out), _stream(stream)))
    return out


def qsigmoid(codes, q_in, q_out, bits, out=None, stream=None):
    torch = _torch()
    codes = _contig(codes, "codes")
    if out is None:
        out = torch.empty_like(codes)
    _check("qmm_qsigmoid", lib().qmm_qsigmoid(_ptr(codes), codes.numel(), _qp(q_in), _qp(q_out), bits, _ptr(out),
                                              _stream(stream)))
    return out


def qmul(a, qa, b, qb, qc, bits, out=None, stream=None):
    torch = _torch()
    a, b = _contig(a, "a"), _contig(b, "b")
    if a.numel() != b.numel():
        raise ValueError("a and b differ in size")
    if out is None:
        out = torch.empty_like(a)
    _check("qmm_qmul", lib().qmm_qmul(_ptr(a), _qp(qa), _ptr(b), _qp(qb), a.numel(), _qp(qc), bits, _ptr(out),
                                      _stream(stream)))
    return out


def qswiglu(gate, up, qparams, bits, out=None, stream=None):
    """Fused quantized SwiGLU chain; qparams: five (scale, zero_point) pairs
    (gate, sigmoid, silu, up, out)."""
    torch = _torch()
    gate, up = _contig(gate, "gate"), _contig(up, "up")
    if gate.numel() != up.numel() or gate.dtype != up.dtype:
        raise ValueError("gate and up differ in size or dtype")
    if out is None:
        out = torch.empty_like(gate)
    arr = (qmm_qparams * 5)(*[_qp(q) for q in qparams])
    _check("qmm_qswiglu", lib().qmm_qswiglu(_ptr(gate), _ptr(up), dtype_code(gate), gate.numel(), bits, arr,
                                            _ptr(out), _stream(stream)))
    return out


def hbm_read_probe(buf, sink, groups, stream=None):
    """Read every byte of `buf` once with 128-bit loads (measurement helper)."""
    _check("qmm_hbm_read_probe", lib().qmm_hbm_read_probe(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink),
                                                          groups, _stream(stream)))


def launch_timing_begin(n: int):
    """Time the next n kernel launches the library makes from this thread."""
    _check("qmm_launch_timing_begin", lib().qmm_launch_timing_begin(n))


def launch_timing_end(n_max: int = 65536):
    """Stop launch timing; the execution time in us of each timed launch, in order."""
    buf = (c_float * n_max)()
    count = c_int(0)
    _check("qmm_launch_timing_end", lib().qmm_launch_timing_end(buf, n_max, ctypes.byref(count)))
    return [float(buf[i]) for i in range(min(count.value, n_max))]


def set_tuning(mode: int, forced_index: int = 0):
    _check("qmm_set_tuning", lib().qmm_set_tuning(mode, forced_index))


def num_candidates(entry: int) -> int:
    return lib().qmm_num_candidates(entry)


def nbits_gemv_matrix_core_form(M: int, K: int, N: int, bits: int, block: int) -> bool:
    return bool(lib().qmm_nbits_gemv_matrix_core_form(M, K, N, bits, block))


def tuned_choice(entry: int) -> int:
    return lib().qmm_tuned_choice(entry)


def clear_tuning():
    lib().qmm_clear_tuning()


def tuner_pick(times_us, rounds, ncand):
    arr = (c_double * len(times_us))(*times_us)
    return lib().qmm_tuner_pick(arr, rounds, ncand)


def tuner_pick_single_launch(times_us, rounds, ncand):
    arr = (c_double * len(times_us))(*times_us)
    return lib().qmm_tuner_pick_single_launch(arr, rounds, ncand)
