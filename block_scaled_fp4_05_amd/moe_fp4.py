"""Python binding of libmoe_fp4.so (the C ABI in include/moe_fp4.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels.  PyTorch supplies device memory and the current stream.  If the
compiled library is missing the calls raise; there is no CPU fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# MOE_FP4_LIB may name another build of the same sources (the host-sanitizer
# build of the CPU tests); by default the in-tree library.
LIB_PATH = os.environ.get("MOE_FP4_LIB") or os.path.join(_PKG, "libmoe_fp4.so")

OK, ERR_NULL, ERR_SHAPE, ERR_ALIGN, ERR_UNSUPPORTED, ERR_HIP, ERR_ARG = range(7)
OUT_BF16, OUT_FP32 = 0, 1
IN_BF16, IN_FP32 = 0, 1
SCALE_STATIC, SCALE_DYNAMIC = 0, 1

# Every symbol include/moe_fp4.h declares.
EXPORTED = ("moe_fp4_quantize", "moe_grouped_gemm_fp4", "moe_grouped_gemm_fp4_packed",
            "moe_grouped_gemm_fp4_finalize", "moe_grouped_gemm_fp4_swiglu", "moe_fp4_combine",
            "moe_fp4_pack_weights", "moe_fp4_unpack_weights", "moe_grouped_gemm_fp4_plan",
            "moe_grouped_gemm_fp4_workspace_size", "moe_fp4_stage_bytes",
            "moe_fp4_status_string", "moe_fp4_abi_version")


class MoeFp4Error(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {status_string(status)} (status {status})")
        self.status = status


class Plan(ctypes.Structure):
    _fields_ = [("tile_m", ctypes.c_int32), ("tile_n", ctypes.c_int32),
                ("k_step", ctypes.c_int32), ("waves_per_group", ctypes.c_int32),
                ("lds_bytes", ctypes.c_int64)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load the compiled library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with block_scaled_fp4_05_amd.build")
    L = ctypes.CDLL(LIB_PATH)
    vp, i64, i32, i = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int
    L.moe_fp4_quantize.argtypes = [vp, i, i64, i64, i64, vp, vp, vp, i, vp]
    L.moe_fp4_quantize.restype = i
    L.moe_grouped_gemm_fp4.argtypes = [vp, vp, vp, i64, vp, vp, vp, vp, vp, i32, i64, i64, i64,
                                       vp, i64, vp]
    L.moe_grouped_gemm_fp4.restype = i
    L.moe_grouped_gemm_fp4_packed.argtypes = L.moe_grouped_gemm_fp4.argtypes
    L.moe_grouped_gemm_fp4_packed.restype = i
    L.moe_grouped_gemm_fp4_finalize.argtypes = [vp, vp, vp, i64, vp, vp, vp, vp, i, vp, i32, i64,
                                                 i64, i64, vp, vp, vp, i64, i64, vp]
    L.moe_grouped_gemm_fp4_finalize.restype = i
    L.moe_grouped_gemm_fp4_swiglu.argtypes = [vp, vp, vp, i64, vp, vp, vp, vp, i, vp, i32, i64,
                                               i64, i64, vp, vp, vp, vp]
    L.moe_grouped_gemm_fp4_swiglu.restype = i
    L.moe_fp4_combine.argtypes = [vp, i64, i64, vp, vp, i32, i64, i64, vp, i64, vp, i, i64, vp]
    L.moe_fp4_combine.restype = i
    for f in (L.moe_fp4_pack_weights, L.moe_fp4_unpack_weights):
        f.argtypes = [vp, vp, i32, i64, i64, vp]
        f.restype = i
    L.moe_grouped_gemm_fp4_plan.argtypes = [i32, i64, i64, i64, ctypes.POINTER(Plan)]
    L.moe_grouped_gemm_fp4_plan.restype = i
    L.moe_grouped_gemm_fp4_workspace_size.argtypes = [i32, i64, i64, i64]
    L.moe_grouped_gemm_fp4_workspace_size.restype = ctypes.c_size_t
    L.moe_fp4_stage_bytes.argtypes = [i64, i64, i64]
    L.moe_fp4_stage_bytes.restype = i64
    L.moe_fp4_status_string.argtypes = [i]
    L.moe_fp4_status_string.restype = ctypes.c_char_p
    L.moe_fp4_abi_version.argtypes = []
    L.moe_fp4_abi_version.restype = i
    _lib = L
    return L


def status_string(status: int) -> str:
    return lib().moe_fp4_status_string(int(status)).decode()


def abi_version() -> int:
    return lib().moe_fp4_abi_version()


def stage_bytes(bm: int, bn: int, bk: int) -> int:
    return lib().moe_fp4_stage_bytes(bm, bn, bk)


def workspace_size(num_experts: int, m_total: int, n: int, k: int) -> int:
    """Device workspace bytes of the grouped GEMM for these sizes (always 0)."""
    return lib().moe_grouped_gemm_fp4_workspace_size(num_experts, m_total, n, k)


def plan(num_experts: int, m_total: int, n: int, k: int) -> dict:
    p = Plan()
    st = lib().moe_grouped_gemm_fp4_plan(num_experts, m_total, n, k, ctypes.byref(p))
    if st != OK:
        raise MoeFp4Error(st, "moe_grouped_gemm_fp4_plan")
    return {f: getattr(p, f) for f, _ in Plan._fields_}


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream, dev):
    """The launch stream (default: the current stream of the current device), which
    must belong to the tensors' device `dev`: the kernels run on the stream's device."""
    if stream is None:
        stream = torch.cuda.current_stream()
    if stream.device_index != dev:
        raise ValueError(f"stream on cuda:{stream.device_index}, tensors on cuda:{dev}")
    return ctypes.c_void_p(stream.cuda_stream)


class _AtLeast(int):
    """A shape entry that admits any extent of at least this value."""

    def __repr__(self):
        return f">={int(self)}"


def _need(t, name, dtype, shape=None, contiguous=True, rows=False):
    """Check a tensor argument before its pointer is handed to the library: its dtype,
    its shape (None entries are free, _AtLeast(x) entries admit x or more), and its
    layout: contiguous, or with rows=True only unit stride along the last axis (rows
    at any leading dimension).  Raises ValueError.  (Plain loops: it runs on every
    call of a decode step.)"""
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name}: expected a tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if shape is not None:
        ts = t.shape
        ok = len(ts) == len(shape)
        if ok:
            for i in range(len(shape)):
                w = shape[i]
                if w is not None and ((ts[i] < w) if type(w) is _AtLeast else (ts[i] != w)):
                    ok = False
                    break
        if not ok:
            raise ValueError(f"{name}: shape {tuple(ts)}, expected {tuple(shape)}")
    if rows:
        if t.dim() != 2 or (t.shape[1] > 1 and t.stride(1) != 1):
            raise ValueError(f"{name}: rows must have unit column stride")
    elif contiguous and not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")


def _same_cuda(names, *tensors):
    """All given tensors (None skipped) are CUDA tensors on one device, which is
    returned; `names` lists them, space-separated, for the error message."""
    dev = -1
    for t in tensors:
        if t is None:
            continue
        d = t.get_device()
        if d < 0 or (dev >= 0 and d != dev):
            devs = {nm: str(x.device) for nm, x in zip(names.split(), tensors) if x is not None}
            if d < 0:
                bad = [nm for nm, v in devs.items() if not v.startswith("cuda")]
                raise ValueError(f"{bad[0]}: must be a CUDA tensor (got {devs[bad[0]]})")
            raise ValueError(f"tensors on several devices: {devs}")
        dev = d
    return dev


def quantize_raw(x_ptr, in_dtype, rows, k, ld_x, q_ptr, sf_ptr, scale_ptr, scale_mode, stream_ptr):
    """Direct call with raw pointers; returns the status code."""
    return lib().moe_fp4_quantize(x_ptr, in_dtype, rows, k, ld_x, q_ptr, sf_ptr, scale_ptr,
                                  scale_mode, stream_ptr)


def gemm_raw(*args):
    """Direct call with raw pointers (C argument order); returns the status code."""
    return lib().moe_grouped_gemm_fp4(*args)


def gemm_packed_raw(*args):
    """moe_grouped_gemm_fp4_packed with raw pointers; returns the status code."""
    return lib().moe_grouped_gemm_fp4_packed(*args)


def pack_weights(w_q: torch.Tensor, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Row-major weight codes [E][n][k/2] (uint8, CUDA) -> the packed layout the
    packed GEMM reads (same shape and size; a byte permutation)."""
    _need(w_q, "w_q", torch.uint8, (None, None, None))
    E, n, kb = w_q.shape
    if out is None:
        out = torch.empty_like(w_q)
    _need(out, "out", torch.uint8, (E, n, kb))
    dev = _same_cuda("w_q out", w_q, out)
    st = lib().moe_fp4_pack_weights(_ptr(w_q), _ptr(out), E, n, 2 * kb, _stream(stream, dev))
    if st != OK:
        raise MoeFp4Error(st, "moe_fp4_pack_weights")
    return out


def unpack_weights(w_packed: torch.Tensor, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Inverse of pack_weights."""
    _need(w_packed, "w_packed", torch.uint8, (None, None, None))
    E, n, kb = w_packed.shape
    if out is None:
        out = torch.empty_like(w_packed)
    _need(out, "out", torch.uint8, (E, n, kb))
    dev = _same_cuda("w_packed out", w_packed, out)
    st = lib().moe_fp4_unpack_weights(_ptr(w_packed), _ptr(out), E, n, 2 * kb, _stream(stream, dev))
    if st != OK:
        raise MoeFp4Error(st, "moe_fp4_unpack_weights")
    return out


def quantize(x: torch.Tensor, tensor_scale: torch.Tensor | None = None, q=None, sf=None,
             stream=None, dynamic: bool | None = None):
    """NVFP4-quantise a 2-D BF16 or FP32 CUDA tensor [rows][k].

    tensor_scale None -> dynamic: a new 1-element float32 tensor receives g.
    Otherwise a 1-element float32 CUDA tensor: by default it holds a calibrated g
    (static); with dynamic=True it receives the computed g instead.
    Returns (q uint8[rows][k/2], sf uint8[rows][k/16], tensor_scale float32[1]).
    """
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be 2-D with unit column stride")
    if x.dtype == torch.bfloat16:
        dt = IN_BF16
    elif x.dtype == torch.float32:
        dt = IN_FP32
    else:
        raise ValueError("x must be bfloat16 or float32")
    rows, k = x.shape
    dev = x.device
    if q is None:
        q = torch.empty((rows, k // 2), dtype=torch.uint8, device=dev)
    if sf is None:
        sf = torch.empty((rows, k // 16), dtype=torch.uint8, device=dev)
    if dynamic is None:
        dynamic = tensor_scale is None
    mode = SCALE_DYNAMIC if dynamic else SCALE_STATIC
    if tensor_scale is None:
        if not dynamic:
            raise ValueError("a static quantisation needs tensor_scale")
        tensor_scale = torch.empty(1, dtype=torch.float32, device=dev)
    _need(q, "q", torch.uint8, (_AtLeast(rows), k // 2))
    _need(sf, "sf", torch.uint8, (_AtLeast(rows), k // 16))
    _need(tensor_scale, "tensor_scale", torch.float32, (_AtLeast(1),))
    dev = _same_cuda("x q sf tensor_scale", x, q, sf, tensor_scale)
    st = lib().moe_fp4_quantize(_ptr(x), dt, rows, k, x.stride(0), _ptr(q), _ptr(sf),
                                _ptr(tensor_scale), mode, _stream(stream, dev))
    if st != OK:
        raise MoeFp4Error(st, "moe_fp4_quantize")
    return q, sf, tensor_scale


def _gemm_operands(a_q, a_sf, a_scale, w_q, w_sf, w_scale, offsets, a_row_index, m_total):
    """Check the operands shared by the grouped-GEMM entry points; returns
    (E, n, k, a_rows, m_total)."""
    _need(w_q, "w_q", torch.uint8, (None, None, None))
    E, n, kb = w_q.shape
    _need(a_q, "a_q", torch.uint8, (None, kb))
    a_rows = a_q.shape[0]
    _need(a_sf, "a_sf", torch.uint8, (a_rows, kb // 8))
    _need(a_scale, "a_scale", torch.float32, (_AtLeast(1),))
    _need(w_sf, "w_sf", torch.uint8, (E, n, kb // 8))
    _need(w_scale, "w_scale", torch.float32, (E,))
    _need(offsets, "offsets", torch.int32, (E + 1,))
    if m_total is None:
        m_total = a_row_index.shape[0] if a_row_index is not None else a_rows
    if a_row_index is not None:
        _need(a_row_index, "a_row_index", torch.int32, (m_total,))
    return E, n, 2 * kb, a_rows, m_total


def grouped_gemm(a_q, a_sf, a_scale, w_q, w_sf, w_scale, offsets, a_row_index=None, out=None,
                 m_total: int | None = None, stream=None, packed: bool = False):
    """NVFP4 grouped GEMM.  Shapes: a_q [a_rows][k/2], a_sf [a_rows][k/16], a_scale [1],
    w_q [E][n][k/2], w_sf [E][n][k/16], w_scale [E], offsets int32 [E+1],
    a_row_index int32 [m_total] or None.  m_total defaults to a_row_index's length,
    else a_rows.  packed: w_q is in the packed layout (pack_weights).  Returns out,
    a BF16 tensor [m_total][n] (or the given `out`)."""
    E, n, k, a_rows, m_total = _gemm_operands(a_q, a_sf, a_scale, w_q, w_sf, w_scale, offsets,
                                              a_row_index, m_total)
    if out is None:
        out = torch.empty((m_total, n), dtype=torch.bfloat16, device=w_q.device)
    _need(out, "out", torch.bfloat16, (_AtLeast(m_total), _AtLeast(n)), rows=True)
    dev = _same_cuda("a_q a_sf a_scale w_q w_sf w_scale offsets a_row_index out", a_q, a_sf, a_scale, w_q, w_sf, w_scale, offsets, a_row_index, out)
    fn = lib().moe_grouped_gemm_fp4_packed if packed else lib().moe_grouped_gemm_fp4
    st = fn(_ptr(a_q), _ptr(a_sf), _ptr(a_scale), a_rows, _ptr(a_row_index), _ptr(w_q), _ptr(w_sf),
            _ptr(w_scale), _ptr(offsets), E, m_total, n, k, _ptr(out), out.stride(0), _stream(stream, dev))
    if st != OK:
        raise MoeFp4Error(st, "moe_grouped_gemm_fp4_packed" if packed else "moe_grouped_gemm_fp4")
    return out


def finalize_raw(*args):
    """moe_grouped_gemm_fp4_finalize with raw pointers (C argument order); returns the status."""
    return lib().moe_grouped_gemm_fp4_finalize(*args)


def grouped_gemm_finalize(a_q, a_sf, a_scale, w_q, w_sf, w_scale, offsets, out_token, row_weight,
                          out, a_row_index=None, m_total: int | None = None, packed: bool = False,
                          stream=None):
    """Grouped GEMM with the finalize epilogue: routed row r adds row_weight[r] times its
    result into row out_token[r] of `out` (float32 CUDA tensor [num_tokens][ldo],
    accumulated into).  Other arguments as grouped_gemm.  Returns out."""
    E, n, k, a_rows, m_total = _gemm_operands(a_q, a_sf, a_scale, w_q, w_sf, w_scale, offsets,
                                              a_row_index, m_total)
    _need(out_token, "out_token", torch.int32, (m_total,))
    _need(row_weight, "row_weight", torch.float32, (m_total,))
    _need(out, "out", torch.float32, (None, _AtLeast(n)), rows=True)
    dev = _same_cuda("a_q a_sf a_scale w_q w_sf w_scale offsets a_row_index out_token row_weight out", a_q, a_sf, a_scale, w_q, w_sf, w_scale, offsets, a_row_index, out_token, row_weight, out)
    st = lib().moe_grouped_gemm_fp4_finalize(
        _ptr(a_q), _ptr(a_sf), _ptr(a_scale), a_rows, _ptr(a_row_index), _ptr(w_q), _ptr(w_sf),
        _ptr(w_scale), 1 if packed else 0, _ptr(offsets), E, m_total, n, k, _ptr(out_token),
        _ptr(row_weight), _ptr(out), out.stride(0), out.shape[0], _stream(stream, dev))
    if st != OK:
        raise MoeFp4Error(st, "moe_grouped_gemm_fp4_finalize")
    return out


def swiglu_raw(*args):
    """moe_grouped_gemm_fp4_swiglu with raw pointers (C argument order); returns the status."""
    return lib().moe_grouped_gemm_fp4_swiglu(*args)


def grouped_gemm_swiglu(a_q, a_sf, a_scale, w_q, w_sf, w_scale, offsets, h_scale,
                        a_row_index=None, h_q=None, h_sf=None, m_total: int | None = None,
                        packed: bool = False, stream=None):
    """Gate+up grouped GEMM with the SwiGLU + NVFP4 epilogue.  w_q [E][2I][k/2]: rows
    0..I-1 the gate, I..2I-1 the up projection; h_scale float32 CUDA tensor [1], the
    intermediate's static tensor scale.  Other arguments as grouped_gemm.  Returns
    (h_q uint8 [m_total][I/2], h_sf uint8 [m_total][I/16]), the down projection's
    activations (or the given buffers)."""
    E, n, k, a_rows, m_total = _gemm_operands(a_q, a_sf, a_scale, w_q, w_sf, w_scale, offsets,
                                              a_row_index, m_total)
    dev = w_q.device
    if h_q is None:
        h_q = torch.empty((m_total, n // 4), dtype=torch.uint8, device=dev)
    if h_sf is None:
        h_sf = torch.empty((m_total, n // 32), dtype=torch.uint8, device=dev)
    _need(h_scale, "h_scale", torch.float32, (_AtLeast(1),))
    _need(h_q, "h_q", torch.uint8, (_AtLeast(m_total), n // 4))
    _need(h_sf, "h_sf", torch.uint8, (_AtLeast(m_total), n // 32))
    dev = _same_cuda("a_q a_sf a_scale w_q w_sf w_scale offsets a_row_index h_scale h_q h_sf", a_q, a_sf, a_scale, w_q, w_sf, w_scale, offsets, a_row_index, h_scale, h_q, h_sf)
    st = lib().moe_grouped_gemm_fp4_swiglu(
        _ptr(a_q), _ptr(a_sf), _ptr(a_scale), a_rows, _ptr(a_row_index), _ptr(w_q), _ptr(w_sf),
        _ptr(w_scale), 1 if packed else 0, _ptr(offsets), E, m_total, n, k, _ptr(h_scale),
        _ptr(h_q), _ptr(h_sf), _stream(stream, dev))
    if st != OK:
        raise MoeFp4Error(st, "moe_grouped_gemm_fp4_swiglu")
    return h_q, h_sf


def combine_raw(*args):
    """moe_fp4_combine with raw pointers (C argument order); returns the status."""
    return lib().moe_fp4_combine(*args)


def combine(rows, token_rows, token_weights, out=None, residual=None, out_dtype=torch.bfloat16,
            stream=None):
    """Token-order combine: out[t] = (residual[t] +) sum_s token_weights[t][s] * rows[token_rows[t][s]]
    in FP32, slots in order.  rows: BF16 CUDA tensor [m_total][>= n] (the grouped GEMM's
    output); token_rows int32 / token_weights float32 [num_tokens][topk].  Returns out
    ([num_tokens][n] of out_dtype, bfloat16 or float32)."""
    _need(rows, "rows", torch.bfloat16, (None, None), rows=True)
    m_total, n = rows.shape
    _need(token_rows, "token_rows", torch.int32, (None, None))
    T, topk = token_rows.shape
    _need(token_weights, "token_weights", torch.float32, (T, topk))
    if residual is not None:
        _need(residual, "residual", torch.float32, (T, _AtLeast(n)), rows=True)
    if out is None:
        out = torch.empty((T, n), dtype=out_dtype, device=rows.device)
    if out.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError(f"out: dtype {out.dtype}, expected bfloat16 or float32")
    _need(out, "out", out.dtype, (T, _AtLeast(n)), rows=True)
    dev = _same_cuda("rows token_rows token_weights residual out", rows, token_rows, token_weights, residual, out)
    dt = OUT_FP32 if out.dtype == torch.float32 else OUT_BF16
    st = lib().moe_fp4_combine(_ptr(rows), rows.stride(0), m_total, _ptr(token_rows),
                               _ptr(token_weights), topk, T, n, _ptr(residual),
                               residual.stride(0) if residual is not None else 0, _ptr(out), dt,
                               out.stride(0), _stream(stream, dev))
    if st != OK:
        raise MoeFp4Error(st, "moe_fp4_combine")
    return out
