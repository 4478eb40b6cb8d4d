"""Python face of the CPU oracle (``fp4_oracle.c``).

TEST INFRASTRUCTURE ONLY.  Imported by ``tests/``, by ``__graft_entry__.smoke``
and by the CPU-baseline leg of ``bench.py``; never by the library.  It shares
no code with the HIP path.

Every function takes and returns numpy arrays.  Layouts (row-major):
  x           float32 [rows][ld_x]
  q           uint8   [rows][k/2]   element 2i in the low nibble of byte i
  sf          uint8   [rows][k/16]  E4M3 block scales
  w_q         uint8   [E][n][k/2]
  w_sf        uint8   [E][n][k/16]
  w_scale     float32 [E]
  offsets     int32   [E+1]         rows of expert e are [offsets[e], offsets[e+1])
  a_row_index int32   [m_total] or None (identity)
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fp4_oracle.c")
LIB_PATH = os.environ.get("FP4_ORACLE_LIB") or os.path.join(_HERE, "liboracle_fp4.so")

_lib = None


def build(force: bool = False, src: str | None = None, out: str | None = None) -> str:
    """Compile the oracle with gcc (-O2, OpenMP, no FP contraction).

    FP4_ORACLE_LIB may name another build of the same source (used to check, on
    the CPU, that the pins fail on a deliberately broken copy); `src` and `out`
    compile such a copy."""
    src = src or _SRC
    out = out or LIB_PATH
    if force or not os.path.exists(out):
        tmp = out + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c99", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
               "-Wall", "-shared", "-fPIC", src, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, out)
    return out


def _load():
    global _lib
    if _lib is not None:
        return _lib
    build(force=False)
    lib = ctypes.CDLL(LIB_PATH)
    c_u8p = ctypes.POINTER(ctypes.c_uint8)
    c_i32p = ctypes.POINTER(ctypes.c_int32)
    c_i64p = ctypes.POINTER(ctypes.c_int64)
    c_f32p = ctypes.POINTER(ctypes.c_float)
    c_f64p = ctypes.POINTER(ctypes.c_double)
    c_u16p = ctypes.POINTER(ctypes.c_uint16)
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = ctypes.c_int
    lib.oracle_e2m1_decode.argtypes = [ctypes.c_int]
    lib.oracle_e2m1_decode.restype = ctypes.c_double
    lib.oracle_e2m1_encode.argtypes = [ctypes.c_float]
    lib.oracle_e2m1_encode.restype = ctypes.c_int
    lib.oracle_e4m3_decode.argtypes = [ctypes.c_int]
    lib.oracle_e4m3_decode.restype = ctypes.c_double
    lib.oracle_e4m3_encode.argtypes = [ctypes.c_float]
    lib.oracle_e4m3_encode.restype = ctypes.c_int
    lib.oracle_bf16_bits_from_double.argtypes = [ctypes.c_double]
    lib.oracle_bf16_bits_from_double.restype = ctypes.c_uint16
    lib.oracle_quantize.argtypes = [c_f32p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                    c_f32p, ctypes.c_int, c_u8p, c_u8p]
    lib.oracle_quantize.restype = ctypes.c_int
    common = [c_u8p, c_u8p, ctypes.c_float, ctypes.c_int64, c_i32p, c_u8p, c_u8p, c_f32p,
              c_i32p, ctypes.c_int32, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
              c_i64p, ctypes.c_int64]
    lib.oracle_grouped_gemm_exact.argtypes = common + [c_f64p, c_u16p]
    lib.oracle_grouped_gemm_exact.restype = ctypes.c_int
    lib.oracle_grouped_gemm_f64.argtypes = common + [c_f64p]
    lib.oracle_grouped_gemm_f64.restype = ctypes.c_int
    _lib = lib
    return lib


def _ptr(a, ctype):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def num_threads() -> int:
    """OpenMP threads the oracle's parallel loops use."""
    return _load().oracle_num_threads()


# ------------------------------------------------------------------ codecs --

def e2m1_decode(code: int) -> float:
    return _load().oracle_e2m1_decode(int(code))


def e2m1_encode(y: float) -> int:
    return _load().oracle_e2m1_encode(float(y))


def e4m3_decode(code: int) -> float:
    return _load().oracle_e4m3_decode(int(code))


def e4m3_encode(r: float) -> int:
    return _load().oracle_e4m3_encode(float(r))


def e2m1_encode_array(y: np.ndarray) -> np.ndarray:
    f = _load().oracle_e2m1_encode
    return np.array([f(float(v)) for v in np.asarray(y, dtype=np.float32).ravel()],
                    dtype=np.uint8).reshape(np.shape(y))


def e4m3_encode_array(r: np.ndarray) -> np.ndarray:
    f = _load().oracle_e4m3_encode
    return np.array([f(float(v)) for v in np.asarray(r, dtype=np.float32).ravel()],
                    dtype=np.uint8).reshape(np.shape(r))


def bf16_bits(x: float) -> int:
    return _load().oracle_bf16_bits_from_double(float(x))


def bf16_bits_array(x: np.ndarray) -> np.ndarray:
    f = _load().oracle_bf16_bits_from_double
    return np.array([f(float(v)) for v in np.asarray(x, dtype=np.float64).ravel()],
                    dtype=np.uint16).reshape(np.shape(x))


def bf16_bits_to_float(bits: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32)


# ---------------------------------------------------------------- quantise --

def quantize(x: np.ndarray, g: float | None = None):
    """NVFP4-quantise a float32 matrix [rows][k].

    g None -> dynamic tensor scale (computed and returned); else static g.
    Returns (q uint8[rows][k/2], sf uint8[rows][k/16], g float32).
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    if x.ndim != 2:
        raise ValueError("x must be 2-D")
    rows, k = x.shape
    if k % 16:
        raise ValueError("k must be a multiple of 16")
    q = np.zeros((rows, k // 2), dtype=np.uint8)
    sf = np.zeros((rows, k // 16), dtype=np.uint8)
    gbuf = np.array([0.0 if g is None else g], dtype=np.float32)
    rc = _load().oracle_quantize(_ptr(x, ctypes.c_float), rows, k, k, _ptr(gbuf, ctypes.c_float),
                                 1 if g is None else 0, _ptr(q, ctypes.c_uint8),
                                 _ptr(sf, ctypes.c_uint8))
    if rc != 0:
        raise ValueError("oracle_quantize rejected its arguments")
    return q, sf, np.float32(gbuf[0])


# ------------------------------------------------------------ grouped GEMM --

def _gemm_args(a_q, a_sf, a_scale, w_q, w_sf, w_scale, offsets, a_row_index, rows_sel):
    a_q = np.ascontiguousarray(a_q, dtype=np.uint8)
    a_sf = np.ascontiguousarray(a_sf, dtype=np.uint8)
    w_q = np.ascontiguousarray(w_q, dtype=np.uint8)
    w_sf = np.ascontiguousarray(w_sf, dtype=np.uint8)
    w_scale = np.ascontiguousarray(w_scale, dtype=np.float32)
    offsets = np.ascontiguousarray(offsets, dtype=np.int32)
    E, n, kb = w_q.shape
    k = kb * 2
    m_total = int(offsets[-1])
    if a_row_index is not None:
        a_row_index = np.ascontiguousarray(a_row_index, dtype=np.int32)
    if rows_sel is not None:
        rows_sel = np.ascontiguousarray(rows_sel, dtype=np.int64)
        nsel = rows_sel.shape[0]
    else:
        nsel = m_total
    return (a_q, a_sf, float(a_scale), w_q, w_sf, w_scale, offsets, a_row_index, rows_sel,
            E, n, k, m_total, nsel)


def grouped_gemm(a_q, a_sf, a_scale, w_q, w_sf, w_scale, offsets, a_row_index=None,
                 rows_sel=None):
    """Exact grouped GEMM.  Returns (R float64 [nsel][n], out_bf16_bits uint16 [nsel][n])."""
    (a_q, a_sf, a_scale, w_q, w_sf, w_scale, offsets, a_row_index, rows_sel,
     E, n, k, m_total, nsel) = _gemm_args(a_q, a_sf, a_scale, w_q, w_sf, w_scale, offsets,
                                          a_row_index, rows_sel)
    R = np.zeros((nsel, n), dtype=np.float64)
    out = np.zeros((nsel, n), dtype=np.uint16)
    rc = _load().oracle_grouped_gemm_exact(
        _ptr(a_q, ctypes.c_uint8), _ptr(a_sf, ctypes.c_uint8), a_scale, a_q.shape[0],
        _ptr(a_row_index, ctypes.c_int32), _ptr(w_q, ctypes.c_uint8), _ptr(w_sf, ctypes.c_uint8),
        _ptr(w_scale, ctypes.c_float), _ptr(offsets, ctypes.c_int32), E, m_total, n, k,
        _ptr(rows_sel, ctypes.c_int64), nsel, _ptr(R, ctypes.c_double), _ptr(out, ctypes.c_uint16))
    if rc != 0:
        raise ValueError("oracle_grouped_gemm_exact rejected its arguments")
    return R, out


def grouped_gemm_f64(a_q, a_sf, a_scale, w_q, w_sf, w_scale, offsets, a_row_index=None,
                     rows_sel=None):
    """FP64-accumulating evaluation of the same definition.  Returns R float64 [nsel][n]."""
    (a_q, a_sf, a_scale, w_q, w_sf, w_scale, offsets, a_row_index, rows_sel,
     E, n, k, m_total, nsel) = _gemm_args(a_q, a_sf, a_scale, w_q, w_sf, w_scale, offsets,
                                          a_row_index, rows_sel)
    R = np.zeros((nsel, n), dtype=np.float64)
    rc = _load().oracle_grouped_gemm_f64(
        _ptr(a_q, ctypes.c_uint8), _ptr(a_sf, ctypes.c_uint8), a_scale, a_q.shape[0],
        _ptr(a_row_index, ctypes.c_int32), _ptr(w_q, ctypes.c_uint8), _ptr(w_sf, ctypes.c_uint8),
        _ptr(w_scale, ctypes.c_float), _ptr(offsets, ctypes.c_int32), E, m_total, n, k,
        _ptr(rows_sel, ctypes.c_int64), nsel, _ptr(R, ctypes.c_double))
    if rc != 0:
        raise ValueError("oracle_grouped_gemm_f64 rejected its arguments")
    return R


def row_error(got_bf16_bits: np.ndarray, ref_bf16_bits: np.ndarray, R: np.ndarray):
    """Per-row relative error of a BF16 result against the oracle.

    err[r] = ||got[r] - ref[r]||_2 / ||R[r]||_2 where ref = bf16(R) (the oracle's rounded
    output) and R the unrounded oracle value; 0 when both rows are zero, inf when the
    reference row is zero but the result is not.  Returns (err, ||R[r]||_2).
    """
    ref = bf16_bits_to_float(ref_bf16_bits).astype(np.float64)
    got = bf16_bits_to_float(got_bf16_bits).astype(np.float64)
    diff = np.linalg.norm(got - ref, axis=1)
    norm = np.linalg.norm(R, axis=1)
    safe = np.where(norm > 0, norm, 1.0)
    err = np.where(norm > 0, diff / safe, np.where(diff > 0, np.inf, 0.0))
    return err, norm


def combine(R: np.ndarray, out_token: np.ndarray, row_weight: np.ndarray, num_tokens: int,
            init: np.ndarray | None = None) -> np.ndarray:
    """MoE finalize step: every routed row's GEMM result, times the row's routing
    weight, summed into its token's output row.

    The pages name the epilogue that performs the final output write FINALIZE
    ("Peering into the CUTLASS Kernel", section "Input Knowledge Required", item 5);
    in the Mixture-of-Experts down projection that write is read here as the
    routing-weighted sum of a token's expert rows (the step after the plain store
    of the grouped GEMM):

        out[t][j] = init[t][j] + sum over rows r with out_token[r] = t of
                    row_weight[r] * R[r][j]

    R float64 [m_total][n] (the exact grouped-GEMM result, unrounded), out_token int
    [m_total] in [0, num_tokens), row_weight float32 [m_total]; init float [num_tokens][n]
    or None (zeros).  Evaluated in FP64.  Returns float64 [num_tokens][n].
    """
    R = np.asarray(R, dtype=np.float64)
    out_token = np.asarray(out_token, dtype=np.int64)
    row_weight = np.asarray(row_weight, dtype=np.float32).astype(np.float64)
    if R.ndim != 2 or out_token.shape != (R.shape[0],) or row_weight.shape != (R.shape[0],):
        raise ValueError("combine: R [m][n], out_token [m], row_weight [m]")
    if np.any(out_token < 0) or np.any(out_token >= num_tokens):
        raise ValueError("combine: out_token outside [0, num_tokens)")
    out = (np.zeros((num_tokens, R.shape[1])) if init is None
           else np.array(init, dtype=np.float64, copy=True))
    np.add.at(out, out_token, row_weight[:, None] * R)
    return out


def token_row_error(got: np.ndarray, ref: np.ndarray):
    """Per-row relative L2 error of an FP32 token-order result against the FP64
    reference: err[t] = ||got[t] - ref[t]||_2 / ||ref[t]||_2; 0 when both rows are zero,
    inf when the reference row is zero but the result is not.  Returns (err, ||ref[t]||)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    diff = np.linalg.norm(got - ref, axis=1)
    norm = np.linalg.norm(ref, axis=1)
    safe = np.where(norm > 0, norm, 1.0)
    err = np.where(norm > 0, diff / safe, np.where(diff > 0, np.inf, 0.0))
    return err, norm


# ------------------------------------------------- gate+up activation step --

def silu(x: np.ndarray) -> np.ndarray:
    """SiLU (the Swish gate of SwiGLU): x * sigmoid(x) = x / (1 + exp(-x)), in FP64.
    Very negative x gives exp(-x) = inf and a result of -0.0, its limit."""
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(over="ignore"):
        return x / (1.0 + np.exp(-x))


def swiglu(R: np.ndarray) -> np.ndarray:
    """The gate+up activation of a Mixture-of-Experts FFN.

    The pages allow the FINALIZE epilogue to apply an activation and a
    quantisation to the GEMM result ("Peering into the CUTLASS Kernel", section
    "Input Knowledge Required", item 5) without naming either.  Read here as the
    gated-SiLU step between the two projections: the gate+up GEMM has n = 2I
    output columns, the first I are the gate and the last I the up projection, and

        h[r][i] = silu(R[r][i]) * R[r][I + i],   0 <= i < I.

    R float64 [rows][2I] (the exact grouped-GEMM result, unrounded).  Evaluated in
    FP64.  Returns float64 [rows][I]."""
    R = np.asarray(R, dtype=np.float64)
    if R.ndim != 2 or R.shape[1] % 2:
        raise ValueError("swiglu: R must be [rows][2I]")
    inter = R.shape[1] // 2
    return silu(R[:, :inter]) * R[:, inter:]


def swiglu_quantize(R: np.ndarray, g: float):
    """The gate+up projection's output as the down projection reads it: the SwiGLU
    activation of the exact GEMM result (swiglu), rounded once to FP32, then
    NVFP4-quantised (quantize) with the static tensor scale g.  A single fused pass
    cannot know the intermediate's amax before it has produced every row, so the
    tensor scale is the caller's calibrated value.
    Returns (h float64 [rows][I], q uint8 [rows][I/2], sf uint8 [rows][I/16])."""
    h = swiglu(R)
    if h.shape[1] % 16:
        raise ValueError("swiglu_quantize: I must be a multiple of 16")
    q, sf, _ = quantize(h.astype(np.float32), g=float(np.float32(g)))
    return h, q, sf
