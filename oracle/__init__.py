"""fp64 CPU oracle for split-KV MLA decode over a paged FP8 E4M3 cache.

TEST INFRASTRUCTURE. Only the test suite, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package. It shares no code with the
HIP library (``decode_attention_gather_amd``) and neither imports the other.

The arithmetic lives in ``mla_oracle.c`` (plain C, fp64, unsplit softmax); this module
only builds it with gcc and marshals numpy arrays through ctypes. The definition it
computes is stated in the C file's header, with the passages it follows:
TensorRT-LLM issue #20510 "CuTe DSL FP8 MLA decode slower after #19338" (Setup, Repro 1)
for geometry, dtypes, scales and the causal MTP shape, and PR #20380
"trtllm-gen FMHA: split the KV partials of a row across thread groups in
fmhaReductionKernel" (Description) for the (max, sum, O) row state.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mla_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_libs = {}

D_QK = 576
D_V = 512
PAGE = 32


def build(force: bool = True) -> str:
    """Compile the oracle with gcc into oracle/liboracle.so and return its path."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-D_GNU_SOURCE", "-fPIC", "-shared", "-pthread",
               "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load(path: str | None = None):
    """Load the oracle library (or a variant built elsewhere, for mutation tests)."""
    key = path or _LIB_PATH
    if key not in _libs:
        if path is None and (not os.path.exists(_LIB_PATH) or
                             os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)):
            build(force=True)  # missing, or older than its source
        lib = ctypes.CDLL(key)
        lib.oracle_e4m3_to_double.restype = ctypes.c_double
        lib.oracle_e4m3_to_double.argtypes = [ctypes.c_uint8]
        lib.oracle_hw_threads.restype = ctypes.c_int
        lib.oracle_mla_decode_rows.restype = ctypes.c_int
        p = ctypes.c_void_p
        lib.oracle_mla_decode_rows.argtypes = [
            p, p, p, p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int64,
            ctypes.c_int64, ctypes.c_double, ctypes.c_double, p, ctypes.c_int64, p, p,
            ctypes.c_int]
        lib.oracle_mla_decode_rows_ex.restype = ctypes.c_int
        lib.oracle_mla_decode_rows_ex.argtypes = [
            p, p, p, p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int64,
            ctypes.c_int64, ctypes.c_double, ctypes.c_double, p, ctypes.c_int, p,
            ctypes.c_int64, p, p, ctypes.c_int]
        lib.oracle_mla_decode_rows_bounded.restype = ctypes.c_int
        lib.oracle_mla_decode_rows_bounded.argtypes = [
            p, p, p, p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int64,
            ctypes.c_int64, ctypes.c_double, ctypes.c_double, p, ctypes.c_int, p, p,
            ctypes.c_int64, p, p, ctypes.c_int]
        lib.oracle_bf16_to_double.restype = ctypes.c_double
        lib.oracle_bf16_to_double.argtypes = [ctypes.c_uint16]
        lib.oracle_round_bf16.restype = None
        lib.oracle_round_bf16.argtypes = [p, ctypes.c_int64, p]
        lib.oracle_mxfp8_quantize.restype = ctypes.c_int
        lib.oracle_mxfp8_quantize.argtypes = [p, ctypes.c_int64, p, p]
        _libs[key] = lib
    return _libs[key]


def e4m3_decode(code: int, lib_path: str | None = None) -> float:
    """fp64 value of one OCP E4M3FN code (NaN for 0x7F / 0xFF)."""
    return _load(lib_path).oracle_e4m3_to_double(int(code) & 0xFF)


def bf16_decode(code: int, lib_path: str | None = None) -> float:
    """fp64 value of one BF16 bit pattern."""
    return _load(lib_path).oracle_bf16_to_double(int(code) & 0xFFFF)


def e4m3_table(lib_path: str | None = None) -> np.ndarray:
    return np.array([e4m3_decode(c, lib_path) for c in range(256)], dtype=np.float64)


def hw_threads() -> int:
    return _load().oracle_hw_threads()


def _np(x, dtype):
    if hasattr(x, "detach"):  # torch tensor (CPU)
        x = x.detach().cpu().numpy()
    a = np.ascontiguousarray(x)
    if a.dtype != dtype:
        a = a.view(dtype) if a.dtype.itemsize == np.dtype(dtype).itemsize else a.astype(dtype)
    return np.ascontiguousarray(a)


def mla_decode(q, kv_cache, block_table, kv_lens, *, q_len: int, num_heads: int,
               softmax_scale: float, output_scale: float = 1.0, rows=None,
               nthreads: int = 0, lib_path: str | None = None, sinks=None,
               kv_dtype: str = "e4m3", kv_bounds=None):
    """Return (O fp64 [nrows, 512], LSE fp64 [nrows]).

    q: uint8 E4M3 codes [B, q_len, H, 576]; kv_cache: uint8 [P, 32, 576]
    (kv_dtype "bf16": int16 / uint16 BF16 bit patterns of the same shapes);
    block_table: int32 [B, stride]; kv_lens: int32 [B]. ``rows`` lists flat row ids
    r = (b*q_len + j)*H + h (None: every row in order). The scales are used as given
    (pass the fp32-rounded value when the GPU side takes fp32). ``sinks``: per-head
    sink logits [H] (None: no sink), in the units of the scaled scores. ``kv_bounds``:
    int32 [B, 2] per-request key windows [start, end) (None: no window); a row with no
    visible key gives O = 0 and LSE = -inf (the sink's logit with a sink).
    """
    lib = _load(lib_path)
    assert kv_dtype in ("e4m3", "bf16")
    bf16 = kv_dtype == "bf16"
    elem = np.uint16 if bf16 else np.uint8
    qa = _np(q, elem)
    kva = _np(kv_cache, elem)
    bta = _np(block_table, np.int32)
    kla = _np(kv_lens, np.int32)
    B = kla.shape[0]
    assert qa.size == B * q_len * num_heads * D_QK, "q shape"
    assert kva.size % (PAGE * D_QK) == 0, "kv shape"
    num_pages = kva.size // (PAGE * D_QK)
    bt2 = bta.reshape(B, -1)
    stride = bt2.shape[1]
    if rows is None:
        nrows = B * q_len * num_heads
        rows_arr = None
        rows_ptr = None
    else:
        rows_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        nrows = rows_arr.size
        rows_ptr = rows_arr.ctypes.data
    o = np.empty((nrows, D_V), dtype=np.float64)
    lse = np.empty((nrows,), dtype=np.float64)
    if kv_bounds is not None:
        kb = _np(kv_bounds, np.int32).reshape(-1)
        assert kb.size == 2 * B, "kv_bounds: [B, 2]"
        sk = None
        if sinks is not None:
            sk = np.ascontiguousarray(np.asarray(sinks, dtype=np.float64).reshape(-1))
            assert sk.size == num_heads, "one sink per head"
        rc = lib.oracle_mla_decode_rows_bounded(
            qa.ctypes.data, kva.ctypes.data, bt2.ctypes.data, kla.ctypes.data, B, q_len,
            num_heads, stride, num_pages, float(softmax_scale), float(output_scale),
            None if sk is None else sk.ctypes.data, int(bf16), kb.ctypes.data, rows_ptr,
            nrows, o.ctypes.data, lse.ctypes.data, int(nthreads))
    elif sinks is None and not bf16:
        rc = lib.oracle_mla_decode_rows(
            qa.ctypes.data, kva.ctypes.data, bt2.ctypes.data, kla.ctypes.data, B, q_len,
            num_heads, stride, num_pages, float(softmax_scale), float(output_scale), rows_ptr,
            nrows, o.ctypes.data, lse.ctypes.data, int(nthreads))
    else:
        sk = None
        if sinks is not None:
            sk = np.ascontiguousarray(np.asarray(sinks, dtype=np.float64).reshape(-1))
            assert sk.size == num_heads, "one sink per head"
        rc = lib.oracle_mla_decode_rows_ex(
            qa.ctypes.data, kva.ctypes.data, bt2.ctypes.data, kla.ctypes.data, B, q_len,
            num_heads, stride, num_pages, float(softmax_scale), float(output_scale),
            None if sk is None else sk.ctypes.data, int(bf16), rows_ptr, nrows,
            o.ctypes.data, lse.ctypes.data, int(nthreads))
    if rc != 0:
        raise ValueError(f"oracle_mla_decode_rows failed with code {rc}")
    return o, lse


def round_bf16(x, lib_path: str | None = None) -> np.ndarray:
    """fp64 array of the BF16 values nearest to x (ties to even)."""
    a = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    out = np.empty_like(a)
    _load(lib_path).oracle_round_bf16(a.ctypes.data, a.size, out.ctypes.data)
    return out


def mxfp8_quantize(x, lib_path: str | None = None):
    """MXFP8 form of rows of 512 BF16 values: (codes uint8 [n, 512], E8M0 scales uint8
    [n, 16]), one scale per 32 consecutive elements."""
    a = np.ascontiguousarray(np.asarray(x, dtype=np.float64).reshape(-1, D_V))
    n = a.shape[0]
    codes = np.empty((n, D_V), dtype=np.uint8)
    scales = np.empty((n, D_V // 32), dtype=np.uint8)
    rc = _load(lib_path).oracle_mxfp8_quantize(a.ctypes.data, n, codes.ctypes.data,
                                               scales.ctypes.data)
    if rc != 0:
        raise ValueError(f"oracle_mxfp8_quantize failed with code {rc}")
    return codes, scales
