"""Thin ctypes binding of libmla_decode.so (declared in include/mla_decode.h).

Argument marshalling only: every step of the computation runs in the library's HIP
kernels. Tensors are PyTorch tensors used as device buffers (``data_ptr()``); the
stream defaults to PyTorch's current stream. Importing this module raises if the
built library is missing — there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import List, Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmla_decode.so")

MLA_OK = 0
MLA_ERR_INVALID_ARG = -1
MLA_ERR_UNSUPPORTED_SHAPE = -2
MLA_ERR_WORKSPACE = -3
MLA_ERR_NOMEM = -4
MLA_ERR_HIP_BASE = -1000

D_QK, D_V, PAGE = 576, 512, 32

EXPORTS = [
    "mla_decode_plan", "mla_decode_plan_ex", "mla_decode_plan_graph",
    "mla_decode_plan_graph_ex", "mla_decode_plan_destroy",
    "mla_decode_workspace_size", "mla_decode_plan_get_info", "mla_decode_plan_with_merge_bound",
    "mla_decode_partial",
    "mla_decode_merge", "mla_decode_merge_f32", "mla_decode", "mla_decode_varq",
    "mla_decode_graph", "mla_decode_merge_ex", "mla_decode_ex", "mla_decode_graph_ex",
    "mla_decode_partial_ex", "mla_decode_bounded", "mla_decode_graph_bounded",
    "mla_decode_noalloc", "mla_decode_strerror",
]

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is not built; run `python -m decode_attention_gather_amd.build` "
        "(hipcc, gfx950). There is no non-HIP fallback.")

_lib = ctypes.CDLL(LIB_PATH)
_p = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_f32 = ctypes.c_float
_sz = ctypes.c_size_t


class PlanInfo(ctypes.Structure):
    _fields_ = [("batch", _i32), ("q_len", _i32), ("num_heads", _i32),
                ("rows_per_request", _i32), ("row_tiles", _i32), ("total_splits", _i32),
                ("work_items", _i32), ("merge_groups", _i32), ("max_splits", _i32),
                ("merge_slices", _i32), ("split_workgroups", _i32)]


_lib.mla_decode_plan.restype = ctypes.c_int
_lib.mla_decode_plan.argtypes = [_p, _i32, _i32, _i32, _i32, _i32, _i32, ctypes.POINTER(_p)]
_lib.mla_decode_plan_ex.restype = ctypes.c_int
_lib.mla_decode_plan_ex.argtypes = [_p, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                    ctypes.POINTER(_p)]
_lib.mla_decode_plan_graph_ex.restype = ctypes.c_int
_lib.mla_decode_plan_graph_ex.argtypes = [_i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                          ctypes.POINTER(_p)]
_lib.mla_decode_plan_graph.restype = ctypes.c_int
_lib.mla_decode_plan_graph.argtypes = [_i32, _i32, _i32, _i32, _i32, _i32, _i32, ctypes.POINTER(_p)]
_lib.mla_decode_graph.restype = ctypes.c_int
_lib.mla_decode_graph.argtypes = [_p, _p, _p, _p, _i64, _p, _p, _p, _p, _p, _sz, _p, _p, _p]
_lib.mla_decode_varq.restype = ctypes.c_int
_lib.mla_decode_varq.argtypes = [_p, _p, _p, _p, _i64, _p, _p, _f32, _f32, _p, _sz, _p, _p, _p]
_lib.mla_decode_plan_with_merge_bound.restype = ctypes.c_int
_lib.mla_decode_plan_with_merge_bound.argtypes = [_p, _i32, ctypes.POINTER(_p)]
_lib.mla_decode_plan_destroy.restype = None
_lib.mla_decode_plan_destroy.argtypes = [_p]
_lib.mla_decode_workspace_size.restype = _sz
_lib.mla_decode_workspace_size.argtypes = [_p]
_lib.mla_decode_plan_get_info.restype = ctypes.c_int
_lib.mla_decode_plan_get_info.argtypes = [_p, ctypes.POINTER(PlanInfo), _p, _p]
_lib.mla_decode_partial.restype = ctypes.c_int
_lib.mla_decode_partial.argtypes = [_p, _p, _p, _p, _i64, _p, _f32, _p, _sz, _p]
_lib.mla_decode_merge.restype = ctypes.c_int
_lib.mla_decode_merge.argtypes = [_p, _p, _sz, _f32, _p, _p, _p]
_lib.mla_decode_merge_f32.restype = ctypes.c_int
_lib.mla_decode_merge_f32.argtypes = [_p, _p, _sz, _f32, _p, _p, _p]
_lib.mla_decode.restype = ctypes.c_int
_lib.mla_decode.argtypes = [_p, _p, _p, _p, _i64, _p, _f32, _f32, _p, _sz, _p, _p, _p]
_lib.mla_decode_merge_ex.restype = ctypes.c_int
_lib.mla_decode_merge_ex.argtypes = [_p, _p, _sz, _f32, _p, _p, _p, _p, _p, _p]
_lib.mla_decode_ex.restype = ctypes.c_int
_lib.mla_decode_ex.argtypes = [_p, _p, _p, _p, _i64, _p, _p, _f32, _f32, _p, _p, _sz, _p, _p,
                               _p, _p, _p]
_lib.mla_decode_graph_ex.restype = ctypes.c_int
_lib.mla_decode_graph_ex.argtypes = [_p, _p, _p, _p, _i64, _p, _p, _p, _p, _p, _p, _sz, _p, _p,
                                     _p, _p, _p]
_lib.mla_decode_partial_ex.restype = ctypes.c_int
_lib.mla_decode_partial_ex.argtypes = [_p, _p, _p, _p, _i64, _p, _p, _p, _f32, _p, _sz, _p]
_lib.mla_decode_bounded.restype = ctypes.c_int
_lib.mla_decode_bounded.argtypes = [_p, _p, _p, _p, _i64, _p, _p, _p, _f32, _f32, _p, _p, _sz,
                                    _p, _p, _p, _p, _p]
_lib.mla_decode_graph_bounded.restype = ctypes.c_int
_lib.mla_decode_graph_bounded.argtypes = [_p, _p, _p, _p, _i64, _p, _p, _p, _p, _p, _p, _p, _sz,
                                          _p, _p, _p, _p, _p]
_lib.mla_decode_noalloc.restype = ctypes.c_int
_lib.mla_decode_noalloc.argtypes = [_p, _p, _p, _p, _i64, _p, _f32, _f32, _p, _p, _p]
_lib.mla_decode_strerror.restype = ctypes.c_char_p
_lib.mla_decode_strerror.argtypes = [ctypes.c_int]


class MlaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {strerror(status)} (status {status})")


def strerror(status: int) -> str:
    return _lib.mla_decode_strerror(int(status)).decode()


def lib_handle():
    return _lib


def _check(status: int, where: str):
    if status != MLA_OK:
        raise MlaError(status, where)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream))


MLA_KV_E4M3, MLA_KV_BF16 = 0, 1


def _kv_dtype_code(kv_dtype: str) -> int:
    codes = {"e4m3": MLA_KV_E4M3, "bf16": MLA_KV_BF16}
    if kv_dtype not in codes:
        raise ValueError(f"kv_dtype must be one of {sorted(codes)}")
    return codes[kv_dtype]


class Plan:
    """Owns an mla_decode_plan_t; freed on close() / garbage collection. kv_dtype: "e4m3"
    (q and cache hold E4M3 codes) or "bf16" (BF16 values)."""

    def __init__(self, kv_lens: Sequence[int], *, q_len: int, num_heads: int, split_kv: int = 0,
                 max_split_kv: int = 256, num_cus: int = 0, kv_dtype: str = "e4m3"):
        lens = (ctypes.c_int32 * len(kv_lens))(*[int(x) for x in kv_lens])
        h = ctypes.c_void_p()
        _check(_lib.mla_decode_plan_ex(lens, len(kv_lens), q_len, num_heads, split_kv,
                                       max_split_kv, num_cus, _kv_dtype_code(kv_dtype),
                                       ctypes.byref(h)), "mla_decode_plan_ex")
        self.kv_dtype = kv_dtype
        self._h = h
        self._destroy = _lib.mla_decode_plan_destroy  # kept: module globals may be gone at exit
        self.batch = len(kv_lens)
        self.q_len = q_len
        self.num_heads = num_heads

    @classmethod
    def graph(cls, batch: int, *, q_len: int, num_heads: int, max_kv_len: int,
              split_kv: int = 0, max_split_kv: int = 256, num_cus: int = 0,
              kv_dtype: str = "e4m3") -> "Plan":
        """A graph plan: shapes and bounds only; the splits are planned on the device from
        the device lengths on every decode_graph() call (capturable in a HIP graph)."""
        self = cls.__new__(cls)
        h = ctypes.c_void_p()
        _check(_lib.mla_decode_plan_graph_ex(batch, q_len, num_heads, max_kv_len, split_kv,
                                             max_split_kv, num_cus, _kv_dtype_code(kv_dtype),
                                             ctypes.byref(h)), "mla_decode_plan_graph_ex")
        self.kv_dtype = kv_dtype
        self._h = h
        self._destroy = _lib.mla_decode_plan_destroy
        self.batch = batch
        self.q_len = q_len
        self.num_heads = num_heads
        return self

    def with_merge_bound(self, max_groups: int) -> "Plan":
        """A copy whose merge uses at most max_groups (1, 2, 4, 8, 16) wavefront groups."""
        other = type(self).__new__(type(self))
        h = ctypes.c_void_p()
        _check(_lib.mla_decode_plan_with_merge_bound(self._h, int(max_groups), ctypes.byref(h)),
               "mla_decode_plan_with_merge_bound")
        other.__dict__.update({k: v for k, v in self.__dict__.items() if k != "_h"})
        other._h = h
        return other

    @property
    def handle(self):
        return self._h

    def close(self):
        if getattr(self, "_h", None):
            self._destroy(self._h)
            self._h = None

    def __del__(self):
        self.close()

    def workspace_size(self) -> int:
        return int(_lib.mla_decode_workspace_size(self._h))

    def info(self):
        inf = PlanInfo()
        splits = (ctypes.c_int32 * self.batch)()
        chunk = (ctypes.c_int32 * self.batch)()
        _check(_lib.mla_decode_plan_get_info(self._h, ctypes.byref(inf), splits, chunk),
               "mla_decode_plan_get_info")
        return inf, list(splits), list(chunk)

    def alloc_workspace(self, device="cuda") -> torch.Tensor:
        # torch's caching allocator returns 256-byte aligned blocks
        return torch.empty(max(1, self.workspace_size()), dtype=torch.uint8, device=device)


def _check_kv(plan: Plan, q, kv_cache):
    """q and the cache must hold the plan's element type (1 byte E4M3, 2 bytes BF16) in
    the [.., 576] / [P, 32, 576] layouts: the kernels address them by that size."""
    es = 2 if getattr(plan, "kv_dtype", "e4m3") == "bf16" else 1
    for name, t in (("q", q), ("kv_cache", kv_cache)):
        if t.element_size() != es or t.shape[-1] != D_QK or not t.is_contiguous():
            raise TypeError(f"{name}: expected contiguous {plan.kv_dtype} elements "
                            f"({es} byte(s)) with a last dimension of {D_QK}, got "
                            f"{t.dtype} {tuple(t.shape)}")
    if kv_cache.dim() != 3 or kv_cache.shape[1] != PAGE:
        raise TypeError(f"kv_cache: expected [pages, {PAGE}, {D_QK}], got {tuple(kv_cache.shape)}")


def partial(plan: Plan, q, kv_cache, block_table, kv_lens, softmax_scale: float, workspace,
            stream=None):
    _check_kv(plan, q, kv_cache)
    _check(_lib.mla_decode_partial(plan.handle, _ptr(q), _ptr(kv_cache), _ptr(block_table),
                                   block_table.stride(0), _ptr(kv_lens), float(softmax_scale),
                                   _ptr(workspace), workspace.numel(), _stream(stream)),
           "mla_decode_partial")


def merge(plan: Plan, workspace, output_scale: float, o, lse=None, stream=None):
    fn = _lib.mla_decode_merge_f32 if o.dtype == torch.float32 else _lib.mla_decode_merge
    if o.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("o must be bfloat16 or float32")
    _check(fn(plan.handle, _ptr(workspace), workspace.numel(), float(output_scale), _ptr(o),
              _ptr(lse), _stream(stream)), "mla_decode_merge")


def decode(plan: Plan, q, kv_cache, block_table, kv_lens, softmax_scale: float,
           output_scale: float, workspace, o, lse=None, stream=None, q_lens=None):
    """q_lens (device int32 [B], optional): a ragged batch (mla_decode_varq)."""
    _check_kv(plan, q, kv_cache)
    if o.dtype != torch.bfloat16:
        raise TypeError("o must be bfloat16")
    if q_lens is not None:
        _check(_lib.mla_decode_varq(plan.handle, _ptr(q), _ptr(kv_cache), _ptr(block_table),
                                    block_table.stride(0), _ptr(kv_lens), _ptr(q_lens),
                                    float(softmax_scale), float(output_scale), _ptr(workspace),
                                    workspace.numel(), _ptr(o), _ptr(lse), _stream(stream)),
               "mla_decode_varq")
        return
    _check(_lib.mla_decode(plan.handle, _ptr(q), _ptr(kv_cache), _ptr(block_table),
                           block_table.stride(0), _ptr(kv_lens), float(softmax_scale),
                           float(output_scale), _ptr(workspace), workspace.numel(), _ptr(o),
                           _ptr(lse), _stream(stream)), "mla_decode")


def _check_i32(name, t, numel=None):
    if t is None:
        return
    if t.dtype != torch.int32 or not t.is_cuda or not t.is_contiguous():
        raise TypeError(f"{name} must be a contiguous int32 device tensor")
    if numel is not None and t.numel() != numel:
        raise TypeError(f"{name}: expected {numel} elements, got {t.numel()}")


def partial_ex(plan: Plan, q, kv_cache, block_table, kv_lens, softmax_scale: float, workspace,
               q_lens=None, kv_bounds=None, stream=None):
    """Partial pass with optional q_lens (int32 [B]) and kv_bounds (int32 [B, 2])."""
    _check_kv(plan, q, kv_cache)
    _check_i32("q_lens", q_lens, plan.batch)
    _check_i32("kv_bounds", kv_bounds, 2 * plan.batch)
    _check(_lib.mla_decode_partial_ex(plan.handle, _ptr(q), _ptr(kv_cache), _ptr(block_table),
                                      block_table.stride(0), _ptr(kv_lens), _ptr(q_lens),
                                      _ptr(kv_bounds), float(softmax_scale), _ptr(workspace),
                                      workspace.numel(), _stream(stream)), "mla_decode_partial_ex")


def decode_bounded(plan: Plan, q, kv_cache, block_table, kv_lens, kv_bounds, softmax_scale: float,
                   output_scale: float, workspace, o=None, lse=None, q_lens=None, sinks=None,
                   o_fp8=None, o_fp8_scales=None, stream=None):
    """decode_ex confined to per-request key windows kv_bounds (int32 [B, 2], device)."""
    _check_kv(plan, q, kv_cache)
    _epilogue_args(o, sinks, o_fp8, o_fp8_scales)
    _check_i32("q_lens", q_lens, plan.batch)
    _check_i32("kv_bounds", kv_bounds, 2 * plan.batch)
    _check(_lib.mla_decode_bounded(plan.handle, _ptr(q), _ptr(kv_cache), _ptr(block_table),
                                   block_table.stride(0), _ptr(kv_lens), _ptr(q_lens),
                                   _ptr(kv_bounds), float(softmax_scale), float(output_scale),
                                   _ptr(sinks), _ptr(workspace), workspace.numel(), _ptr(o),
                                   _ptr(lse), _ptr(o_fp8), _ptr(o_fp8_scales), _stream(stream)),
           "mla_decode_bounded")


def decode_graph_bounded(plan: Plan, q, kv_cache, block_table, kv_lens, kv_bounds, softmax_scale,
                         output_scale, workspace, o=None, lse=None, q_lens=None, sinks=None,
                         o_fp8=None, o_fp8_scales=None, stream=None):
    """decode_graph_ex confined to per-request key windows kv_bounds (int32 [B, 2])."""
    _check_kv(plan, q, kv_cache)
    _epilogue_args(o, sinks, o_fp8, o_fp8_scales)
    _check_i32("q_lens", q_lens, plan.batch)
    _check_i32("kv_bounds", kv_bounds, 2 * plan.batch)
    for name, t in (("softmax_scale", softmax_scale), ("output_scale", output_scale)):
        if t.dtype != torch.float32 or not t.is_cuda:
            raise TypeError(f"{name} must be a float32 device tensor")
    _check(_lib.mla_decode_graph_bounded(plan.handle, _ptr(q), _ptr(kv_cache), _ptr(block_table),
                                         block_table.stride(0), _ptr(kv_lens), _ptr(q_lens),
                                         _ptr(kv_bounds), _ptr(softmax_scale), _ptr(output_scale),
                                         _ptr(sinks), _ptr(workspace), workspace.numel(), _ptr(o),
                                         _ptr(lse), _ptr(o_fp8), _ptr(o_fp8_scales),
                                         _stream(stream)), "mla_decode_graph_bounded")


NOALLOC_SCRATCH_BYTES = 64 << 20


def decode_noalloc(plan: Plan, q, kv_cache, block_table, kv_lens, softmax_scale: float,
                   output_scale: float, o, lse=None, stream=None):
    """mla_decode with the library's per-GPU scratch array in place of a workspace (for
    callers that cannot allocate); calls that overlap on one GPU race."""
    _check_kv(plan, q, kv_cache)
    if o.dtype != torch.bfloat16:
        raise TypeError("o must be bfloat16")
    _check(_lib.mla_decode_noalloc(plan.handle, _ptr(q), _ptr(kv_cache), _ptr(block_table),
                                   block_table.stride(0), _ptr(kv_lens), float(softmax_scale),
                                   float(output_scale), _ptr(o), _ptr(lse), _stream(stream)),
           "mla_decode_noalloc")


def decode_graph(plan: Plan, q, kv_cache, block_table, kv_lens, softmax_scale, output_scale,
                 workspace, o, lse=None, stream=None, q_lens=None):
    """Device-planned decode: kv_lens, softmax_scale and output_scale are device tensors
    (int32 [B], float32 [1], float32 [1]); nothing here reads them on the host."""
    _check_kv(plan, q, kv_cache)
    if o.dtype != torch.bfloat16:
        raise TypeError("o must be bfloat16")
    for name, t in (("softmax_scale", softmax_scale), ("output_scale", output_scale)):
        if t.dtype != torch.float32 or not t.is_cuda:
            raise TypeError(f"{name} must be a float32 device tensor")
    _check(_lib.mla_decode_graph(plan.handle, _ptr(q), _ptr(kv_cache), _ptr(block_table),
                                 block_table.stride(0), _ptr(kv_lens), _ptr(q_lens),
                                 _ptr(softmax_scale),
                                 _ptr(output_scale), _ptr(workspace), workspace.numel(), _ptr(o),
                                 _ptr(lse), _stream(stream)), "mla_decode_graph")


def _epilogue_args(o, sinks, o_fp8, o_fp8_scales):
    if o is not None and o.dtype != torch.bfloat16:
        raise TypeError("o must be bfloat16")
    if sinks is not None and (sinks.dtype != torch.float32 or not sinks.is_cuda):
        raise TypeError("sinks must be a float32 device tensor [H]")
    for name, t in (("o_fp8", o_fp8), ("o_fp8_scales", o_fp8_scales)):
        if t is not None and t.dtype != torch.uint8:
            raise TypeError(f"{name} must be uint8")


def merge_ex(plan: Plan, workspace, output_scale: float, o=None, lse=None, sinks=None,
             o_fp8=None, o_fp8_scales=None, stream=None):
    """Merge with the epilogue options: per-head sinks, and the MXFP8 form of O
    (o_fp8 uint8 [rows, 512] E4M3 codes, o_fp8_scales uint8 [rows, 16] E8M0)."""
    _epilogue_args(o, sinks, o_fp8, o_fp8_scales)
    _check(_lib.mla_decode_merge_ex(plan.handle, _ptr(workspace), workspace.numel(),
                                    float(output_scale), _ptr(sinks), _ptr(o), _ptr(lse),
                                    _ptr(o_fp8), _ptr(o_fp8_scales), _stream(stream)),
           "mla_decode_merge_ex")


def decode_ex(plan: Plan, q, kv_cache, block_table, kv_lens, softmax_scale: float,
              output_scale: float, workspace, o=None, lse=None, q_lens=None, sinks=None,
              o_fp8=None, o_fp8_scales=None, stream=None):
    _check_kv(plan, q, kv_cache)
    _epilogue_args(o, sinks, o_fp8, o_fp8_scales)
    _check(_lib.mla_decode_ex(plan.handle, _ptr(q), _ptr(kv_cache), _ptr(block_table),
                              block_table.stride(0), _ptr(kv_lens), _ptr(q_lens),
                              float(softmax_scale), float(output_scale), _ptr(sinks),
                              _ptr(workspace), workspace.numel(), _ptr(o), _ptr(lse),
                              _ptr(o_fp8), _ptr(o_fp8_scales), _stream(stream)), "mla_decode_ex")


def decode_graph_ex(plan: Plan, q, kv_cache, block_table, kv_lens, softmax_scale, output_scale,
                    workspace, o=None, lse=None, q_lens=None, sinks=None, o_fp8=None,
                    o_fp8_scales=None, stream=None):
    _check_kv(plan, q, kv_cache)
    _epilogue_args(o, sinks, o_fp8, o_fp8_scales)
    for name, t in (("softmax_scale", softmax_scale), ("output_scale", output_scale)):
        if t.dtype != torch.float32 or not t.is_cuda:
            raise TypeError(f"{name} must be a float32 device tensor")
    _check(_lib.mla_decode_graph_ex(plan.handle, _ptr(q), _ptr(kv_cache), _ptr(block_table),
                                    block_table.stride(0), _ptr(kv_lens), _ptr(q_lens),
                                    _ptr(softmax_scale), _ptr(output_scale), _ptr(sinks),
                                    _ptr(workspace), workspace.numel(), _ptr(o), _ptr(lse),
                                    _ptr(o_fp8), _ptr(o_fp8_scales), _stream(stream)),
           "mla_decode_graph_ex")


@dataclass
class DeviceCase:
    """A decode batch resident on the GPU (see decode_attention_gather_amd.inputs.Case)."""
    q: torch.Tensor
    kv: torch.Tensor
    block_table: torch.Tensor
    kv_lens: torch.Tensor
    kv_lens_host: List[int]
    q_len: int
    num_heads: int
    softmax_scale: float
    output_scale: float
    kv_dtype: str = "e4m3"


def to_device(case, device="cuda") -> DeviceCase:
    return DeviceCase(q=case.q.to(device), kv=case.kv.to(device),
                      block_table=case.block_table.to(device), kv_lens=case.kv_lens.to(device),
                      kv_lens_host=[int(x) for x in case.kv_lens.tolist()], q_len=case.q_len,
                      num_heads=case.num_heads, softmax_scale=case.softmax_scale,
                      output_scale=case.output_scale,
                      kv_dtype=getattr(case, "kv_dtype", "e4m3"))


def run_decode(dc: DeviceCase, plan: Plan, workspace=None, f32_out: bool = False):
    """Run partial + merge; returns (O [B*q*H, 512], LSE [B*q*H])."""
    rows = len(dc.kv_lens_host) * dc.q_len * dc.num_heads
    dev = dc.q.device
    if workspace is None:
        workspace = plan.alloc_workspace(dev)
    o = torch.empty((rows, D_V), dtype=torch.float32 if f32_out else torch.bfloat16, device=dev)
    lse = torch.empty((rows,), dtype=torch.float32, device=dev)
    if f32_out:
        partial(plan, dc.q, dc.kv, dc.block_table, dc.kv_lens, dc.softmax_scale, workspace)
        merge(plan, workspace, dc.output_scale, o, lse)
    else:
        decode(plan, dc.q, dc.kv, dc.block_table, dc.kv_lens, dc.softmax_scale,
               dc.output_scale, workspace, o, lse)
    return o, lse
