"""Thin ctypes binding over librkv.so (the C ABI in include/rkv.h).

Argument marshalling only: torch tensors become device pointers and sizes,
the current HIP stream is passed through, and a non-OK status raises.  All
arithmetic happens in the HIP kernels behind the C ABI.  There is no fallback:
if the library is missing, loading fails loudly.
"""

from __future__ import annotations

import ctypes
import os
import re

import numpy as np
import torch

HERE = os.path.dirname(os.path.abspath(__file__))
DEFAULT_LIB_PATH = os.path.join(HERE, "librkv.so")
# the same library built with RKV_DEBUG: kernels report out-of-range values
DEBUG_LIB_PATH = os.path.join(HERE, "librkv_debug.so")
STAMPS_LIB_PATH = os.path.join(HERE, "librkv_stamps.so")
LIB_PATH = os.environ.get("RKV_LIB") or DEFAULT_LIB_PATH
HEADER = os.path.join(os.path.dirname(HERE), "include", "rkv.h")

(RKV_OK, RKV_ERR_INVALID_ARG, RKV_ERR_UNSUPPORTED, RKV_ERR_WORKSPACE, RKV_ERR_HIP,
 RKV_ERR_BOUNDS) = range(6)
ATTN_AUTO, ATTN_MFMA, ATTN_VALU = 0, 1, 2
BLOCK = 128
HEAD_DIM = 128
RKV_MAX_BLOCKS = 8192
RKV_MAX_QUERY_ROWS = 1 << 18     # batch * n_q_heads per call
RKV_MAX_LIST_ENTRIES = 1 << 23   # batch * n_kv_heads * longest per-list row


class Params(ctypes.Structure):
    _fields_ = [("block_size", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("init_tokens", ctypes.c_int32), ("local_tokens", ctypes.c_int32),
                ("topk_ppm", ctypes.c_int32), ("dense_boundary", ctypes.c_int32),
                ("scale", ctypes.c_float), ("attn_impl", ctypes.c_int32),
                ("split_waves", ctypes.c_int32), ("select_mode", ctypes.c_int32),
                ("copy_lanes", ctypes.c_int32)]

    def __repr__(self):
        return "Params(" + ", ".join(f"{n}={getattr(self, n)}"
                                     for n, _ in self._fields_) + ")"


class RkvError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"rkv status {status}: {msg}")
        self.status = status


SELECT_PER_HEAD = 0
SELECT_PER_SEQUENCE = 1
MAX_COPY_LANES = 8  # rkv_params.copy_lanes

_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t
_PP = ctypes.POINTER(Params)

_SIGS = {
    "rkv_params_default": (Params, [_I32, _I32]),
    "rkv_abi_version": (_I32, []),
    "rkv_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "rkv_last_error": (ctypes.c_char_p, []),
    "rkv_build_reps": (ctypes.c_int, [_PP, _P, _I64, _P, _I32, _P, _P, _I32, _P, _P]),
    "rkv_append_kv": (ctypes.c_int, [_PP, _P, _P, _P, _P, _I64, _P, _I32, _P, _I32,
                                     _P, _P]),
    "rkv_select_workspace_size": (_SZ, [_PP, _I32, _I32]),
    "rkv_topk_capacity": (_I32, [_PP, _I32]),
    "rkv_select": (ctypes.c_int, [_PP, _P, _P, _P, _P, _P, _I32, _I32, _P, _P, _I32,
                                  _P, _P, _I32, _P, _SZ, _P]),
    "rkv_append_select": (ctypes.c_int, [_PP, _P, _P, _P, _P, _I64, _P, _P, _P, _P,
                                         _P, _I32, _I32, _P, _P, _I32, _P, _P, _I32,
                                         _P, _SZ, _P]),
    "rkv_merge_table": (ctypes.c_int, [_PP, _P, _I32, _P, _P, _P, _I32, _I32, _P,
                                       _I64, _P, _P, _I32, _P]),
    "rkv_stage_blocks": (ctypes.c_int, [_PP, _P, _P, _I64, _P, _I32, _P, _P, _I32,
                                        _I32, _P, _P, _I64, _I64, _P]),
    "rkv_offload_blocks": (ctypes.c_int, [_PP, _P, _P, _I64, _P, _I32, _P, _I32, _P,
                                          _P, _P, _I64, _P]),
    "rkv_stage_workspace_size": (_SZ, [_PP, _I32, _I32]),
    "rkv_stage_resident": (ctypes.c_int, [_PP, _P, _P, _I64, _P, _P, _I32, _P, _P,
                                          _P, _I32, _I32, _I32, _P, _P, _P, _P, _I64,
                                          _I64, _P, _P, _I32, _P, _P, _SZ, _P]),
    "rkv_stage_plan": (ctypes.c_int, [_PP, _P, _P, _I32, _P, _P, _P, _I32, _I32, _I32, _P,
                                      _P, _I64, _I64, _P, _P, _I32, _P, _P, _P, _P, _SZ,
                                      _P]),
    "rkv_stage_copy": (ctypes.c_int, [_PP, _P, _P, _I64, _P, _I32, _I32, _I32, _I32, _P,
                                      _P, _I64, _I64, _P, _SZ, _P]),
    "rkv_stage_host_list_size": (_SZ, [_PP, _I32, _I32]),
    "rkv_stage_blocks_async": (ctypes.c_int, [_PP, _P, _P, _I64, _P, _I32, _P, _P, _I32,
                                              _I32, _P, _P, _I64, _I64, _P, _SZ, _P, _P,
                                              _P]),
    "rkv_stage_resident_async": (ctypes.c_int, [_PP, _P, _P, _I64, _P, _P, _P, _I32, _P,
                                                _P, _P, _I32, _I32, _I32, _P, _P, _P, _P,
                                                _I64, _I64, _P, _P, _I32, _P, _P, _SZ, _P,
                                                _SZ, _P, _P, _P]),
    "rkv_attn_workspace_size": (_SZ, [_PP, _I32, _I32]),
    "rkv_decode_attn": (ctypes.c_int, [_PP, _P, _P, _P, _I64, _P, _P, _I32, _P, _I32,
                                       _P, _P, _SZ, _P]),
    "rkv_decode_attn_lse": (ctypes.c_int, [_PP, _P, _P, _P, _I64, _P, _P, _I32, _P, _I32,
                                           _P, _P, _P, _P, _P, _SZ, _P]),
    "rkv_attn_cascade_workspace_size": (_SZ, [_PP, _I32, _I32, _I32]),
    "rkv_decode_attn_cascade": (ctypes.c_int, [_PP, _P, _P, _P, _I64, _P, _P, _I32, _P,
                                               _P, _I32, _P, _I32, _I32, _P, _I32, _P,
                                               _P, _SZ, _P]),
    "rkv_select_attend": (ctypes.c_int, [_PP, _P, _P, _P, _I64, _P, _I32, _P, _P, _I32,
                                         _P, _P, _P, _I32, _P, _P, _I32, _P, _P, _SZ,
                                         _P]),
    "rkv_decode_step": (ctypes.c_int, [_PP, _P, _P, _P, _P, _I64, _P, _P, _P, _P, _P,
                                       _I32, _I32, _P, _P, _I32, _P, _P, _I32, _P, _P,
                                       _SZ, _P, _SZ, _P]),
    "rkv_decode_step_static": (ctypes.c_int, [_PP, _P, _P, _P, _P, _I64, _P, _P, _P,
                                              _P, _P, _I32, _I32, _P, _P, _I32, _P,
                                              _P, _I32, _P, _P]),
    "rkv_read_probe": (ctypes.c_int, [_P, _SZ, _P, _P]),
    "rkv_debug_set_report": (ctypes.c_int, [_P]),
    "rkv_debug_check": (ctypes.c_int, [_P, _P]),
    "rkv_debug_wave_stamps": (ctypes.c_int, [_P, _I32]),
}
RKV_STATIC_SCRATCH_BYTES = 64 << 20

_lib = None


def use_library(path: str) -> None:
    """Load the library at `path` for the calls made from now on (the
    RKV_DEBUG build, DEBUG_LIB_PATH, or back to DEFAULT_LIB_PATH).  Prepared
    calls keep the library they were prepared with."""
    global _lib, LIB_PATH
    if path != LIB_PATH:
        LIB_PATH = path
        _lib = None
    lib()


def lib() -> ctypes.CDLL:
    """Load librkv.so once; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it first "
                "(python -c 'import __graft_entry__ as g; g.build()')")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name, None)
            if f is None:  # an older library without this export
                continue
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def header_functions() -> list:
    """Names of the functions include/rkv.h declares."""
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:[\w\s\*]+?)\b(rkv_\w+)\s*\(", text, re.M)))


def _check(status: int):
    if status != RKV_OK:
        raise RkvError(status, lib().rkv_last_error().decode())


def params(n_q_heads: int, n_kv_heads: int, **kw) -> Params:
    p = lib().rkv_params_default(n_q_heads, n_kv_heads)
    for k, v in kw.items():
        if not hasattr(p, k):
            raise AttributeError(k)
        setattr(p, k, v)
    return p


def _ptr(t, dtype=None, name="tensor", shape=None, dev=None):
    """Device pointer of a contiguous GPU tensor (None for None), after
    checking its dtype, its exact shape and its device when given: the C
    ABI takes plain pointers, so a buffer smaller than its declared layout
    would otherwise be read or written past its end on the device."""
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if dev is not None and t.device != dev:
        raise ValueError(f"{name} is on {t.device}, the other buffers on {dev}")
    return t.data_ptr()


def _stream(t: torch.Tensor):
    return torch.cuda.current_stream(t.device).cuda_stream


def _pool_shape(p: Params, pool):
    """[n_pages][n_kv_heads][128][128] (K token-major, V dim-major)."""
    return (pool.shape[0], p.n_kv_heads, BLOCK, HEAD_DIM)


def build_reps(p: Params, k_pages, block_table, lens, reps, block_begin=None):
    batch, mb = block_table.shape
    d = k_pages.device
    _check(lib().rkv_build_reps(
        ctypes.byref(p), _ptr(k_pages, torch.int16, "k_pages", _pool_shape(p, k_pages), d),
        k_pages.shape[0],
        _ptr(block_table, torch.int32, "block_table", None, d), mb,
        _ptr(lens, torch.int32, "lens", (batch,), d),
        _ptr(block_begin, torch.int32, "block_begin", (batch,), d), batch,
        _ptr(reps, torch.float32, "reps", (batch, p.n_kv_heads, mb, HEAD_DIM), d),
        _stream(k_pages)))


def append_kv(p: Params, k_new, v_new, k_pages, v_pages, block_table, lens,
              reps=None):
    batch, mb = block_table.shape
    d = k_pages.device
    kv = (batch, p.n_kv_heads, HEAD_DIM)
    _check(lib().rkv_append_kv(
        ctypes.byref(p), _ptr(k_new, torch.int16, "k_new", kv, d),
        _ptr(v_new, torch.int16, "v_new", kv, d),
        _ptr(k_pages, torch.int16, "k_pages", _pool_shape(p, k_pages), d),
        _ptr(v_pages, torch.int16, "v_pages", _pool_shape(p, k_pages), d), k_pages.shape[0],
        _ptr(block_table, torch.int32, "block_table", None, d), mb,
        _ptr(lens, torch.int32, "lens", (batch,), d), batch,
        _ptr(reps, torch.float32, "reps", (batch, p.n_kv_heads, mb, HEAD_DIM), d),
        _stream(k_pages)))


def select_workspace_size(p: Params, batch: int, max_blocks: int) -> int:
    return lib().rkv_select_workspace_size(ctypes.byref(p), batch, max_blocks)


def select(p: Params, q, reps, block_table, lens, sel_ids, n_sel,
           merged=None, n_merged=None, prompt_lens=None, workspace=None):
    batch, mb = block_table.shape
    d = q.device
    hkv = p.n_kv_heads
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().rkv_select(
        ctypes.byref(p), _ptr(q, torch.int16, "q", (batch, p.n_q_heads, HEAD_DIM), d),
        _ptr(reps, torch.float32, "reps", (batch, hkv, mb, HEAD_DIM), d),
        _ptr(block_table, torch.int32, "block_table", None, d),
        _ptr(lens, torch.int32, "lens", (batch,), d),
        _ptr(prompt_lens, torch.int32, "prompt_lens", (batch,), d), batch, mb,
        _ptr(sel_ids, torch.int32, "sel_ids", (batch, hkv, sel_ids.shape[-1]), d),
        _ptr(n_sel, torch.int32, "n_sel", (batch, hkv), d), sel_ids.shape[-1],
        _ptr(merged, torch.int32, "merged",
             None if merged is None else (batch, hkv, merged.shape[-1]), d),
        _ptr(n_merged, torch.int32, "n_merged", (batch, hkv), d),
        merged.shape[-1] if merged is not None else 0,
        _ptr(workspace, None, "workspace", None, d), ws_bytes, _stream(q)))


def append_select(p: Params, k_new, v_new, k_pages, v_pages, q, reps, block_table,
                  lens, sel_ids, n_sel, merged=None, n_merged=None,
                  prompt_lens=None, workspace=None):
    batch, mb = block_table.shape
    d = q.device
    hkv = p.n_kv_heads
    kv = (batch, hkv, HEAD_DIM)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().rkv_append_select(
        ctypes.byref(p), _ptr(k_new, torch.int16, "k_new", kv, d),
        _ptr(v_new, torch.int16, "v_new", kv, d),
        _ptr(k_pages, torch.int16, "k_pages", _pool_shape(p, k_pages), d),
        _ptr(v_pages, torch.int16, "v_pages", _pool_shape(p, k_pages), d), k_pages.shape[0],
        _ptr(q, torch.int16, "q", (batch, p.n_q_heads, HEAD_DIM), d),
        _ptr(reps, torch.float32, "reps", (batch, hkv, mb, HEAD_DIM), d),
        _ptr(block_table, torch.int32, "block_table", None, d),
        _ptr(lens, torch.int32, "lens", (batch,), d),
        _ptr(prompt_lens, torch.int32, "prompt_lens", (batch,), d), batch, mb,
        _ptr(sel_ids, torch.int32, "sel_ids", (batch, hkv, sel_ids.shape[-1]), d),
        _ptr(n_sel, torch.int32, "n_sel", (batch, hkv), d), sel_ids.shape[-1],
        _ptr(merged, torch.int32, "merged",
             None if merged is None else (batch, hkv, merged.shape[-1]), d),
        _ptr(n_merged, torch.int32, "n_merged", (batch, hkv), d),
        merged.shape[-1] if merged is not None else 0,
        _ptr(workspace, None, "workspace", None, d), ws_bytes, _stream(q)))


def merge_table(p: Params, block_table, lens, sel_ids, n_sel, merged, n_merged,
                host_table=None, stage_page0: int = -1):
    batch, mb = block_table.shape
    d = block_table.device
    hkv = p.n_kv_heads
    _check(lib().rkv_merge_table(
        ctypes.byref(p), _ptr(block_table, torch.int32, "block_table", None, d), mb,
        _ptr(lens, torch.int32, "lens", (batch,), d),
        _ptr(sel_ids, torch.int32, "sel_ids", (batch, hkv, sel_ids.shape[-1]), d),
        _ptr(n_sel, torch.int32, "n_sel", (batch, hkv), d), sel_ids.shape[-1], batch,
        _ptr(host_table, torch.int32, "host_table", (batch, mb), d), stage_page0,
        _ptr(merged, torch.int32, "merged", (batch, hkv, merged.shape[-1]), d),
        _ptr(n_merged, torch.int32, "n_merged", (batch, hkv), d), merged.shape[-1],
        _stream(block_table)))


def _host_ptr(t, name, shape=None):
    if not isinstance(t, torch.Tensor) or t.is_cuda or not t.is_pinned():
        raise ValueError(f"{name} must be a pinned host tensor")
    if t.dtype != torch.int16 or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous int16 tensor")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t.data_ptr()


def stage_blocks(p: Params, host_k, host_v, host_table, sel_ids, n_sel,
                 k_pages, v_pages, stage_page0: int):
    batch, mb = host_table.shape
    d = k_pages.device
    hkv = p.n_kv_heads
    _check(lib().rkv_stage_blocks(
        ctypes.byref(p), _host_ptr(host_k, "host_k", _pool_shape(p, host_k)),
        _host_ptr(host_v, "host_v", _pool_shape(p, host_k)),
        host_k.shape[0], _ptr(host_table, torch.int32, "host_table", None, d), mb,
        _ptr(sel_ids, torch.int32, "sel_ids", (batch, hkv, sel_ids.shape[-1]), d),
        _ptr(n_sel, torch.int32, "n_sel", (batch, hkv), d), sel_ids.shape[-1], batch,
        _ptr(k_pages, torch.int16, "k_pages", _pool_shape(p, k_pages), d),
        _ptr(v_pages, torch.int16, "v_pages", _pool_shape(p, k_pages), d),
        k_pages.shape[0], stage_page0, _stream(k_pages)))


def offload_blocks(p: Params, k_pages, v_pages, block_table, lens, host_table,
                   host_k, host_v):
    batch, mb = block_table.shape
    d = k_pages.device
    _check(lib().rkv_offload_blocks(
        ctypes.byref(p), _ptr(k_pages, torch.int16, "k_pages", _pool_shape(p, k_pages), d),
        _ptr(v_pages, torch.int16, "v_pages", _pool_shape(p, k_pages), d), k_pages.shape[0],
        _ptr(block_table, torch.int32, "block_table", None, d), mb,
        _ptr(lens, torch.int32, "lens", (batch,), d), batch,
        _ptr(host_table, torch.int32, "host_table", (batch, mb), d),
        _host_ptr(host_k, "host_k", _pool_shape(p, host_k)),
        _host_ptr(host_v, "host_v", _pool_shape(p, host_k)), host_k.shape[0],
        _stream(k_pages)))


def stage_workspace_size(p: Params, batch: int, k_cap: int) -> int:
    return lib().rkv_stage_workspace_size(ctypes.byref(p), batch, k_cap)


def stage_resident(p: Params, host_k, host_v, host_table, block_table, lens,
                   sel_ids, n_sel, slot_ids, slot_cursor, k_pages, v_pages,
                   stage_page0: int, merged, n_merged, workspace, n_staged=None):
    batch, mb = block_table.shape
    d = k_pages.device
    hkv = p.n_kv_heads
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib().rkv_stage_resident(
        ctypes.byref(p), _host_ptr(host_k, "host_k", _pool_shape(p, host_k)),
        _host_ptr(host_v, "host_v", _pool_shape(p, host_k)),
        host_k.shape[0], _ptr(host_table, torch.int32, "host_table", (batch, mb), d),
        _ptr(block_table, torch.int32, "block_table", None, d), mb,
        _ptr(lens, torch.int32, "lens", (batch,), d),
        _ptr(sel_ids, torch.int32, "sel_ids", (batch, hkv, sel_ids.shape[-1]), d),
        _ptr(n_sel, torch.int32, "n_sel", (batch, hkv), d), sel_ids.shape[-1], batch,
        slot_ids.shape[-1],
        _ptr(slot_ids, torch.int32, "slot_ids", (batch, hkv, slot_ids.shape[-1]), d),
        _ptr(slot_cursor, torch.int32, "slot_cursor", (batch, hkv), d),
        _ptr(k_pages, torch.int16, "k_pages", _pool_shape(p, k_pages), d),
        _ptr(v_pages, torch.int16, "v_pages", _pool_shape(p, k_pages), d),
        k_pages.shape[0], stage_page0,
        _ptr(merged, torch.int32, "merged", (batch, hkv, merged.shape[-1]), d),
        _ptr(n_merged, torch.int32, "n_merged", (batch, hkv), d), merged.shape[-1],
        None if n_staged is None else _ptr(n_staged, torch.int32, "n_staged",
                                           (batch, hkv), d),
        _ptr(workspace, None, "workspace", None, d), ws_bytes, _stream(k_pages)))


def stage_plan(p: Params, host_table, block_table, lens, sel_ids, n_sel, slot_ids,
               slot_cursor, n_pages: int, stage_page0: int, merged, n_merged, workspace,
               merged_new=None, n_new=None, n_staged=None):
    """The residency planner alone (rkv_stage_plan); with merged_new / n_new,
    split mode: merged keeps the entries in HBM before the copies, merged_new
    the staging pages of the blocks copied now."""
    batch, mb = block_table.shape
    d = block_table.device
    hkv = p.n_kv_heads
    ws_bytes = workspace.numel() * workspace.element_size()
    k_cap = sel_ids.shape[-1]
    _check(lib().rkv_stage_plan(
        ctypes.byref(p), _ptr(host_table, torch.int32, "host_table", (batch, mb), d),
        _ptr(block_table, torch.int32, "block_table", None, d), mb,
        _ptr(lens, torch.int32, "lens", (batch,), d),
        _ptr(sel_ids, torch.int32, "sel_ids", (batch, hkv, k_cap), d),
        _ptr(n_sel, torch.int32, "n_sel", (batch, hkv), d), k_cap, batch,
        slot_ids.shape[-1],
        _ptr(slot_ids, torch.int32, "slot_ids", (batch, hkv, slot_ids.shape[-1]), d),
        _ptr(slot_cursor, torch.int32, "slot_cursor", (batch, hkv), d),
        n_pages, stage_page0,
        _ptr(merged, torch.int32, "merged", (batch, hkv, merged.shape[-1]), d),
        _ptr(n_merged, torch.int32, "n_merged", (batch, hkv), d), merged.shape[-1],
        None if merged_new is None else _ptr(merged_new, torch.int32, "merged_new",
                                             (batch, hkv, k_cap), d),
        None if n_new is None else _ptr(n_new, torch.int32, "n_new", (batch, hkv), d),
        None if n_staged is None else _ptr(n_staged, torch.int32, "n_staged",
                                           (batch, hkv), d),
        _ptr(workspace, None, "workspace", None, d), ws_bytes, _stream(block_table)))


def stage_copy(p: Params, host_k, host_v, host_table, k_cap: int, slot_cap: int,
               k_pages, v_pages, stage_page0: int, workspace):
    """The copies of the list the last stage_plan left in `workspace`
    (rkv_stage_copy), on the current stream."""
    batch, mb = host_table.shape
    d = k_pages.device
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib().rkv_stage_copy(
        ctypes.byref(p), _host_ptr(host_k, "host_k", _pool_shape(p, host_k)),
        _host_ptr(host_v, "host_v", _pool_shape(p, host_k)), host_k.shape[0],
        _ptr(host_table, torch.int32, "host_table", (batch, mb), d), mb, k_cap, batch,
        slot_cap, _ptr(k_pages, torch.int16, "k_pages", _pool_shape(p, k_pages), d),
        _ptr(v_pages, torch.int16, "v_pages", _pool_shape(p, k_pages), d),
        k_pages.shape[0], stage_page0, _ptr(workspace, None, "workspace", None, d),
        ws_bytes, _stream(k_pages)))


def stage_host_list_size(p: Params, batch: int, k_cap: int) -> int:
    return lib().rkv_stage_host_list_size(ctypes.byref(p), batch, k_cap)


def _host_i32(t, name, shape):
    if not isinstance(t, torch.Tensor) or t.is_cuda or t.dtype != torch.int32 \
            or not t.is_contiguous() or tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must be a contiguous int32 host tensor of shape {shape}")
    return t.data_ptr()


def _pinned_buf(t, name, nbytes):
    if not isinstance(t, torch.Tensor) or t.is_cuda or not t.is_pinned() \
            or not t.is_contiguous() or t.numel() * t.element_size() < nbytes:
        raise ValueError(f"{name} must be a pinned host tensor of at least {nbytes} bytes")
    return t.data_ptr(), t.numel() * t.element_size()


def _event(ev):
    return None if ev is None else ev.cuda_event


def stage_blocks_async(p: Params, host_k, host_v, host_table_host, sel_ids, n_sel,
                       k_pages, v_pages, stage_page0: int, host_list, side, done=None):
    """rkv_stage_blocks_async: kept ids to the host, then copy-engine copies
    of the kept host blocks on `side` (a torch stream); `done` an event."""
    batch, mb = host_table_host.shape
    d = k_pages.device
    hkv = p.n_kv_heads
    k_cap = sel_ids.shape[-1]
    lp, lb = _pinned_buf(host_list, "host_list", stage_host_list_size(p, batch, k_cap))
    _check(lib().rkv_stage_blocks_async(
        ctypes.byref(p), _host_ptr(host_k, "host_k", _pool_shape(p, host_k)),
        _host_ptr(host_v, "host_v", _pool_shape(p, host_k)), host_k.shape[0],
        _host_i32(host_table_host, "host_table_host", (batch, mb)), mb,
        _ptr(sel_ids, torch.int32, "sel_ids", (batch, hkv, k_cap), d),
        _ptr(n_sel, torch.int32, "n_sel", (batch, hkv), d), k_cap, batch,
        _ptr(k_pages, torch.int16, "k_pages", _pool_shape(p, k_pages), d),
        _ptr(v_pages, torch.int16, "v_pages", _pool_shape(p, k_pages), d),
        k_pages.shape[0], stage_page0, lp, lb, _stream(k_pages), side.cuda_stream,
        _event(done)))


def stage_resident_async(p: Params, host_k, host_v, host_table, host_table_host,
                         block_table, lens, sel_ids, n_sel, slot_ids, slot_cursor,
                         k_pages, v_pages, stage_page0: int, merged, n_merged, workspace,
                         host_list, side, done=None, n_staged=None):
    """rkv_stage_resident_async: the residency planner on the current stream,
    its copy list to the host, copy-engine copies on `side`."""
    batch, mb = block_table.shape
    d = k_pages.device
    hkv = p.n_kv_heads
    k_cap = sel_ids.shape[-1]
    ws_bytes = workspace.numel() * workspace.element_size()
    lp, lb = _pinned_buf(host_list, "host_list", stage_host_list_size(p, batch, k_cap))
    _check(lib().rkv_stage_resident_async(
        ctypes.byref(p), _host_ptr(host_k, "host_k", _pool_shape(p, host_k)),
        _host_ptr(host_v, "host_v", _pool_shape(p, host_k)), host_k.shape[0],
        _ptr(host_table, torch.int32, "host_table", (batch, mb), d),
        _host_i32(host_table_host, "host_table_host", (batch, mb)),
        _ptr(block_table, torch.int32, "block_table", None, d), mb,
        _ptr(lens, torch.int32, "lens", (batch,), d),
        _ptr(sel_ids, torch.int32, "sel_ids", (batch, hkv, k_cap), d),
        _ptr(n_sel, torch.int32, "n_sel", (batch, hkv), d), k_cap, batch,
        slot_ids.shape[-1],
        _ptr(slot_ids, torch.int32, "slot_ids", (batch, hkv, slot_ids.shape[-1]), d),
        _ptr(slot_cursor, torch.int32, "slot_cursor", (batch, hkv), d),
        _ptr(k_pages, torch.int16, "k_pages", _pool_shape(p, k_pages), d),
        _ptr(v_pages, torch.int16, "v_pages", _pool_shape(p, k_pages), d),
        k_pages.shape[0], stage_page0,
        _ptr(merged, torch.int32, "merged", (batch, hkv, merged.shape[-1]), d),
        _ptr(n_merged, torch.int32, "n_merged", (batch, hkv), d), merged.shape[-1],
        None if n_staged is None else _ptr(n_staged, torch.int32, "n_staged",
                                           (batch, hkv), d),
        _ptr(workspace, None, "workspace", None, d), ws_bytes, lp, lb,
        _stream(k_pages), side.cuda_stream, _event(done)))


def attn_workspace_size(p: Params, batch: int, m_cap: int) -> int:
    return lib().rkv_attn_workspace_size(ctypes.byref(p), batch, m_cap)


def decode_attn(p: Params, q, k_pages, v_pages, merged, n_merged, lens, out,
                workspace):
    batch = lens.shape[0]
    d = q.device
    hkv = p.n_kv_heads
    rows = (batch, p.n_q_heads, HEAD_DIM)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib().rkv_decode_attn(
        ctypes.byref(p), _ptr(q, torch.int16, "q", rows, d),
        _ptr(k_pages, torch.int16, "k_pages", _pool_shape(p, k_pages), d),
        _ptr(v_pages, torch.int16, "v_pages", _pool_shape(p, k_pages), d),
        k_pages.shape[0],
        _ptr(merged, torch.int32, "merged", (batch, hkv, merged.shape[-1]), d),
        _ptr(n_merged, torch.int32, "n_merged", (batch, hkv), d), merged.shape[-1],
        _ptr(lens, torch.int32, "lens", (batch,), d), batch,
        _ptr(out, torch.float32, "out", rows, d), _ptr(workspace, None, "workspace", None, d),
        ws_bytes, _stream(q)))


def decode_attn_lse(p: Params, q, k_pages, v_pages, merged, n_merged, lens, out,
                    workspace, prev_out=None, prev_lse=None, lse=None):
    """rkv_decode_attn_lse: attention over the merged lists, folded with a
    previous part (prev_out, prev_lse) and leaving the rows' log-sum-exp."""
    batch = lens.shape[0]
    d = q.device
    hkv = p.n_kv_heads
    rows = (batch, p.n_q_heads, HEAD_DIM)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib().rkv_decode_attn_lse(
        ctypes.byref(p), _ptr(q, torch.int16, "q", rows, d),
        _ptr(k_pages, torch.int16, "k_pages", _pool_shape(p, k_pages), d),
        _ptr(v_pages, torch.int16, "v_pages", _pool_shape(p, k_pages), d),
        k_pages.shape[0],
        _ptr(merged, torch.int32, "merged", (batch, hkv, merged.shape[-1]), d),
        _ptr(n_merged, torch.int32, "n_merged", (batch, hkv), d), merged.shape[-1],
        _ptr(lens, torch.int32, "lens", (batch,), d), batch,
        None if prev_out is None else _ptr(prev_out, torch.float32, "prev_out", rows, d),
        None if prev_lse is None else _ptr(prev_lse, torch.float32, "prev_lse",
                                           rows[:2], d),
        _ptr(out, torch.float32, "out", rows, d),
        None if lse is None else _ptr(lse, torch.float32, "lse", rows[:2], d),
        _ptr(workspace, None, "workspace", None, d), ws_bytes, _stream(q)))


def attn_cascade_workspace_size(p: Params, batch: int, m_cap: int,
                                shared_blocks: int) -> int:
    return lib().rkv_attn_cascade_workspace_size(ctypes.byref(p), batch, m_cap,
                                                 shared_blocks)


def decode_attn_cascade(p: Params, q, k_pages, v_pages, merged, n_merged, sel_ids,
                        n_sel, block_table, shared_blocks: int, lens, out, workspace):
    batch = lens.shape[0]
    d = q.device
    hkv = p.n_kv_heads
    rows = (batch, p.n_q_heads, HEAD_DIM)
    ws_bytes = workspace.numel() * workspace.element_size()
    max_blocks = block_table.shape[-1]
    _check(lib().rkv_decode_attn_cascade(
        ctypes.byref(p), _ptr(q, torch.int16, "q", rows, d),
        _ptr(k_pages, torch.int16, "k_pages", _pool_shape(p, k_pages), d),
        _ptr(v_pages, torch.int16, "v_pages", _pool_shape(p, k_pages), d),
        k_pages.shape[0],
        _ptr(merged, torch.int32, "merged", (batch, hkv, merged.shape[-1]), d),
        _ptr(n_merged, torch.int32, "n_merged", (batch, hkv), d), merged.shape[-1],
        _ptr(sel_ids, torch.int32, "sel_ids", (batch, hkv, sel_ids.shape[-1]), d),
        _ptr(n_sel, torch.int32, "n_sel", (batch, hkv), d), sel_ids.shape[-1],
        _ptr(block_table, torch.int32, "block_table", (batch, max_blocks), d),
        max_blocks, shared_blocks,
        _ptr(lens, torch.int32, "lens", (batch,), d), batch,
        _ptr(out, torch.float32, "out", rows, d), _ptr(workspace, None, "workspace", None, d),
        ws_bytes, _stream(q)))


def _dyn(t, dtype, shape, name, dev):
    """Pointer of a per-step tensor whose dtype / shape / device were fixed
    when the call was prepared (cheap checks only)."""
    if t.dtype is not dtype or tuple(t.shape) != shape or t.device != dev \
            or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {dtype} tensor of shape {shape} "
                         f"on {dev}")
    return t.data_ptr()


class PreparedStep:
    """The two per-step calls of a decode session with every buffer that
    does not change between steps validated and converted once; a call then
    re-reads only the per-step tensors (q, k_new, v_new, lens) and the
    current stream.  Same arguments, same checks on the C side."""

    def __init__(self, p: Params, k_pages, v_pages, reps, block_table, sel_ids,
                 n_sel, merged, n_merged, prompt_lens, ws_select, out, ws_attn):
        L = lib()
        self._L = L
        self._p = p
        self._pp = ctypes.byref(p)
        self._dev = k_pages.device
        batch, max_blocks = block_table.shape
        hq, hkv = p.n_q_heads, p.n_kv_heads
        self._q_shape = (batch, hq, HEAD_DIM)
        self._kv_shape = (batch, hkv, HEAD_DIM)
        self._lens_shape = (batch,)
        d = self._dev
        pool = _pool_shape(p, k_pages)
        if merged is None or n_merged is None:
            raise ValueError("a prepared step needs the merged table and its counts")
        m_cap = merged.shape[-1]
        ws_sel = 0 if ws_select is None else ws_select.numel() * ws_select.element_size()
        self._sel_args = (
            _ptr(k_pages, torch.int16, "k_pages", pool, d),
            _ptr(v_pages, torch.int16, "v_pages", pool, d),
            k_pages.shape[0], _ptr(reps, torch.float32, "reps",
                                   (batch, hkv, max_blocks, HEAD_DIM), d),
            _ptr(block_table, torch.int32, "block_table", None, d),
            _ptr(prompt_lens, torch.int32, "prompt_lens", (batch,), d), batch, max_blocks,
            _ptr(sel_ids, torch.int32, "sel_ids", (batch, hkv, sel_ids.shape[-1]), d),
            _ptr(n_sel, torch.int32, "n_sel", (batch, hkv), d),
            sel_ids.shape[-1], _ptr(merged, torch.int32, "merged", (batch, hkv, m_cap), d),
            _ptr(n_merged, torch.int32, "n_merged", (batch, hkv), d), m_cap,
            _ptr(ws_select, None, "workspace", None, d), ws_sel)
        self._attn_args = (
            _ptr(k_pages, torch.int16, "k_pages", pool, d),
            _ptr(v_pages, torch.int16, "v_pages", pool, d),
            k_pages.shape[0], _ptr(merged, torch.int32, "merged", (batch, hkv, m_cap), d),
            _ptr(n_merged, torch.int32, "n_merged", (batch, hkv), d), m_cap,
            batch, _ptr(out, torch.float32, "out", (batch, hq, HEAD_DIM), d),
            _ptr(ws_attn, None, "workspace", None, d),
            ws_attn.numel() * ws_attn.element_size())
        # keep every buffer alive as long as the prepared call
        self._keep = (k_pages, v_pages, reps, block_table, sel_ids, n_sel, merged,
                      n_merged, prompt_lens, ws_select, out, ws_attn)

    def append_select(self, q, k_new, v_new, lens):
        (kp, vp, n_pages, reps, bt, plens, batch, max_blocks, sel, nsel, k_cap,
         merged, nmerged, m_cap, ws, ws_bytes) = self._sel_args
        _check(self._L.rkv_append_select(
            self._pp, _dyn(k_new, torch.int16, self._kv_shape, "k_new", self._dev),
            _dyn(v_new, torch.int16, self._kv_shape, "v_new", self._dev), kp, vp, n_pages,
            _dyn(q, torch.int16, self._q_shape, "q", self._dev), reps, bt,
            _dyn(lens, torch.int32, self._lens_shape, "lens", self._dev), plens, batch,
            max_blocks,
            sel, nsel, k_cap, merged, nmerged, m_cap, ws, ws_bytes,
            torch.cuda.current_stream(self._dev).cuda_stream))

    def decode_step(self, q, k_new, v_new, lens):
        """rkv_decode_step: append + scores, then the selection and the
        attention (folded into one launch for a batch of one)."""
        (kp, vp, n_pages, reps, bt, plens, batch, max_blocks, sel, nsel, k_cap,
         merged, nmerged, m_cap, ws, ws_bytes) = self._sel_args
        out, wa, wa_bytes = self._attn_args[7:]
        _check(self._L.rkv_decode_step(
            self._pp, _dyn(k_new, torch.int16, self._kv_shape, "k_new", self._dev),
            _dyn(v_new, torch.int16, self._kv_shape, "v_new", self._dev), kp, vp, n_pages,
            _dyn(q, torch.int16, self._q_shape, "q", self._dev), reps, bt,
            _dyn(lens, torch.int32, self._lens_shape, "lens", self._dev), plens, batch,
            max_blocks, sel, nsel, k_cap, merged, nmerged, m_cap, out, ws, ws_bytes,
            wa, wa_bytes, torch.cuda.current_stream(self._dev).cuda_stream))

    def select_attend(self, q, lens):
        """rkv_select_attend on the scores the last selection left in the
        select workspace."""
        (kp, vp, n_pages, reps, bt, plens, batch, max_blocks, sel, nsel, k_cap,
         merged, nmerged, m_cap, ws, ws_bytes) = self._sel_args
        out, wa, wa_bytes = self._attn_args[7:]
        if ws is None:
            raise ValueError("no select workspace holds scores")
        _check(self._L.rkv_select_attend(
            self._pp, _dyn(q, torch.int16, self._q_shape, "q", self._dev), kp, vp, n_pages,
            bt, max_blocks, _dyn(lens, torch.int32, self._lens_shape, "lens", self._dev),
            plens, batch, ws, sel, nsel, k_cap, merged, nmerged, m_cap, out, wa, wa_bytes,
            torch.cuda.current_stream(self._dev).cuda_stream))

    def decode_attn(self, q, lens):
        kp, vp, n_pages, merged, nmerged, m_cap, batch, out, ws, ws_bytes = self._attn_args
        _check(self._L.rkv_decode_attn(
            self._pp, _dyn(q, torch.int16, self._q_shape, "q", self._dev), kp, vp, n_pages,
            merged, nmerged, m_cap,
            _dyn(lens, torch.int32, self._lens_shape, "lens", self._dev),
            batch, out, ws, ws_bytes, torch.cuda.current_stream(self._dev).cuda_stream))


def decode_step_static(p: Params, q, k_new, v_new, k_pages, v_pages, reps,
                       block_table, lens, sel_ids, n_sel, merged, n_merged, out,
                       prompt_lens=None):
    """rkv_decode_step_static: the decode step with the library's static
    scratch as its workspaces (no allocation behind the call)."""
    batch, mb = block_table.shape
    d = q.device
    hkv = p.n_kv_heads
    kv = (batch, hkv, HEAD_DIM)
    pool = _pool_shape(p, k_pages)
    _check(lib().rkv_decode_step_static(
        ctypes.byref(p), _ptr(k_new, torch.int16, "k_new", kv, d),
        _ptr(v_new, torch.int16, "v_new", kv, d),
        _ptr(k_pages, torch.int16, "k_pages", pool, d),
        _ptr(v_pages, torch.int16, "v_pages", pool, d), k_pages.shape[0],
        _ptr(q, torch.int16, "q", (batch, p.n_q_heads, HEAD_DIM), d),
        _ptr(reps, torch.float32, "reps", (batch, hkv, mb, HEAD_DIM), d),
        _ptr(block_table, torch.int32, "block_table", None, d),
        _ptr(lens, torch.int32, "lens", (batch,), d),
        _ptr(prompt_lens, torch.int32, "prompt_lens", (batch,), d), batch, mb,
        _ptr(sel_ids, torch.int32, "sel_ids", (batch, hkv, sel_ids.shape[-1]), d),
        _ptr(n_sel, torch.int32, "n_sel", (batch, hkv), d), sel_ids.shape[-1],
        _ptr(merged, torch.int32, "merged", (batch, hkv, merged.shape[-1]), d),
        _ptr(n_merged, torch.int32, "n_merged", (batch, hkv), d), merged.shape[-1],
        _ptr(out, torch.float32, "out", (batch, p.n_q_heads, HEAD_DIM), d),
        _stream(q)))


def debug_set_report(word):
    """RKV_DEBUG builds: kernels launched from now on record the first
    out-of-range device value into `word` (an int64 device tensor of one
    element, zero-filled); None stops it."""
    _check(lib().rkv_debug_set_report(
        None if word is None else _ptr(word, torch.int64, "word", (1,))))


def debug_check(word):
    """Waits for the current stream, reads and clears `word`; raises
    RkvError(RKV_ERR_BOUNDS) when a kernel reported a value."""
    _check(lib().rkv_debug_check(_ptr(word, torch.int64, "word", (1,)), _stream(word)))


WAVE_STAMP_SLOTS = 16
WAVE_STAMP_WAVES = 4096


def wave_stamps(waves):
    """rkv_debug_wave_stamps: the per-wave timestamps of the last
    folded-selection launches, as a uint64 array [waves, WAVE_STAMP_SLOTS]
    (a library built with RKV_WAVE_STAMPS only)."""
    out = np.zeros((int(waves), WAVE_STAMP_SLOTS), dtype=np.uint64)
    _check(lib().rkv_debug_wave_stamps(out.ctypes.data if waves else None, int(waves)))
    return out


def read_probe(buf, sink):
    """Stream-read `buf` once on the device (bandwidth measurement helper)."""
    _check(lib().rkv_read_probe(_ptr(buf, None, "buffer"),
                                buf.numel() * buf.element_size(),
                                _ptr(sink, None, "sink"), _stream(buf)))


def ceil_div(a: int, b: int) -> int:
    return -(-a // b)


def topk_capacity(p: Params, max_blocks: int) -> int:
    """Smallest k_cap rkv_select accepts (rkv_topk_capacity)."""
    return int(lib().rkv_topk_capacity(ctypes.byref(p), max_blocks))


__all__ = ["Params", "RkvError", "lib", "params", "build_reps", "append_kv",
           "select", "merge_table", "decode_attn", "attn_workspace_size",
           "select_workspace_size", "topk_capacity", "header_functions", "read_probe",
           "stage_blocks", "append_select",
           "ATTN_AUTO", "ATTN_MFMA", "ATTN_VALU"]
