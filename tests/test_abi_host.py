"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every function include/rkv.h declares, returns the page's defaults, and
rejects bad arguments before anything is enqueued."""

import ctypes
import os
import re

import numpy as np
import pytest

from sparse_retrieval_kv_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

FAKE = 0x10000  # aligned, never dereferenced: every call below fails validation
ODD = 0x10002


@pytest.fixture(scope="module")
def L():
    return B.lib()


def test_every_declared_function_is_exported(L):
    names = B.header_functions()
    assert len(names) >= 11
    for n in names:
        assert hasattr(L, n), n
    assert L.rkv_abi_version() == 6


def test_defaults_follow_the_page(L):
    p = L.rkv_params_default(32, 8)
    assert (p.block_size, p.head_dim, p.init_tokens, p.local_tokens,
            p.topk_ppm, p.dense_boundary) == (128, 128, 1024, 7192, 200000, 32768)
    assert p.scale == pytest.approx(128 ** -0.5)
    assert (p.n_q_heads, p.n_kv_heads, p.attn_impl, p.split_waves) == (32, 8, 0, 0)
    assert (p.select_mode, p.copy_lanes) == (B.SELECT_PER_HEAD, 0)
    # the binding's struct has the header's size (every field mirrored)
    assert ctypes.sizeof(B.Params) == 13 * 4
    assert L.rkv_status_string(0) == b"ok"
    assert L.rkv_status_string(3) == b"workspace too small"


def _attn(L, p, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, n_pages=10, merged=FAKE, n_merged=FAKE,
             m_cap=16, lens=FAKE, batch=2, out=FAKE, ws=FAKE, ws_bytes=0)
    a.update(kw)
    return L.rkv_decode_attn(ctypes.byref(p), a["q"], a["k"], a["v"], a["n_pages"],
                             a["merged"], a["n_merged"], a["m_cap"], a["lens"],
                             a["batch"], a["out"], a["ws"], a["ws_bytes"], None)


def test_param_validation(L):
    base = L.rkv_params_default(32, 8)

    def with_(**kw):
        p = L.rkv_params_default(32, 8)
        for k, v in kw.items():
            setattr(p, k, v)
        return p

    cases = [
        (with_(block_size=64), B.RKV_ERR_UNSUPPORTED),
        (with_(head_dim=64), B.RKV_ERR_UNSUPPORTED),
        (with_(n_q_heads=30), B.RKV_ERR_INVALID_ARG),
        (with_(n_q_heads=0), B.RKV_ERR_INVALID_ARG),
        (with_(n_q_heads=64, n_kv_heads=2), B.RKV_ERR_UNSUPPORTED),
        (with_(topk_ppm=1_000_001), B.RKV_ERR_INVALID_ARG),
        (with_(topk_ppm=-1), B.RKV_ERR_INVALID_ARG),
        (with_(init_tokens=-1), B.RKV_ERR_INVALID_ARG),
        (with_(dense_boundary=-5), B.RKV_ERR_INVALID_ARG),
        (with_(scale=float("inf")), B.RKV_ERR_INVALID_ARG),
        (with_(attn_impl=7), B.RKV_ERR_INVALID_ARG),
        (with_(split_waves=-1), B.RKV_ERR_INVALID_ARG),
        (with_(split_waves=(1 << 16) + 1), B.RKV_ERR_INVALID_ARG),
        (with_(select_mode=2), B.RKV_ERR_INVALID_ARG),
        (with_(select_mode=-1), B.RKV_ERR_INVALID_ARG),
        (with_(copy_lanes=-1), B.RKV_ERR_INVALID_ARG),
        (with_(copy_lanes=B.MAX_COPY_LANES + 1), B.RKV_ERR_INVALID_ARG),
    ]
    for p, want in cases:
        assert _attn(L, p) == want, p
        assert L.rkv_last_error() != b""
    assert _attn(L, base, ws_bytes=0) == B.RKV_ERR_WORKSPACE
    assert b"workspace" in L.rkv_last_error()
    need = L.rkv_attn_workspace_size(ctypes.byref(base), 2, 16)
    assert need > 0
    assert _attn(L, base, ws_bytes=need - 1) == B.RKV_ERR_WORKSPACE
    assert _attn(L, base, q=None, ws_bytes=need) == B.RKV_ERR_INVALID_ARG
    assert _attn(L, base, out=ODD, ws_bytes=need) == B.RKV_ERR_INVALID_ARG
    assert _attn(L, base, m_cap=0, ws_bytes=need) == B.RKV_ERR_INVALID_ARG
    assert _attn(L, base, n_pages=0, ws_bytes=need) == B.RKV_ERR_INVALID_ARG
    assert _attn(L, base, batch=-1, ws_bytes=need) == B.RKV_ERR_INVALID_ARG
    assert L.rkv_decode_attn(None, FAKE, FAKE, FAKE, 10, FAKE, FAKE, 16, FAKE, 2,
                             FAKE, FAKE, need, None) == B.RKV_ERR_INVALID_ARG


def test_select_and_merge_capacity_rules(L):
    p = L.rkv_params_default(32, 8)

    def sel(k_cap, m_cap, merged=FAKE, n_merged=FAKE, max_blocks=100, q=FAKE):
        return L.rkv_select(ctypes.byref(p), q, FAKE, FAKE, FAKE, None, 4,
                            max_blocks, FAKE, FAKE, k_cap, merged, n_merged, m_cap,
                            None, 0, None)

    # dense switch possible (boundary 32768): k_cap must cover max_blocks
    assert sel(99, 100) == B.RKV_ERR_INVALID_ARG
    assert b"k_cap" in L.rkv_last_error()
    assert sel(100, 99) == B.RKV_ERR_INVALID_ARG
    assert sel(100, 100, n_merged=None) == B.RKV_ERR_INVALID_ARG
    assert sel(100, 100, q=None) == B.RKV_ERR_INVALID_ARG
    assert sel(100, 100, max_blocks=0) == B.RKV_ERR_INVALID_ARG
    assert sel(100, 100, max_blocks=8193) == B.RKV_ERR_INVALID_ARG
    # no dense switch: ceil(max_blocks * ppm / 1e6) suffices
    p.dense_boundary = 0
    assert sel(19, 100) == B.RKV_ERR_INVALID_ARG    # ceil(100 * 0.2) = 20
    p.topk_ppm = 1_000_000
    assert sel(99, 100) == B.RKV_ERR_INVALID_ARG
    assert L.rkv_merge_table(ctypes.byref(p), FAKE, 100, FAKE, FAKE, FAKE, 20, 4,
                             None, -1, FAKE, FAKE, 99, None) == B.RKV_ERR_INVALID_ARG
    assert L.rkv_merge_table(ctypes.byref(p), FAKE, 100, FAKE, None, FAKE, 20, 4,
                             None, -1, FAKE, FAKE, 100, None) == B.RKV_ERR_INVALID_ARG
    assert L.rkv_merge_table(ctypes.byref(p), FAKE, 100, FAKE, FAKE, FAKE, 20, 4,
                             FAKE, 2**31 - 10, FAKE, FAKE, 100, None) == B.RKV_ERR_INVALID_ARG
    assert L.rkv_merge_table(ctypes.byref(p), FAKE, 100, FAKE, FAKE, FAKE, 20, 4,
                             FAKE, -1, FAKE, FAKE, 100, None) == B.RKV_ERR_INVALID_ARG


def test_select_attend_and_decode_step_validation(L):
    """Every case breaks exactly one rule; nothing is enqueued."""
    p = L.rkv_params_default(32, 8)
    big = L.rkv_attn_workspace_size(ctypes.byref(p), 1, 100)
    assert big > 0

    def sa(**kw):
        a = dict(q=FAKE, table=FAKE, max_blocks=100, lens=FAKE, scores=FAKE,
                 sel=FAKE, k_cap=100, merged=FAKE, n_merged=FAKE, m_cap=100,
                 out=FAKE, ws=FAKE, ws_bytes=big)
        a.update(kw)
        return L.rkv_select_attend(ctypes.byref(p), a["q"], FAKE, FAKE, 1000,
                                   a["table"], a["max_blocks"], a["lens"], None, 1,
                                   a["scores"], a["sel"], FAKE, a["k_cap"],
                                   a["merged"], a["n_merged"], a["m_cap"], a["out"],
                                   a["ws"], a["ws_bytes"], None)

    assert sa(scores=None) == B.RKV_ERR_INVALID_ARG
    assert b"scores" in L.rkv_last_error()
    assert sa(scores=FAKE + 2) == B.RKV_ERR_INVALID_ARG
    assert sa(merged=None) == B.RKV_ERR_INVALID_ARG
    assert sa(n_merged=None) == B.RKV_ERR_INVALID_ARG
    assert sa(k_cap=99) == B.RKV_ERR_INVALID_ARG     # dense switch possible
    assert sa(m_cap=99) == B.RKV_ERR_INVALID_ARG
    assert sa(max_blocks=0) == B.RKV_ERR_INVALID_ARG
    assert sa(q=ODD) == B.RKV_ERR_INVALID_ARG
    assert sa(ws_bytes=big - 1) == B.RKV_ERR_WORKSPACE
    assert sa(ws=ODD) == B.RKV_ERR_INVALID_ARG

    sel_need = L.rkv_select_workspace_size(ctypes.byref(p), 1, 100)
    assert sel_need == 8 * 100 * 4

    def step(**kw):
        a = dict(k_new=FAKE, reps=FAKE, sel_ws=FAKE, sel_bytes=sel_need,
                 attn_ws=FAKE + 0x100000, attn_bytes=big, k_cap=100)
        a.update(kw)
        return L.rkv_decode_step(ctypes.byref(p), a["k_new"], FAKE, FAKE, FAKE, 1000,
                                 FAKE, a["reps"], FAKE, FAKE, None, 1, 100, FAKE,
                                 FAKE, a["k_cap"], FAKE, FAKE, 100, FAKE,
                                 a["sel_ws"], a["sel_bytes"], a["attn_ws"],
                                 a["attn_bytes"], None)

    assert step(k_new=None) == B.RKV_ERR_INVALID_ARG
    assert step(reps=ODD) == B.RKV_ERR_INVALID_ARG
    assert step(sel_bytes=sel_need - 4) == B.RKV_ERR_WORKSPACE
    assert b"select workspace" in L.rkv_last_error()
    assert step(attn_bytes=big - 1) == B.RKV_ERR_WORKSPACE
    assert step(attn_ws=FAKE) == B.RKV_ERR_INVALID_ARG   # same buffer as select
    # overlapping byte ranges, either way round
    assert step(attn_ws=FAKE + 16) == B.RKV_ERR_INVALID_ARG
    assert b"overlap" in L.rkv_last_error()
    assert step(sel_ws=FAKE + 0x100000 + 256) == B.RKV_ERR_INVALID_ARG
    assert step(sel_ws=FAKE + 0x100000 - sel_need + 16) == B.RKV_ERR_INVALID_ARG
    assert step(k_cap=99) == B.RKV_ERR_INVALID_ARG


def test_stage_validation(L):
    p = L.rkv_params_default(32, 8)

    def stage(stage_page0=0, n_pages=1000, k_cap=100, batch=4, host_k=FAKE):
        return L.rkv_stage_blocks(ctypes.byref(p), host_k, FAKE, 50, FAKE, 200,
                                  FAKE, FAKE, k_cap, batch, FAKE, FAKE, n_pages,
                                  stage_page0, None)

    assert stage(stage_page0=601) == B.RKV_ERR_INVALID_ARG   # 601 + 400 > 1000
    assert b"staging" in L.rkv_last_error()
    assert stage(stage_page0=-1) == B.RKV_ERR_INVALID_ARG
    assert stage(k_cap=0) == B.RKV_ERR_INVALID_ARG
    assert stage(host_k=None) == B.RKV_ERR_INVALID_ARG
    assert stage(host_k=ODD) == B.RKV_ERR_INVALID_ARG


def test_stage_resident_validation(L):
    p = L.rkv_params_default(32, 8)
    need = L.rkv_stage_workspace_size(ctypes.byref(p), 4, 100)
    assert need >= 4 * 8 * 100 * 8 + 4 * 8 * 4

    def res(stage_page0=0, n_pages=1000, k_cap=100, batch=4, host_k=FAKE,
            slot_ids=FAKE, slot_cursor=FAKE, slot_cap=None, m_cap=200,
            ws_bytes=None, merged=FAKE):
        ws = need if ws_bytes is None else ws_bytes
        sc = k_cap if slot_cap is None else slot_cap
        return L.rkv_stage_resident(ctypes.byref(p), host_k, FAKE, 50, FAKE, FAKE,
                                    200, FAKE, FAKE, FAKE, k_cap, batch, sc, slot_ids,
                                    slot_cursor, FAKE, FAKE, n_pages, stage_page0,
                                    merged, FAKE, m_cap, None, FAKE, ws, None)

    assert res(stage_page0=601) == B.RKV_ERR_INVALID_ARG   # 601 + 400 > 1000
    assert b"staging" in L.rkv_last_error()
    assert res(slot_cap=200, stage_page0=201) == B.RKV_ERR_INVALID_ARG  # 201 + 800
    assert res(slot_cap=0) == B.RKV_ERR_INVALID_ARG
    assert res(slot_cap=8193, n_pages=10**6) == B.RKV_ERR_INVALID_ARG
    assert res(k_cap=0) == B.RKV_ERR_INVALID_ARG
    assert res(k_cap=8193, n_pages=10**6) == B.RKV_ERR_INVALID_ARG
    assert res(slot_ids=None) == B.RKV_ERR_INVALID_ARG
    assert res(slot_cursor=None) == B.RKV_ERR_INVALID_ARG
    assert res(merged=None) == B.RKV_ERR_INVALID_ARG
    assert res(m_cap=199) == B.RKV_ERR_INVALID_ARG
    assert res(host_k=ODD) == B.RKV_ERR_INVALID_ARG
    assert res(ws_bytes=need - 1) == B.RKV_ERR_WORKSPACE
    # fake host pools are not pinned, mapped host memory
    assert res() == B.RKV_ERR_INVALID_ARG
    assert b"pinned" in L.rkv_last_error()


def test_copy_engine_staging_validation(L):
    """The copy-engine staging calls check their host-side arguments before
    anything is enqueued (fake pools are not pinned host memory)."""
    p = L.rkv_params_default(32, 8)
    n = L.rkv_stage_host_list_size(ctypes.byref(p), 4, 100)
    assert n == 4 * 8 * 100 * 8 + 4 * 8 * 4
    assert L.rkv_stage_host_list_size(None, 4, 100) == 0

    def blocks(host_table_host=FAKE, stage_page0=0, k_cap=100):
        return L.rkv_stage_blocks_async(ctypes.byref(p), FAKE, FAKE, 50, host_table_host,
                                        200, FAKE, FAKE, k_cap, 4, FAKE, FAKE, 1000,
                                        stage_page0, FAKE, n, None, None, None)

    assert blocks(host_table_host=None) == B.RKV_ERR_INVALID_ARG
    assert blocks(stage_page0=601) == B.RKV_ERR_INVALID_ARG
    assert b"staging" in L.rkv_last_error()
    assert blocks(k_cap=0) == B.RKV_ERR_INVALID_ARG
    assert blocks() == B.RKV_ERR_INVALID_ARG
    assert b"pinned" in L.rkv_last_error()

    need = L.rkv_stage_workspace_size(ctypes.byref(p), 4, 100)

    def resident(host_table_host=FAKE, ws_bytes=need, slot_cap=100):
        return L.rkv_stage_resident_async(
            ctypes.byref(p), FAKE, FAKE, 50, FAKE, host_table_host, FAKE, 200, FAKE, FAKE,
            FAKE, 100, 4, slot_cap, FAKE, FAKE, FAKE, FAKE, 1000, 0, FAKE, FAKE, 200, None,
            FAKE, ws_bytes, FAKE, n, None, None, None)

    assert resident(host_table_host=None) == B.RKV_ERR_INVALID_ARG
    assert resident(ws_bytes=need - 1) == B.RKV_ERR_WORKSPACE
    assert resident(slot_cap=0) == B.RKV_ERR_INVALID_ARG
    assert resident() == B.RKV_ERR_INVALID_ARG
    assert b"pinned" in L.rkv_last_error()


def test_release_build_has_no_bounds_reports(L):
    assert L.rkv_debug_set_report(None) == B.RKV_ERR_UNSUPPORTED
    assert b"RKV_DEBUG" in L.rkv_last_error()
    assert L.rkv_debug_set_report(ODD) == B.RKV_ERR_INVALID_ARG
    assert L.rkv_debug_check(None, None) == B.RKV_ERR_INVALID_ARG
    assert L.rkv_status_string(B.RKV_ERR_BOUNDS) == b"out-of-range device value"


def test_debug_build_exports_the_same_calls():
    if not os.path.exists(B.DEBUG_LIB_PATH):
        pytest.skip("debug library not built")
    D = ctypes.CDLL(B.DEBUG_LIB_PATH)
    for n in B.header_functions():
        assert hasattr(D, n), n


def test_release_build_has_no_wave_stamps(L):
    buf = np.zeros(16, dtype=np.uint64)
    assert L.rkv_debug_wave_stamps(buf.ctypes.data, 1) == B.RKV_ERR_UNSUPPORTED
    assert b"RKV_WAVE_STAMPS" in L.rkv_last_error()
    assert L.rkv_debug_wave_stamps(None, 1) == B.RKV_ERR_INVALID_ARG
    assert L.rkv_debug_wave_stamps(buf.ctypes.data, -1) == B.RKV_ERR_INVALID_ARG
    assert L.rkv_debug_wave_stamps(buf.ctypes.data, 4097) == B.RKV_ERR_INVALID_ARG
    assert B.WAVE_STAMP_SLOTS == 16 and B.WAVE_STAMP_WAVES == 4096


def test_stamps_build_exports_the_same_calls():
    if not os.path.exists(B.STAMPS_LIB_PATH):
        pytest.skip("stamps library not built")
    D = ctypes.CDLL(B.STAMPS_LIB_PATH)
    for n in B.header_functions():
        assert hasattr(D, n), n


def test_reps_and_append_validation(L):
    p = L.rkv_params_default(8, 2)
    assert L.rkv_build_reps(ctypes.byref(p), None, 10, FAKE, 8, FAKE, None, 1,
                            FAKE, None) == B.RKV_ERR_INVALID_ARG
    assert L.rkv_build_reps(ctypes.byref(p), FAKE, 10, FAKE, 8, FAKE, None, 1,
                            ODD, None) == B.RKV_ERR_INVALID_ARG
    assert L.rkv_append_kv(ctypes.byref(p), FAKE, FAKE, FAKE, ODD, 10, FAKE, 8,
                           FAKE, 1, None, None) == B.RKV_ERR_INVALID_ARG
    p.block_size = 256
    assert L.rkv_append_kv(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, 10, FAKE, 8,
                           FAKE, 1, None, None) == B.RKV_ERR_UNSUPPORTED


def test_call_extent_limits(L):
    """Calls whose launch grids would pass a dispatch's 32-bit work-item count
    are refused up front; at the limits they go on to the next check."""
    p = L.rkv_params_default(32, 8)
    rows, entries = B.RKV_MAX_QUERY_ROWS, B.RKV_MAX_LIST_ENTRIES
    with open(B.HEADER) as f:
        text = f.read()
    for name, val in (("RKV_MAX_QUERY_ROWS", rows), ("RKV_MAX_LIST_ENTRIES", entries),
                      ("RKV_MAX_BLOCKS", B.RKV_MAX_BLOCKS)):
        m = re.search(r"#define %s \(?1 << (\d+)\)?|#define %s (\d+)" % (name, name), text)
        assert m, name
        assert val == (1 << int(m.group(1)) if m.group(1) else int(m.group(2))), name
    batch = rows // 32                       # batch * n_q_heads at the limit
    assert _attn(L, p, batch=batch + 1, m_cap=1) == B.RKV_ERR_UNSUPPORTED
    assert b"n_q_heads" in L.rkv_last_error()
    assert _attn(L, p, batch=batch, m_cap=1) == B.RKV_ERR_WORKSPACE
    # batch * n_kv_heads * m_cap: 1024 * 8 * 1024 is the limit
    assert _attn(L, p, batch=1024, m_cap=1025) == B.RKV_ERR_UNSUPPORTED
    assert _attn(L, p, batch=1024, m_cap=1024) == B.RKV_ERR_WORKSPACE
    assert L.rkv_build_reps(ctypes.byref(p), FAKE, 10, FAKE, 1025, FAKE, None, 1024,
                            FAKE, None) == B.RKV_ERR_UNSUPPORTED
    assert L.rkv_build_reps(ctypes.byref(p), FAKE, 10, FAKE, 1024, FAKE, None, 1024,
                            ODD, None) == B.RKV_ERR_INVALID_ARG
    assert L.rkv_select(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, None, 1024, 1025,
                        FAKE, FAKE, 1025, FAKE, FAKE, 1025, FAKE, 0,
                        None) == B.RKV_ERR_UNSUPPORTED
    assert L.rkv_stage_blocks(ctypes.byref(p), FAKE, FAKE, 50, FAKE, 200, FAKE, FAKE,
                              entries // 32 + 1, 4, FAKE, FAKE, 10**9, 0,
                              None) == B.RKV_ERR_UNSUPPORTED


def test_static_scratch_limit(L):
    """rkv_decode_step_static refuses, before touching the device, a shape
    whose workspaces do not fit the static scratch (65536 split waves of 16
    query heads: 65538 partial slots of 16 x 520 bytes)."""
    assert B.RKV_STATIC_SCRATCH_BYTES == 64 << 20
    p = L.rkv_params_default(16, 1)
    p.split_waves = 1 << 16
    p.dense_boundary = 0
    need = (L.rkv_attn_workspace_size(ctypes.byref(p), 2, 100) +
            L.rkv_select_workspace_size(ctypes.byref(p), 2, 100))
    assert need > B.RKV_STATIC_SCRATCH_BYTES
    st = L.rkv_decode_step_static(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, 1000, FAKE,
                                  FAKE, FAKE, FAKE, None, 2, 100, FAKE, FAKE, 100, FAKE,
                                  FAKE, 100, FAKE, None)
    assert st == B.RKV_ERR_UNSUPPORTED
    assert b"static" in L.rkv_last_error()
    assert L.rkv_decode_step_static(None, FAKE, FAKE, FAKE, FAKE, 1000, FAKE, FAKE, FAKE,
                                    FAKE, None, 2, 100, FAKE, FAKE, 100, FAKE, FAKE, 100,
                                    FAKE, None) == B.RKV_ERR_INVALID_ARG


def test_workspace_sizes_are_monotone(L):
    p = L.rkv_params_default(32, 8)
    a = L.rkv_attn_workspace_size(ctypes.byref(p), 1, 513)
    b = L.rkv_attn_workspace_size(ctypes.byref(p), 16, 1025)
    assert 0 < a < b
    assert L.rkv_attn_workspace_size(None, 1, 10) == 0
    assert L.rkv_select_workspace_size(ctypes.byref(p), 16, 1025) == 16 * p.n_kv_heads * 1025 * 4
    assert L.rkv_select_workspace_size(None, 16, 1025) == 0


def test_binding_refuses_host_tensors(L):
    import torch
    p = B.params(8, 2)
    t = torch.zeros(4, dtype=torch.int32)
    with pytest.raises(ValueError):
        B.merge_table(p, t.view(1, 4), t[:1], t.view(1, 1, 4), t[:2].view(1, 2),
                      t.view(1, 1, 4), t[:2].view(1, 2))


def test_binding_fails_loudly_without_the_library(tmp_path):
    """With no built library the product path raises instead of falling
    back to anything else."""
    import subprocess
    import sys
    code = ("import os, sys; sys.path.insert(0, os.getcwd()); "
            "from sparse_retrieval_kv_amd import binding as B\n"
            "try:\n    B.lib()\nexcept ImportError as e:\n    print('refused:', e)\n"
            "else:\n    print('loaded')\n")
    env = dict(os.environ, RKV_LIB=str(tmp_path / "missing" / "librkv.so"))
    out = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env,
                         capture_output=True, text=True, timeout=120)
    assert "refused:" in out.stdout, out.stdout + out.stderr


def test_bench_refuses_more_than_one_gpu():
    import subprocess
    import sys
    out = subprocess.run([sys.executable, "bench.py", "--gpus", "2"], cwd=ROOT,
                         capture_output=True, text=True, timeout=300)
    assert out.returncode == 2
    assert "one GPU" in out.stderr


def _cascade(L, p, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, n_pages=10, merged=FAKE, n_merged=FAKE, m_cap=16,
             sel=FAKE, n_sel=FAKE, k_cap=16, table=FAKE, max_blocks=16, shared=8,
             lens=FAKE, batch=2, out=FAKE, ws=FAKE, ws_bytes=1 << 30)
    a.update(kw)
    return L.rkv_decode_attn_cascade(
        ctypes.byref(p), a["q"], a["k"], a["v"], a["n_pages"], a["merged"],
        a["n_merged"], a["m_cap"], a["sel"], a["n_sel"], a["k_cap"], a["table"],
        a["max_blocks"], a["shared"], a["lens"], a["batch"], a["out"], a["ws"],
        a["ws_bytes"], None)


def test_cascade_attention_validation(L):
    """rkv_decode_attn_cascade rejects bad arguments before enqueuing."""
    p = L.rkv_params_default(32, 8)
    for name in ("q", "merged", "n_merged", "sel", "n_sel", "table", "lens", "out"):
        assert _cascade(L, p, **{name: None}) == B.RKV_ERR_INVALID_ARG, name
    assert _cascade(L, p, shared=17) == B.RKV_ERR_INVALID_ARG
    assert _cascade(L, p, shared=-1) == B.RKV_ERR_INVALID_ARG
    assert _cascade(L, p, max_blocks=0) == B.RKV_ERR_INVALID_ARG
    assert _cascade(L, p, k_cap=0) == B.RKV_ERR_INVALID_ARG
    assert _cascade(L, p, batch=-1) == B.RKV_ERR_INVALID_ARG
    assert _cascade(L, p, q=FAKE + 4) == B.RKV_ERR_INVALID_ARG
    assert _cascade(L, p, ws_bytes=16) == B.RKV_ERR_WORKSPACE
    assert _cascade(L, p, ws=FAKE + 8) == B.RKV_ERR_INVALID_ARG
    valu = L.rkv_params_default(32, 8)
    valu.attn_impl = B.ATTN_VALU
    assert _cascade(L, valu) == B.RKV_ERR_UNSUPPORTED
    assert _cascade(L, p, batch=1 << 20) == B.RKV_ERR_UNSUPPORTED


def test_cascade_workspace_size(L):
    """The cascade workspace adds the cascade pieces, masks and private tables
    to the plain attention workspace; with nothing shared, or a single
    sequence, it is the plain one."""
    p = L.rkv_params_default(64, 8)
    plain = L.rkv_attn_workspace_size(ctypes.byref(p), 8, 1025)
    assert L.rkv_attn_cascade_workspace_size(ctypes.byref(p), 8, 1025, 0) == plain
    one = L.rkv_attn_workspace_size(ctypes.byref(p), 1, 1025)
    assert L.rkv_attn_cascade_workspace_size(ctypes.byref(p), 1, 1025, 128) == one
    big = L.rkv_attn_cascade_workspace_size(ctypes.byref(p), 8, 1025, 128)
    # at least the private tables (lists x m_cap int32) and masks on top
    assert big >= plain + 64 * 1025 * 4 + 64 * 4 * 4
    assert L.rkv_attn_cascade_workspace_size(ctypes.byref(p), 8, 1025, -1) == 0


def test_split_staging_and_lse_attention_validation(L):
    """rkv_stage_plan, rkv_stage_copy and rkv_decode_attn_lse reject bad
    arguments before enqueuing."""
    p = L.rkv_params_default(32, 8)
    ws = L.rkv_stage_workspace_size(ctypes.byref(p), 2, 50)

    def plan(**kw):
        a = dict(host_table=FAKE, table=FAKE, max_blocks=100, lens=FAKE, sel=FAKE,
                 n_sel=FAKE, k_cap=50, batch=2, slot_cap=60, slots=FAKE, cursor=FAKE,
                 n_pages=1000, page0=500, merged=FAKE, n_merged=FAKE, m_cap=100,
                 merged_new=FAKE, n_new=FAKE, n_staged=None, ws=FAKE, ws_bytes=ws)
        a.update(kw)
        return L.rkv_stage_plan(ctypes.byref(p), a["host_table"], a["table"],
                                a["max_blocks"], a["lens"], a["sel"], a["n_sel"],
                                a["k_cap"], a["batch"], a["slot_cap"], a["slots"],
                                a["cursor"], a["n_pages"], a["page0"], a["merged"],
                                a["n_merged"], a["m_cap"], a["merged_new"], a["n_new"],
                                a["n_staged"], a["ws"], a["ws_bytes"], None)

    assert plan(merged_new=None) == B.RKV_ERR_INVALID_ARG  # n_new without merged_new
    assert plan(n_new=None) == B.RKV_ERR_INVALID_ARG
    assert plan(host_table=None) == B.RKV_ERR_INVALID_ARG
    assert plan(m_cap=99) == B.RKV_ERR_INVALID_ARG
    assert plan(page0=1000 - 119) == B.RKV_ERR_INVALID_ARG  # 2 x 60 slots do not fit
    assert plan(ws_bytes=ws - 1) == B.RKV_ERR_WORKSPACE
    assert plan(k_cap=0) == B.RKV_ERR_INVALID_ARG

    def copy(**kw):
        a = dict(hk=FAKE, hv=FAKE, n_host=100, host_table=FAKE, max_blocks=100, k_cap=50,
                 batch=2, slot_cap=60, k=FAKE, v=FAKE, n_pages=1000, page0=500, ws=FAKE,
                 ws_bytes=ws)
        a.update(kw)
        return L.rkv_stage_copy(ctypes.byref(p), a["hk"], a["hv"], a["n_host"],
                                a["host_table"], a["max_blocks"], a["k_cap"], a["batch"],
                                a["slot_cap"], a["k"], a["v"], a["n_pages"], a["page0"],
                                a["ws"], a["ws_bytes"], None)

    assert copy(hk=None) == B.RKV_ERR_INVALID_ARG
    assert copy(host_table=None) == B.RKV_ERR_INVALID_ARG
    assert copy(page0=-1) == B.RKV_ERR_INVALID_ARG
    assert copy(ws_bytes=0) == B.RKV_ERR_WORKSPACE
    assert copy(slot_cap=0) == B.RKV_ERR_INVALID_ARG

    need = L.rkv_attn_workspace_size(ctypes.byref(p), 2, 16)

    def attn(**kw):
        a = dict(q=FAKE, k=FAKE, v=FAKE, n_pages=10, merged=FAKE, n_merged=FAKE, m_cap=16,
                 lens=FAKE, batch=2, prev_out=FAKE + 4096, prev_lse=FAKE + 8192,
                 out=FAKE, lse=None, ws=FAKE, ws_bytes=need)
        a.update(kw)
        return L.rkv_decode_attn_lse(ctypes.byref(p), a["q"], a["k"], a["v"],
                                     a["n_pages"], a["merged"], a["n_merged"], a["m_cap"],
                                     a["lens"], a["batch"], a["prev_out"], a["prev_lse"],
                                     a["out"], a["lse"], a["ws"], a["ws_bytes"], None)

    assert attn(prev_lse=None) == B.RKV_ERR_INVALID_ARG  # given together
    assert attn(prev_out=None) == B.RKV_ERR_INVALID_ARG
    assert attn(prev_out=FAKE) == B.RKV_ERR_INVALID_ARG  # prev_out is out
    assert attn(prev_out=FAKE + 4100) == B.RKV_ERR_INVALID_ARG  # misaligned
    assert attn(out=None) == B.RKV_ERR_INVALID_ARG
    assert attn(ws_bytes=need - 1) == B.RKV_ERR_WORKSPACE
    assert attn(m_cap=0) == B.RKV_ERR_INVALID_ARG


def test_topk_capacity_rule(L):
    """rkv_topk_capacity: max_blocks when a list can be dense, else
    ceil(max_blocks * ppm / 10^6) in exact integers; rkv_select accepts
    exactly that k_cap and rejects one less."""
    from fractions import Fraction
    import math
    p = L.rkv_params_default(32, 8)
    assert L.rkv_topk_capacity(ctypes.byref(p), 1000) == 1000  # dense boundary on
    p.dense_boundary = 0
    for mb in (0, 1, 5, 999, 1000, 8192):
        for ppm in (1, 199_999, 200_000, 333_333, 999_999):
            p.topk_ppm = ppm
            want = math.ceil(Fraction(mb * ppm, 1_000_000))
            assert L.rkv_topk_capacity(ctypes.byref(p), mb) == want, (mb, ppm)
    p.topk_ppm = 1_000_000
    assert L.rkv_topk_capacity(ctypes.byref(p), 77) == 77
    assert L.rkv_topk_capacity(None, 77) == 0
    assert L.rkv_topk_capacity(ctypes.byref(p), -1) == 0
