"""Test harness helpers: the oracle's view of a synthetic batch and
comparison utilities.  The oracle's inputs come from the generator (pool
contents written before any library call, plus the generator's appended
tokens), never from the library's outputs."""

from __future__ import annotations

import numpy as np
import torch

import oracle as O
from sparse_retrieval_kv_amd import synth

GAP = 1e-3  # relative k-th / (k+1)-th score gap below which a selection is a near tie


def u16(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy().view(np.uint16)


def oracle_params(spec, **kw) -> O.Params:
    d = dict(init_tokens=spec.init_tokens, local_tokens=spec.local_tokens,
             topk_ppm=spec.topk_ppm, dense_boundary=spec.dense_boundary)
    d.update(kw)
    return O.Params(spec.n_q_heads, spec.n_kv_heads, **d)


def seq_pages_host(batch: synth.Batch, b: int, heads=None, host=None):
    """Host copy of sequence b's pages (all heads or the given ones), taken
    from the generator's pools (device pools, and for blocks placed in host
    memory the host pools `host`).  Returns (k [nb,H,128,128], v, heads)."""
    L_final = int(batch.context[b]) + batch.spec.steps - 1
    nb = -(-L_final // 128)
    pages = torch.as_tensor(batch.table_np[b, :nb].astype(np.int64),
                            device=batch.k_pages.device)
    hs = list(range(batch.spec.n_kv_heads)) if heads is None else list(heads)
    hidx = torch.as_tensor(hs, device=batch.k_pages.device)
    k = u16(batch.k_pages.index_select(0, pages).index_select(1, hidx))
    v = u16(batch.v_pages.index_select(0, pages).index_select(1, hidx))
    if host is not None:
        ht = host.host_table_np[b, :nb]
        on_host = np.nonzero(ht >= 0)[0]
        hp = torch.as_tensor(ht[on_host].astype(np.int64))
        hh = torch.as_tensor(hs)
        k[on_host] = u16(host.host_k.index_select(0, hp).index_select(1, hh))
        v[on_host] = u16(host.host_v.index_select(0, hp).index_select(1, hh))
    return k, v, hs


def logical_at_step(batch: synth.Batch, b: int, t: int, pages=None):
    """float64 logical K, V [H, L_t, d] of sequence b after step t's append,
    plus L_t.  Prefill positions come from the pools, decoded positions from
    the generator's appended tokens."""
    if pages is None:
        pages = seq_pages_host(batch, b)
    kp, vp, hs = pages
    L = int(batch.context[b]) + t
    K, V = O.logical_kv(kp, vp, np.arange(kp.shape[0]), L)
    first = int(batch.context[b]) - 1
    for s in range(t + 1):
        kn, vn = batch.new_kv_bits(s)
        K[:, first + s] = O.bf16_to_f64(u16(kn[b])[hs])
        V[:, first + s] = O.bf16_to_f64(u16(vn[b])[hs])
    return K, V, L


def q_f64(batch: synth.Batch, t: int) -> np.ndarray:
    return O.bf16_to_f64(u16(batch.q_bits(t)))


def close_report(got: np.ndarray, ref: np.ndarray, atol=2e-3, rtol=1e-2):
    """BJ-style elementwise check plus relative L2 error."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = np.abs(got - ref)
    ok = bool(np.all(err <= atol + rtol * np.abs(ref)))
    rel_l2 = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))
    return ok, float(err.max(initial=0.0)), rel_l2


def check_selection(sel_gpu, hr, n_init, ctx):
    """The GPU's kept blocks of one list against the oracle's step: exactly k
    distinct offload blocks in ascending order; the oracle's set whenever its
    k-th/(k+1)-th relative gap exceeds 1e-3, otherwise a valid top-k of the
    oracle's scores (every kept score >= every dropped one - 1e-3 |s_k|)."""
    ref = hr.selected
    sel_gpu = np.asarray(sel_gpu, dtype=np.int64)
    n_off = len(hr.scores)
    assert len(sel_gpu) == len(ref) == hr.k, (ctx, len(sel_gpu), hr.k)
    assert np.all((sel_gpu >= n_init) & (sel_gpu < n_init + n_off)), (ctx, sel_gpu)
    assert np.all(np.diff(sel_gpu) > 0), ctx
    if hr.gap_rel > GAP:
        assert np.array_equal(sel_gpu, ref), (ctx, hr.gap_rel)
        return
    # near tie (then 0 < k < n_off): the GPU set only has to be a valid top-k
    s = hr.scores
    mask = np.zeros(n_off, bool)
    mask[sel_gpu - n_init] = True
    assert int(mask.sum()) == hr.k, ctx
    tol = GAP * abs(np.sort(s)[::-1][hr.k - 1])
    assert s[mask].min() >= s[~mask].max() - tol, ctx


def check_merged(sess, batch, b, h, regions, sel, host, ctx):
    """The GPU's merged list of (b, h) must be init ∪ sel ∪ local from the
    oracle's regions and the GPU's (validated) selection, logical ids and
    page ids exactly: blocks in HBM at their block-table page, host-resident
    blocks (host tier) at a staging page holding that block.  Returns the
    expected logical list."""
    expect = O.merged_blocks(regions, np.asarray(sel, dtype=np.int64))
    mlog, mpages = gpu_merged_logical(sess, batch, b, h, host is not None)
    assert np.array_equal(mlog, expect), (ctx, mlog, expect)
    if host is None:
        assert np.array_equal(mpages, batch.table_np[b, expect]), ctx
    else:
        on_host = host.host_table_np[b, expect] >= 0
        assert np.array_equal(mpages[~on_host], batch.table_np[b, expect[~on_host]]), ctx
        assert np.all(mpages[on_host] >= sess.stage_page0), ctx
    return expect


def gpu_selection(sess, b, h):
    n = int(sess.n_sel[b, h])
    return sess.sel_ids[b, h, :n].cpu().numpy()


def gpu_merged_logical(sess, batch, b, h, staged=False):
    """The GPU's merged list of (b, h) as logical blocks (and page ids).
    Staging page stage_page0 + b*k_cap + r stands for the block slot r holds:
    the r-th kept block without residency, slot_ids[b][h][r] with it.  A page
    that stands for no block of the sequence maps to -1."""
    n = int(sess.n_merged[b, h])
    pages = sess.merged[b, h, :n].cpu().numpy()
    inv = {int(p): j for j, p in enumerate(batch.table_np[b]) if p >= 0}
    if staged:
        if getattr(sess, "resident", False):
            held = sess.slot_ids[b, h].cpu().numpy()
            base = sess.stage_page0 + b * sess.slot_cap
        else:
            held = gpu_selection(sess, b, h)
            base = sess.stage_page0 + b * sess.k_cap
        for r, j in enumerate(held):
            if j >= 0:
                inv[int(base + r)] = int(j)
    return np.array([inv.get(int(p), -1) for p in pages], dtype=np.int64), pages
