"""The RKV_DEBUG build (librkv_debug.so) through the C ABI: kernels that meet
an out-of-range device value clamp or skip it exactly as the release build
does and record the first one; rkv_debug_check turns it into
RKV_ERR_BOUNDS.  Every kernel still exits normally: the same session keeps
computing correct steps afterwards (checked against the oracle)."""

import os

import numpy as np
import pytest
import torch

import oracle as O
from sparse_retrieval_kv_amd import binding as B
from sparse_retrieval_kv_amd import synth
from sparse_retrieval_kv_amd.decode import DecodeSession
from tests.helpers import (close_report, gpu_merged_logical, logical_at_step,
                           oracle_params, q_f64)

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def debug_lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if not os.path.exists(B.DEBUG_LIB_PATH):
        pytest.fail("librkv_debug.so is not built")
    B.use_library(B.DEBUG_LIB_PATH)
    word = torch.zeros(1, dtype=torch.int64, device=DEV)
    B.debug_set_report(word)
    yield word
    B.debug_set_report(None)
    B.use_library(B.DEFAULT_LIB_PATH)


def i32(x):
    return torch.as_tensor(np.asarray(x, dtype=np.int32), device=DEV)


def expect_report(word, kind):
    with pytest.raises(B.RkvError) as e:
        B.debug_check(word)
    assert e.value.status == B.RKV_ERR_BOUNDS
    assert kind in str(e.value), str(e.value)
    B.debug_check(word)  # cleared


def _session():
    spec = synth.custom("bounds", batch=1, n_q_heads=8, n_kv_heads=2, context=(3000,),
                        steps=3, init_tokens=256, local_tokens=512, dense_boundary=0,
                        config_id=150)
    batch = synth.make_batch(spec, DEV)
    prm = B.params(8, 2, init_tokens=256, local_tokens=512, dense_boundary=0)
    sess = DecodeSession(prm, batch.k_pages, batch.v_pages, batch.block_table,
                         i32(batch.context))
    sess.build_reps(i32(batch.context - 1))
    return spec, batch, prm, sess


def _check_step(spec, batch, sess, t):
    """Selections, merged tables and outputs of step t against the oracle."""
    K, V, L = logical_at_step(batch, 0, t)
    res = O.decode_step(q_f64(batch, t)[0], K, V, L, int(batch.context[0]),
                        oracle_params(spec))
    out = sess.out[0].cpu().numpy()
    for h, hr in enumerate(res.heads):
        n = int(sess.n_sel[0, h])
        assert np.array_equal(sess.sel_ids[0, h, :n].cpu().numpy(), hr.selected)
        ok, mx, rl2 = close_report(out[h * 4:(h + 1) * 4], res.out[h * 4:(h + 1) * 4])
        assert ok and rl2 <= 1e-4, (h, mx, rl2)


def test_clean_steps_report_nothing(debug_lib):
    spec, batch, prm, sess = _session()
    print("[case] debug build, clean steps", flush=True)
    for t in range(2):
        kn, vn = batch.new_kv_bits(t)
        sess.step(batch.q_bits(t), kn, vn, i32(batch.lens_at(t)))
        B.debug_check(debug_lib)
        _check_step(spec, batch, sess, t)


def test_bad_page_ids_are_reported_and_skipped(debug_lib):
    spec, batch, prm, sess = _session()
    print("[case] debug build, out-of-range page ids", flush=True)
    lens = i32(batch.context)
    kn, vn = batch.new_kv_bits(0)
    sess.append(kn, vn, lens)
    sess.select(batch.q_bits(0), lens)
    B.debug_check(debug_lib)
    mlog, _ = gpu_merged_logical(sess, batch, 0, 1)
    sess.merged[0, 1, 3] = batch.n_pages + 7
    sess.attend(batch.q_bits(0), lens)
    expect_report(debug_lib, "page id")
    # the attention skipped that block: the oracle over the other blocks
    K, V, L = logical_at_step(batch, 0, 0)
    keep = np.delete(mlog, [3])
    tok = (keep[:, None] * 128 + np.arange(128)).reshape(-1)
    tok = tok[tok < L]
    ref = O.attend(q_f64(batch, 0)[0, 4:8], K[1, tok], V[1, tok], 1 / np.sqrt(128))
    ok, mx, rl2 = close_report(sess.out[0, 4:8].cpu().numpy(), ref)
    assert ok and rl2 <= 1e-4, (mx, rl2)
    # -1 marks a block the merge left out: skipped, not reported
    sess.merged[0, 1, 3] = -1
    sess.attend(batch.q_bits(0), lens)
    B.debug_check(debug_lib)


def test_bad_lengths_counts_and_block_ids_are_reported(debug_lib):
    spec, batch, prm, sess = _session()
    print("[case] debug build, out-of-range lengths, counts and block ids", flush=True)
    lens = i32(batch.context)
    mb = batch.table_np.shape[1]
    too_long = i32([mb * 128 + 5])
    sess.select(batch.q_bits(0), too_long)
    expect_report(debug_lib, "length")
    # kept ids outside the offload range and a count above its capacity
    sess.select(batch.q_bits(0), lens)
    B.debug_check(debug_lib)
    sel = sess.sel_ids.clone()
    sel[0, 0, 0] = 1  # an init block
    B.merge_table(prm, sess.block_table, lens, sel, sess.n_sel, sess.merged,
                  sess.n_merged)
    expect_report(debug_lib, "block id")
    n_sel = sess.n_sel.clone()
    n_sel[0, 1] = sess.sel_ids.shape[-1] + 3
    B.merge_table(prm, sess.block_table, lens, sess.sel_ids, n_sel, sess.merged,
                  sess.n_merged)
    expect_report(debug_lib, "count")
    # every kernel exited normally: the session goes on computing correct steps
    for t in range(2):
        kn, vn = batch.new_kv_bits(t)
        sess.step(batch.q_bits(t), kn, vn, i32(batch.lens_at(t)))
        B.debug_check(debug_lib)
        _check_step(spec, batch, sess, t)
