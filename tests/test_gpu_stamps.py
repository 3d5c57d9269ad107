"""The RKV_WAVE_STAMPS build (librkv_stamps.so) through the C ABI: its decode
step computes what the release build computes, bit for bit, and the per-wave
timestamps rkv_debug_wave_stamps returns are well formed -- every wave of
the folded-selection launch leaves one row, its events in program order
inside [start, done], and one stamp per unit it attended."""

import os

import numpy as np
import pytest
import torch

from sparse_retrieval_kv_amd import binding as B
from sparse_retrieval_kv_amd import synth
from sparse_retrieval_kv_amd.decode import DecodeSession

pytestmark = pytest.mark.gpu
DEV = "cuda"

START, SCORES, SEARCH, VREQ, LIST, DONE, HWID, UNIT0 = range(8)


@pytest.fixture(scope="module")
def stamps_path():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if not os.path.exists(B.STAMPS_LIB_PATH):
        pytest.fail("librkv_stamps.so is not built")
    yield B.STAMPS_LIB_PATH
    B.use_library(B.DEFAULT_LIB_PATH)


def i32(x):
    return torch.as_tensor(np.asarray(x, dtype=np.int32), device=DEV)


def run_steps(spec, steps):
    """Decode `steps` steps of a fresh batch; per step the output bits, the
    selections and the merged tables (valid entries), the merged-table
    lengths of the last step."""
    batch = synth.make_batch(spec, DEV)
    prm = B.params(spec.n_q_heads, spec.n_kv_heads, init_tokens=spec.init_tokens,
                   local_tokens=spec.local_tokens, topk_ppm=spec.topk_ppm,
                   dense_boundary=spec.dense_boundary)
    sess = DecodeSession(prm, batch.k_pages, batch.v_pages, batch.block_table,
                         i32(batch.context))
    sess.build_reps(i32(batch.context - 1))
    rec = []
    for t in range(steps):
        kn, vn = batch.new_kv_bits(t)
        sess.step(batch.q_bits(t), kn, vn, i32(batch.lens_at(t)))
        torch.cuda.synchronize()
        n_sel = sess.n_sel.cpu().numpy()
        n_m = sess.n_merged.cpu().numpy()
        sel = sess.sel_ids.cpu().numpy()
        mer = sess.merged.cpu().numpy()
        rec.append((sess.out.cpu().numpy().view(np.uint32).copy(),
                    [sel[0, h, :n_sel[0, h]].tolist() for h in range(spec.n_kv_heads)],
                    [mer[0, h, :n_m[0, h]].tolist() for h in range(spec.n_kv_heads)]))
    return rec, n_m[0].copy()


def test_stamps_build_matches_release_and_stamps_are_well_formed(stamps_path):
    spec = synth.CONFIGS[2]  # Llama-3-8B-shaped layer, 1 x 64K
    print("[case] stamps build vs release, 8B layer (1 x 64K), 2 steps", flush=True)
    B.use_library(B.DEFAULT_LIB_PATH)
    ref, _ = run_steps(spec, 2)
    B.use_library(stamps_path)
    got, n_merged = run_steps(spec, 2)
    for t, (a, b) in enumerate(zip(ref, got)):
        assert np.array_equal(a[0], b[0]), f"output differs at step {t}"
        assert a[1] == b[1], f"selection differs at step {t}"
        assert a[2] == b[2], f"merged table differs at step {t}"

    st = B.wave_stamps(B.WAVE_STAMP_WAVES).astype(np.int64)
    rows = st[st[:, START] > 0]
    # the grid is a whole number of waves per KV head, and only the rows of
    # the launch were written (the array starts zeroed when the library loads)
    assert len(rows) > 0 and len(rows) % spec.n_kv_heads == 0, len(rows)
    assert not st[len(rows):].any()
    # every event of the wave's start is stamped, in program order, and the
    # wave ends within 10 ms (100 MHz counter)
    ev = rows[:, [START, SCORES, SEARCH, VREQ, LIST, DONE]]
    assert (ev > 0).all()
    assert (np.diff(ev, axis=1) >= 0).all()
    assert (rows[:, DONE] - rows[:, START] < 1_000_000).all()
    # the die field of XCC_ID (low four bits): one of the eight dies
    assert (((rows[:, HWID] >> 32) & 0xF) < 8).all()
    # unit stamps: a prefix of the slots, increasing, after the list is built
    units = rows[:, UNIT0:]
    stamped = units > 0
    n_units = stamped.sum(axis=1)
    assert (stamped == (np.arange(units.shape[1])[None, :] < n_units[:, None])).all()
    for w in range(len(rows)):
        u = units[w, :n_units[w]]
        assert (np.diff(u) >= 0).all() and (u >= rows[w, LIST]).all()
        assert (u <= rows[w, DONE]).all()
    # each unit (half a 128-token block) of the merged tables is attended by
    # exactly one wave, so the stamps count them all
    assert n_units.max() < units.shape[1], "a wave had more units than slots"
    assert int(n_units.sum()) == 2 * int(n_merged.sum())
