"""rkv_decode_step_static (the decode step with the library's static device
scratch as its workspaces, for callers that cannot allocate) against
rkv_decode_step with caller workspaces: the same kernels run, so every
output must be bit-identical.  Two calls in a row, the second on a smaller
input, so the second call finds the first one's contents in the scratch."""

import numpy as np
import pytest
import torch

from sparse_retrieval_kv_amd import binding as B
from sparse_retrieval_kv_amd import synth
from sparse_retrieval_kv_amd.decode import DecodeSession

pytestmark = pytest.mark.gpu
DEV = "cuda"


def i32(x):
    return torch.as_tensor(np.asarray(x, dtype=np.int32), device=DEV)


def _session(batch):
    s = batch.spec
    prm = B.params(s.n_q_heads, s.n_kv_heads, init_tokens=s.init_tokens,
                   local_tokens=s.local_tokens, topk_ppm=s.topk_ppm,
                   dense_boundary=s.dense_boundary)
    sess = DecodeSession(prm, batch.k_pages, batch.v_pages, batch.block_table,
                         i32(batch.context))
    sess.build_reps(i32(batch.context - 1))
    return prm, sess


def _valid(t, n):
    t, n = t.cpu().numpy(), n.cpu().numpy()
    return [t[b, h, :n[b, h]].tolist() for b in range(n.shape[0]) for h in range(n.shape[1])]


def _compare(spec, steps):
    print("[case] static scratch vs caller workspaces:", spec.name, spec.context,
          flush=True)
    ref_b = synth.make_batch(spec, DEV)
    got_b = synth.make_batch(spec, DEV)
    prm, ref = _session(ref_b)
    _, got = _session(got_b)
    for t in range(steps):
        lens = i32(ref_b.lens_at(t))
        kn, vn = ref_b.new_kv_bits(t)
        q = ref_b.q_bits(t)
        got.out.fill_(float("nan"))
        ref.step(q, kn, vn, lens)
        B.decode_step_static(prm, q, kn, vn, got.k_pages, got.v_pages, got.reps,
                             got.block_table, lens, got.sel_ids, got.n_sel,
                             got.merged, got.n_merged, got.out)
        torch.cuda.synchronize()
        assert torch.equal(ref.out, got.out), (spec.name, t)
        assert torch.equal(ref.n_sel, got.n_sel) and torch.equal(ref.n_merged, got.n_merged)
        assert _valid(ref.sel_ids, ref.n_sel) == _valid(got.sel_ids, got.n_sel)
        assert _valid(ref.merged, ref.n_merged) == _valid(got.merged, got.n_merged)
    assert torch.equal(ref_b.k_pages, got_b.k_pages)
    assert torch.equal(ref_b.v_pages, got_b.v_pages)
    assert torch.equal(ref.reps, got.reps)


def test_static_scratch_step_matches_decode_step():
    # first call: a ragged batch of three (range split, top-k launch); then a
    # smaller single sequence (folded selection, strided partition)
    big = synth.custom("no-alloc batch", batch=3, n_q_heads=32, n_kv_heads=8,
                       context=(40000, 9000, 70001), steps=2, dense_boundary=0,
                       shuffle=True, config_id=140)
    small = synth.custom("no-alloc single", batch=1, n_q_heads=16, n_kv_heads=4,
                         context=(20000,), steps=2, dense_boundary=0, config_id=141)
    _compare(big, 2)
    _compare(small, 2)
