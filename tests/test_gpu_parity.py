"""GPU parity of the HIP path (through the C ABI) against the float64 oracle.

Tolerances:
  * representations: the recursive-summation bound of an fp32 sum of 128
    terms, 127 * 2^-24 * sum|K| / 128, plus one fp32 rounding of the result;
  * selections: the oracle's selected set exactly whenever its k-th/(k+1)-th
    relative score gap exceeds 1e-3, otherwise any set whose oracle scores
    dominate the rest within 1e-3 * |s_k|;
  * merged tables and appended slots: bit-exact;
  * attention outputs: |gpu - ref| <= 2e-3 + 1e-2 |ref| elementwise, and a
    relative L2 error <= 1e-4 (fp32 accumulation, weights kept to ~16 bits).
"""

import os
import sys

import numpy as np
import pytest
import torch

import oracle as O
from sparse_retrieval_kv_amd import binding as B
from sparse_retrieval_kv_amd import synth
from sparse_retrieval_kv_amd.decode import DecodeSession, HostTierSession
from tests.helpers import (GAP, check_merged, check_selection, close_report,
                           gpu_merged_logical, gpu_selection, logical_at_step,
                           oracle_params, q_f64, seq_pages_host, u16)

pytestmark = pytest.mark.gpu
DEV = "cuda"
REL_L2 = 1e-4


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def i32(x):
    return torch.as_tensor(np.asarray(x, dtype=np.int32), device=DEV)


def make_session(batch, **pkw):
    s = batch.spec
    kw = dict(init_tokens=s.init_tokens, local_tokens=s.local_tokens,
              topk_ppm=s.topk_ppm, dense_boundary=s.dense_boundary)
    kw.update(pkw)
    prm = B.params(s.n_q_heads, s.n_kv_heads, **kw)
    sess = DecodeSession(prm, batch.k_pages, batch.v_pages, batch.block_table,
                         i32(batch.context))
    return prm, sess


def prefill(batch, sess):
    sess.build_reps(i32(batch.context - 1))


def step(batch, sess, t):
    lens = i32(batch.lens_at(t))
    kn, vn = batch.new_kv_bits(t)
    return sess.step(batch.q_bits(t), kn, vn, lens)


def check_head_output(out_gpu, ref, ctx):
    ok, mx, rl2 = close_report(out_gpu, ref)
    assert ok, (ctx, mx, rl2)
    assert rl2 <= REL_L2, (ctx, mx, rl2)


def oracle_full_check(batch, sess, t, seqs=None, heads=None, host=None, q=None):
    """Check selections, merged tables and outputs of step t for the given
    sequences / KV heads (default: all) against the oracle.  `q` replaces the
    step's queries (bf16 bits on the device) when the step ran on others."""
    spec = batch.spec
    G = spec.group
    out = sess.out.cpu().numpy()
    qall = q_f64(batch, t) if q is None else O.bf16_to_f64(u16(q))
    for b in (range(spec.batch) if seqs is None else seqs):
        hs = list(range(spec.n_kv_heads)) if heads is None else heads
        pages = seq_pages_host(batch, b, hs, host)
        K, V, L = logical_at_step(batch, b, t, pages)
        prm1 = oracle_params(spec)
        prm1 = O.Params(G, 1, prm1.init_tokens, prm1.local_tokens, prm1.topk_ppm,
                        prm1.dense_boundary)
        for i, h in enumerate(hs):
            ctx = f"{spec.name} step {t} seq {b} head {h}"
            qh = qall[b, h * G:(h + 1) * G]
            res = O.decode_step(qh, K[i:i + 1], V[i:i + 1], L,
                                int(batch.context[b]), prm1)
            hr = res.heads[0]
            sel = gpu_selection(sess, b, h)
            check_selection(sel, hr, res.regions.n_init, ctx)
            expect = check_merged(sess, batch, b, h, res.regions, sel, host, ctx)
            if np.array_equal(sel, hr.selected):
                ref = res.out
            else:  # a valid near-tie selection: attention over its blocks
                ref = O.decode_step(qh, K[i:i + 1], V[i:i + 1], L,
                                    int(batch.context[b]), prm1,
                                    merged_override=[expect]).out
            check_head_output(out[b, h * G:(h + 1) * G], ref, ctx)


# ---------------------------------------------------------------------------


def test_build_reps_parity_and_block_begin():
    spec = synth.custom("reps", batch=3, n_q_heads=8, n_kv_heads=2,
                        context=(1000, 2000, 129), shuffle=True, config_id=91)
    batch = synth.make_batch(spec, DEV)
    prm, sess = make_session(batch)
    say("build_reps", spec.context)
    prefill(batch, sess)
    torch.cuda.synchronize()
    reps = sess.reps.cpu().numpy()
    for b in range(3):
        K, _, _ = logical_at_step(batch, b, 0)
        Lp = int(batch.context[b]) - 1
        ref = np.stack([O.block_reps(K[h, :Lp]) for h in range(2)])
        nc = ref.shape[1]
        absK = np.abs(K[:, :nc * 128]).reshape(2, nc, 128, 128).sum(axis=2)
        bound = 127 * 2.0 ** -24 * absK / 128 + 2.0 ** -24 * np.abs(ref) + 1e-30
        assert (np.abs(reps[b, :, :nc] - ref) <= bound).all(), b
        assert (reps[b, :, nc:] == 0).all()  # partial / unused blocks untouched
    # rebuild from block 3 / 5 / 0 into zeroed reps: earlier rows stay zero
    sess.reps.zero_()
    sess.build_reps(i32(batch.context - 1), i32([3, 5, 0]))
    torch.cuda.synchronize()
    again = sess.reps.cpu().numpy()
    assert (again[0, :, :3] == 0).all() and (again[1, :, :5] == 0).all()
    assert np.array_equal(again[0, :, 3:7], reps[0, :, 3:7])
    assert np.array_equal(again[1, :, 5:15], reps[1, :, 5:15])
    assert np.array_equal(again[2, :, :1], reps[2, :, :1])


def test_append_writes_slots_and_completed_block_rep():
    spec = synth.custom("append", batch=2, n_q_heads=4, n_kv_heads=2,
                        context=(767, 300), steps=3, config_id=92)
    batch = synth.make_batch(spec, DEV)
    prm, sess = make_session(batch)
    say("append", spec.context)
    for t in range(3):
        kn, vn = batch.new_kv_bits(t)
        sess.append(kn, vn, i32(batch.lens_at(t)))
    torch.cuda.synchronize()
    kp, vp = u16(batch.k_pages), u16(batch.v_pages)
    for b in range(2):
        for t in range(3):
            pos = int(batch.context[b]) - 1 + t
            page, slot = batch.table_np[b, pos // 128], pos % 128
            kn, vn = batch.new_kv_bits(t)
            assert np.array_equal(kp[page, :, slot, :], u16(kn[b]))
            assert np.array_equal(vp[page, :, :, slot], u16(vn[b]))
        nxt = int(batch.context[b]) - 1 + 3
        page, slot = batch.table_np[b, nxt // 128], nxt % 128
        assert (kp[page, :, slot, :] == synth.BF16_QNAN).all()
    # sequence 0 completed block 5 at step 1 (position 767)
    K, _, _ = logical_at_step(batch, 0, 2)
    ref = K[:, 640:768].mean(axis=1)
    got = sess.reps[0, :, 5].cpu().numpy()
    assert np.allclose(got, ref, rtol=0, atol=1e-6)
    assert (sess.reps[1].cpu().numpy() == 0).all()


def test_tiny_config_end_to_end_planted():
    batch = synth.make_batch(synth.CONFIGS[1], DEV)
    prm, sess = make_session(batch)
    say("tiny workload (1 x 4K, 8/2 heads)")
    prefill(batch, sess)
    step(batch, sess, 0)
    torch.cuda.synchronize()
    for h in range(2):
        assert set(batch.planted[0]) <= set(gpu_selection(sess, 0, h).tolist())
        assert int(sess.n_merged[0, h]) == 12
    oracle_full_check(batch, sess, 0)


@pytest.mark.parametrize("ppm,dense_boundary", [(200_000, 0), (70_000, 0),
                                                (1_000_000, 0), (0, 0),
                                                (200_000, 32768)])
def test_mixed_lengths_selection_and_attention(ppm, dense_boundary):
    spec = synth.custom("mixed", batch=4, n_q_heads=16, n_kv_heads=4,
                        context=(20000, 33000, 9000, 40960), steps=2,
                        init_tokens=1000, local_tokens=2000, topk_ppm=ppm,
                        dense_boundary=dense_boundary, shuffle=True, config_id=93)
    batch = synth.make_batch(spec, DEV)
    prm, sess = make_session(batch)
    say("mixed", ppm, dense_boundary)
    prefill(batch, sess)
    for t in range(2):
        step(batch, sess, t)
        torch.cuda.synchronize()
        oracle_full_check(batch, sess, t)


@pytest.mark.parametrize("hq,hkv", [(4, 4), (32, 2), (12, 4)])
def test_group_sizes(hq, hkv):
    spec = synth.custom("groups", batch=2, n_q_heads=hq, n_kv_heads=hkv,
                        context=(5000, 3333), init_tokens=256, local_tokens=700,
                        dense_boundary=0, config_id=94)
    batch = synth.make_batch(spec, DEV)
    prm, sess = make_session(batch)
    say("groups", hq, hkv)
    prefill(batch, sess)
    step(batch, sess, 0)
    torch.cuda.synchronize()
    oracle_full_check(batch, sess, 0)


@pytest.mark.parametrize("hq,hkv,context", [(32, 32, (20000,)), (64, 64, (9000,)),
                                             (40, 40, (12345,)),
                                             (48, 24, (7000, 15000))])
def test_many_kv_heads(hq, hkv, context):
    """Models with many KV heads (G = 1 or 2): the single-sequence partition
    then gives each list 512 / n_kv waves (16, 8, 12) and the lists no longer
    line up with the eight dies; batch 2 takes the range partition."""
    spec = synth.custom(f"kv{hkv}", batch=len(context), n_q_heads=hq, n_kv_heads=hkv,
                        context=context, steps=2, init_tokens=256, local_tokens=1000,
                        dense_boundary=0, config_id=160 + hkv)
    say("many KV heads", hq, hkv, context)
    if len(context) == 1:
        fused_vs_separate(spec, oracle_check=True)
        return
    batch = synth.make_batch(spec, DEV)
    prm, sess = make_session(batch)
    prefill(batch, sess)
    for t in range(2):
        step(batch, sess, t)
        torch.cuda.synchronize()
        oracle_full_check(batch, sess, t)


def test_short_and_degenerate_lengths():
    spec = synth.custom("short", batch=6, n_q_heads=8, n_kv_heads=2,
                        context=(1, 2, 127, 128, 129, 700), init_tokens=128,
                        local_tokens=128, dense_boundary=0, config_id=95)
    batch = synth.make_batch(spec, DEV)
    prm, sess = make_session(batch)
    say("short lengths")
    prefill(batch, sess)
    step(batch, sess, 0)
    torch.cuda.synchronize()
    oracle_full_check(batch, sess, 0)


def test_maximum_table_size():
    """8192 blocks (the library's table limit; 1,048,566 tokens) for one
    sequence: every register slot of the top-k, 254 score chunks, and a
    combine that folds several batches of pieces for one list."""
    L0 = 8192 * 128 - 10
    spec = synth.custom("max", batch=1, n_q_heads=4, n_kv_heads=1, context=(L0,),
                        dense_boundary=0, config_id=98)
    batch = synth.make_batch(spec, DEV)
    assert batch.table_np.shape[1] == 8192
    prm, sess = make_session(batch)
    say("maximum table size (8192 blocks)")
    prefill(batch, sess)
    step(batch, sess, 0)
    torch.cuda.synchronize()
    assert int(sess.n_sel[0, 0]) == -(-(8135 - 8) * 200_000 // 1_000_000)
    oracle_full_check(batch, sess, 0)


def test_zero_length_sequence_gives_zeros():
    spec = synth.custom("empty", batch=2, n_q_heads=8, n_kv_heads=2,
                        context=(1, 1000), config_id=96)
    batch = synth.make_batch(spec, DEV)
    prm, sess = make_session(batch)
    say("zero length")
    lens = i32([0, 1000])
    sess.build_reps(i32([0, 999]))
    kn, vn = batch.new_kv_bits(0)
    sess.append(kn, vn, lens)
    sess.select(batch.q_bits(0), lens)
    sess.attend(batch.q_bits(0), lens)
    torch.cuda.synchronize()
    assert (sess.n_merged[0].cpu().numpy() == 0).all()
    assert (sess.out[0].cpu().numpy() == 0).all()
    assert np.isfinite(sess.out[1].cpu().numpy()).all()


def test_ties_go_to_lower_block_index():
    """Identical blocks give bit-identical scores on both sides; the tie rule
    (smaller logical block first) decides the selection exactly."""
    spec = synth.custom("ties", batch=1, n_q_heads=8, n_kv_heads=2,
                        context=(6000,), init_tokens=128, local_tokens=256,
                        topk_ppm=100_000, dense_boundary=0, config_id=97)
    batch = synth.make_batch(spec, DEV)
    t = batch.table_np[0]
    src = t[10]
    for j in (3, 7, 12, 20, 33, 40):  # six copies of block 10 -> 7 equal reps
        batch.k_pages[t[j]] = batch.k_pages[src]
    prm, sess = make_session(batch)
    say("ties")
    prefill(batch, sess)
    step(batch, sess, 0)
    torch.cuda.synchronize()
    K, V, L = logical_at_step(batch, 0, 0)
    res = O.decode_step(q_f64(batch, 0)[0], K, V, L, L, oracle_params(spec))
    for h in range(2):
        assert np.array_equal(gpu_selection(sess, 0, h), res.heads[h].selected)
    oracle_full_check(batch, sess, 0)


def test_split_sizes_agree_and_runs_are_deterministic():
    spec = synth.custom("splits", batch=2, n_q_heads=32, n_kv_heads=8,
                        context=(30000, 17001), init_tokens=1024,
                        local_tokens=3000, dense_boundary=0, shuffle=True,
                        config_id=98)
    batch = synth.make_batch(spec, DEV)
    lens = i32(batch.lens_at(0))
    kn, vn = batch.new_kv_bits(0)
    outs = []
    for split in (7, 64, 301, 2048, 5000):
        prm, sess = make_session(batch, split_waves=split)
        say("split", split)
        prefill(batch, sess)
        if split == 7:
            sess.append(kn, vn, lens)  # once: the pools are shared
        sess.select(batch.q_bits(0), lens)
        o1 = sess.attend(batch.q_bits(0), lens).clone()
        o2 = sess.attend(batch.q_bits(0), lens).clone()
        torch.cuda.synchronize()
        assert torch.equal(o1, o2)
        outs.append(o1.cpu().numpy())
        if split in (7, 2048, 5000):
            oracle_full_check(batch, sess, 0)
    for o in outs[1:]:
        assert np.allclose(o, outs[0], rtol=1e-5, atol=1e-6)


def test_single_sequence_partition_split_sizes():
    """A batch of one takes the strided partition (wave c of P per list takes
    units c, c + P, ...): from one piece per list (every wave past its 64
    prefetched page ids) to more waves than units, each run deterministic
    and equal to the oracle."""
    spec = synth.custom("strided", batch=1, n_q_heads=32, n_kv_heads=8,
                        context=(30000,), init_tokens=1024, local_tokens=3000,
                        dense_boundary=0, shuffle=True, config_id=89)
    batch = synth.make_batch(spec, DEV)
    lens = i32(batch.lens_at(0))
    kn, vn = batch.new_kv_bits(0)
    outs = []
    for split in (1, 7, 64, 301, 2048, 5000):
        prm, sess = make_session(batch, split_waves=split)
        say("single-sequence split", split)
        prefill(batch, sess)
        if split == 1:
            sess.append(kn, vn, lens)  # once: the pools are shared
        sess.select(batch.q_bits(0), lens)
        o1 = sess.attend(batch.q_bits(0), lens).clone()
        o2 = sess.attend(batch.q_bits(0), lens).clone()
        torch.cuda.synchronize()
        assert torch.equal(o1, o2)
        outs.append(o1.cpu().numpy())
        if split in (1, 301, 5000):
            oracle_full_check(batch, sess, 0)
    for o in outs[1:]:
        assert np.allclose(o, outs[0], rtol=1e-5, atol=1e-6)


def test_attention_workspace_reused_across_shapes():
    """One zero-filled attention workspace serves calls of different shapes
    in turn (a ragged batch on the range split, a single sequence on the
    strided partition with its per-list hand-off counters, then the batch
    again): the combine waves leave the counters at rest, so every call
    gives, bit for bit, what the same call gives with a fresh workspace."""
    specs = [
        synth.custom("ws reuse batch", batch=3, n_q_heads=32, n_kv_heads=8,
                     context=(40000, 9000, 70001), dense_boundary=0, shuffle=True,
                     config_id=142),
        synth.custom("ws reuse single", batch=1, n_q_heads=16, n_kv_heads=4,
                     context=(20000,), dense_boundary=0, config_id=143),
    ]
    cases = []
    for spec in specs:
        batch = synth.make_batch(spec, DEV)
        prm, sess = make_session(batch)
        prefill(batch, sess)
        lens = i32(batch.lens_at(0))
        kn, vn = batch.new_kv_bits(0)
        sess.append(kn, vn, lens)
        sess.select(batch.q_bits(0), lens)
        ref = sess.attend(batch.q_bits(0), lens).clone()
        cases.append((spec, batch, prm, sess, lens, ref))
    size = max(B.attn_workspace_size(c[2], c[1].spec.batch, c[3].merged.shape[-1])
               for c in cases)
    ws = torch.zeros(size, dtype=torch.uint8, device=DEV)
    for i in (0, 1, 0, 1, 1, 0):
        spec, batch, prm, sess, lens, ref = cases[i]
        say("shared attention workspace:", spec.name)
        out = torch.full_like(ref, float("nan"))
        B.decode_attn(prm, batch.q_bits(0), sess.k_pages, sess.v_pages, sess.merged,
                      sess.n_merged, lens, out, ws)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), spec.name


@pytest.mark.parametrize("hq,hkv,dense_boundary,extra,per_seq", [
    (8, 2, 0, 0, False),        # group 4: four sequences per cascade wave
    (16, 2, 0, 0, False),       # group 8: two
    (4, 2, 0, 6, False),        # group 2: eight; shared count named 6 past the truth
    (32, 2, 0, 0, False),       # group 16: one (no reuse, same results)
    (16, 2, 12000, 0, False),   # one prompt below the dense boundary
    (16, 4, 0, 0, True),        # one selection per sequence, shared by its heads
])
def test_cascade_matches_oracle_and_plain_attention(hq, hkv, dense_boundary, extra,
                                                   per_seq):
    """rkv_decode_attn_cascade over a batch with a shared prefix: outputs
    against the oracle (selections and merged tables are the plain path's,
    checked too) and against rkv_decode_attn over the same tables.  The
    batch has a sequence whose last block is the first one past the shared
    prefix and sequences in a partly filled last group."""
    S = 40
    spec = synth.custom(f"cascade {hq}/{hkv}", batch=5, n_q_heads=hq, n_kv_heads=hkv,
                        context=(20000, 9000, S * 128 + 1, 14001, 11111), steps=2,
                        init_tokens=1024, local_tokens=3000,
                        dense_boundary=dense_boundary, shared_prefix_pages=S,
                        shuffle=True, config_id=144)
    batch = synth.make_batch(spec, DEV)
    if per_seq:
        prm, sess = make_session(batch, select_mode=B.SELECT_PER_SEQUENCE)
    else:
        prm, sess = make_session(batch)
    prefill(batch, sess)
    for t in range(spec.steps):
        say("cascade", spec.name, "step", t)
        lens = i32(batch.lens_at(t))
        kn, vn = batch.new_kv_bits(t)
        sess.append_select(batch.q_bits(t), kn, vn, lens)
        plain = sess.attend(batch.q_bits(t), lens).clone()
        sess.out.fill_(float("nan"))
        got = sess.attend_cascade(batch.q_bits(t), lens, S + extra).clone()
        torch.cuda.synchronize()
        assert torch.isfinite(got).all()
        scale = float(plain.abs().max())
        assert float((got - plain).abs().max()) <= 1e-5 * scale + 1e-7
        if per_seq:
            per_sequence_check(batch, sess, t)
        else:
            oracle_full_check(batch, sess, t)


def test_cascade_without_shared_blocks_is_plain_attention():
    """shared_blocks = 0 takes rkv_decode_attn's launches: bit-identical."""
    spec = synth.custom("cascade none", batch=3, n_q_heads=16, n_kv_heads=2,
                        context=(20000, 9000, 14001), steps=1, dense_boundary=0,
                        shared_prefix_pages=20, config_id=145)
    batch = synth.make_batch(spec, DEV)
    prm, sess = make_session(batch)
    prefill(batch, sess)
    lens = i32(batch.lens_at(0))
    kn, vn = batch.new_kv_bits(0)
    sess.append_select(batch.q_bits(0), kn, vn, lens)
    plain = sess.attend(batch.q_bits(0), lens).clone()
    got = sess.attend_cascade(batch.q_bits(0), lens, 0).clone()
    torch.cuda.synchronize()
    assert torch.equal(plain, got)


def _score_rounds(groups, max_blocks, init_tokens, n_cu):
    """Representations per score wave (8 x rounds) the library picks: 32,
    halved while the scan would have fewer than two waves per compute unit."""
    ib = min(-(-init_tokens // 128), max_blocks)
    rounds = 4
    while rounds > 1 and groups * -(-(max_blocks - ib) // (8 * rounds)) < 2 * n_cu:
        rounds //= 2
    return rounds


@pytest.mark.parametrize("batch_n,context,rounds", [
    (1, (20000,), 1), (2, (76800, 70001), 2), (8, (38400,) * 8, 4)])
def test_score_chunk_sizes(batch_n, context, rounds):
    """The scan's three chunk sizes (8, 16 and 32 representations per wave)
    give the oracle's selections, merged tables and outputs."""
    spec = synth.custom(f"score chunks {rounds}", batch=batch_n, n_q_heads=32,
                        n_kv_heads=8, context=context, shuffle=True,
                        dense_boundary=0, config_id=88)
    batch = synth.make_batch(spec, DEV)
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    mb = batch.table_np.shape[1]
    got = _score_rounds(batch_n * spec.n_kv_heads, mb, spec.init_tokens, n_cu)
    if n_cu == 256:
        assert got == rounds, (got, rounds)
    say("score chunk", 8 * got, "batch", batch_n, "max_blocks", mb)
    prm, sess = make_session(batch)
    prefill(batch, sess)
    step(batch, sess, 0)
    torch.cuda.synchronize()
    seqs = sorted({0, batch_n - 1})
    oracle_full_check(batch, sess, 0, seqs=seqs, heads=[0, 5])


def test_binding_rejects_mismatched_buffers():
    """The binding checks every tensor against the layout the C ABI assumes
    (exact shape, dtype, device) before the call, so an undersized or
    misplaced buffer raises instead of being read past its end."""
    spec = synth.custom("binding shapes", batch=2, n_q_heads=8, n_kv_heads=2,
                        context=(3000, 1000), dense_boundary=0, config_id=87)
    batch = synth.make_batch(spec, DEV)
    prm, sess = make_session(batch)
    lens = i32(batch.lens_at(0))
    q = batch.q_bits(0)
    short_out = torch.zeros((2, 7, 128), dtype=torch.float32, device=DEV)
    with pytest.raises(ValueError, match="out"):
        B.decode_attn(prm, q, sess.k_pages, sess.v_pages, sess.merged, sess.n_merged,
                      lens, short_out, sess.ws_attn)
    with pytest.raises(ValueError, match="reps"):
        B.select(prm, q, sess.reps[:, :, :-1].contiguous(), sess.block_table, lens,
                 sess.sel_ids, sess.n_sel, sess.merged, sess.n_merged, None,
                 sess.ws_select)
    with pytest.raises(ValueError, match="lens"):
        B.build_reps(prm, sess.k_pages, sess.block_table, lens[:1], sess.reps)
    with pytest.raises(ValueError, match="q"):
        sess.attend(q[:, :4].contiguous(), lens)          # prepared fast path
    with pytest.raises(ValueError, match="lens"):
        sess.attend(q, lens.cpu())                       # host tensor
    # the buffers are untouched and a well-formed step still runs
    prefill(batch, sess)
    step(batch, sess, 0)
    torch.cuda.synchronize()
    oracle_full_check(batch, sess, 0)


def test_many_short_lists():
    """More (sequence, KV head) lists than split waves (96 x 8 = 768 > 512),
    ragged and short: most waves' ranges cover several whole lists, so the
    piece numbering, the piece counts and the combine are exercised across
    many list boundaries.  Sampled sequences against the oracle."""
    rng = np.random.default_rng(86)
    ctx = tuple(int(x) for x in rng.integers(1, 3000, size=96))
    spec = synth.custom("many lists", batch=96, n_q_heads=32, n_kv_heads=8,
                        context=ctx, init_tokens=128, local_tokens=256,
                        dense_boundary=0, shuffle=True, config_id=86)
    batch = synth.make_batch(spec, DEV)
    prm, sess = make_session(batch)
    prefill(batch, sess)
    step(batch, sess, 0)
    torch.cuda.synchronize()
    seqs = [0, 1, 47, int(np.argmax(batch.context)), int(np.argmin(batch.context)), 95]
    oracle_full_check(batch, sess, 0, seqs=sorted(set(seqs)))


def _permuted_copy(batch, seed=5):
    """Same logical contents at different physical pages."""
    rng = np.random.default_rng(seed)
    P = batch.n_pages
    perm = rng.permutation(P)
    kp = torch.empty_like(batch.k_pages)
    vp = torch.empty_like(batch.v_pages)
    idx = torch.as_tensor(perm, device=DEV)
    kp[idx] = batch.k_pages
    vp[idx] = batch.v_pages
    table = np.where(batch.table_np >= 0, perm[np.maximum(batch.table_np, 0)], -1)
    return kp, vp, torch.as_tensor(table.astype(np.int32), device=DEV)


def test_page_permutation_and_shared_pages_bitwise():
    spec = synth.custom("perm", batch=3, n_q_heads=16, n_kv_heads=4,
                        context=(12000, 12000, 9000), init_tokens=512,
                        local_tokens=1500, dense_boundary=0,
                        shared_prefix_pages=20, config_id=99)
    batch = synth.make_batch(spec, DEV)
    say("permutation / shared pages")

    def run(kp, vp, table):
        prm = B.params(16, 4, init_tokens=512, local_tokens=1500, dense_boundary=0)
        sess = DecodeSession(prm, kp, vp, table, i32(batch.context))
        sess.build_reps(i32(batch.context - 1))
        kn, vn = batch.new_kv_bits(0)
        out = sess.step(batch.q_bits(0), kn, vn, i32(batch.lens_at(0)))
        torch.cuda.synchronize()
        return out.clone(), sess.sel_ids.clone(), sess.n_sel.clone()

    base = run(batch.k_pages.clone(), batch.v_pages.clone(), batch.block_table)
    perm = run(*_permuted_copy(batch))
    assert torch.equal(base[0], perm[0]) and torch.equal(base[1], perm[1])
    # private copies of the 20 shared prefix pages for sequences 1 and 2
    t = batch.table_np.copy()
    extra = []
    kp, vp = batch.k_pages.clone(), batch.v_pages.clone()
    nxt = batch.n_pages
    for b in (1, 2):
        for j in range(20):
            extra.append(int(t[b, j]))
            t[b, j] = nxt
            nxt += 1
    src = torch.as_tensor(extra, device=DEV)
    kp = torch.cat([kp, batch.k_pages[src]])
    vp = torch.cat([vp, batch.v_pages[src]])
    private = run(kp, vp, torch.as_tensor(t, device=DEV))
    assert torch.equal(base[0], private[0]) and torch.equal(base[1], private[1])


def test_invalid_page_ids_are_skipped():
    spec = synth.custom("badpage", batch=1, n_q_heads=8, n_kv_heads=2,
                        context=(3000,), init_tokens=256, local_tokens=512,
                        dense_boundary=0, config_id=100)
    batch = synth.make_batch(spec, DEV)
    prm, sess = make_session(batch)
    say("invalid page ids")
    prefill(batch, sess)
    lens = i32(batch.context)
    kn, vn = batch.new_kv_bits(0)
    sess.append(kn, vn, lens)
    sess.select(batch.q_bits(0), lens)
    torch.cuda.synchronize()
    mlog, _ = gpu_merged_logical(sess, batch, 0, 1)
    sess.merged[0, 1, 3] = -5
    sess.merged[0, 1, 4] = batch.n_pages + 7
    sess.attend(batch.q_bits(0), lens)
    torch.cuda.synchronize()
    K, V, L = logical_at_step(batch, 0, 0)
    keep = np.delete(mlog, [3, 4])
    G = 4
    q = q_f64(batch, 0)[0, G:2 * G]
    tok = (keep[:, None] * 128 + np.arange(128)).reshape(-1)
    tok = tok[tok < int(batch.context[0])]
    ref = O.attend(q, K[1, tok], V[1, tok], 1 / np.sqrt(128))
    assert L == int(batch.context[0])
    check_head_output(sess.out[0, G:2 * G].cpu().numpy(), ref, "bad pages")


def test_llama_layer_full_size_steps():
    batch = synth.make_batch(synth.CONFIGS[2], DEV)
    prm, sess = make_session(batch)
    say("8B layer (1 x 64K, 64 steps)")
    prefill(batch, sess)
    for t in range(64):
        step(batch, sess, t)
        if t in (0, 31, 63):
            torch.cuda.synchronize()
            for h in range(8):
                assert set(batch.planted[0]) <= set(gpu_selection(sess, 0, h).tolist())
            oracle_full_check(batch, sess, t)


def run_to_step(batch, sess, t_check):
    """Prefill, then decode steps 0 .. t_check (every step through the
    library, so the pools and representations evolve as in a real decode)."""
    prefill(batch, sess)
    for t in range(t_check + 1):
        step(batch, sess, t)
    torch.cuda.synchronize()


@pytest.mark.parametrize("t_check", [0, 15, 31])
def test_batched_ragged_full_size(t_check):
    """Batched workload (16 x U[32K, 128K], shuffled pool): every sequence
    and KV head against the oracle at the first, middle and last step."""
    batch = synth.make_batch(synth.CONFIGS[3], DEV)
    prm, sess = make_session(batch)
    say("batched (16 x 32K-128K, shuffled)", batch.context.tolist(), "step", t_check)
    run_to_step(batch, sess, t_check)
    oracle_full_check(batch, sess, t_check)


@pytest.mark.parametrize("t_check", [0, 7, 15])
def test_70b_shared_prefix_full_size(t_check):
    """70B-shaped layer (8 x 128K, 64/8 heads, 16K shared prefix): every
    sequence and KV head against the oracle at the first, middle and last
    step."""
    batch = synth.make_batch(synth.CONFIGS[4], DEV)
    prm, sess = make_session(batch)
    say("70B layer (8 x 128K, 64/8, shared prefix) step", t_check)
    run_to_step(batch, sess, t_check)
    oracle_full_check(batch, sess, t_check)


@pytest.mark.parametrize("t_check", [0, 15])
def test_70b_shared_prefix_cascade_full_size(t_check):
    """The 70B-shaped layer (8 x 128K, 64/8 heads, 128 shared prefix pages)
    with the cascade attention: every sequence and KV head against the
    oracle at the first and last step, and within rounding of
    rkv_decode_attn."""
    spec = synth.CONFIGS[4]
    batch = synth.make_batch(spec, DEV)
    prm, sess = make_session(batch)
    prefill(batch, sess)
    for t in range(t_check + 1):
        lens = i32(batch.lens_at(t))
        kn, vn = batch.new_kv_bits(t)
        sess.append_select(batch.q_bits(t), kn, vn, lens)
        got = sess.attend_cascade(batch.q_bits(t), lens, spec.shared_prefix_pages)
    say("70B cascade step", t_check)
    got = got.clone()
    plain = sess.attend(batch.q_bits(t_check), i32(batch.lens_at(t_check))).clone()
    torch.cuda.synchronize()
    scale = float(plain.abs().max())
    assert float((got - plain).abs().max()) <= 1e-5 * scale + 1e-7
    sess.out.copy_(got)
    oracle_full_check(batch, sess, t_check)


@pytest.mark.parametrize("t_check", [0, 15])
def test_70b_shared_prefix_full_size_per_sequence(t_check):
    """The per-sequence selection reading on the 70B-shaped layer at full
    size: every sequence against the head-summed oracle step."""
    batch = synth.make_batch(synth.CONFIGS[4], DEV)
    prm, sess = make_session(batch, select_mode=B.SELECT_PER_SEQUENCE)
    say("70B layer, per-sequence selection, step", t_check)
    run_to_step(batch, sess, t_check)
    per_sequence_check(batch, sess, t_check)


@pytest.mark.parametrize("t_check", [0, 31])
def test_batched_ragged_full_size_per_sequence(t_check):
    """The per-sequence selection reading on the batched workload (16 x
    U[32K, 128K], shuffled pool) at full size: every sequence against the
    head-summed oracle step, at the first and the last step."""
    batch = synth.make_batch(synth.CONFIGS[3], DEV)
    prm, sess = make_session(batch, select_mode=B.SELECT_PER_SEQUENCE)
    say("batched, per-sequence selection, step", t_check)
    run_to_step(batch, sess, t_check)
    per_sequence_check(batch, sess, t_check)


@pytest.mark.parametrize("hq,hkv", [(4, 4), (8, 4), (16, 4), (64, 8)])
def test_valu_variant_matches_oracle_and_mfma(hq, hkv):
    spec = synth.custom("valu", batch=2, n_q_heads=hq, n_kv_heads=hkv,
                        context=(9000, 4321), init_tokens=512, local_tokens=1000,
                        dense_boundary=0, config_id=101)
    batch = synth.make_batch(spec, DEV)
    say("valu", hq, hkv)
    outs = {}
    for impl in (B.ATTN_MFMA, B.ATTN_VALU):
        prm, sess = make_session(batch, attn_impl=impl)
        prefill(batch, sess)
        if impl == B.ATTN_MFMA:
            kn, vn = batch.new_kv_bits(0)
            sess.append(kn, vn, i32(batch.lens_at(0)))
        sess.select(batch.q_bits(0), i32(batch.lens_at(0)))
        sess.attend(batch.q_bits(0), i32(batch.lens_at(0)))
        torch.cuda.synchronize()
        oracle_full_check(batch, sess, 0)
        outs[impl] = sess.out.cpu().numpy()
    assert np.allclose(outs[B.ATTN_MFMA], outs[B.ATTN_VALU], rtol=1e-4, atol=1e-5)


def make_host_session(spec, resident=True, slot_mult=1, slot_cap=None,
                      copy_mode="kernel", **pkw):
    """Host-tier session: prefill representations are built with every block
    in HBM, then the offload blocks move to pinned host memory."""
    max_blocks = -(-(max(spec.context) + spec.steps - 1) // 128)
    batch = synth.make_batch(spec, DEV, extra_pages=slot_mult * spec.batch * max_blocks)
    kw = dict(init_tokens=spec.init_tokens, local_tokens=spec.local_tokens,
              topk_ppm=spec.topk_ppm, dense_boundary=spec.dense_boundary)
    kw.update(pkw)
    prm = B.params(spec.n_q_heads, spec.n_kv_heads, **kw)
    k_cap = max(1, B.topk_capacity(prm, max_blocks))
    sess = HostTierSession(prm, batch.k_pages, batch.v_pages, batch.block_table,
                           i32(batch.context), resident=resident,
                           slot_cap=slot_mult * k_cap if slot_cap is None else slot_cap,
                           copy_mode=copy_mode)
    assert sess.stage_page0 >= batch.n_pages  # staging pages are the extra ones
    prefill(batch, sess)
    torch.cuda.synchronize()
    host = synth.move_offload_to_host(batch)
    sess.attach_host(host.host_k, host.host_v, host.host_table)
    return batch, host, sess


@pytest.mark.parametrize("copy_mode", ["kernel", "memcpy"])
@pytest.mark.parametrize("resident", [True, False])
def test_host_tier_small(resident, copy_mode):
    # host blocks [8, 90) of the offload range [8, 100): blocks 90..99 stay in
    # HBM and are read in place when kept
    spec = synth.scaled(synth.CONFIGS[5], batch=2, context=(20000, 20000), steps=3,
                        plant_range=(8, 90), plant_count=5, local_tokens=7192,
                        dense_boundary=0, config_id=102)
    say(f"host tier small (resident={resident}, copies by {copy_mode})")
    batch, host, sess = make_host_session(spec, resident=resident, copy_mode=copy_mode)
    for t in range(3):
        step(batch, sess, t)
        torch.cuda.synchronize()
        for b in range(2):
            for h in range(8):
                assert set(batch.planted[b]) <= set(gpu_selection(sess, b, h).tolist())
        oracle_full_check(batch, sess, t, host=host)


@pytest.mark.parametrize("slot_mult", [1, 2])
def test_host_tier_overlapped_step(slot_mult):
    """The step whose copies overlap the attention over the blocks already in
    HBM (the planner in split mode, rkv_stage_copy on the side stream,
    rkv_decode_attn_lse over the resident entries, then over the newly
    staged ones with the first part folded in): the same selections and slot
    state as the plain step, outputs within rounding of it and against the
    oracle, and split tables that hold exactly the plain table's pages (the
    resident ones in the plain order, the trailing block last)."""
    spec = synth.scaled(synth.CONFIGS[5], batch=2, context=(20000, 23000), steps=6,
                        plant_range=(8, 90), plant_count=5, local_tokens=7192,
                        topk_ppm=200_000, dense_boundary=0, config_id=104)
    say(f"host tier overlapped step (slots {slot_mult} x k_cap)")
    batch_a, _, sess_a = make_host_session(spec, resident=True, slot_mult=slot_mult)
    batch_b, host_b, sess_b = make_host_session(spec, resident=True, slot_mult=slot_mult)
    for t in range(6):
        step(batch_a, sess_a, t)
        lens = i32(batch_b.lens_at(t))
        kn, vn = batch_b.new_kv_bits(t)
        sess_b.out.fill_(float("nan"))
        sess_b.step_overlapped(batch_b.q_bits(t), kn, vn, lens)
        torch.cuda.synchronize()
        assert torch.equal(sess_a.n_sel, sess_b.n_sel), t
        assert torch.equal(sess_a.slot_ids, sess_b.slot_ids), t
        assert torch.equal(sess_a.slot_cursor, sess_b.slot_cursor), t
        assert torch.equal(sess_a.n_staged, sess_b.n_staged), t
        ma, na = sess_a.merged.cpu().numpy(), sess_a.n_merged.cpu().numpy()
        mr, nr = sess_b.merged.cpu().numpy(), sess_b.n_merged.cpu().numpy()
        mn, nn = sess_b.merged_new.cpu().numpy(), sess_b.n_new.cpu().numpy()
        for b in range(2):
            for h in range(8):
                plain = [int(x) for x in ma[b, h, :na[b, h]] if x >= 0]
                res = [int(x) for x in mr[b, h, :nr[b, h]]]
                new = [int(x) for x in mn[b, h, :nn[b, h]]]
                assert sorted(plain) == sorted(res + new), (t, b, h)
                assert [x for x in plain if x not in set(new)] == res, (t, b, h)
                assert res[-1] == plain[-1], (t, b, h)
        scale = float(sess_a.out.abs().max())
        assert float((sess_b.out - sess_a.out).abs().max()) <= 1e-5 * scale + 1e-7, t
        if t in (0, 5):
            # the oracle check reads the whole merged table: the plain one
            sess_b.merged.copy_(sess_a.merged)
            sess_b.n_merged.copy_(sess_a.n_merged)
            oracle_full_check(batch_b, sess_b, t, host=host_b)


def mirror_residency(slots, cursor, kept, on_host):
    """The slot policy of rkv_stage_resident, restated: slots holding a kept
    host block keep it; the other kept host blocks, ascending, take the slots
    holding no kept block in slot order from the cursor, which then moves
    past the last slot filled.  Returns (blocks copied, new cursor)."""
    S = len(slots)
    held = {}
    for r, j in enumerate(slots):
        if j >= 0 and j in kept and on_host[j] and j not in held:
            held[j] = r
    free = [(cursor + i) % S for i in range(S) if (cursor + i) % S not in held.values()]
    new = [j for j in sorted(kept) if on_host[j] and j not in held]
    n = min(len(new), len(free))
    for j, r in zip(new[:n], free[:n]):
        slots[r] = j
    if n:
        cursor = (free[n - 1] + 1) % S
    return new[:n], cursor


@pytest.mark.parametrize("slot_mult", [1, 2])
def test_host_tier_residency_matches_full_staging(slot_mult):
    """Residency changes which bytes move, not the results: every step's
    output and selection equal those of staging every kept block, and the
    slot state, copy counts and merged page ids follow the stated policy
    (with k_cap slots, and with twice as many)."""
    spec = synth.scaled(synth.CONFIGS[5], batch=2, context=(20000, 23000), steps=6,
                        plant_range=(8, 90), plant_count=5, local_tokens=7192,
                        topk_ppm=200_000, dense_boundary=0, config_id=104)
    say(f"host tier residency vs full staging (slots {slot_mult} x k_cap)")
    batch_r, host_r, sess_r = make_host_session(spec, resident=True, slot_mult=slot_mult)
    batch_f, _, sess_f = make_host_session(spec, resident=False)
    k_cap, S = sess_r.k_cap, sess_r.slot_cap
    assert S == slot_mult * k_cap
    slots = {(b, h): [-1] * S for b in range(2) for h in range(8)}
    cursors = {(b, h): 0 for b in range(2) for h in range(8)}
    kept_total = copied_total = 0
    for t in range(6):
        step(batch_r, sess_r, t)
        step(batch_f, sess_f, t)
        torch.cuda.synchronize()
        assert torch.equal(sess_r.out, sess_f.out), t
        assert torch.equal(sess_r.n_sel, sess_f.n_sel), t
        sel = sess_r.sel_ids.cpu().numpy()
        n_sel = sess_r.n_sel.cpu().numpy()
        slot_gpu = sess_r.slot_ids.cpu().numpy()
        cur_gpu = sess_r.slot_cursor.cpu().numpy()
        staged = sess_r.n_staged.cpu().numpy()
        merged = sess_r.merged.cpu().numpy()
        lens = batch_r.lens_at(t)
        for b in range(2):
            on_host = host_r.host_table_np[b] >= 0
            n_init = min(8, -(-int(lens[b]) // 128))
            for h in range(8):
                kept = [int(j) for j in sel[b, h, :n_sel[b, h]]]
                assert np.array_equal(kept, sess_f.sel_ids.cpu().numpy()[b, h, :n_sel[b, h]])
                new, cursors[(b, h)] = mirror_residency(slots[(b, h)], cursors[(b, h)],
                                                        set(kept), on_host)
                assert slot_gpu[b, h].tolist() == slots[(b, h)], (t, b, h)
                assert cur_gpu[b, h] == cursors[(b, h)], (t, b, h)
                assert staged[b, h] == len(new), (t, b, h)
                for q, j in enumerate(kept):
                    if on_host[j]:
                        r = slots[(b, h)].index(j)
                        assert merged[b, h, n_init + q] == sess_r.stage_page0 + b * S + r
                    else:
                        assert merged[b, h, n_init + q] == batch_r.table_np[b, j]
                if t > 0:
                    kept_total += sum(1 for j in kept if on_host[j])
                    copied_total += len(new)
    assert copied_total < kept_total


@pytest.mark.parametrize("resident", [True, False])
@pytest.mark.parametrize("select_mode", [B.SELECT_PER_HEAD, B.SELECT_PER_SEQUENCE])
def test_host_tier_copy_engine_equals_gather_kernel(select_mode, resident):
    """The copy engines -- on the side stream, or spread over 3 or 4 copy
    lanes -- and the gather kernel stage the same bytes to the same slots:
    pools, slot state, merged tables and outputs bit-identical over four
    steps (with residency: 2x slots)."""
    spec = synth.scaled(synth.CONFIGS[5], batch=2, context=(20000, 23000), steps=4,
                        plant_range=(8, 90), plant_count=5, local_tokens=7192,
                        dense_boundary=0, config_id=110)
    say(f"host tier: copy engines vs gather kernel, select mode {select_mode}, "
        f"resident {resident}")
    runs = {}
    for mode, lanes in (("kernel", 0), ("memcpy", 0), ("memcpy", 4), ("memcpy", 3)):
        batch, host, sess = make_host_session(spec, resident=resident, slot_mult=2,
                                              copy_mode=mode, select_mode=select_mode,
                                              copy_lanes=lanes)
        rec = []
        for t in range(4):
            step(batch, sess, t)
            torch.cuda.synchronize()
            rec.append((sess.out.clone(), sess.merged.clone(), sess.n_merged.clone(),
                        sess.slot_ids.clone(), sess.n_staged.clone()))
        rec.append((batch.k_pages.clone(), batch.v_pages.clone()))
        runs[(mode, lanes)] = rec
        del batch, host, sess
    for key in (("memcpy", 0), ("memcpy", 4), ("memcpy", 3)):
        for a, b in zip(runs[("kernel", 0)], runs[key]):
            for x, y in zip(a, b):
                assert torch.equal(x, y), key


def test_host_tier_too_few_slots_is_reported():
    """slot_cap below the kept count: the blocks that find no slot are left
    out (page -1) and every such list reports n_staged = -1."""
    spec = synth.scaled(synth.CONFIGS[5], batch=2, context=(20000, 23000), steps=1,
                        plant_range=(8, 90), plant_count=5, local_tokens=7192,
                        dense_boundary=0, config_id=109)
    say("host tier with too few staging slots")
    batch, host, sess = make_host_session(spec, resident=True, slot_cap=3)
    step(batch, sess, 0)
    torch.cuda.synchronize()
    staged = sess.n_staged.cpu().numpy()
    merged = sess.merged.cpu().numpy()
    sel = sess.sel_ids.cpu().numpy()
    n_sel = sess.n_sel.cpu().numpy()
    lens = batch.lens_at(0)
    for b in range(2):
        on_host = host.host_table_np[b] >= 0
        n_init = min(8, -(-int(lens[b]) // 128))
        for h in range(8):
            kept = [int(j) for j in sel[b, h, :n_sel[b, h]]]
            n_host = sum(1 for j in kept if on_host[j])
            assert n_host > 3 and staged[b, h] == -1, (b, h)
            pages = [int(merged[b, h, n_init + q]) for q, j in enumerate(kept) if on_host[j]]
            assert sum(p >= 0 for p in pages) == 3 and pages.count(-1) == n_host - 3


def test_host_tier_overlapped_step_with_too_few_slots():
    """The overlapped step with slot_cap below the kept count: the blocks
    without a slot are in neither split table, exactly as the plain step
    leaves them out (page -1), and the outputs agree within rounding."""
    spec = synth.scaled(synth.CONFIGS[5], batch=2, context=(20000, 23000), steps=1,
                        plant_range=(8, 90), plant_count=5, local_tokens=7192,
                        dense_boundary=0, config_id=109)
    say("host tier overlapped step with too few staging slots")
    batch_a, _, sess_a = make_host_session(spec, resident=True, slot_cap=3)
    batch_b, _, sess_b = make_host_session(spec, resident=True, slot_cap=3)
    step(batch_a, sess_a, 0)
    lens = i32(batch_b.lens_at(0))
    kn, vn = batch_b.new_kv_bits(0)
    sess_b.step_overlapped(batch_b.q_bits(0), kn, vn, lens)
    torch.cuda.synchronize()
    assert torch.equal(sess_a.n_staged, sess_b.n_staged)
    assert (sess_b.n_staged.cpu().numpy() == -1).all()
    assert (sess_b.n_new.cpu().numpy() == 3).all()
    ma, na = sess_a.merged.cpu().numpy(), sess_a.n_merged.cpu().numpy()
    mr, nr = sess_b.merged.cpu().numpy(), sess_b.n_merged.cpu().numpy()
    mn = sess_b.merged_new.cpu().numpy()
    for b in range(2):
        for h in range(8):
            plain = [int(x) for x in ma[b, h, :na[b, h]] if x >= 0]
            split = [int(x) for x in mr[b, h, :nr[b, h]]] + [int(x) for x in mn[b, h, :3]]
            assert sorted(plain) == sorted(split), (b, h)
    scale = float(sess_a.out.abs().max())
    assert float((sess_b.out - sess_a.out).abs().max()) <= 1e-5 * scale + 1e-7


@pytest.mark.parametrize("concurrent", [False, True])
def test_offload_prefill_native(concurrent):
    """rkv_offload_blocks copies exactly the offload blocks that have a host
    page (bit-exact), leaves every other host page alone, and the decode
    path then runs from the natively filled pools (oracle check)."""
    spec = synth.scaled(synth.CONFIGS[5], batch=2, context=(20000, 23000), steps=2,
                        plant_range=(8, 90), plant_count=5, local_tokens=7192,
                        dense_boundary=0, config_id=105)
    say("native prefill offload")
    max_blocks = -(-(max(spec.context) + spec.steps - 1) // 128)
    batch = synth.make_batch(spec, DEV, extra_pages=spec.batch * max_blocks)
    host = synth.plan_host_pools(batch)
    n_host = host.host_k.shape[0]
    # one extra host page, assigned to an init block: outside the offload
    # range, so it must stay untouched
    hk = torch.full((n_host + 1,) + tuple(host.host_k.shape[1:]), 0x1234,
                    dtype=torch.int16, pin_memory=True)
    hv = torch.full_like(hk, 0x4321, pin_memory=True)
    table = host.host_table_np.copy()
    table[0, 0] = n_host
    host_table = torch.from_numpy(table).to(DEV)
    prm = B.params(spec.n_q_heads, spec.n_kv_heads, init_tokens=spec.init_tokens,
                   local_tokens=spec.local_tokens, topk_ppm=spec.topk_ppm,
                   dense_boundary=spec.dense_boundary)
    sess = HostTierSession(prm, batch.k_pages, batch.v_pages, batch.block_table,
                           i32(batch.context))
    ref = DecodeSession(prm, batch.k_pages, batch.v_pages, batch.block_table,
                        i32(batch.context))
    prefill_lens = i32(batch.context - 1)
    ref.build_reps(prefill_lens)
    sess.offload_prefill(hk, hv, host_table, prefill_lens, concurrent=concurrent)
    torch.cuda.synchronize()
    assert torch.equal(sess.reps, ref.reps)
    kp, vp = batch.k_pages.cpu(), batch.v_pages.cpu()
    for b in range(2):
        for j in range(8, 90):
            hp, page = int(table[b, j]), int(batch.table_np[b, j])
            assert torch.equal(hk[hp], kp[page]) and torch.equal(hv[hp], vp[page]), (b, j)
    assert bool((hk[n_host] == 0x1234).all()) and bool((hv[n_host] == 0x4321).all())
    # decode from the natively filled pools (the extra page is not used:
    # block 0 is an init block, read from HBM)
    pools = synth.HostPools(hk[:n_host], hv[:n_host], host.host_table, host.host_table_np)
    synth.poison_device_copies(batch, pools)
    sess.attach_host(pools.host_k, pools.host_v, pools.host_table)
    for t in range(2):
        step(batch, sess, t)
        torch.cuda.synchronize()
        oracle_full_check(batch, sess, t, host=pools)


@pytest.mark.parametrize("t_check", [0, 7, 15])
def test_host_tier_full_size(t_check):
    """Host tier (4 x 256K, offload blocks in pinned host memory, residency):
    every sequence and KV head against the oracle at the first, middle and
    last step."""
    say("host tier (4 x 256K) step", t_check)
    batch, host, sess = make_host_session(synth.CONFIGS[5])
    for t in range(t_check + 1):
        step(batch, sess, t)
    torch.cuda.synchronize()
    oracle_full_check(batch, sess, t_check, host=host)


def test_host_tier_full_size_per_sequence_copy_lanes():
    """Host tier at full size (4 x 256K) with the per-sequence selection and
    whole-page staging by the copy engines over four copy lanes, with
    residency: every sequence against the head-summed oracle at step 7."""
    say("host tier (4 x 256K), per-sequence selection, copy engines over 4 lanes")
    batch, host, sess = make_host_session(synth.CONFIGS[5], copy_mode="memcpy",
                                          select_mode=B.SELECT_PER_SEQUENCE,
                                          copy_lanes=4)
    for t in range(8):
        step(batch, sess, t)
    torch.cuda.synchronize()
    per_sequence_check(batch, sess, 7, host=host)


def per_sequence_check(batch, sess, t, seqs=None, host=None):
    """Per-sequence selection mode: one oracle step over all KV heads of each
    sequence (scores summed over the heads), every head's GPU selection equal
    to the others' and checked against it, merged tables and outputs per
    head."""
    spec = batch.spec
    G = spec.group
    out = sess.out.cpu().numpy()
    qall = q_f64(batch, t)
    prm = oracle_params(spec, per_sequence=True)
    for b in (range(spec.batch) if seqs is None else seqs):
        hs = list(range(spec.n_kv_heads))
        K, V, L = logical_at_step(batch, b, t, seq_pages_host(batch, b, hs, host))
        res = O.decode_step(qall[b], K, V, L, int(batch.context[b]), prm)
        sel0 = gpu_selection(sess, b, 0)
        for h in hs:
            ctx = f"{spec.name} per-sequence step {t} seq {b} head {h}"
            sel = gpu_selection(sess, b, h)
            assert np.array_equal(sel, sel0), ctx
            hr = res.heads[h]
            check_selection(sel, hr, res.regions.n_init, ctx)
            expect = check_merged(sess, batch, b, h, res.regions, sel, host, ctx)
            q = qall[b, h * G:(h + 1) * G]
            if np.array_equal(sel, hr.selected):
                ref = res.out[h * G:(h + 1) * G]
            else:
                prm1 = O.Params(G, 1, prm.init_tokens, prm.local_tokens, prm.topk_ppm,
                                prm.dense_boundary)
                ref = O.decode_step(q, K[h:h + 1], V[h:h + 1], L, int(batch.context[b]),
                                    prm1, merged_override=[expect]).out
            check_head_output(out[b, h * G:(h + 1) * G], ref, ctx)


def test_per_sequence_selection_mixed():
    spec = synth.custom("perseq", batch=3, n_q_heads=16, n_kv_heads=4,
                        context=(767, 9000, 20480), steps=2, init_tokens=256,
                        local_tokens=1000, dense_boundary=0, config_id=106)
    say("per-sequence selection, mixed lengths")
    batch = synth.make_batch(spec, DEV)
    prm, sess = make_session(batch, select_mode=B.SELECT_PER_SEQUENCE)
    prefill(batch, sess)
    for t in range(2):
        step(batch, sess, t)
        torch.cuda.synchronize()
        per_sequence_check(batch, sess, t)


def test_per_sequence_selection_llama_layer():
    say("per-sequence selection, 8B layer (1 x 64K), steps 0 and 5")
    spec = synth.scaled(synth.CONFIGS[2], steps=6)
    batch = synth.make_batch(spec, DEV)
    prm, sess = make_session(batch, select_mode=B.SELECT_PER_SEQUENCE)
    prefill(batch, sess)
    for t in range(6):
        step(batch, sess, t)
        if t in (0, 5):
            torch.cuda.synchronize()
            per_sequence_check(batch, sess, t)


def test_decode_step_replays_from_a_hip_graph():
    """A whole decode step (append + select + attention, four kernels, no
    memsets, no host syncs) captured in a HIP graph: every replay, with eager
    work and synchronisations in between, equals the eager step bit for
    bit."""
    spec = synth.custom("graph", batch=2, n_q_heads=16, n_kv_heads=4,
                        context=(9000, 20480), steps=1, init_tokens=256,
                        local_tokens=1000, dense_boundary=0, config_id=107)
    say("HIP graph replay of a decode step")
    batch = synth.make_batch(spec, DEV)
    prm, sess = make_session(batch)
    prefill(batch, sess)
    lens = i32(batch.lens_at(0))
    kn, vn = batch.new_kv_bits(0)
    q = batch.q_bits(0)
    sess.step(q, kn, vn, lens)
    torch.cuda.synchronize()
    eager = (sess.out.clone(), sess.merged.clone(), sess.n_merged.clone(),
             sess.sel_ids.clone())
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        sess.step(q, kn, vn, lens)  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        sess.step(q, kn, vn, lens)
    for r in range(3):
        sess.out.zero_()
        sess.merged.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        # merged lists count only their first n_merged entries
        live = (torch.arange(sess.merged.shape[-1], device=DEV)
                < sess.n_merged[..., None])
        assert torch.equal(sess.n_merged, eager[2]), r
        assert torch.equal(sess.merged[live], eager[1][live]), r
        assert torch.equal(sess.out, eager[0]), r
        assert torch.equal(sess.sel_ids, eager[3]), r


@pytest.mark.parametrize("copy_mode", ["kernel", "memcpy"])
def test_per_sequence_selection_with_resident_host_tier(copy_mode):
    """Per-sequence selection: every KV head keeps the same blocks, so the
    copy-engine mode copies whole pages."""
    spec = synth.scaled(synth.CONFIGS[5], batch=2, context=(20000, 23000), steps=3,
                        plant_range=(8, 90), plant_count=5, local_tokens=7192,
                        dense_boundary=0, config_id=108)
    say(f"per-sequence selection + resident host tier, copies by {copy_mode}")
    batch, host, sess = make_host_session(spec, resident=True, copy_mode=copy_mode,
                                          select_mode=B.SELECT_PER_SEQUENCE)
    for t in range(3):
        step(batch, sess, t)
        torch.cuda.synchronize()
        per_sequence_check(batch, sess, t, host=host)


def random_case(seed):
    """One seeded random configuration of the method and launch."""
    rng = np.random.default_rng(7000 + seed)
    G = int(rng.choice([1, 2, 4, 8, 16]))
    hkv = int(rng.choice([1, 2, 4]))
    bsz = int(rng.integers(1, 5))
    ctx = tuple(int(x) for x in rng.integers(1, 24000, size=bsz))
    spec = synth.custom(f"random{seed}", batch=bsz, n_q_heads=G * hkv, n_kv_heads=hkv,
                        context=ctx, steps=2,
                        init_tokens=int(rng.choice([0, 128, 256, 1000, 1024])),
                        local_tokens=int(rng.choice([0, 1, 128, 1000, 7192])),
                        topk_ppm=int(rng.choice([1, 50_000, 200_000, 999_999, 1_000_000])),
                        dense_boundary=int(rng.choice([0, 0, 5000, 32768])),
                        shuffle=bool(rng.integers(0, 2)), config_id=300 + seed)
    impls = [B.ATTN_MFMA] + ([B.ATTN_VALU] if G in (1, 2, 4, 8) else [])
    launch = dict(split_waves=int(rng.choice([0, 7, 64, 512, 1000])),
                  attn_impl=int(rng.choice(impls)),
                  select_mode=int(rng.choice([B.SELECT_PER_HEAD, B.SELECT_PER_SEQUENCE])))
    return spec, launch


RANDOM_CASES = int(os.environ.get("RKV_RANDOM_CASES", "16"))


@pytest.mark.parametrize("seed", range(RANDOM_CASES))
def test_random_configurations(seed):
    spec, launch = random_case(seed)
    say(f"random configuration {seed}: {spec.batch} x {spec.context}, "
        f"{spec.n_q_heads}/{spec.n_kv_heads}, init {spec.init_tokens}, "
        f"local {spec.local_tokens}, ppm {spec.topk_ppm}, dense {spec.dense_boundary}, "
        f"{launch}")
    batch = synth.make_batch(spec, DEV)
    prm, sess = make_session(batch, **launch)
    prefill(batch, sess)
    for t in range(2):
        step(batch, sess, t)
        torch.cuda.synchronize()
        if launch["select_mode"] == B.SELECT_PER_SEQUENCE:
            per_sequence_check(batch, sess, t)
        else:
            oracle_full_check(batch, sess, t)


def test_append_select_equals_append_then_select():
    """The fused launch gives bit-identical pools, representations,
    selections and merged tables to rkv_append_kv followed by rkv_select."""
    spec = synth.custom("fused", batch=3, n_q_heads=16, n_kv_heads=4,
                        context=(767, 9000, 20480), steps=2, init_tokens=256,
                        local_tokens=1000, dense_boundary=0, config_id=103)
    say("append_select vs append + select")
    results = []
    for fused in (False, True):
        batch = synth.make_batch(spec, DEV)
        prm, sess = make_session(batch)
        prefill(batch, sess)
        for t in range(2):
            lens = i32(batch.lens_at(t))
            kn, vn = batch.new_kv_bits(t)
            if fused:
                sess.append_select(batch.q_bits(t), kn, vn, lens)
            else:
                sess.append(kn, vn, lens)
                sess.select(batch.q_bits(t), lens)
        torch.cuda.synchronize()
        results.append((batch.k_pages.clone(), batch.v_pages.clone(), sess.reps.clone(),
                        sess.sel_ids.clone(), sess.n_sel.clone(), sess.merged.clone(),
                        sess.n_merged.clone()))
    for x, y in zip(*results):
        assert torch.equal(x, y)
    # sequence 0 completed block 5 at step 1: its representation exists
    assert results[1][2][0, :, 5].abs().sum() > 0


# ---------------------------------------------------------------------------
# rkv_decode_step (for a batch of one: the top-k and merge inside the
# attention launch) against rkv_append_select + rkv_decode_attn.  Every
# selection, merged table, pool, representation and output must be
# bit-identical: both attend the same pages in the same order with the same
# arithmetic, and the selection is defined by its values alone.
# ---------------------------------------------------------------------------

def _valid_rows(sel, n):
    return [sel[i, :int(n[i])].tolist() for i in range(n.shape[0])]


def _snapshot(sess):
    n_sel = sess.n_sel.cpu().numpy()
    n_m = sess.n_merged.cpu().numpy()
    sel = sess.sel_ids.cpu().numpy()
    mer = sess.merged.cpu().numpy()
    return (sess.out.cpu().numpy().copy(), n_sel.copy(), n_m.copy(),
            [_valid_rows(sel[b], n_sel[b]) for b in range(sel.shape[0])],
            [_valid_rows(mer[b], n_m[b]) for b in range(mer.shape[0])])


def fused_vs_separate(spec, launch=None, steps=None, zero_q=False, mutate=None,
                      oracle_check=False):
    launch = launch or {}
    steps = spec.steps if steps is None else steps
    runs = []
    for mode in ("step", "separate"):
        batch = synth.make_batch(spec, DEV)
        if mutate is not None:
            mutate(batch)
        prm, sess = make_session(batch, **launch)
        prefill(batch, sess)
        rec = []
        for t in range(steps):
            lens = i32(batch.lens_at(t))
            kn, vn = batch.new_kv_bits(t)
            q = batch.q_bits(t)
            if zero_q:
                q = torch.zeros_like(q)
            if mode == "step":
                sess.step(q, kn, vn, lens)
            else:
                sess.step_separate(q, kn, vn, lens)
            torch.cuda.synchronize()
            rec.append(_snapshot(sess))
            if mode == "step" and oracle_check:
                oracle_full_check(batch, sess, t, q=q if zero_q else None)
        rec.append((u16(batch.k_pages), u16(batch.v_pages), sess.reps.cpu().numpy()))
        runs.append(rec)
        del batch, sess
    for t, (a, b) in enumerate(zip(runs[0][:-1], runs[1][:-1])):
        assert np.array_equal(a[0], b[0]), f"out differs at step {t}"
        assert np.array_equal(a[1], b[1]) and np.array_equal(a[2], b[2]), t
        assert a[3] == b[3], f"selection differs at step {t}"
        assert a[4] == b[4], f"merged table differs at step {t}"
    for x, y in zip(runs[0][-1], runs[1][-1]):
        assert np.array_equal(x, y)
    return runs


def test_decode_step_llama_layer_equals_separate_calls():
    say("decode step vs separate calls, 8B layer (1 x 64K), 3 steps")
    fused_vs_separate(synth.CONFIGS[2], steps=3)


def test_decode_step_tiny_planted_against_oracle():
    say("decode step, tiny workload (1 x 4K), against the oracle and separate calls")
    fused_vs_separate(synth.CONFIGS[1], oracle_check=True)


def test_decode_step_all_scores_tied():
    """q = 0: every score is 0 (or -0), so the k-th largest key ties with
    every other key and the lowest blocks are kept."""
    spec = synth.custom("tied", batch=1, n_q_heads=16, n_kv_heads=4, context=(40000,),
                        steps=2, dense_boundary=0, config_id=120)
    say("decode step, all scores tied")
    runs = fused_vs_separate(spec, zero_q=True, oracle_check=True)
    n_init = 8
    n_sel = runs[0][0][1][0]
    sel = runs[0][0][3][0]
    for h in range(4):
        assert sel[h] == list(range(n_init, n_init + int(n_sel[h])))


def test_decode_step_partial_ties_at_the_threshold():
    spec = synth.custom("ties2", batch=1, n_q_heads=8, n_kv_heads=2, context=(30000,),
                        steps=2, init_tokens=128, local_tokens=256, dense_boundary=0,
                        config_id=121)

    def dup(batch):
        t = batch.table_np[0]
        for j in range(30, 230, 2):  # 100 copies of block 20 -> ties around k
            batch.k_pages[t[j]] = batch.k_pages[t[20]]

    say("decode step, duplicated blocks (ties)")
    for ppm in (50_000, 200_000, 500_000):
        fused_vs_separate(synth.scaled(spec, topk_ppm=ppm), mutate=dup,
                          oracle_check=True)


@pytest.mark.parametrize("ctx,expect_fused", [(131071, True), (131072, False)])
def test_decode_step_block_limit(ctx, expect_fused):
    """1024 blocks (the last shape the folded selection takes) and 1025."""
    spec = synth.custom(f"limit{ctx}", batch=1, n_q_heads=8, n_kv_heads=1,
                        context=(ctx,), steps=2, dense_boundary=0, config_id=122)
    say("decode step at the block limit", ctx, "fused" if expect_fused else "two launches")
    fused_vs_separate(spec)


def random_batch1_case(seed):
    rng = np.random.default_rng(9100 + seed)
    G = int(rng.choice([1, 2, 4, 8, 16]))
    hkv = int(rng.choice([1, 2, 4, 8]))
    L = int(rng.choice([int(rng.integers(1, 3000)), int(rng.integers(3000, 131000))]))
    spec = synth.custom(f"b1random{seed}", batch=1, n_q_heads=G * hkv, n_kv_heads=hkv,
                        context=(L,), steps=2,
                        init_tokens=int(rng.choice([0, 128, 256, 1000, 1024])),
                        local_tokens=int(rng.choice([0, 1, 128, 1000, 7192])),
                        topk_ppm=int(rng.choice([0, 1, 50_000, 200_000, 999_999,
                                                 1_000_000])),
                        dense_boundary=int(rng.choice([0, 0, 5000, 32768])),
                        shuffle=bool(rng.integers(0, 2)), config_id=500 + seed)
    launch = dict(split_waves=int(rng.choice([0, 0, 7, 64, 512, 1000])))
    return spec, launch


SINGLE_SEQUENCE_CASES = int(os.environ.get("RKV_SINGLE_SEQUENCE_CASES", "12"))


@pytest.mark.parametrize("seed", range(SINGLE_SEQUENCE_CASES))
def test_decode_step_random_single_sequence(seed):
    spec, launch = random_batch1_case(seed)
    say(f"decode step random single sequence {seed}: L {spec.context[0]}, "
        f"{spec.n_q_heads}/{spec.n_kv_heads}, init {spec.init_tokens}, "
        f"local {spec.local_tokens}, ppm {spec.topk_ppm}, "
        f"dense {spec.dense_boundary}, {launch}")
    # the default 12 check seeds 0-3 against the oracle too; a wider sweep
    # (RKV_SINGLE_SEQUENCE_CASES) checks every seed past 11 against it
    fused_vs_separate(spec, launch, oracle_check=seed < 4 or seed >= 12)


def test_decode_step_batch_and_valu_take_the_two_launch_path():
    spec = synth.custom("b3", batch=3, n_q_heads=16, n_kv_heads=4,
                        context=(767, 9000, 20480), steps=2, init_tokens=256,
                        local_tokens=1000, dense_boundary=0, config_id=123)
    say("decode step, batch of three and VALU")
    fused_vs_separate(spec)
    spec1 = synth.custom("b1valu", batch=1, n_q_heads=16, n_kv_heads=4,
                         context=(20000,), steps=2, dense_boundary=0, config_id=124)
    fused_vs_separate(spec1, dict(attn_impl=B.ATTN_VALU))
    fused_vs_separate(spec1, dict(select_mode=B.SELECT_PER_SEQUENCE))


def test_select_attend_from_the_select_workspace():
    """rkv_select_attend over the scores a selection left in its workspace
    repeats that selection and attention bit for bit."""
    for spec in (synth.custom("sa1", batch=1, n_q_heads=32, n_kv_heads=8,
                              context=(50000,), steps=1, dense_boundary=0,
                              config_id=125),
                 synth.custom("sa2", batch=2, n_q_heads=32, n_kv_heads=8,
                              context=(50000, 20000), steps=1, dense_boundary=0,
                              config_id=126)):
        say("select_attend from the workspace", spec.name)
        batch = synth.make_batch(spec, DEV)
        prm, sess = make_session(batch)
        prefill(batch, sess)
        lens = i32(batch.lens_at(0))
        kn, vn = batch.new_kv_bits(0)
        q = batch.q_bits(0)
        sess.step_separate(q, kn, vn, lens)
        torch.cuda.synchronize()
        ref = _snapshot(sess)
        sess.out.zero_()
        sess.merged.zero_()
        sess.sel_ids.zero_()
        sess.select_attend(q, lens)
        torch.cuda.synchronize()
        got = _snapshot(sess)
        assert np.array_equal(got[0], ref[0])
        assert got[3] == ref[3] and got[4] == ref[4]


@pytest.mark.parametrize("ctx", [72727, 72728, 72856, 72857])
def test_decode_step_search_register_edge(ctx):
    """The folded search runs over 8 registers while the offload range ends
    at or before block 512 and over 16 past it: contexts around that edge
    (local 7192 tokens: the offload range ends at block 512 for
    L in [72728, 72855])."""
    spec = synth.custom(f"edge{ctx}", batch=1, n_q_heads=32, n_kv_heads=8,
                        context=(ctx,), steps=2, dense_boundary=0,
                        config_id=130 + ctx % 97)
    say("decode step at the 8/16-register edge", ctx)
    fused_vs_separate(spec, oracle_check=ctx in (72728, 72857))
