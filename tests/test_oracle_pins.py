"""Pins of the float64 CPU oracle against facts fixed outside itself.

Each test ties one oracle function to something independent of its code:
the hand-worked region table (tests/golden/regions.txt), token-level brute
force, exact rational arithmetic, brute force over all k-subsets, plain-loop
attention, torch's own scaled_dot_product_attention, closed forms, and the
invariants the method must satisfy (page permutation, shared pages, planted
blocks).  No test here needs a GPU.
"""

import itertools
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as O
from sparse_retrieval_kv_amd import synth


def _golden_rows(golden_dir):
    rows = []
    with open(os.path.join(golden_dir, "regions.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if not line:
                continue
            lhs, rhs = line.split("|")
            rows.append((tuple(int(x) for x in lhs.split()),
                         tuple(int(x) for x in rhs.split())))
    return rows


def test_regions_and_k_match_hand_worked_table(golden_dir):
    rows = _golden_rows(golden_dir)
    assert len(rows) >= 15
    for (L, init, local, ppm), (nb, n_init, ls, n_off, k) in rows:
        r = O.block_regions(L, init, local)
        assert (r.nb, r.n_init, r.local_start, r.n_off) == (nb, n_init, ls, n_off), L
        assert O.topk_count(r.n_off, ppm) == k, (L, ppm)


def _brute_regions(L, init, local, block=128):
    """Block roles from token positions: a block is init if it holds a token
    below ``init``; local if it holds a token in the last ``local`` positions
    or is the last block; offload otherwise."""
    nb = -(-L // block)
    roles = []
    for j in range(nb):
        toks = range(j * block, min((j + 1) * block, L))
        is_init = any(t < init for t in toks)
        is_local = any(t >= L - local for t in toks) or j == nb - 1
        roles.append("init" if is_init else ("local" if is_local else "off"))
    return roles


def test_regions_match_token_level_brute_force():
    rng = np.random.default_rng(7)
    cases = [(int(rng.integers(1, 6000)), int(rng.integers(0, 1500)),
              int(rng.integers(0, 3000))) for _ in range(400)]
    cases += [(L, i, l) for L in (1, 127, 128, 129, 255, 256, 257)
              for i in (0, 1, 128, 129) for l in (0, 1, 127, 128, 129)]
    for L, init, local in cases:
        roles = _brute_regions(L, init, local)
        r = O.block_regions(L, init, local)
        assert r.nb == len(roles)
        assert [j for j, x in enumerate(roles) if x == "init"] == list(range(r.n_init))
        assert [j for j, x in enumerate(roles) if x == "off"] == \
            list(range(r.n_init, r.n_init + r.n_off)), (L, init, local)
        local_blocks = [j for j, x in enumerate(roles) if x == "local"]
        assert local_blocks == list(range(max(r.local_start, r.n_init), r.nb))
        merged = O.merged_blocks(r, np.zeros(0, dtype=np.int64))
        assert list(merged) == [j for j, x in enumerate(roles) if x != "off"]


def test_topk_count_is_exact_ceiling():
    for n in list(range(0, 3000, 7)) + [447, 959, 1983, 8191]:
        for ppm in (0, 1, 70_000, 199_999, 200_000, 333_333, 999_999, 1_000_000):
            want = math.ceil(Fraction(n * ppm, 1_000_000))
            assert O.topk_count(n, ppm) == want
    # the ratio is a fraction of the offload blocks: k >= 1 once n >= 1
    assert all(O.topk_count(n, 1) == 1 for n in range(1, 100))


def test_dense_switch_comparator():
    assert O.is_dense(32767, 32768, 200_000)
    assert not O.is_dense(32768, 32768, 200_000)
    assert not O.is_dense(4096, 0, 200_000)
    assert O.is_dense(10**6, 32768, 1_000_000)


def test_top_k_equals_subset_brute_force():
    rng = np.random.default_rng(11)
    for trial in range(300):
        n = int(rng.integers(1, 8))
        s = rng.integers(-3, 4, size=n).astype(np.float64)  # many ties
        if trial % 3 == 0:
            s = rng.standard_normal(n)
        for k in range(0, n + 1):
            valid = []
            for sub in itertools.combinations(range(n), k):
                rest = [j for j in range(n) if j not in sub]
                if not sub or not rest or min(s[list(sub)]) >= max(s[rest]):
                    valid.append(sub)
            want = min(valid)  # ties resolved toward the smaller index
            got = tuple(int(x) for x in O.top_k(s, k))
            assert got == want, (s, k, got, want)


def test_selection_gap_examples():
    s = np.array([5.0, 1.0, 4.0, 2.0])
    assert O.selection_gap(s, 2) == pytest.approx((4.0 - 2.0) / 4.0)
    assert O.selection_gap(s, 0) == float("inf")
    assert O.selection_gap(s, 4) == float("inf")
    assert O.selection_gap(np.array([1.0, 1.0]), 1) == 0.0


def test_ip_scores_sum_over_group_brute_force():
    rng = np.random.default_rng(3)
    q = rng.standard_normal((4, 9))
    reps = rng.standard_normal((6, 9))
    got = O.ip_scores(q, reps)
    for j in range(6):
        want = math.fsum(q[g, d] * reps[j, d] for g in range(4) for d in range(9))
        assert got[j] == pytest.approx(want, rel=1e-12, abs=1e-12)


def test_block_reps_brute_force_and_closed_form():
    rng = np.random.default_rng(5)
    L = 3 * 128 + 50
    K = rng.standard_normal((L, 4))
    reps = O.block_reps(K)
    assert reps.shape == (3, 4)  # the partial block gets no representation
    for j in range(3):
        for d in range(4):
            want = math.fsum(K[j * 128 + t, d] for t in range(128)) / 128
            assert reps[j, d] == pytest.approx(want, rel=1e-13, abs=1e-15)
    Kc = np.tile(np.array([0.75, -2.0, 3.5, 0.0]), (256, 1))
    assert np.array_equal(O.block_reps(Kc), np.tile(Kc[0], (2, 1)))


def _loop_attention(q_rows, K, V, scale):
    out = []
    for q in q_rows:
        z = [scale * sum(q[d] * k[d] for d in range(len(q))) for k in K]
        m = max(z)
        w = [math.exp(x - m) for x in z]
        tot = math.fsum(w)
        out.append([math.fsum(w[t] * V[t][d] for t in range(len(K))) / tot
                    for d in range(len(V[0]))])
    return np.array(out)


def test_attend_equals_plain_loop():
    rng = np.random.default_rng(9)
    for T in (1, 2, 37):
        q = rng.standard_normal((3, 16))
        K = rng.standard_normal((T, 16)) * 3
        V = rng.standard_normal((T, 16))
        got = O.attend(q, K, V, 0.25)
        want = _loop_attention(q.tolist(), K.tolist(), V.tolist(), 0.25)
        np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-13)


def test_attend_equals_torch_sdpa():
    rng = np.random.default_rng(10)
    q = rng.standard_normal((4, 128))
    K = rng.standard_normal((700, 128))
    V = rng.standard_normal((700, 128))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None, None], torch.from_numpy(K)[None, None],
        torch.from_numpy(V)[None, None])[0, 0].numpy()
    np.testing.assert_allclose(O.attend(q, K, V, 1 / math.sqrt(128)), ref,
                               rtol=1e-11, atol=1e-12)


def test_attend_closed_forms():
    rng = np.random.default_rng(12)
    q = rng.standard_normal((2, 8))
    K = rng.standard_normal((50, 8))
    c = rng.standard_normal(8)
    Vc = np.tile(c, (50, 1))
    np.testing.assert_allclose(O.attend(q, K, Vc, 0.3), np.tile(c, (2, 1)),
                               rtol=1e-13, atol=1e-14)
    V = rng.standard_normal((50, 8))
    Keq = np.tile(rng.standard_normal(8), (50, 1))
    np.testing.assert_allclose(O.attend(q, Keq, V, 0.3),
                               np.tile(V.mean(axis=0), (2, 1)), rtol=1e-12)
    np.testing.assert_allclose(O.attend(np.zeros((2, 8)), K, V, 0.3),
                               np.tile(V.mean(axis=0), (2, 1)), rtol=1e-12)
    assert np.array_equal(O.attend(q, K[:0], V[:0], 0.3), np.zeros((2, 8)))


# ---------------------------------------------------------------------------
# Whole-step invariants on paged inputs.
# ---------------------------------------------------------------------------

def _scatter_pages(K, V, table_row, n_pages, block=128):
    """Write logical [Hkv, L, d] bf16 bits into pools with an explicit loop
    over tokens: K page slice [token][dim], V page slice [dim][token]."""
    hkv, L, d = K.shape
    kp = np.zeros((n_pages, hkv, block, d), dtype=np.uint16)
    vp = np.zeros((n_pages, hkv, d, block), dtype=np.uint16)
    for t in range(L):
        page, slot = table_row[t // block], t % block
        kp[page, :, slot, :] = K[:, t, :]
        vp[page, :, :, slot] = V[:, t, :]
    return kp, vp


def _bits(x):
    return synth.to_bf16_bits(torch.from_numpy(x.astype(np.float32))).numpy() \
        .view(np.uint16)


def _random_seq(rng, hkv, L):
    return (_bits(rng.standard_normal((hkv, L, 128))),
            _bits(rng.standard_normal((hkv, L, 128))))


def test_logical_kv_round_trip_and_bf16_decode():
    rng = np.random.default_rng(21)
    L = 128 * 5 + 17
    Kb, Vb = _random_seq(rng, 2, L)
    table = rng.permutation(9)[:6]
    kp, vp = _scatter_pages(Kb, Vb, table, 9)
    K, V = O.logical_kv(kp, vp, table, L)
    assert np.array_equal(K, O.bf16_to_f64(Kb))
    assert np.array_equal(V, O.bf16_to_f64(Vb))
    # bf16 decoding: a few exact values
    bits = np.array([0x3F80, 0xBF80, 0x4049, 0x0000, 0x8000, 0x7F80], np.uint16)
    vals = O.bf16_to_f64(bits)
    assert list(vals[:5]) == [1.0, -1.0, 3.140625, 0.0, -0.0]
    assert math.isinf(vals[5])


def _step_from_pages(kp, vp, table, L, q, prm, prompt_len=None):
    K, V = O.logical_kv(kp, vp, table, L)
    return O.decode_step(q, K, V, L, prompt_len if prompt_len is not None else L,
                         prm)


def test_page_permutation_invariance():
    rng = np.random.default_rng(22)
    L, hkv, hq = 40 * 128 + 77, 2, 8
    Kb, Vb = _random_seq(rng, hkv, L)
    q = rng.standard_normal((hq, 128))
    prm = O.Params(hq, hkv, init_tokens=256, local_tokens=512, dense_boundary=0)
    nb = -(-L // 128)
    ident = np.arange(nb)
    perm = rng.permutation(nb + 10)[:nb]
    a = _step_from_pages(*_scatter_pages(Kb, Vb, ident, nb), ident, L, q, prm)
    b = _step_from_pages(*_scatter_pages(Kb, Vb, perm, nb + 10), perm, L, q, prm)
    assert np.array_equal(a.out, b.out)
    for ha, hb in zip(a.heads, b.heads):
        assert np.array_equal(ha.selected, hb.selected)


def test_shared_prefix_pages_equal_private_copies():
    rng = np.random.default_rng(23)
    hkv, hq, L = 2, 4, 30 * 128 + 5
    prefix_blocks = 8
    K0, V0 = _random_seq(rng, hkv, L)
    K1, V1 = _random_seq(rng, hkv, L)
    K1[:, :prefix_blocks * 128] = K0[:, :prefix_blocks * 128]
    V1[:, :prefix_blocks * 128] = V0[:, :prefix_blocks * 128]
    nb = -(-L // 128)
    # shared: both tables name the same physical prefix pages
    t0 = np.arange(nb)
    t1 = np.concatenate([np.arange(prefix_blocks), nb + np.arange(nb - prefix_blocks)])
    n_pages = nb + nb - prefix_blocks
    kp = np.zeros((n_pages, hkv, 128, 128), np.uint16)
    vp = np.zeros((n_pages, hkv, 128, 128), np.uint16)
    for K, V, t in ((K0, V0, t0), (K1, V1, t1)):
        a, b = _scatter_pages(K, V, t, n_pages)
        used = np.unique(t)
        kp[used], vp[used] = a[used], b[used]
    q = rng.standard_normal((hq, 128))
    prm = O.Params(hq, hkv, init_tokens=128, local_tokens=1000, dense_boundary=0)
    shared = _step_from_pages(kp, vp, t1, L, q, prm)
    private = _step_from_pages(*_scatter_pages(K1, V1, np.arange(nb), nb),
                               np.arange(nb), L, q, prm)
    assert np.array_equal(shared.out, private.out)


def test_dense_equals_sdpa_over_all_tokens():
    rng = np.random.default_rng(24)
    hkv, hq, L = 2, 8, 20 * 128 + 33
    Kb, Vb = _random_seq(rng, hkv, L)
    K, V = O.bf16_to_f64(Kb), O.bf16_to_f64(Vb)
    q = rng.standard_normal((hq, 128))
    G = hq // hkv
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[:, None, :],
        torch.from_numpy(np.repeat(K, G, axis=0)),
        torch.from_numpy(np.repeat(V, G, axis=0)))[:, 0].numpy()
    base = dict(init_tokens=256, local_tokens=512)
    for prm, plen in ((O.Params(hq, hkv, topk_ppm=1_000_000, dense_boundary=0, **base), L),
                      (O.Params(hq, hkv, dense_boundary=L + 1, **base), L),
                      (O.Params(hq, hkv, dense_boundary=32768, **base), 100)):
        res = O.decode_step(q, K, V, L, plen, prm)
        assert all(h.dense for h in res.heads)
        np.testing.assert_allclose(res.out, ref, rtol=1e-11, atol=1e-12)
    # the sparse path at the same sizes differs from dense
    sp = O.decode_step(q, K, V, L, L, O.Params(hq, hkv, dense_boundary=0, **base))
    assert not np.allclose(sp.out, ref, rtol=1e-6, atol=1e-8)


def test_zero_query_selects_first_blocks_and_averages():
    rng = np.random.default_rng(25)
    hkv, hq, L = 1, 2, 16 * 128
    Kb, Vb = _random_seq(rng, hkv, L)
    K, V = O.bf16_to_f64(Kb), O.bf16_to_f64(Vb)
    prm = O.Params(hq, hkv, init_tokens=128, local_tokens=256, dense_boundary=0)
    res = O.decode_step(np.zeros((hq, 128)), K, V, L, L, prm)
    h = res.heads[0]
    # all scores tie at 0: the tie rule picks the lowest offload blocks
    assert list(h.selected) == list(range(1, 1 + h.k))
    tok = np.concatenate([np.arange(j * 128, (j + 1) * 128) for j in h.merged])
    np.testing.assert_allclose(res.out, np.tile(V[0, tok].mean(axis=0), (hq, 1)),
                               rtol=1e-12)


def test_attended_set_covers_init_and_window_tokens():
    rng = np.random.default_rng(26)
    for _ in range(50):
        L = int(rng.integers(1, 9000))
        init, local = int(rng.integers(0, 2000)), int(rng.integers(0, 3000))
        reg = O.block_regions(L, init, local)
        merged = O.merged_blocks(reg, np.zeros(0, dtype=np.int64))
        toks = set()
        for j in merged:
            toks.update(range(j * 128, min((j + 1) * 128, L)))
        assert set(range(min(init, L))) <= toks
        assert set(range(max(L - local, 0), L)) <= toks
        assert L - 1 in toks


def _oracle_batch_step(batch, t, **overrides):
    """Oracle result of step t for every sequence of a synth batch."""
    spec = batch.spec
    kw = dict(init_tokens=spec.init_tokens, local_tokens=spec.local_tokens,
              topk_ppm=spec.topk_ppm, dense_boundary=spec.dense_boundary)
    kw.update(overrides)
    prm = O.Params(spec.n_q_heads, spec.n_kv_heads, **kw)
    kp = batch.k_pages.cpu().numpy().view(np.uint16)
    vp = batch.v_pages.cpu().numpy().view(np.uint16)
    q = O.bf16_to_f64(batch.q_bits(t).cpu().numpy().view(np.uint16))
    res = []
    for b in range(spec.batch):
        L = int(batch.context[b]) + t
        K, V = O.logical_kv(kp, vp, batch.table_np[b], L)
        for s in range(t + 1):
            kn, vn = batch.new_kv_bits(s)
            pos = int(batch.context[b]) - 1 + s
            K[:, pos] = O.bf16_to_f64(kn[b].cpu().numpy().view(np.uint16))
            V[:, pos] = O.bf16_to_f64(vn[b].cpu().numpy().view(np.uint16))
        res.append(O.decode_step(q[b], K, V, L, int(batch.context[b]), prm))
    return res


def test_planted_blocks_selected_tiny_config():
    batch = synth.make_batch(synth.CONFIGS[1], "cpu")
    (res,) = _oracle_batch_step(batch, 0)
    assert (res.regions.n_init, res.regions.nb - res.regions.local_start,
            res.regions.n_off) == (2, 4, 26)
    for h in res.heads:
        assert h.k == 6
        assert set(batch.planted[0]) <= set(h.selected.tolist())
        assert not np.isnan(res.out).any()


def test_planting_follows_the_query_group():
    """Blocks planted toward KV group 1's queries are selected for KV head 1;
    a wrong query-head-to-group mapping would not select them."""
    rng = np.random.default_rng(27)
    hkv, hq, L = 2, 8, 32 * 128
    G = hq // hkv
    q = rng.standard_normal((hq, 128))
    K = rng.standard_normal((hkv, L, 128))
    V = rng.standard_normal((hkv, L, 128))
    planted = [5, 17]
    for j in planted:
        K[1, j * 128:(j + 1) * 128] += 0.5 * q[G:2 * G].mean(axis=0)
    prm = O.Params(hq, hkv, init_tokens=256, local_tokens=512, dense_boundary=0)
    res = O.decode_step(q, K, V, L, L, prm)
    assert set(planted) <= set(res.heads[1].selected.tolist())
    s = res.heads[1].scores
    lo = res.regions.n_init
    assert min(s[j - lo] for j in planted) > np.sort(s)[-3]


def test_multistep_planted_selected_llama_layer_scaled():
    """Shared-direction planting (queries (u + z_t)/sqrt 2, planted keys
    N(0,1) + 0.5 u/sqrt 2) keeps planted blocks selected over many steps."""
    spec = synth.scaled(synth.CONFIGS[2], context=(16384,), steps=4,
                        plant_range=(8, 71), plant_count=3, dense_boundary=0)
    batch = synth.make_batch(spec, "cpu")
    for t in (0, 3):
        (res,) = _oracle_batch_step(batch, t)
        for h in res.heads:
            assert set(batch.planted[0]) <= set(h.selected.tolist())


def test_synth_shared_prefix_refcounts_and_layout():
    spec = synth.scaled(synth.CONFIGS[4], batch=3, context=(2048,) * 3, steps=2,
                        shared_prefix_pages=4)
    batch = synth.make_batch(spec, "cpu")
    t = batch.table_np
    assert (t[:, :4] == t[0, :4]).all()
    assert (batch.refcount[t[0, :4]] == 3).all()
    private = t[:, 4:17].reshape(-1)
    assert len(np.unique(private)) == private.size
    assert (batch.refcount[private] == 1).all()
    # first decode slot onward is poisoned with NaN until appended
    kp = batch.k_pages.numpy().view(np.uint16)
    last = t[0, 2047 // 128]
    assert (kp[last, :, 2047 % 128:, :] == synth.BF16_QNAN).all()
    assert (kp[last, :, :2047 % 128, :] != synth.BF16_QNAN).all()


def test_attend_rows_independent_at_extreme_scales():
    """Each query row is normalised on its own: a zero row next to a row with
    huge logits still gives the plain mean of V (no shared shift)."""
    rng = np.random.default_rng(28)
    K = rng.standard_normal((64, 16))
    V = rng.standard_normal((64, 16))
    q = np.stack([np.zeros(16), 1e4 * rng.standard_normal(16)])
    out = O.attend(q, K, V, 1.0)
    np.testing.assert_allclose(out[0], V.mean(axis=0), rtol=1e-12)
    assert np.isfinite(out).all()


# ----------------------------------------------------------------------------
# Per-sequence selection (scores summed over all KV heads, one top-k per
# sequence): the other reading of one record per block.
# ----------------------------------------------------------------------------

def test_per_sequence_selection_brute_force():
    """The per-sequence set maximises the all-heads score of plain loops over
    every k-subset (ties to the smaller block), and every KV head attends it."""
    rng = np.random.default_rng(31)
    hkv, hq, L = 3, 6, 12 * 128
    G = hq // hkv
    prm = O.Params(hq, hkv, init_tokens=128, local_tokens=128, topk_ppm=400_000,
                   dense_boundary=0, per_sequence=True)
    for trial in range(6):
        q = rng.standard_normal((hq, 128))
        K = rng.standard_normal((hkv, L, 128))
        V = rng.standard_normal((hkv, L, 128))
        res = O.decode_step(q, K, V, L, L, prm)
        lo, n = res.regions.n_init, res.regions.n_off
        assert (lo, n) == (1, 10)
        k = res.heads[0].k
        assert k == 4
        # all-heads score of each offload block from plain loops
        tot = []
        for j in range(lo, lo + n):
            terms = []
            for h in range(hkv):
                rep = [math.fsum(K[h, j * 128 + t, d] for t in range(128)) / 128
                       for d in range(128)]
                for g in range(G):
                    terms.extend(q[h * G + g, d] * rep[d] for d in range(128))
            tot.append(math.fsum(terms))
        best = max(itertools.combinations(range(n), k),
                   key=lambda sub: (math.fsum(tot[i] for i in sub),
                                    [-i for i in sub]))
        want = [lo + i for i in best]
        for h in res.heads:
            assert h.selected.tolist() == want
            assert np.array_equal(h.merged, res.heads[0].merged)


def test_per_sequence_equals_per_head_with_one_kv_head():
    rng = np.random.default_rng(32)
    L = 30 * 128 + 5
    q = rng.standard_normal((4, 128))
    K = rng.standard_normal((1, L, 128))
    V = rng.standard_normal((1, L, 128))
    a = O.decode_step(q, K, V, L, L, O.Params(4, 1, init_tokens=256,
                                              local_tokens=512, dense_boundary=0))
    b = O.decode_step(q, K, V, L, L, O.Params(4, 1, init_tokens=256, local_tokens=512,
                                              dense_boundary=0, per_sequence=True))
    assert np.array_equal(a.out, b.out)
    assert np.array_equal(a.heads[0].selected, b.heads[0].selected)


def test_per_sequence_planted_blocks_and_dense_switch():
    """Blocks planted toward one KV group dominate the all-heads sum, so the
    per-sequence set holds them for every head; with ratio 1.0 both readings
    attend every block and agree."""
    batch = synth.make_batch(synth.CONFIGS[1], "cpu")
    (res,) = _oracle_batch_step(batch, 0, per_sequence=True)
    for h in res.heads:
        assert set(batch.planted[0]) <= set(h.selected.tolist())
    (dense_a,) = _oracle_batch_step(batch, 0, topk_ppm=1_000_000)
    (dense_b,) = _oracle_batch_step(batch, 0, topk_ppm=1_000_000, per_sequence=True)
    assert not np.isnan(dense_a.out).any()
    assert np.array_equal(dense_a.out, dense_b.out)
