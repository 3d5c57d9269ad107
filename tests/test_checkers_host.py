"""The GPU parity checkers themselves, on the CPU: selections and merged
tables with planted mistakes (an id outside the offload range, a repeat, a
wrong count, a dropped or extra init / window block, a wrong page id, an
invalid near-tie set) must be rejected, and valid ones (the oracle's own, or
another valid top-k at a near tie) accepted.  The lists under test are built
from the oracle's results; nothing here runs the library."""

from types import SimpleNamespace

import numpy as np
import pytest
import torch

import oracle as O
from tests.helpers import GAP, check_merged, check_selection


def head_result(scores, k, n_init=2, n_off=None):
    s = np.asarray(scores, dtype=np.float64)
    n_off = len(s) if n_off is None else n_off
    sel = O.top_k(s, k) + n_init
    return O.HeadResult(sel, None, s, k, O.selection_gap(s, k), False)


def test_selection_checker_accepts_the_oracle_and_rejects_mistakes():
    rng = np.random.default_rng(1)
    s = rng.standard_normal(40)
    hr = head_result(s, 8)
    assert hr.gap_rel > GAP
    check_selection(hr.selected.copy(), hr, 2, "ok")
    bad = {
        "below init": np.r_[1, hr.selected[1:]],
        "past offload": np.r_[hr.selected[:-1], 42],
        "repeat": np.r_[hr.selected[:-1], hr.selected[-2]],
        "too few": hr.selected[:-1],
        "too many": np.sort(np.r_[hr.selected, 41 if 41 not in hr.selected else 2]),
        "one swapped": np.sort(np.r_[hr.selected[:-1],
                                     [j for j in range(2, 42) if j not in hr.selected][0]]),
    }
    for name, sel in bad.items():
        with pytest.raises(AssertionError):
            check_selection(np.asarray(sel), hr, 2, name)


def test_selection_checker_near_ties():
    # scores 9 > 5 > 5(1 - 1e-4) > 0 ...: k = 2 is a near tie between blocks
    # 3 and 4 (offload positions 1 and 2)
    s = np.array([9.0, 5.0, 5.0 * (1 - 1e-4), 0.0, -1.0, -2.0])
    hr = head_result(s, 2)
    assert hr.gap_rel <= GAP
    check_selection(np.array([2, 3]), hr, 2, "oracle set")
    check_selection(np.array([2, 4]), hr, 2, "other valid set")
    for name, sel in {"dropped best": [3, 4], "low block": [2, 5],
                      "below init": [1, 2], "wrap-around id": [-4, 2],
                      "repeat": [2, 2], "count": [2]}.items():
        with pytest.raises(AssertionError):
            check_selection(np.array(sel), hr, 2, name)


def fake_session(merged_rows):
    n = max(len(r) for r in merged_rows)
    m = torch.full((1, len(merged_rows), n), -9, dtype=torch.int32)
    nm = torch.zeros((1, len(merged_rows)), dtype=torch.int32)
    for h, r in enumerate(merged_rows):
        m[0, h, :len(r)] = torch.as_tensor(np.asarray(r, dtype=np.int32))
        nm[0, h] = len(r)
    return SimpleNamespace(merged=m, n_merged=nm)


def test_merged_checker_rejects_dropped_extra_and_wrong_pages():
    L = 20 * 128 + 5
    reg = O.block_regions(L, 256, 600)           # init 2, local from block 15
    assert (reg.n_init, reg.local_start, reg.nb) == (2, 15, 21)
    table = np.random.default_rng(3).permutation(100)[:21].astype(np.int32)
    batch = SimpleNamespace(table_np=table[None, :])
    sel = np.array([4, 7, 11])
    good = O.merged_blocks(reg, sel)
    sess = fake_session([table[good]])
    assert np.array_equal(check_merged(sess, batch, 0, 0, reg, sel, None, "ok"), good)
    mistakes = {
        "dropped init": table[good[1:]],
        "dropped window": table[good[:-2]],
        "duplicated window": table[np.r_[good, good[-1]]],
        "extra block": table[np.sort(np.r_[good, 9])],
        "other selection": table[O.merged_blocks(reg, np.array([4, 7, 12]))],
        "wrong page": np.r_[table[good[:-1]], 99],
    }
    for name, pages in mistakes.items():
        with pytest.raises(AssertionError):
            check_merged(fake_session([pages]), batch, 0, 0, reg, sel, None, name)
