"""Pins of the oracle's token permutation (dispatch by expert).

The pages ask for tokens to be regrouped by expert with scatter/gather
("MoE架构揭秘", section 4.1, the comment on the per-slot loop) and describe a
router output packed with token ids ("GPT-4 Has 1.8 Trillion Parameters...",
section 4.2, routing optimisation).  The layout is this build's: rows ordered
by (expert asc, token asc), shared expert s of token t at row T*k + s*T + t.
"""
import numpy as np
import pytest

import oracle
from workloads import LayerShape


def shape(**kw):
    base = dict(name="p", T=1, H=8, E=4, S=0, k=2, I=8)
    base.update(kw)
    return LayerShape(**base)


def test_hand_example():
    cfg = shape(E=4, k=2, S=1)
    idx = np.array([[2, 0], [0, 3], [2, -1]], np.int32)
    counts, offsets, row_token, slot_row = oracle.permute(cfg, idx)
    assert counts.tolist() == [2, 0, 2, 1]
    assert offsets.tolist() == [0, 2, 2, 4, 5]
    assert row_token.tolist() == [0, 1, 0, 2, 1, -1, 0, 1, 2]
    assert slot_row.tolist() == [[2, 0], [1, 4], [3, -1]]


@pytest.mark.parametrize("T,E,k,S,drop", [(1, 8, 2, 0, 0.0), (257, 16, 4, 1, 0.1), (1000, 256, 8, 2, 0.02),
                                          (64, 3, 3, 0, 0.5)])
def test_invariants(T, E, k, S, drop):
    rng = np.random.default_rng(T + E)
    cfg = shape(T=T, E=E, k=k, S=S)
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    idx[rng.random((T, k)) < drop] = -1
    counts, offsets, row_token, slot_row = oracle.permute(cfg, idx)
    valid = idx >= 0
    # counts are the histogram, offsets its exclusive prefix sum
    assert np.array_equal(counts, np.bincount(idx[valid], minlength=E))
    assert np.array_equal(offsets, np.concatenate([[0], np.cumsum(counts)]))
    # every assigned (token, slot) owns exactly one row, inside its expert's segment
    rows = slot_row[valid]
    assert len(set(rows.tolist())) == rows.size == offsets[-1]
    assert np.all(slot_row[~valid] == -1)
    tt, jj = np.nonzero(valid)
    for t, j in zip(tt, jj):
        r = slot_row[t, j]
        e = idx[t, j]
        assert offsets[e] <= r < offsets[e + 1] and row_token[r] == t
    # tokens ascend inside each segment
    for e in range(E):
        seg = row_token[offsets[e]:offsets[e + 1]]
        assert np.all(np.diff(seg) > 0)
    # unused routed rows are -1 and shared rows are identity per shared expert
    assert np.all(row_token[offsets[-1]:T * k] == -1)
    for s in range(S):
        assert np.array_equal(row_token[T * k + s * T:T * k + (s + 1) * T], np.arange(T))


def test_rejects_out_of_range_index():
    cfg = shape(E=4, k=1)
    with pytest.raises(ValueError):
        oracle.permute(cfg, np.array([[4]], np.int32))
