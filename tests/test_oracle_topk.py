"""Pins for the oracle's top-K selection.

Definition (SemiAnalysis GLM-5.3 article, "Lightning Indexer"): keep the K
highest-scoring visible tokens; a query that sees fewer than K tokens keeps
them all.  Tie rule (reading): equal scores go to the lower token index.
Pins: brute-force selection by repeated arg-max (a different algorithm from
the oracle's sort), the defining dominance property, forced ties, and the
boundary lengths n in {K-1, K, K+1}.
"""
import numpy as np
import pytest


def _argmax_select(scores, k):
    """Pick the best remaining token k times: max score, lowest index on ties."""
    remaining = list(range(len(scores)))
    out = []
    for _ in range(min(k, len(scores))):
        best = remaining[0]
        for s in remaining[1:]:
            if scores[s] > scores[best]:
                best = s
        out.append(best)
        remaining.remove(best)
    return out


@pytest.mark.parametrize("seed", range(6))
def test_matches_bruteforce(orc, seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 60))
    k = int(rng.integers(1, 40))
    # few distinct values so ties are common
    scores = rng.integers(-3, 4, size=n).astype(np.float64) * 0.25
    got = orc.topk(scores, k)
    assert got.tolist() == _argmax_select(scores.tolist(), k)


@pytest.mark.parametrize("n,k", [(15, 16), (16, 16), (17, 16), (1, 1), (1, 5), (64, 63), (65, 64)])
def test_boundary_lengths(orc, n, k):
    rng = np.random.default_rng(n * 100 + k)
    scores = rng.standard_normal(n)
    got = orc.topk(scores, k)
    assert len(got) == min(n, k)
    assert len(set(got.tolist())) == len(got)
    if n <= k:
        assert got.tolist() == list(range(n))
    sel = set(got.tolist())
    worst_sel = min((scores[s], -s) for s in sel)
    rest = [(scores[s], -s) for s in range(n) if s not in sel]
    assert all(r < worst_sel for r in rest)


def test_all_equal_scores_take_lowest_indices(orc):
    got = orc.topk(np.full(1000, 0.125), 37)
    assert sorted(got.tolist()) == list(range(37))


def test_duplicate_scores(orc):
    scores = np.array([1.0, 5.0, 2.0, 5.0, 2.0, 2.0, 0.0])
    assert sorted(orc.topk(scores, 3).tolist()) == [1, 2, 3]
    assert sorted(orc.topk(scores, 4).tolist()) == [1, 2, 3, 4]


def test_query_positions_hand_worked():
    """The causal visibility reading against hand-worked rows (request,
    position, visible count), requests with no query rows included."""
    import json
    import os
    import types

    import numpy as np

    import oracle
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "positions_hand.json")
    for case in json.load(open(path))["cases"]:
        ql = np.asarray(case["q_lens"], dtype=np.int32)
        qsl = np.concatenate([[0], np.cumsum(ql)]).astype(np.int32)
        wl = types.SimpleNamespace(context_lens=np.asarray(case["context_lens"], dtype=np.int32), q_lens=ql,
                                   query_start_loc=qsl)
        want = [tuple(r) for r in case["rows"]]
        assert oracle.query_positions(wl) == want
        assert [oracle.row_position(wl, t) for t in range(len(want))] == want
