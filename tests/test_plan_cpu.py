"""Per-rank work report of a ring (cpattn_ring_plan), host only: checked
against the tables the pages print for small causal rings.

* ML-systems lesson (sequence/context parallelism), worked example (c): N = 4
  ranks, 8 causal tokens; contiguous blocks give 3, 7, 11, 15 pairs per rank
  and a ring time of 15 pair-times (round maxima 3, 4, 4, 4); the zig-zag
  layout gives 9 per rank, round maxima 3, 2, 2, 2 (ring time 9), and the
  golden file lists every pair of every (round, rank).
* "Context Parallelism in ART", section 05: eight causal tokens on two ranks,
  contiguous halves 10 / 26, folded (first and last quarter vs the middle)
  18 / 18.
"""
import json
import os

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


@pytest.fixture(scope="module")
def cp():
    from context_blockwise_attention_amd import build as b
    if not b.up_to_date():
        b.build()
    import context_blockwise_attention_amd as cpattn
    cpattn.lib()
    return cpattn


def _zigzag_chunks(n, N):
    c = n // (2 * N)
    pos, sizes = [], []
    for r in range(N):
        for chunk in (r, 2 * N - 1 - r):
            pos.append((chunk * c, 1))
            sizes.append(c)
    return sizes, pos


def test_contiguous_ring_table(cp):
    g = json.load(open(os.path.join(GOLDEN, "causal_ring_n4_s8.json")))["contiguous"]
    m = cp.Mask.causal(8)
    w = cp.ring_plan([2] * 4, [(2 * r, 1) for r in range(4)], m)
    assert w.sum(axis=1).tolist() == g["per_rank"]
    assert w.max(axis=0).tolist() == g["round_max"]
    assert int(w.max(axis=0).sum()) == g["ring_time"]


def test_zigzag_ring_table(cp):
    g = json.load(open(os.path.join(GOLDEN, "causal_ring_n4_s8.json")))["zigzag"]
    m = cp.Mask.causal(8)
    sizes, pos = _zigzag_chunks(8, 4)
    w = cp.ring_plan(sizes, pos, m, chunks_per_rank=2)
    # every (round, rank) count equals the number of pairs the page lists
    for k in range(4):
        for r in range(4):
            assert w[r, k] == len(g["pairs"][k][r])
    assert w.sum(axis=1).tolist() == g["per_rank"]
    assert w.max(axis=0).tolist() == g["round_max"]
    assert int(w.max(axis=0).sum()) == g["ring_time"]


def test_fold_example(cp):
    g = json.load(open(os.path.join(GOLDEN, "fold_8_tokens.json")))
    m = cp.Mask.causal(8)
    w = cp.ring_plan([4, 4], [(0, 1), (4, 1)], m)
    assert w.sum(axis=1).tolist() == g["two_rank_contiguous"]
    sizes, pos = _zigzag_chunks(8, 2)
    w = cp.ring_plan(sizes, pos, m, chunks_per_rank=2)
    assert w.sum(axis=1).tolist() == g["fold_first_last_vs_middle"]


@pytest.mark.parametrize("N", [2, 4, 8])
def test_causal_totals_and_balance(cp, N):
    """Any layout covers the s(s+1)/2 causal pairs; zig-zag ranks differ by
    at most the chunk imbalance, contiguous ranks grow linearly."""
    s = 4096
    m = cp.Mask.causal(s)
    c = s // N
    w = cp.ring_plan([c] * N, [(r * c, 1) for r in range(N)], m)
    assert int(w.sum()) == s * (s + 1) // 2
    per = w.sum(axis=1)
    assert np.all(np.diff(per) == c * c)           # rank r: c(c+1)/2 + r c^2
    sizes, pos = _zigzag_chunks(s, N)
    wz = cp.ring_plan(sizes, pos, m, chunks_per_rank=2)
    assert int(wz.sum()) == s * (s + 1) // 2
    assert len(set(wz.sum(axis=1).tolist())) == 1   # every rank the same work


def test_striped_rank0_closed_form(cp):
    n, P = 64, 4
    m = cp.Mask.causal(n * P)
    w = cp.ring_plan([n] * P, [(r, P) for r in range(P)], m)
    assert int(w[0].sum()) == n * (n + 1) // 2 + (P - 1) * n * (n - 1) // 2


def test_plan_rejects_bad_arguments(cp):
    m = cp.Mask.causal(16)
    with pytest.raises(cp.CpattnError) as e:
        cp.ring_plan([8, 8], [(0, 1), (10, 1)], m)      # positions past the mask
    assert e.value.code == cp.EINVAL
    with pytest.raises(cp.CpattnError) as e:
        cp.ring_plan([-1, 8], [(0, 1), (8, 1)], m)
    assert e.value.code == cp.EINVAL


@pytest.mark.parametrize("window", [1, 5, 23])
@pytest.mark.parametrize("C", [1, 2])
def test_plan_with_causal_window(cp, window, C):
    """Sliding window on a causal sequence ("Context Parallelism in ART",
    section 06): the plan counts only pairs with y - window < x <= y."""
    s, N = 64, 4
    m = cp.Mask.causal(s).with_window(window)
    c = s // (N * C)
    chunks = list(range(N)) if C == 1 else [ch for r in range(N) for ch in (r, 2 * N - 1 - r)]
    w = cp.ring_plan([c] * (N * C), [(ch * c, 1) for ch in chunks], m, chunks_per_rank=C)
    y, x = np.meshgrid(np.arange(s), np.arange(s), indexing="ij")
    vis = (x <= y) & (y - x < window)
    for r in range(N):
        for kk in range(N):
            b = (r - kk) % N
            qs = np.concatenate([np.arange(ch * c, (ch + 1) * c) for ch in chunks[r * C:(r + 1) * C]])
            ks = np.concatenate([np.arange(ch * c, (ch + 1) * c) for ch in chunks[b * C:(b + 1) * C]])
            assert w[r, kk] == int(vis[np.ix_(qs, ks)].sum())
    assert int(w.sum()) == int(vis.sum())


def test_window_rejects_bad_arguments(cp):
    m = cp.Mask.causal(16)
    for bad in (0, -3, (1 << 30) + 1):
        with pytest.raises(cp.CpattnError) as e:
            m.with_window(bad)
        assert e.value.code == cp.EINVAL
