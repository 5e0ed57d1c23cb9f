"""Host-side counts that bench.py reports (visible pairs per row, per
(query block, key block) pair, and the tiles the partial kernel executes),
checked by brute force on small random packed trees: a dense boolean
visibility matrix built from the tree's definition ("Context Parallelism in
ART", sections 01-02: a packed token sees its own segment up to itself and
every token of every strict ancestor segment)."""
import numpy as np
import pytest

import bench


def _random_preorder_tree(rng, n_seg, min_len, max_len):
    """Random rooted forest emitted in DFS preorder; returns (seg, parent)."""
    par = [-1]
    for s in range(1, n_seg):
        par.append(int(rng.integers(-1, s)))          # any earlier node, or a new root
    kids = {s: [] for s in range(-1, n_seg)}
    for s, p in enumerate(par):
        kids[p].append(s)
    order, stack = [], list(reversed(kids[-1]))
    while stack:
        s = stack.pop()
        order.append(s)
        stack.extend(reversed(kids[s]))
    new = {s: i for i, s in enumerate(order)}
    parent = np.array([-1 if par[s] < 0 else new[par[s]] for s in order], dtype=np.int64)
    lens = rng.integers(min_len, max_len + 1, size=n_seg)
    seg = np.repeat(np.arange(n_seg), lens)
    return seg, parent


def _dense_visible(seg, parent):
    n = len(seg)
    anc = [set() for _ in range(len(parent))]
    for s, p in enumerate(parent):
        if p >= 0:
            anc[s] = anc[p] | {p}
    vis = np.zeros((n, n), dtype=bool)
    for y in range(n):
        for x in range(n):
            vis[y, x] = (seg[x] == seg[y] and x <= y) or seg[x] in anc[seg[y]]
    return vis


@pytest.mark.parametrize("seed", range(4))
def test_counts_match_brute_force(seed):
    rng = np.random.default_rng(seed)
    seg, parent = _random_preorder_tree(rng, int(rng.integers(3, 9)), 5, 60)
    n = len(seg)
    bm, bn, N = 16, 8, 4
    c = -(-n // (N * bm)) * bm                       # block size, a multiple of both tiles
    pad = N * c - n                                  # trailing rows: one more root segment
    seg = np.r_[seg, np.full(pad, len(parent))]
    parent = np.r_[parent, -1]
    n = len(seg)
    vis = _dense_visible(seg, parent)
    assert np.array_equal(bench.tree_visible_pairs(seg, parent, np.arange(n)), vis.sum(axis=1))
    blocks = vis.reshape(N, c, N, c).sum(axis=(1, 3))
    assert np.array_equal(bench.block_pair_counts(seg, parent, c, N), blocks)
    tiles = vis.reshape(n // bm, bm, n // bn, bn).any(axis=(1, 3)).sum()
    assert bench.computed_tiles(seg, parent, c, bm=bm, bn=bn) == tiles


def test_tree64k_counts():
    """The 64K row: closed-form visible pairs, and the executed-tile count
    (prompt 24576 + five 8192 completions, 256 x 64 tiles: a completion's
    query tile t sees the 384 prompt tiles and its own first 4(t+1), the
    prompt's query tile t its first 4(t+1))."""
    import workloads
    seg, parent = workloads.tree_prompt_completions()
    P, C = 24576, 8192
    tp, tc = P // 256, C // 256
    expect = sum(4 * (t + 1) for t in range(tp)) + 5 * sum(P // 64 + 4 * (t + 1) for t in range(tc))
    assert bench.computed_tiles(seg, parent, 16384) == expect
    A = int(bench.tree_visible_pairs(seg, parent, np.arange(len(seg))).sum())
    assert A == 1476427776
