"""Sliding-window attention on logical (root-to-leaf) positions
("Context Parallelism in ART", section 06), GPU against the fp64 reference
(whose window is pinned to the page's example, trajectory brute force and
banded torch attention), element by element:

* causal partials with windows from 1 to beyond the block, ragged sizes and
  offsets, fp32 and bf16, d 64 and 128; striped positions;
* random packed trees, windows 1 .. 400, bf16 and fp32;
* rings of packed trees (contiguous and zig-zag) with a window;
* the 64K tree row, ring of 4, window 4096: sampled rows, and the plan's
  pair count against the closed form sum_y min(W, lpos(y) + 1);
* the plan on random trees against a dense trajectory count.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from test_gpu_parity import TOL, _cmp, _dev, _preorder_tree

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def cp():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import context_blockwise_attention_amd as cpattn
    cpattn.lib()
    return cpattn


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("window", [1, 37, 300, 5000])
@pytest.mark.parametrize("nq,nk,qbase,kbase", [(300, 300, 0, 0), (257, 190, 190, 0), (200, 333, 150, 100)])
def test_partial_causal_window(cp, dtype, d, window, nq, nk, qbase, kbase):
    H = 2
    q, _, _ = workloads.qkv(21, H, nq, d, dtype)
    _, k, v = workloads.qkv(22, H, nk, d, dtype)
    mask = cp.Mask.causal(max(qbase + nq, kbase + nk)).with_window(window)
    o, l = cp.partial(_dev(q), _dev(k), _dev(v), mask, (qbase, 1), (kbase, 1))
    O, L = oracle.attention(q, k, v, qbase + np.arange(nq), kbase + np.arange(nk), oracle.Causal(window=window))
    _cmp(o, l, O, L, dtype, "causal window %d" % window)


@pytest.mark.parametrize("window", [3, 250])
def test_partial_striped_window(cp, window):
    H, n, d, P = 2, 600, 128, 4
    q, k, v = workloads.qkv(23, H, n * P, d, "bf16")
    lay = workloads.striped(n * P, P)
    mask = cp.Mask.causal(n * P).with_window(window)
    for b in range(P):
        qq, kk, vv = q[:, lay[1]], k[:, lay[b]], v[:, lay[b]]
        o, l = cp.partial(_dev(qq), _dev(kk), _dev(vv), mask, (1, P), (b, P))
        O, L = oracle.attention(qq, kk, vv, lay[1], lay[b], oracle.Causal(window=window))
        _cmp(o, l, O, L, "bf16", "stripe %d window %d" % (b, window))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("seed,window", [(0, 1), (1, 3), (2, 50), (3, 400), (4, 129)])
def test_partial_tree_window(cp, dtype, seed, window):
    rng = np.random.default_rng(30 + seed)
    seg, parent = _preorder_tree(rng, 9, 1, 200)
    n = len(seg)
    H, d = 2, 128
    q, k, v = workloads.qkv(40 + seed, H, n, d, dtype)
    mask = cp.Mask.tree(seg, parent).with_window(window)
    o, l = cp.partial(_dev(q), _dev(k), _dev(v), mask)
    O, L = oracle.attention(q, k, v, np.arange(n), np.arange(n), oracle.Tree(seg, parent, window=window))
    _cmp(o, l, O, L, dtype, "tree seed %d window %d" % (seed, window))


@pytest.mark.parametrize("C", [1, 2])
def test_ring_tree_window(cp, C):
    seg, parent = workloads.tree_prompt_completions(384, (128, 200, 96, 160))
    N = 4
    n = len(seg) // (N * C) * (N * C)
    seg = seg[:n]
    H, d, window = 2, 128, 150
    q, k, v = workloads.qkv(45, H, n, d, "bf16")
    qd, kd, vd = _dev(q), _dev(k), _dev(v)
    mask = cp.Mask.tree(seg, parent).with_window(window)
    c = n // (N * C)
    chunks = list(range(N)) if C == 1 else [ch for r in range(N) for ch in (r, 2 * N - 1 - r)]
    view = lambda t, ch: t[:, ch * c:(ch + 1) * c]
    out = cp.ring_emulate_chunks([view(qd, ch) for ch in chunks], [view(kd, ch) for ch in chunks],
                                 [view(vd, ch) for ch in chunks], [(ch * c, 1) for ch in chunks], mask,
                                 chunks_per_rank=C)
    O, L = oracle.attention(q, k, v, np.arange(n), np.arange(n), oracle.Tree(seg, parent, window=window))
    for i, ch in enumerate(chunks):
        sl = slice(ch * c, (ch + 1) * c)
        _cmp(out[i][0], out[i][1], O[:, sl], L[:, sl], "bf16", "chunk %d" % ch)


def _logical_positions(seg, parent):
    lens = np.bincount(seg, minlength=len(parent))
    anc = np.zeros(len(parent), dtype=np.int64)
    for s in range(len(parent)):
        p = parent[s]
        anc[s] = 0 if p < 0 else anc[p] + lens[p]
    first = np.flatnonzero(np.r_[True, seg[1:] != seg[:-1]])
    start = np.zeros(len(parent), dtype=np.int64)
    start[seg[first]] = first
    x = np.arange(len(seg))
    return anc[seg] + x - start[seg]


def test_tree64k_ring_window(cp):
    H, d, N, window = 32, 128, 4, 4096
    seg, parent = workloads.tree_prompt_completions(24576, (8192,) * 5)
    n = len(seg)
    c = n // N
    print("tree64k window: generating inputs", flush=True)
    q, k, v = workloads.qkv(0, H, n, d, "bf16")
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    mask = cp.Mask.tree(seg, parent).with_window(window)
    w = cp.ring_plan([c] * N, [(r * c, 1) for r in range(N)], mask)
    lp = _logical_positions(seg, parent)
    assert int(w.sum()) == int(np.minimum(window, lp + 1).sum())
    blk = lambda t: [t[:, r * c:(r + 1) * c] for r in range(N)]
    out = cp.ring_emulate(blk(qd), blk(kd), blk(vd), [(r * c, 1) for r in range(N)], mask)
    O = torch.cat([out[r][0] for r in range(N)], 1)
    L = torch.cat([out[r][1] for r in range(N)], 1)
    torch.cuda.synchronize()
    worst_o = worst_l = 0.0
    allpos = np.arange(n)
    for h in range(H):
        rows = workloads.sample_rows(0, h, n, forced=(0, n - 1, 4095, 4096, 24575, 24576, 24576 + 4095, n - 8192))
        O_ref, L_ref = oracle.attention(q[h:h + 1], k[h:h + 1], v[h:h + 1], allpos, allpos,
                                        oracle.Tree(seg, parent, window=window), rows=rows)
        idx = torch.from_numpy(rows).cuda()
        worst_o = max(worst_o, float(np.abs(O[h].index_select(0, idx).double().cpu().numpy() - O_ref[0]).max()))
        worst_l = max(worst_l, float(np.abs(L[h].index_select(0, idx).double().cpu().numpy() - L_ref[0]).max()))
    print("tree64k window %d: sampled rows max|dO| %.2e max|dLSE| %.2e" % (window, worst_o, worst_l), flush=True)
    assert worst_o <= TOL["bf16"][0] and worst_l <= TOL["bf16"][1]
    mask.free()


@pytest.mark.parametrize("seed,window", [(0, 2), (1, 9), (2, 40)])
def test_plan_tree_window_vs_trajectories(cp, seed, window):
    from test_gpu_zigzag import _dense_tree_visibility
    rng = np.random.default_rng(60 + seed)
    seg, parent = _preorder_tree(rng, 7, 1, 30)
    n = len(seg) // 8 * 8
    seg = seg[:n]
    parent = parent[:int(seg.max()) + 1]
    lp = _logical_positions(seg, parent)
    vis = _dense_tree_visibility(seg, parent) & ((lp[:, None] - lp[None, :]) < window)
    mask = cp.Mask.tree(seg, parent).with_window(window)
    N, C = 4, 2
    c = n // (N * C)
    chunks = [ch for r in range(N) for ch in (r, 2 * N - 1 - r)]
    w = cp.ring_plan([c] * (N * C), [(ch * c, 1) for ch in chunks], mask, chunks_per_rank=C)
    for r in range(N):
        for kk in range(N):
            b = (r - kk) % N
            qs = np.concatenate([np.arange(ch * c, (ch + 1) * c) for ch in chunks[r * C:(r + 1) * C]])
            ks = np.concatenate([np.arange(ch * c, (ch + 1) * c) for ch in chunks[b * C:(b + 1) * C]])
            assert w[r, kk] == int(vis[np.ix_(qs, ks)].sum())
