"""GPU parity of the zig-zag (folded) ring: 2N chunks, rank r holds chunks r
and 2N-1-r (ML-systems lesson, causal load balancing), through
cpattn_ring_emulate_chunks, against the fp64 reference computing plain
unpartitioned attention; and the per-rank work report on packed trees.

* tiny causal ring, fp32 (1 head, d 64, 256 tokens, N = 4 -> 8 chunks of 32):
  every row, tolerance 1e-5;
* the causal ring workload in zig-zag layout (32 heads, d 128, 32768 tokens,
  N = 8 -> 16 chunks of 2048, bf16): 256 sampled rows per head (2e-2 / 1e-3)
  and the exact count pin on every row (1e-5);
* the same packed-tree row in zig-zag and in contiguous layout give the same
  output;
* cpattn_ring_plan on random packed trees equals a brute-force count over the
  dense visibility matrix built from the trajectories.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from test_gpu_fullsize import _bits_v, _check_counts, _cmp_sampled, _expected_counts, _print, _sample

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def cp():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import context_blockwise_attention_amd as cpattn
    cpattn.lib()
    return cpattn


def _zigzag_ring(cp, q, k, v, N, mask):
    """Runs every rank; returns (O, L) in position order."""
    n = k.shape[1]
    c = n // (2 * N)
    chunks = [ch for r in range(N) for ch in (r, 2 * N - 1 - r)]
    Q = [q[:, ch * c:(ch + 1) * c] for ch in chunks]
    K = [k[:, ch * c:(ch + 1) * c] for ch in chunks]
    V = [v[:, ch * c:(ch + 1) * c] for ch in chunks]
    out = cp.ring_emulate_chunks(Q, K, V, [(ch * c, 1) for ch in chunks], mask, chunks_per_rank=2)
    H, d = q.shape[0], q.shape[2]
    O = torch.empty((H, n, d), dtype=torch.float32, device=q.device)
    L = torch.empty((H, n), dtype=torch.float32, device=q.device)
    for i, ch in enumerate(chunks):
        O[:, ch * c:(ch + 1) * c], L[:, ch * c:(ch + 1) * c] = out[i]
    return O, L


def test_tiny_causal_zigzag_fp32(cp):
    H, n, d, N = 1, 256, 64, 4
    q, k, v = workloads.qkv(0, H, n, d, "f32")
    mask = cp.Mask.causal(n)
    O, L = _zigzag_ring(cp, q.cuda(), k.cuda(), v.cuda(), N, mask)
    torch.cuda.synchronize()
    pos = np.arange(n)
    Oref, Lref = oracle.attention(q, k, v, pos, pos, oracle.Causal())
    do = float(np.abs(O.double().cpu().numpy() - Oref).max())
    dl = float(np.abs(L.double().cpu().numpy() - Lref).max())
    _print("tiny zig-zag fp32: max|dO| %.2e max|dLSE| %.2e" % (do, dl))
    assert do <= 1e-5 and dl <= 1e-5


def test_causal_ring_zigzag_8x2x2048(cp):
    w = workloads.WORKLOADS["causal_ring"]
    H, n, d, N = w.heads, w.n_tok, w.d, w.n_blocks
    _print("causal_ring zig-zag: generating inputs")
    q, k, v = workloads.qkv(0, H, n, d, "bf16")
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    mask = cp.Mask.causal(n)
    O, L = _zigzag_ring(cp, qd, kd, vd, N, mask)
    torch.cuda.synchronize()
    c = n // (2 * N)
    forced = [0, n - 1] + [b * c for b in range(2 * N)] + [b * c - 1 for b in range(1, 2 * N)]
    pos = np.arange(n)
    _cmp_sampled(O, L, _sample(0, H, n, forced), q, k, v, pos, pos, oracle.Causal(), "causal_ring zig-zag")
    vb = _bits_v(pos, H, d).cuda()
    O, L = _zigzag_ring(cp, torch.zeros_like(qd), kd, vb, N, mask)
    counts, n_vis = _expected_counts(n, pos)
    _check_counts(O, L, counts, n_vis, d, "causal_ring zig-zag")


def test_tree_zigzag_equals_contiguous(cp):
    H, d, N = 4, 128, 4
    seg, parent = workloads.tree_prompt_completions(1536, (512, 384, 640))
    n = len(seg)
    q, k, v = workloads.qkv(3, H, n, d, "bf16")
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    mask = cp.Mask.tree(seg, parent)
    Oz, Lz = _zigzag_ring(cp, qd, kd, vd, N, mask)
    c = n // N
    out = cp.ring_emulate([qd[:, r * c:(r + 1) * c] for r in range(N)], [kd[:, r * c:(r + 1) * c] for r in range(N)],
                          [vd[:, r * c:(r + 1) * c] for r in range(N)], [(r * c, 1) for r in range(N)], mask)
    Oc = torch.cat([out[r][0] for r in range(N)], 1)
    Lc = torch.cat([out[r][1] for r in range(N)], 1)
    torch.cuda.synchronize()
    pos = np.arange(n)
    Oref, Lref = oracle.attention(q, k, v, pos, pos, oracle.Tree(seg, parent))
    for O, L, what in ((Oz, Lz, "zig-zag"), (Oc, Lc, "contiguous")):
        do = float(np.abs(O.double().cpu().numpy() - Oref).max())
        dl = float(np.abs(L.double().cpu().numpy() - Lref).max())
        _print("tree %s: max|dO| %.2e max|dLSE| %.2e" % (what, do, dl))
        assert do <= 2e-2 and dl <= 1e-3
    # the two layouts merge different partials in different orders: equal up to rounding
    assert float((Oz - Oc).abs().max()) <= 2e-2


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_tree_zigzag_gqa(cp, dtype):
    """Zig-zag chunks with grouped-query heads (8 query heads over 2 K/V
    heads) on a packed tree, every row against the reference with the K/V
    heads repeated."""
    H, hkv, d, N = 8, 2, 128, 4
    g = H // hkv
    seg, parent = workloads.tree_prompt_completions(384, (256, 192, 192))
    n = len(seg)
    q, _, _ = workloads.qkv(9, H, n, d, dtype)
    _, k, v = workloads.qkv(10, hkv, n, d, dtype)
    mask = cp.Mask.tree(seg, parent)
    O, L = _zigzag_ring(cp, q.cuda(), k.cuda(), v.cuda(), N, mask)
    torch.cuda.synchronize()
    pos = np.arange(n)
    Oref, Lref = oracle.attention(q, k.repeat_interleave(g, 0), v.repeat_interleave(g, 0), pos, pos,
                                  oracle.Tree(seg, parent))
    do = float(np.abs(O.double().cpu().numpy() - Oref).max())
    dl = float(np.abs(L.double().cpu().numpy() - Lref).max())
    _print("tree zig-zag gqa %s: max|dO| %.2e max|dLSE| %.2e" % (dtype, do, dl))
    tol_o, tol_l = (1e-5, 1e-5) if dtype == "f32" else (2e-2, 1e-3)
    assert do <= tol_o and dl <= tol_l
    mask.free()


def _dense_tree_visibility(seg, parent):
    """vis[y, x]: key x visible to query y, from the trajectories: x's segment
    is y's segment (and x <= y) or a strict ancestor of it."""
    n = len(seg)
    anc = []
    for s in range(len(parent)):
        a, p = set(), parent[s]
        while p >= 0:
            a.add(p)
            p = parent[p]
        anc.append(a)
    vis = np.zeros((n, n), dtype=bool)
    for y in range(n):
        for x in range(n):
            vis[y, x] = (seg[x] == seg[y] and x <= y) or (seg[x] in anc[seg[y]])
    return vis


@pytest.mark.parametrize("seed", [0, 1])
def test_plan_on_random_trees_matches_brute_force(cp, seed):
    rng = np.random.default_rng(seed)
    # a preorder tree: each new segment's parent is on the open path
    lengths, parents, path = [], [], []
    while sum(lengths) < 192:
        depth = int(rng.integers(0, len(path) + 1))
        path = path[:depth]
        parents.append(path[-1] if path else -1)
        lengths.append(int(rng.integers(1, 24)))
        path.append(len(lengths) - 1)
    seg, par = workloads.tree_from_lengths(lengths, parents)
    n = len(seg) // 8 * 8
    seg = seg[:n]
    par = par[:int(seg.max()) + 1]
    vis = _dense_tree_visibility(seg, par)
    mask = cp.Mask.tree(seg, par)
    for N, C in ((4, 1), (4, 2), (2, 2)):
        c = n // (N * C)
        chunks = list(range(N)) if C == 1 else [ch for r in range(N) for ch in (r, 2 * N - 1 - r)]
        w = cp.ring_plan([c] * (N * C), [(ch * c, 1) for ch in chunks], mask, chunks_per_rank=C)
        for r in range(N):
            for kk in range(N):
                b = (r - kk) % N
                qrows = np.concatenate([np.arange(ch * c, (ch + 1) * c) for ch in chunks[r * C:(r + 1) * C]])
                kcols = np.concatenate([np.arange(ch * c, (ch + 1) * c) for ch in chunks[b * C:(b + 1) * C]])
                assert w[r, kk] == int(vis[np.ix_(qrows, kcols)].sum()), (N, C, r, kk)
    mask.free()
