"""GPU parity: the HIP path through the C ABI against the fp64 CPU reference,
element by element, at sizes that span several tiles and a ragged tail.

Tolerances: fp32 inputs 1e-5 max-abs on O and LSE; bf16 inputs 2e-2 on O and
1e-3 on LSE (max-abs).
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu

TOL = {"f32": (1e-5, 1e-5), "bf16": (2e-2, 1e-3)}


@pytest.fixture(scope="module")
def cp():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import context_blockwise_attention_amd as cpattn
    cpattn.lib()
    return cpattn


def _dev(t):
    return t.contiguous().to("cuda")


def _cmp(o, l, O_ref, L_ref, dtype, what=""):
    tol_o, tol_l = TOL[dtype]
    o = o.detach().cpu().numpy().astype(np.float64)
    l = l.detach().cpu().numpy().astype(np.float64)
    fin = np.isfinite(L_ref)
    assert np.array_equal(np.isfinite(l), fin), "%s: empty-row pattern differs" % what
    assert np.all(l[~fin] == -np.inf) and np.all(o[~fin] == 0), "%s: empty rows must be (0, -inf)" % what
    do = np.abs(o - O_ref).max() if o.size else 0.0
    dl = np.abs(l[fin] - L_ref[fin]).max() if fin.any() else 0.0
    assert do <= tol_o and dl <= tol_l, "%s: max|dO| %.3e (tol %.0e), max|dLSE| %.3e (tol %.0e)" % (
        what, do, tol_o, dl, tol_l)
    return do, dl


def _blocks_of(t, layout):
    return [t[:, torch.from_numpy(p)] for p in layout]


# ----------------------------------------------------------------------------
# tiny causal fp32 ring: every partial, every running merge, the final result
# ----------------------------------------------------------------------------
def test_tiny_causal_fp32_every_round(cp):
    w = workloads.WORKLOADS["tiny_causal"]
    q, k, v = workloads.qkv(0, w.heads, w.n_tok, w.d, "f32")
    N = w.n_blocks
    lay = workloads.contiguous(w.n_tok, N)
    c = w.n_tok // N
    mask = cp.Mask.causal(w.n_tok)
    Q, K, V = [_dev(x) for x in _blocks_of(q, lay)], [_dev(x) for x in _blocks_of(k, lay)], \
        [_dev(x) for x in _blocks_of(v, lay)]
    for r in range(N):
        _, _, rounds = oracle.ring(q[:, lay[r]], lay[r], _blocks_of(k, lay), _blocks_of(v, lay), lay, r,
                                   oracle.Causal(), keep_rounds=True)
        run = None
        for kk, (b, (Op, Lp), (Or, Lr)) in enumerate(rounds):
            o, l = cp.partial(Q[r], K[b], V[b], mask, (r * c, 1), (b * c, 1))
            _cmp(o, l, Op, Lp, "f32", "rank %d round %d partial" % (r, kk))
            if run is None:
                run = (o.clone(), l.clone())
            else:
                cp.partial(Q[r], K[b], V[b], mask, (r * c, 1), (b * c, 1), out=run, accumulate=True)
            _cmp(run[0], run[1], Or, Lr, "f32", "rank %d round %d running" % (r, kk))
    out = cp.ring_emulate(Q, K, V, [(r * c, 1) for r in range(N)], mask)
    O, L = oracle.attention(q, k, v, np.arange(w.n_tok), np.arange(w.n_tok), oracle.Causal())
    for r in range(N):
        _cmp(out[r][0], out[r][1], O[:, lay[r]], L[:, lay[r]], "f32", "rank %d final" % r)


# ----------------------------------------------------------------------------
# single partials: causal, full-visibility offsets, ragged tails, both d
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("nq,nk,qbase,kbase", [(300, 300, 0, 0), (257, 190, 190, 0), (128, 64, 64, 0),
                                                (1, 1000, 999, 0), (200, 333, 0, 100)])
def test_partial_causal(cp, dtype, d, nq, nk, qbase, kbase):
    H = 2
    q, _, _ = workloads.qkv(1, H, nq, d, dtype)
    _, k, v = workloads.qkv(2, H, nk, d, dtype)
    mask = cp.Mask.causal(max(qbase + nq, kbase + nk))
    o, l = cp.partial(_dev(q), _dev(k), _dev(v), mask, (qbase, 1), (kbase, 1))
    O, L = oracle.attention(q, k, v, qbase + np.arange(nq), kbase + np.arange(nk), oracle.Causal())
    _cmp(o, l, O, L, dtype, "causal partial")


@pytest.mark.parametrize("H,nq", [(2, 2900), (9, 2600)])
def test_partial_causal_qtile_blocks(cp, H, nq):
    """More than eight 256-row query tiles in a count that is not a multiple
    of eight: the workgroups take a job's q-tiles in blocks of eight with the
    second half reversed, and a trailing partial block keeps its order.  With
    2 heads (fewer than the XCDs) and 9 (two head slots per XCD, some of them
    empty).  Every row against the oracle."""
    d = 128
    q, k, v = workloads.qkv(4, H, nq, d, "bf16")
    mask = cp.Mask.causal(nq)
    o, l = cp.partial(_dev(q), _dev(k), _dev(v), mask, (0, 1), (0, 1))
    O, L = oracle.attention(q, k, v, np.arange(nq), np.arange(nq), oracle.Causal())
    _cmp(o, l, O, L, "bf16", "causal partial, %d heads x %d rows" % (H, nq))


@pytest.mark.parametrize("P", [2, 4])
def test_partial_striped(cp, P):
    H, n, d = 2, 1200, 128
    q, k, v = workloads.qkv(3, H, n * P, d, "bf16")
    lay = workloads.striped(n * P, P)
    mask = cp.Mask.causal(n * P)
    for b in range(P):
        qq, kk, vv = q[:, lay[0]], k[:, lay[b]], v[:, lay[b]]
        o, l = cp.partial(_dev(qq), _dev(kk), _dev(vv), mask, (0, P), (b, P))
        O, L = oracle.attention(qq, kk, vv, lay[0], lay[b], oracle.Causal())
        _cmp(o, l, O, L, "bf16", "stripe %d" % b)


def _preorder_tree(rng, n_seg, lo, hi):
    parent = [-1]
    for s in range(1, n_seg):
        parent.append(int(rng.integers(-1, s)))
    kids = {s: [] for s in range(n_seg)}
    roots = []
    for s, p in enumerate(parent):
        (kids[p] if p >= 0 else roots).append(s)
    order = []

    def visit(s):
        order.append(s)
        for c in kids[s]:
            visit(c)

    for r in roots:
        visit(r)
    new = {s: i for i, s in enumerate(order)}
    par = [(-1 if parent[s] < 0 else new[parent[s]]) for s in order]
    lens = rng.integers(lo, hi + 1, size=n_seg).tolist()
    return workloads.tree_from_lengths(lens, par)


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_partial_tree_random(cp, seed):
    rng = np.random.default_rng(seed)
    seg, parent = _preorder_tree(rng, 9, 1, 200)
    n = len(seg)
    H, d = 2, 128
    q, k, v = workloads.qkv(10 + seed, H, n, d, "bf16")
    mask = cp.Mask.tree(seg, parent)
    o, l = cp.partial(_dev(q), _dev(k), _dev(v), mask)
    O, L = oracle.attention(q, k, v, np.arange(n), np.arange(n), oracle.Tree(seg, parent))
    _cmp(o, l, O, L, "bf16", "tree seed %d" % seed)


@pytest.mark.parametrize("N", [1, 3, 4])
def test_ring_tree_all_ranks(cp, N):
    seg, parent = workloads.tree_prompt_completions(384, (128, 200, 96, 160))
    n = len(seg) // N * N
    seg = seg[:n]
    H, d = 2, 128
    q, k, v = workloads.qkv(5, H, n, d, "bf16")
    lay = workloads.contiguous(n, N)
    c = n // N
    mask = cp.Mask.tree(seg, parent)
    Q, K, V = [_dev(x) for x in _blocks_of(q, lay)], [_dev(x) for x in _blocks_of(k, lay)], \
        [_dev(x) for x in _blocks_of(v, lay)]
    out = cp.ring_emulate(Q, K, V, [(r * c, 1) for r in range(N)], mask)
    O, L = oracle.attention(q, k, v, np.arange(n), np.arange(n), oracle.Tree(seg, parent))
    for r in range(N):
        _cmp(out[r][0], out[r][1], O[:, lay[r]], L[:, lay[r]], "bf16", "rank %d" % r)


def _merge_parts(n_parts, rows, d, seed):
    rng = np.random.default_rng(seed)
    parts = []
    for p in range(n_parts):
        O = rng.standard_normal((3, rows, d))
        L = rng.standard_normal((3, rows)) * 4
        L[p % 3, p * 5 % rows:(p * 5 % rows + 7)] = -np.inf   # rows this part never saw
        O[p % 3, p * 5 % rows:(p * 5 % rows + 7)] = 0
        L[:, 0] = -np.inf                                       # a row empty in every part
        O[:, 0] = 0
        parts.append((O.astype(np.float32), L.astype(np.float32)))
    return parts


def test_merge_kernel(cp):
    parts = _merge_parts(5, 77, 128, 0)
    Om, Lm = oracle.merge([(a.astype(np.float64), b.astype(np.float64)) for a, b in parts])
    dev = [(torch.from_numpy(a).cuda(), torch.from_numpy(b).cuda()) for a, b in parts]
    o, l = cp.merge(dev)
    _cmp(o, l, Om, Lm, "f32", "merge")


# every part count the kernel unrolls (1..8), the grouped form (9, 17, 64
# parts), rows of 1-float units (d % 4 != 0), short rows, and rows that span
# several waves (d = 1024: 256 threads per row)
@pytest.mark.parametrize("n_parts,d", [(1, 128), (2, 128), (3, 64), (4, 128), (6, 100), (7, 36), (8, 128),
                                       (9, 128), (17, 20), (64, 8), (4, 1024), (12, 1024), (3, 2), (2, 1)])
def test_merge_kernel_shapes(cp, n_parts, d):
    parts = _merge_parts(n_parts, 45, d, 100 + n_parts)
    Om, Lm = oracle.merge([(a.astype(np.float64), b.astype(np.float64)) for a, b in parts])
    dev = [(torch.from_numpy(a).cuda(), torch.from_numpy(b).cuda()) for a, b in parts]
    o, l = cp.merge(dev)
    _cmp(o, l, Om, Lm, "f32", "merge of %d parts, d %d" % (n_parts, d))
    # the output may alias part 0 (documented in-place use)
    cp.merge(dev, out=dev[0])
    _cmp(dev[0][0], dev[0][1], Om, Lm, "f32", "in-place merge of %d parts, d %d" % (n_parts, d))


def test_merge_kernel_misaligned_parts(cp):
    """Parts and output at a 4-byte offset from a 16-byte boundary (contiguous
    tensors that start one float into their storage), d a multiple of 4: the
    kernel takes its one-float path instead of 16-byte units."""
    n_parts, rows, d = 3, 45, 128
    parts = _merge_parts(n_parts, rows, d, 7)
    Om, Lm = oracle.merge([(a.astype(np.float64), b.astype(np.float64)) for a, b in parts])

    def shifted(a):
        buf = torch.empty(a.size + 1, dtype=torch.float32, device="cuda")
        t = buf[1:].view(a.shape)
        t.copy_(torch.from_numpy(a))
        assert t.is_contiguous() and t.data_ptr() % 16 == 4
        return t

    dev = [(shifted(a), torch.from_numpy(b).cuda()) for a, b in parts]
    out = (shifted(np.zeros((3, rows, d), dtype=np.float32)), torch.empty((3, rows), device="cuda"))
    o, l = cp.merge(dev, out=out)
    _cmp(o, l, Om, Lm, "f32", "merge of misaligned parts")
