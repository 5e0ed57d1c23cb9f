"""Backward on the GPU (global softmax derivative, "Context Parallelism in
ART", section 04) against the fp64 reference's backward, which is pinned by
finite differences, the staged-sum invariant and the page's counterexample.

The reference gradients use the reference's complete (O, L); the GPU uses the
GPU forward's complete (O, L) and its own D = dot(dO, O).  Tolerances:
fp32 inputs 1e-4 max-abs; bf16 inputs 1e-2 x the largest reference magnitude
of each gradient (P and dS are rounded to bf16 for the MFMAs, a relative
2^-8 per product term) plus the fp32 bound 1e-4, which only matters where a
gradient cancels to zero in exact arithmetic (a window of 1: each query sees
only itself, p = 1 and dS = dot(dO, v) - D = 0 up to fp32 rounding).

* partial backward, causal and tree, fp32 and bf16, d 64 and 128, ragged
  sizes and offsets, every element of dQ, dK, dV;
* grouped-query K/V (8 query heads over 2);
* ring backward of a packed tree (N = 4), every element;
* sliding windows on logical positions: causal partials (windows 1 .. past
  the block, ragged offsets), a packed tree, and the ring of a packed tree;
* striped position maps (stride 4), with and without a window, every pair of
  stripes against the complete forward's (O, L);
* the zig-zag (chunked) ring backward (N = 4, two chunks per rank), causal
  and packed tree, also with grouped-query heads and with sliding windows,
  every element;
* random preorder trees (nested segments, ragged lengths), with and without
  windows, split into unequal key/query blocks, every element;
* a windowed prompt with 80 completions, whose key blocks see more query
  tiles than the dK/dV kernel's list holds (the whole-range walk; checked on
  the host), fp32 and bf16;
* the 64K tree ring at full size, without and with a 4096-position window:
  the output gradient is nonzero on 256 sampled rows per head only, so dK and
  dV of every key come from those rows (checked on every key of every head)
  and dQ on those rows.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def cp():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import context_blockwise_attention_amd as cpattn
    cpattn.lib()
    return cpattn


def _check(name, got, ref, dtype):
    got = got.double().cpu().numpy() if isinstance(got, torch.Tensor) else got
    err = float(np.abs(got - ref).max()) if ref.size else 0.0
    tol = 1e-4 if dtype == "f32" else 1e-2 * float(np.abs(ref).max()) + 1e-4
    print("  %s: max|err| %.2e (tol %.1e, max|ref| %.2e)" % (name, err, tol, float(np.abs(ref).max())), flush=True)
    assert err <= tol, name


def _grad_out(seed, H, n, d, dtype):
    g = torch.Generator().manual_seed(seed)
    t = torch.randn((H, n, d), generator=g)
    return t.to(torch.bfloat16) if dtype == "bf16" else t


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("maskname,nq,nk,qbase,kbase", [("causal", 300, 300, 0, 0), ("causal", 200, 333, 150, 100),
                                                        ("tree", 300, 300, 0, 0)])
def test_partial_backward(cp, dtype, d, maskname, nq, nk, qbase, kbase):
    H = 2
    q, _, _ = workloads.qkv(51, H, nq, d, dtype)
    _, k, v = workloads.qkv(52, H, nk, d, dtype)
    G = _grad_out(53, H, nq, d, dtype)
    if maskname == "causal":
        npos = max(qbase + nq, kbase + nk)
        mask, omask = cp.Mask.causal(npos), oracle.Causal()
    else:
        seg, parent = workloads.tree_prompt_completions(100, (80, 70, 50))
        mask, omask = cp.Mask.tree(seg, parent), oracle.Tree(seg, parent)
    qpos, kpos = qbase + np.arange(nq), kbase + np.arange(nk)
    qd, kd, vd, gd = q.cuda(), k.cuda(), v.cuda(), G.cuda()
    o, l = cp.partial(qd, kd, vd, mask, (qbase, 1), (kbase, 1))
    delta = cp.backward_delta(o, gd)
    dq, dk, dv = cp.partial_backward(qd, kd, vd, mask, l, delta, gd, (qbase, 1), (kbase, 1))
    torch.cuda.synchronize()
    O, L = oracle.attention(q, k, v, qpos, kpos, omask)
    rq, rk, rv = oracle.attention_backward(q, k, v, qpos, kpos, O, L, G.double().numpy(), omask)
    _check("dq", dq, rq, dtype)
    _check("dk", dk, rk, dtype)
    _check("dv", dv, rv, dtype)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("window", [1, 37, 300])
@pytest.mark.parametrize("nq,nk,qbase,kbase", [(300, 300, 0, 0), (200, 333, 150, 100)])
def test_partial_backward_causal_window(cp, dtype, d, window, nq, nk, qbase, kbase):
    H = 2
    q, _, _ = workloads.qkv(61, H, nq, d, dtype)
    _, k, v = workloads.qkv(62, H, nk, d, dtype)
    G = _grad_out(63, H, nq, d, dtype)
    mask = cp.Mask.causal(max(qbase + nq, kbase + nk)).with_window(window)
    omask = oracle.Causal(window=window)
    qpos, kpos = qbase + np.arange(nq), kbase + np.arange(nk)
    qd, kd, vd, gd = q.cuda(), k.cuda(), v.cuda(), G.cuda()
    o, l = cp.partial(qd, kd, vd, mask, (qbase, 1), (kbase, 1))
    delta = cp.backward_delta(o, gd)
    dq, dk, dv = cp.partial_backward(qd, kd, vd, mask, l, delta, gd, (qbase, 1), (kbase, 1))
    torch.cuda.synchronize()
    O, L = oracle.attention(q, k, v, qpos, kpos, omask)
    rq, rk, rv = oracle.attention_backward(q, k, v, qpos, kpos, O, L, G.double().numpy(), omask)
    _check("dq", dq, rq, dtype)
    _check("dk", dk, rk, dtype)
    _check("dv", dv, rv, dtype)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("window", [3, 90, 250])
def test_partial_backward_tree_window(cp, dtype, window):
    H, d = 2, 128
    seg, parent = workloads.tree_prompt_completions(160, (96, 64, 80))
    n = len(seg)
    q, k, v = workloads.qkv(64, H, n, d, dtype)
    G = _grad_out(65, H, n, d, dtype)
    mask = cp.Mask.tree(seg, parent).with_window(window)
    omask = oracle.Tree(seg, parent, window=window)
    qd, kd, vd, gd = q.cuda(), k.cuda(), v.cuda(), G.cuda()
    o, l = cp.partial(qd, kd, vd, mask)
    delta = cp.backward_delta(o, gd)
    dq, dk, dv = cp.partial_backward(qd, kd, vd, mask, l, delta, gd)
    torch.cuda.synchronize()
    pos = np.arange(n)
    O, L = oracle.attention(q, k, v, pos, pos, omask)
    rq, rk, rv = oracle.attention_backward(q, k, v, pos, pos, O, L, G.double().numpy(), omask)
    _check("dq", dq, rq, dtype)
    _check("dk", dk, rk, dtype)
    _check("dv", dv, rv, dtype)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_ring_backward_tree_window(cp, dtype):
    N, H, d, window = 4, 2, 128, 150
    seg, parent = workloads.tree_prompt_completions(384, (128, 200, 96, 160))
    n = len(seg) // N * N
    seg = seg[:n]
    c = n // N
    q, k, v = workloads.qkv(66, H, n, d, dtype)
    G = _grad_out(67, H, n, d, dtype)
    qd, kd, vd, gd = q.cuda(), k.cuda(), v.cuda(), G.cuda()
    mask = cp.Mask.tree(seg, parent).with_window(window)
    blk = lambda t: [t[:, r * c:(r + 1) * c] for r in range(N)]
    pos = [(r * c, 1) for r in range(N)]
    out = cp.ring_emulate(blk(qd), blk(kd), blk(vd), pos, mask)
    deltas = [cp.backward_delta(out[r][0], blk(gd)[r].contiguous()) for r in range(N)]
    grads = cp.ring_backward(blk(qd), blk(kd), blk(vd), pos, mask, [out[r][1] for r in range(N)], deltas, blk(gd))
    torch.cuda.synchronize()
    allpos = np.arange(n)
    omask = oracle.Tree(seg, parent, window=window)
    O, L = oracle.attention(q, k, v, allpos, allpos, omask)
    rq, rk, rv = oracle.attention_backward(q, k, v, allpos, allpos, O, L, G.double().numpy(), omask)
    for name, i, ref in (("dq", 0, rq), ("dk", 1, rk), ("dv", 2, rv)):
        got = torch.cat([grads[r][i] for r in range(N)], 1)
        _check(name, got, ref, dtype)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("window", [0, 45])
def test_partial_backward_striped(cp, dtype, window):
    """Striped layout (global position P idx + r): every (query stripe, key
    stripe) pair, strides > 1 in both position maps."""
    H, n, d, P = 2, 150, 128, 4
    q, k, v = workloads.qkv(68, H, n * P, d, dtype)
    G = _grad_out(69, H, n * P, d, dtype)
    lay = workloads.striped(n * P, P)
    mask = cp.Mask.causal(n * P)
    if window:
        mask = mask.with_window(window)
    omask = oracle.Causal(window=window)
    for a in (0, 3):
        for b in range(P):
            qq, gg = q[:, lay[a]].contiguous(), G[:, lay[a]].contiguous()
            kk, vv = k[:, lay[b]].contiguous(), v[:, lay[b]].contiguous()
            qd, kd, vd, gd = qq.cuda(), kk.cuda(), vv.cuda(), gg.cuda()
            # the complete forward of the stripe's queries (all key stripes), then this pair's gradients
            O, L = oracle.attention(qq, k, v, lay[a], np.arange(n * P), omask)
            ot = torch.from_numpy(O.astype(np.float32)).cuda()
            lt = torch.from_numpy(L.astype(np.float32)).cuda()
            delta = cp.backward_delta(ot, gd)
            dq, dk, dv = cp.partial_backward(qd, kd, vd, mask, lt, delta, gd, (a, P), (b, P))
            torch.cuda.synchronize()
            rq, rk, rv = oracle.attention_backward(qq, kk, vv, lay[a], lay[b], O, L, gg.double().numpy(), omask)
            _check("dq %d/%d" % (a, b), dq, rq, dtype)
            _check("dk %d/%d" % (a, b), dk, rk, dtype)
            _check("dv %d/%d" % (a, b), dv, rv, dtype)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_partial_backward_gqa(cp, dtype):
    H, hkv, n, d = 8, 2, 260, 128
    g = H // hkv
    q, _, _ = workloads.qkv(54, H, n, d, dtype)
    _, k, v = workloads.qkv(55, hkv, n, d, dtype)
    G = _grad_out(56, H, n, d, dtype)
    seg, parent = workloads.tree_prompt_completions(100, (60, 100))
    mask, omask = cp.Mask.tree(seg, parent), oracle.Tree(seg, parent)
    qd, kd, vd, gd = q.cuda(), k.cuda(), v.cuda(), G.cuda()
    o, l = cp.partial(qd, kd, vd, mask)
    delta = cp.backward_delta(o, gd)
    dq, dk, dv = cp.partial_backward(qd, kd, vd, mask, l, delta, gd)
    torch.cuda.synchronize()
    pos = np.arange(n)
    kr, vr = k.repeat_interleave(g, 0), v.repeat_interleave(g, 0)
    O, L = oracle.attention(q, kr, vr, pos, pos, omask)
    rq, rk, rv = oracle.attention_backward(q, kr, vr, pos, pos, O, L, G.double().numpy(), omask)
    _check("dq", dq, rq, dtype)
    _check("dk", dk, rk.reshape(hkv, g, n, d).sum(1), dtype)
    _check("dv", dv, rv.reshape(hkv, g, n, d).sum(1), dtype)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_partial_backward_gqa_window(cp, dtype):
    """Grouped-query heads and a sliding window on a tree, backward."""
    H, hkv, n, d, window = 8, 2, 260, 128, 70
    g = H // hkv
    q, _, _ = workloads.qkv(57, H, n, d, dtype)
    _, k, v = workloads.qkv(58, hkv, n, d, dtype)
    G = _grad_out(59, H, n, d, dtype)
    seg, parent = workloads.tree_prompt_completions(100, (60, 100))
    mask = cp.Mask.tree(seg, parent).with_window(window)
    omask = oracle.Tree(seg, parent, window=window)
    qd, kd, vd, gd = q.cuda(), k.cuda(), v.cuda(), G.cuda()
    o, l = cp.partial(qd, kd, vd, mask)
    delta = cp.backward_delta(o, gd)
    dq, dk, dv = cp.partial_backward(qd, kd, vd, mask, l, delta, gd)
    torch.cuda.synchronize()
    pos = np.arange(n)
    kr, vr = k.repeat_interleave(g, 0), v.repeat_interleave(g, 0)
    O, L = oracle.attention(q, kr, vr, pos, pos, omask)
    rq, rk, rv = oracle.attention_backward(q, kr, vr, pos, pos, O, L, G.double().numpy(), omask)
    _check("dq", dq, rq, dtype)
    _check("dk", dk, rk.reshape(hkv, g, n, d).sum(1), dtype)
    _check("dv", dv, rv.reshape(hkv, g, n, d).sum(1), dtype)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_ring_backward_tree(cp, dtype):
    N, H, d = 4, 2, 128
    seg, parent = workloads.tree_prompt_completions(384, (128, 200, 96, 160))
    n = len(seg) // N * N
    seg = seg[:n]
    c = n // N
    q, k, v = workloads.qkv(57, H, n, d, dtype)
    G = _grad_out(58, H, n, d, dtype)
    qd, kd, vd, gd = q.cuda(), k.cuda(), v.cuda(), G.cuda()
    mask = cp.Mask.tree(seg, parent)
    blk = lambda t: [t[:, r * c:(r + 1) * c] for r in range(N)]
    pos = [(r * c, 1) for r in range(N)]
    out = cp.ring_emulate(blk(qd), blk(kd), blk(vd), pos, mask)
    deltas = [cp.backward_delta(out[r][0], blk(gd)[r].contiguous()) for r in range(N)]
    grads = cp.ring_backward(blk(qd), blk(kd), blk(vd), pos, mask, [out[r][1] for r in range(N)], deltas, blk(gd))
    torch.cuda.synchronize()
    allpos = np.arange(n)
    omask = oracle.Tree(seg, parent)
    O, L = oracle.attention(q, k, v, allpos, allpos, omask)
    rq, rk, rv = oracle.attention_backward(q, k, v, allpos, allpos, O, L, G.double().numpy(), omask)
    for name, i, ref in (("dq", 0, rq), ("dk", 1, rk), ("dv", 2, rv)):
        got = torch.cat([grads[r][i] for r in range(N)], 1)
        _check(name, got, ref, dtype)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("maskname", ["causal", "tree"])
def test_zigzag_ring_backward(cp, dtype, maskname):
    N, H, d = 4, 2, 128
    if maskname == "causal":
        n = 8 * 96
        mask, omask = cp.Mask.causal(n), oracle.Causal()
    else:
        seg, parent = workloads.tree_prompt_completions(320, (160, 200, 88))
        n = len(seg)
        mask, omask = cp.Mask.tree(seg, parent), oracle.Tree(seg, parent)
    c = n // (2 * N)
    q, k, v = workloads.qkv(70, H, n, d, dtype)
    G = _grad_out(71, H, n, d, dtype)
    qd, kd, vd, gd = q.cuda(), k.cuda(), v.cuda(), G.cuda()
    chunks = [ch for r in range(N) for ch in (r, 2 * N - 1 - r)]
    cut = lambda t: [t[:, ch * c:(ch + 1) * c].contiguous() for ch in chunks]
    pos = [(ch * c, 1) for ch in chunks]
    Q, K, V, Gs = cut(qd), cut(kd), cut(vd), cut(gd)
    out = cp.ring_emulate_chunks(Q, K, V, pos, mask, chunks_per_rank=2)
    deltas = [cp.backward_delta(out[i][0], Gs[i]) for i in range(2 * N)]
    grads = cp.ring_backward_chunks(Q, K, V, pos, mask, [out[i][1] for i in range(2 * N)], deltas, Gs,
                                    chunks_per_rank=2)
    torch.cuda.synchronize()
    allpos = np.arange(n)
    O, L = oracle.attention(q[:, :2 * N * c], k[:, :2 * N * c], v[:, :2 * N * c], allpos[:2 * N * c],
                            allpos[:2 * N * c], omask)
    rq, rk, rv = oracle.attention_backward(q[:, :2 * N * c], k[:, :2 * N * c], v[:, :2 * N * c], allpos[:2 * N * c],
                                           allpos[:2 * N * c], O, L, G[:, :2 * N * c].double().numpy(), omask)
    for name, j, ref in (("dq", 0, rq), ("dk", 1, rk), ("dv", 2, rv)):
        got = torch.zeros((H, 2 * N * c, d), dtype=torch.float64)
        for i, ch in enumerate(chunks):
            got[:, ch * c:(ch + 1) * c] = grads[i][j].double().cpu()
        _check(name, got, ref, dtype)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("maskname,window", [("causal", 70), ("tree", 40), ("tree", 150)])
def test_zigzag_ring_backward_window(cp, dtype, maskname, window):
    """Zig-zag chunks (rank r holds chunks r and 2N-1-r) with a sliding window
    on logical positions, backward: the chunk pairs that the window empties
    are skipped, the rest go through the windowed dQ and dK/dV kernels."""
    N, H, d = 4, 2, 128
    if maskname == "causal":
        n = 8 * 96
        mask, omask = cp.Mask.causal(n).with_window(window), oracle.Causal(window=window)
    else:
        seg, parent = workloads.tree_prompt_completions(320, (160, 200, 88))
        n = len(seg)
        mask = cp.Mask.tree(seg, parent).with_window(window)
        omask = oracle.Tree(seg, parent, window=window)
    c = n // (2 * N)
    m = 2 * N * c
    q, k, v = workloads.qkv(75, H, n, d, dtype)
    G = _grad_out(76, H, n, d, dtype)
    qd, kd, vd, gd = q.cuda(), k.cuda(), v.cuda(), G.cuda()
    chunks = [ch for r in range(N) for ch in (r, 2 * N - 1 - r)]
    cut = lambda t: [t[:, ch * c:(ch + 1) * c].contiguous() for ch in chunks]
    pos = [(ch * c, 1) for ch in chunks]
    Q, K, V, Gs = cut(qd), cut(kd), cut(vd), cut(gd)
    out = cp.ring_emulate_chunks(Q, K, V, pos, mask, chunks_per_rank=2)
    deltas = [cp.backward_delta(out[i][0], Gs[i]) for i in range(2 * N)]
    grads = cp.ring_backward_chunks(Q, K, V, pos, mask, [out[i][1] for i in range(2 * N)], deltas, Gs,
                                    chunks_per_rank=2)
    torch.cuda.synchronize()
    allpos = np.arange(m)
    O, L = oracle.attention(q[:, :m], k[:, :m], v[:, :m], allpos, allpos, omask)
    rq, rk, rv = oracle.attention_backward(q[:, :m], k[:, :m], v[:, :m], allpos, allpos, O, L,
                                           G[:, :m].double().numpy(), omask)
    for name, j, ref in (("dq", 0, rq), ("dk", 1, rk), ("dv", 2, rv)):
        got = torch.zeros((H, m, d), dtype=torch.float64)
        for i, ch in enumerate(chunks):
            got[:, ch * c:(ch + 1) * c] = grads[i][j].double().cpu()
        _check(name, got, ref, dtype)
    mask.free()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_zigzag_ring_backward_gqa(cp, dtype):
    """Zig-zag chunks with grouped-query heads (4 query heads over 2 K/V
    heads) on a packed tree, backward: dK/dV of a K/V head sum its group's
    query heads."""
    N, H, hkv, d = 4, 4, 2, 128
    g = H // hkv
    seg, parent = workloads.tree_prompt_completions(320, (160, 200, 88))
    n = len(seg)
    mask, omask = cp.Mask.tree(seg, parent), oracle.Tree(seg, parent)
    c = n // (2 * N)
    q, _, _ = workloads.qkv(72, H, n, d, dtype)
    _, k, v = workloads.qkv(73, hkv, n, d, dtype)
    G = _grad_out(74, H, n, d, dtype)
    qd, kd, vd, gd = q.cuda(), k.cuda(), v.cuda(), G.cuda()
    chunks = [ch for r in range(N) for ch in (r, 2 * N - 1 - r)]
    cut = lambda t: [t[:, ch * c:(ch + 1) * c].contiguous() for ch in chunks]
    pos = [(ch * c, 1) for ch in chunks]
    Q, K, V, Gs = cut(qd), cut(kd), cut(vd), cut(gd)
    out = cp.ring_emulate_chunks(Q, K, V, pos, mask, chunks_per_rank=2)
    deltas = [cp.backward_delta(out[i][0], Gs[i]) for i in range(2 * N)]
    grads = cp.ring_backward_chunks(Q, K, V, pos, mask, [out[i][1] for i in range(2 * N)], deltas, Gs,
                                    chunks_per_rank=2)
    torch.cuda.synchronize()
    m = 2 * N * c
    allpos = np.arange(m)
    kr, vr = k[:, :m].repeat_interleave(g, 0), v[:, :m].repeat_interleave(g, 0)
    O, L = oracle.attention(q[:, :m], kr, vr, allpos, allpos, omask)
    rq, rk, rv = oracle.attention_backward(q[:, :m], kr, vr, allpos, allpos, O, L, G[:, :m].double().numpy(), omask)
    refs = (rq, rk.reshape(hkv, g, m, d).sum(1), rv.reshape(hkv, g, m, d).sum(1))
    for name, j in (("dq", 0), ("dk", 1), ("dv", 2)):
        heads = H if j == 0 else hkv
        got = torch.zeros((heads, m, d), dtype=torch.float64)
        for i, ch in enumerate(chunks):
            got[:, ch * c:(ch + 1) * c] = grads[i][j].double().cpu()
        _check(name, got, refs[j], dtype)
    mask.free()


@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("window", [0, 40, 170])
def test_random_tree_backward(cp, seed, window):
    """Random nested trees: the query block and the key block are unequal
    slices of the row, so tiles straddle runs and the window's run prefixes."""
    from test_gpu_parity import _preorder_tree
    rng = np.random.default_rng(100 + seed)
    seg, parent = _preorder_tree(rng, int(rng.integers(3, 9)), 20, 140)
    n = len(seg)
    H, d, dtype = 2, 128, ("bf16" if seed % 2 == 0 else "f32")
    q, k, v = workloads.qkv(72 + seed, H, n, d, dtype)
    G = _grad_out(75 + seed, H, n, d, dtype)
    mask = cp.Mask.tree(seg, parent)
    if window:
        mask = mask.with_window(window)
    omask = oracle.Tree(seg, parent, window=window)
    a, b = sorted(rng.integers(1, n, size=2).tolist())
    qs, ks = slice(a // 2, n), slice(0, max(b, a // 2 + 1))   # queries from a/2 on, keys up to b
    qq, gg = q[:, qs].contiguous(), G[:, qs].contiguous()
    kk, vv = k[:, ks].contiguous(), v[:, ks].contiguous()
    qpos, kpos = np.arange(n)[qs], np.arange(n)[ks]
    # complete forward of the queries over every key, then this pair's gradients
    O, L = oracle.attention(qq, k, v, qpos, np.arange(n), omask)
    ot = torch.from_numpy(O.astype(np.float32)).cuda()
    lt = torch.from_numpy(L.astype(np.float32)).cuda()
    gd = gg.cuda()
    delta = cp.backward_delta(ot, gd)
    dq, dk, dv = cp.partial_backward(qq.cuda(), kk.cuda(), vv.cuda(), mask, lt, delta, gd, (int(qpos[0]), 1),
                                     (int(kpos[0]), 1))
    torch.cuda.synchronize()
    rq, rk, rv = oracle.attention_backward(qq, kk, vv, qpos, kpos, O, L, gg.double().numpy(), omask)
    _check("dq", dq, rq, dtype)
    _check("dk", dk, rk, dtype)
    _check("dv", dv, rv, dtype)


def _logical_positions(seg, parent):
    """Position of each token along its root-to-leaf path (tokens of the
    strict ancestors, then earlier tokens of its own segment)."""
    seg = np.asarray(seg)
    n_seg = len(parent)
    start = np.full(n_seg, -1)
    length = np.zeros(n_seg, np.int64)
    for x, s_ in enumerate(seg):
        if start[s_] < 0:
            start[s_] = x
        length[s_] += 1
    anc = np.zeros(n_seg, np.int64)
    for s_ in range(n_seg):
        a = parent[s_]
        while a >= 0:
            anc[s_] += length[a]
            a = parent[a]
    return anc[seg] + np.arange(len(seg)) - start[seg]


# query tiles (of 32 rows) a dK/dV workgroup's tile list can hold, and the keys per workgroup
DKV_LIST_CAP, DKV_KEYS, DKV_QTILE = 1024, 128, 32


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_window_tree_many_runs_backward(cp, dtype):
    """A prompt with 80 short completions and a window that reaches into all
    of them: the prompt's key blocks see more query tiles than the dK/dV
    kernel lists, so they take its whole-range walk."""
    H, d, window = 1, 64, 1000
    seg, parent = workloads.tree_prompt_completions(512, (500,) * 80)
    n = len(seg)
    # the first key workgroup (keys 0..127 of the prompt; every completion is
    # in its subtree): distinct 32-row query tiles holding a query within the
    # window of its largest logical key position
    lpos = _logical_positions(seg, parent)
    lkm = int(lpos[DKV_KEYS - 1])
    tiles = np.unique(np.nonzero(lpos < lkm + window)[0] // DKV_QTILE)
    assert len(tiles) > DKV_LIST_CAP, "the case no longer overflows the dK/dV tile list (%d tiles)" % len(tiles)
    q, k, v = workloads.qkv(78, H, n, d, dtype)
    G = _grad_out(79, H, n, d, dtype)
    mask = cp.Mask.tree(seg, parent).with_window(window)
    omask = oracle.Tree(seg, parent, window=window)
    qd, kd, vd, gd = q.cuda(), k.cuda(), v.cuda(), G.cuda()
    o, l = cp.partial(qd, kd, vd, mask)
    delta = cp.backward_delta(o, gd)
    dq, dk, dv = cp.partial_backward(qd, kd, vd, mask, l, delta, gd)
    torch.cuda.synchronize()
    pos = np.arange(n)
    O, L = oracle.attention(q, k, v, pos, pos, omask)
    rq, rk, rv = oracle.attention_backward(q, k, v, pos, pos, O, L, G.double().numpy(), omask)
    _check("dq", dq, rq, dtype)
    _check("dk", dk, rk, dtype)
    _check("dv", dv, rv, dtype)


@pytest.mark.parametrize("window", [0, 4096])
def test_tree64k_ring_backward_sampled(cp, window):
    H, d, N = 32, 128, 4
    seg, parent = workloads.tree_prompt_completions(24576, (8192,) * 5)
    n = len(seg)
    c = n // N
    print("tree64k backward (window %d): generating inputs" % window, flush=True)
    q, k, v = workloads.qkv(0, H, n, d, "bf16")
    rows = [workloads.sample_rows(0, h, n, forced=(0, n - 1, 24575, 24576, n - 8192)) for h in range(H)]
    G = torch.zeros((H, n, d))
    gen = torch.Generator().manual_seed(59)
    for h in range(H):
        G[h, torch.from_numpy(rows[h])] = torch.randn((len(rows[h]), d), generator=gen)
    G = G.to(torch.bfloat16)
    qd, kd, vd, gd = q.cuda(), k.cuda(), v.cuda(), G.cuda()
    mask = cp.Mask.tree(seg, parent)
    if window:
        mask = mask.with_window(window)
    blk = lambda t: [t[:, r * c:(r + 1) * c] for r in range(N)]
    pos = [(r * c, 1) for r in range(N)]
    out = cp.ring_emulate(blk(qd), blk(kd), blk(vd), pos, mask)
    deltas = [cp.backward_delta(out[r][0], blk(gd)[r].contiguous()) for r in range(N)]
    grads = cp.ring_backward(blk(qd), blk(kd), blk(vd), pos, mask, [out[r][1] for r in range(N)], deltas, blk(gd))
    dq = torch.cat([grads[r][0] for r in range(N)], 1)
    dk = torch.cat([grads[r][1] for r in range(N)], 1)
    dv = torch.cat([grads[r][2] for r in range(N)], 1)
    torch.cuda.synchronize()
    allpos = np.arange(n)
    omask = oracle.Tree(seg, parent, window=window)
    worst = {"dq": 0.0, "dk": 0.0, "dv": 0.0}
    for h in range(H):   # every head: dK and dV of every key, dQ of the sampled rows
        O, L = oracle.attention(q[h:h + 1], k[h:h + 1], v[h:h + 1], allpos, allpos, omask, rows=rows[h])
        Gh = G[h:h + 1, torch.from_numpy(rows[h])].double().numpy()
        rq, rk, rv = oracle.attention_backward(q[h:h + 1], k[h:h + 1], v[h:h + 1], allpos, allpos, O, L, Gh,
                                               omask, rows=rows[h])
        idx = torch.from_numpy(rows[h]).cuda()
        for name, got, ref in (("dq", dq[h].index_select(0, idx), rq[0]), ("dk", dk[h], rk[0]), ("dv", dv[h], rv[0])):
            err = float(np.abs(got.double().cpu().numpy() - ref).max())
            scale_ref = float(np.abs(ref).max())
            worst[name] = max(worst[name], err / scale_ref)
            assert err <= 1e-2 * scale_ref, "head %d %s: max|err| %.2e, max|ref| %.2e" % (h, name, err, scale_ref)
    print("tree64k backward (window %d): worst max|err| / max|ref| per head:" % window,
          {k_: "%.2e" % worst[k_] for k_ in worst}, flush=True)
    mask.free()
