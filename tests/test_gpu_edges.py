"""Degenerate inputs (GPU): empty blocks, pairs with no visible key, ranks
that hold no tokens, one-token blocks, zero-row merges.

A partial over no keys is the identity of the merge ("Context Parallelism in
ART", section 03: the log-sum-exp merge, an empty set having weight
exp(-inf) = 0), so every row gets O = 0 and LSE = -inf, and merging it into a
running result (accumulate) leaves that result unchanged bit for bit.  A
backward over no visible pair adds nothing.  A ring rank with no tokens
takes part in the schedule without changing anyone's result.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from test_gpu_parity import _cmp

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def cp():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import context_blockwise_attention_amd as cpattn
    cpattn.lib()
    return cpattn


def _garbage(H, n, d):
    g = torch.Generator(device="cpu").manual_seed(99)
    return (torch.randn((H, n, d), generator=g).cuda(), torch.randn((H, n), generator=g).cuda())


def _is_empty_result(o, l):
    return bool((o == 0).all()) and bool((l == -float("inf")).all())


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
def test_partial_empty_key_block(cp, dtype, d):
    H, nq = 3, 300
    q, k, v = workloads.qkv(71, H, nq, d, dtype, n_kv=0)
    mask = cp.Mask.causal(nq)
    o, l = _garbage(H, nq, d)
    cp.partial(q.cuda(), k.cuda(), v.cuda(), mask, out=(o, l))
    torch.cuda.synchronize()
    assert _is_empty_result(o, l)
    run = _garbage(H, nq, d)
    keep = (run[0].clone(), run[1].clone())
    cp.partial(q.cuda(), k.cuda(), v.cuda(), mask, out=run, accumulate=True)
    torch.cuda.synchronize()
    assert torch.equal(run[0], keep[0]) and torch.equal(run[1], keep[1])


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_partial_empty_query_block(cp, dtype):
    H, nk, d = 2, 200, 128
    q, k, v = workloads.qkv(72, H, 0, d, dtype, n_kv=nk)
    mask = cp.Mask.causal(nk)
    o, l = cp.partial(q.cuda(), k.cuda(), v.cuda(), mask)
    torch.cuda.synchronize()
    assert o.shape == (H, 0, d) and l.shape == (H, 0)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("kind", ["causal", "tree", "window"])
def test_partial_no_visible_pair(cp, dtype, kind):
    """Key blocks that no query of the block can see: keys after every query
    (causal), keys in a sibling subtree (tree), keys beyond the window
    (causal, window 50): every row (0, -inf), as the reference says; with
    accumulate the running result is untouched."""
    H, d, n = 2, 128, 900
    q, k, v = workloads.qkv(73, H, 300, d, dtype, n_kv=300)
    if kind == "causal":
        mask, omask, qb, kb = cp.Mask.causal(n), oracle.Causal(), 0, 600
    elif kind == "tree":
        seg, parent = workloads.tree_prompt_completions(300, (300, 300))
        mask, omask, qb, kb = cp.Mask.tree(seg, parent), oracle.Tree(seg, parent), 300, 600
    else:
        mask, omask, qb, kb = cp.Mask.causal(n).with_window(50), oracle.Causal(window=50), 600, 0
    O, L = oracle.attention(q, k, v, qb + np.arange(300), kb + np.arange(300), omask)
    assert not np.isfinite(L).any(), "the case must have no visible pair"
    o, l = _garbage(H, 300, d)
    cp.partial(q.cuda(), k.cuda(), v.cuda(), mask, (qb, 1), (kb, 1), out=(o, l))
    torch.cuda.synchronize()
    _cmp(o, l, O, L, dtype, "no visible pair, %s" % kind)
    run = _garbage(H, 300, d)
    keep = (run[0].clone(), run[1].clone())
    cp.partial(q.cuda(), k.cuda(), v.cuda(), mask, (qb, 1), (kb, 1), out=run, accumulate=True)
    torch.cuda.synchronize()
    assert torch.equal(run[0], keep[0]) and torch.equal(run[1], keep[1])


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
def test_one_token_blocks(cp, dtype, d):
    """One query against one key at its own position (the only visible key:
    O = V, LSE = the scaled score), and one query against one key after it
    (none visible)."""
    H = 2
    q, k, v = workloads.qkv(74, H, 1, d, dtype)
    mask = cp.Mask.causal(4)
    for kb in (2, 3):
        o, l = cp.partial(q.cuda(), k.cuda(), v.cuda(), mask, (2, 1), (kb, 1))
        torch.cuda.synchronize()
        O, L = oracle.attention(q, k, v, np.array([2]), np.array([kb]), oracle.Causal())
        _cmp(o, l, O, L, dtype, "one token, key at %d" % kb)
    if dtype == "f32":
        # one visible key: its value (its weight is 1 up to the rounding of
        # the scaled score minus the scaled maximum)
        o, l = cp.partial(q.cuda(), k.cuda(), v.cuda(), mask, (2, 1), (2, 1))
        assert float((o.cpu() - v).abs().max()) <= 1e-6 * float(v.abs().max())


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_ring_with_an_empty_rank(cp, dtype):
    """Ring of 4 where rank 1 holds no tokens (a causal row of 3 x 256
    positions split over ranks 0, 2 and 3): the other ranks' results equal
    the reference, forward and backward."""
    H, d, c = 2, 128, 256
    n = 3 * c
    q, k, v = workloads.qkv(75, H, n, d, dtype)
    G = torch.randn((H, n, d), generator=torch.Generator().manual_seed(76))
    G = G.to(torch.bfloat16) if dtype == "bf16" else G
    mask = cp.Mask.causal(n)
    owner = {0: 0, 2: 1, 3: 2}            # rank -> which third of the row it holds
    blk = lambda t, r: (t[:, owner[r] * c:(owner[r] + 1) * c] if r in owner else t[:, :0]).contiguous().cuda()
    Q = [blk(q, r) for r in range(4)]
    K = [blk(k, r) for r in range(4)]
    V = [blk(v, r) for r in range(4)]
    pos = [((owner[r] * c) if r in owner else 0, 1) for r in range(4)]
    out = cp.ring_emulate(Q, K, V, pos, mask)
    torch.cuda.synchronize()
    pos_all = np.arange(n)
    O, L = oracle.attention(q, k, v, pos_all, pos_all, oracle.Causal())
    assert out[1][0].shape == (H, 0, d)
    for r, t in owner.items():
        sl = slice(t * c, (t + 1) * c)
        _cmp(out[r][0], out[r][1], O[:, sl], L[:, sl], dtype, "rank %d" % r)
    Gs = [blk(G, r) for r in range(4)]
    deltas = [cp.backward_delta(out[r][0], Gs[r]) for r in range(4)]
    grads = cp.ring_backward(Q, K, V, pos, mask, [out[r][1] for r in range(4)], deltas, Gs)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.attention_backward(q, k, v, pos_all, pos_all, O, L, G.double().numpy(), oracle.Causal())
    assert all(t.numel() == 0 for t in grads[1])
    for r, t in owner.items():
        sl = slice(t * c, (t + 1) * c)
        for got, want, name in zip(grads[r], (rq[:, sl], rk[:, sl], rv[:, sl]), ("dq", "dk", "dv")):
            err = float(np.abs(got.double().cpu().numpy() - want).max())
            tol = 1e-4 if dtype == "f32" else 1e-2 * float(np.abs(want).max()) + 1e-4
            assert err <= tol, "rank %d %s: max|err| %.2e > %.2e" % (r, name, err, tol)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_backward_empty_and_invisible(cp, dtype):
    """The backward of an empty key block, of an empty query block and of a
    pair with no visible key adds nothing: the gradient buffers keep their
    contents bit for bit."""
    H, d = 2, 128
    q, k, v = workloads.qkv(77, H, 300, d, dtype)
    G = torch.randn((H, 300, d), generator=torch.Generator().manual_seed(78))
    G = G.to(torch.bfloat16) if dtype == "bf16" else G
    mask = cp.Mask.causal(900)
    qd, kd, vd, gd = q.cuda(), k.cuda(), v.cuda(), G.cuda()
    lse = torch.randn((H, 300)).cuda()
    delta = torch.randn((H, 300)).cuda()
    base = [torch.randn((H, 300, d)).cuda() for _ in range(3)]
    cases = {
        "no keys": (qd, kd[:, :0], vd[:, :0], gd, (600, 1), (0, 1), lse, delta),
        "no queries": (qd[:, :0], kd, vd, gd[:, :0], (0, 1), (0, 1), lse[:, :0], delta[:, :0]),
        "keys after every query": (qd, kd, vd, gd, (0, 1), (600, 1), lse, delta),
    }
    for name, (qq, kk, vv, gg, qp, kp, ll, dl) in cases.items():
        grads = tuple(t.clone() for t in base)
        if qq.shape[1] == 0:
            grads = (grads[0][:, :0].contiguous(), grads[1], grads[2])
        if kk.shape[1] == 0:
            grads = (grads[0], grads[1][:, :0].contiguous(), grads[2][:, :0].contiguous())
        keep = tuple(t.clone() for t in grads)
        cp.partial_backward(qq, kk, vv, mask, ll.contiguous(), dl.contiguous(), gg, qp, kp, grads=grads)
        torch.cuda.synchronize()
        for a, b in zip(grads, keep):
            assert torch.equal(a, b), "%s: a gradient buffer changed" % name


def test_zero_row_merge_sink_delta(cp):
    """Merge, sink and D over zero rows are valid calls that do nothing; a
    merge of one part returns that part."""
    d = 128
    e = (torch.empty((3, 0, d), device="cuda"), torch.empty((3, 0), device="cuda"))
    o, l = cp.merge([e, e])
    assert o.shape == (3, 0, d)
    cp.apply_sink(e[0], e[1], torch.zeros(3, device="cuda"))
    dl = cp.backward_delta(e[0], torch.empty((3, 0, d), dtype=torch.bfloat16, device="cuda"))
    assert dl.shape == (3, 0)
    g = torch.Generator().manual_seed(79)
    one = (torch.randn((3, 40, d), generator=g).cuda(), torch.randn((3, 40), generator=g).cuda())
    one[1][0, :5] = -float("inf")
    one[0][0, :5] = 0
    o, l = cp.merge([one])
    torch.cuda.synchronize()
    assert torch.equal(l, one[1])
    assert float((o - one[0]).abs().max()) <= 1e-6 * float(one[0].abs().max())
