"""Token-major and packed layouts (GPU).

Models keep activations token-major: [tokens, heads, d], or Q, K and V (and
the output gradient) packed as [tokens, 3, heads, d].  The C ABI takes such
a tensor through its head and token strides, with no copy: a head-major
[H, n, d] view of it has head stride d and token stride (heads per token) x d.
Every other test uses head-major tensors, whose token stride is d.

The kernels' arithmetic does not depend on where a row is stored, so each
call on a strided view must give bit for bit what the same call gives on
contiguous copies of the same values, and agree with the fp64 reference at
the usual bounds:

* partial attention on packed Q/K/V, bf16 and fp32, d 64 and 128, causal and
  tree, several query and key tiles with ragged tails;
* grouped-query heads with a sliding window, Q, K and V packed in one
  token-major tensor of H + 2 H_kv heads;
* the ring of 4 on a packed tree row (each rank's block a token slice of the
  packed views);
* the backward (D, and dQ, dK, dV of a partial and of the ring, with and
  without a window, grouped heads included), Q, K, V and dO packed.
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


def _packed(*ts):
    """Head-major views [H_i, n, d] into one token-major device tensor
    [n, sum H_i, d] holding the given [H_i, n, d] tensors side by side."""
    x = torch.cat(ts, 0).permute(1, 0, 2).contiguous().cuda()
    views, h0 = [], 0
    for t in ts:
        views.append(x[:, h0:h0 + t.shape[0]].permute(1, 0, 2))
        h0 += t.shape[0]
    Ht, d = x.shape[1], x.shape[2]
    for v in views:
        assert v.stride() == (d, Ht * d, 1) and not v.is_contiguous()
    return views


def _mask(cp, kind, n, window=0):
    if kind == "causal":
        m, om = cp.Mask.causal(n), oracle.Causal(window=window) if window else oracle.Causal()
        return (m.with_window(window) if window else m), om
    seg, parent = workloads.tree_prompt_completions(n - 400, (150, 130, 120))
    assert len(seg) == n
    m = cp.Mask.tree(seg, parent)
    if window:
        return m.with_window(window), oracle.Tree(seg, parent, window=window)
    return m, oracle.Tree(seg, parent)


def _equal(a, b, what):
    for x, y, name in zip(a, b, ("0", "1", "2")):
        assert torch.equal(x, y), "%s: output %s differs from the contiguous call (max |diff| %.3g)" % (
            what, name, float((x - y).abs().nan_to_num(0.0).max()))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("kind", ["causal", "tree"])
def test_partial_packed_qkv(cp, dtype, d, kind):
    H, n = 3, 700
    q, k, v = workloads.qkv(61, H, n, d, dtype)
    mask, omask = _mask(cp, kind, n)
    qv, kv, vv = _packed(q, k, v)
    o, l = cp.partial(qv, kv, vv, mask)
    o2, l2 = cp.partial(q.cuda(), k.cuda(), v.cuda(), mask)
    torch.cuda.synchronize()
    _equal((o, l), (o2, l2), "packed %s d %d %s" % (dtype, d, kind))
    pos = np.arange(n)
    O, L = oracle.attention(q, k, v, pos, pos, omask)
    _cmp(o, l, O, L, dtype, "packed %s d %d %s" % (dtype, d, kind))
    mask.free()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_partial_gqa_window_token_major(cp, dtype):
    H, hkv, n, d, window = 8, 2, 700, 128, 90
    q, _, _ = workloads.qkv(62, H, n, d, dtype)
    _, k, v = workloads.qkv(63, hkv, n, d, dtype)
    mask, omask = _mask(cp, "tree", n, window)
    qv, kv, vv = _packed(q, k, v)
    o, l = cp.partial(qv, kv, vv, mask)
    o2, l2 = cp.partial(q.cuda(), k.cuda(), v.cuda(), mask)
    torch.cuda.synchronize()
    _equal((o, l), (o2, l2), "gqa window token-major %s" % dtype)
    pos = np.arange(n)
    g = H // hkv
    O, L = oracle.attention(q, k.repeat_interleave(g, 0), v.repeat_interleave(g, 0), pos, pos, omask)
    _cmp(o, l, O, L, dtype, "gqa window token-major %s" % dtype)
    mask.free()


def test_ring_packed_tree(cp):
    H, d, N = 4, 128, 4
    seg, parent = workloads.tree_prompt_completions(2048, (1024,) * 3)
    n = len(seg)
    c = n // N
    q, k, v = workloads.qkv(64, H, n, d, "bf16")
    mask = cp.Mask.tree(seg, parent)
    qv, kv, vv = _packed(q, k, v)
    blk = lambda t: [t[:, r * c:(r + 1) * c] for r in range(N)]
    pos = [(r * c, 1) for r in range(N)]
    out = cp.ring_emulate(blk(qv), blk(kv), blk(vv), pos, mask)
    ref = cp.ring_emulate(blk(q.cuda()), blk(k.cuda()), blk(v.cuda()), pos, mask)
    torch.cuda.synchronize()
    for r in range(N):
        _equal(out[r], ref[r], "ring rank %d" % r)
    rows = np.arange(0, n, 37)
    O, L = oracle.attention(q, k, v, np.arange(n), np.arange(n), oracle.Tree(seg, parent), rows=rows)
    o = torch.cat([out[r][0] for r in range(N)], 1)[:, rows]
    l = torch.cat([out[r][1] for r in range(N)], 1)[:, rows]
    _cmp(o, l, O, L, "bf16", "ring on packed views, sampled rows")
    mask.free()


def _grad_out(seed, H, n, d, dtype):
    g = torch.Generator().manual_seed(seed)
    t = torch.randn((H, n, d), generator=g)
    return t.to(torch.bfloat16) if dtype == "bf16" else t


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("window", [0, 120])
def test_partial_backward_packed(cp, dtype, window):
    """D, dQ, dK and dV with Q, K, V and dO packed token-major (grouped heads:
    8 query heads over 2 K/V heads): bitwise the contiguous call's, and
    against the reference."""
    H, hkv, n, d = 8, 2, 700, 128
    g = H // hkv
    q, _, _ = workloads.qkv(65, H, n, d, dtype)
    _, k, v = workloads.qkv(66, hkv, n, d, dtype)
    G = _grad_out(67, H, n, d, dtype)
    mask, omask = _mask(cp, "tree", n, window)
    qv, kv, vv, gv = _packed(q, k, v, G)
    qc, kc, vc, gc = q.cuda(), k.cuda(), v.cuda(), G.cuda()
    o, l = cp.partial(qc, kc, vc, mask)
    delta = cp.backward_delta(o, gc)
    delta_v = cp.backward_delta(o, gv)
    grads = cp.partial_backward(qv, kv, vv, mask, l, delta_v, gv)
    ref = cp.partial_backward(qc, kc, vc, mask, l, delta, gc)
    torch.cuda.synchronize()
    assert torch.equal(delta, delta_v), "D from a packed dO differs"
    _equal(grads, ref, "backward packed %s W %d" % (dtype, window))
    pos = np.arange(n)
    kr, vr = k.repeat_interleave(g, 0), v.repeat_interleave(g, 0)
    O, L = oracle.attention(q, kr, vr, pos, pos, omask)
    rq, rk, rv = oracle.attention_backward(q, kr, vr, pos, pos, O, L, G.double().numpy(), omask)
    rk = rk.reshape(hkv, g, n, d).sum(1)
    rv = rv.reshape(hkv, g, n, d).sum(1)
    for got, want, name in zip(grads, (rq, rk, rv), ("dq", "dk", "dv")):
        got = got.double().cpu().numpy()
        err = float(np.abs(got - want).max())
        tol = 1e-4 if dtype == "f32" else 1e-2 * float(np.abs(want).max()) + 1e-4
        assert err <= tol, "%s %s W %d: max|err| %.2e > %.2e" % (name, dtype, window, err, tol)
    mask.free()


@pytest.mark.parametrize("window", [0, 600])
def test_ring_backward_packed(cp, window):
    H, d, N = 4, 128, 4
    seg, parent = workloads.tree_prompt_completions(2048, (1024,) * 3)
    n = len(seg)
    c = n // N
    q, k, v = workloads.qkv(68, H, n, d, "bf16")
    G = _grad_out(69, H, n, d, "bf16")
    mask = cp.Mask.tree(seg, parent)
    if window:
        mask = mask.with_window(window)
    qv, kv, vv, gv = _packed(q, k, v, G)
    blk = lambda t: [t[:, r * c:(r + 1) * c] for r in range(N)]
    pos = [(r * c, 1) for r in range(N)]
    qc, kc, vc, gc = q.cuda(), k.cuda(), v.cuda(), G.cuda()
    fwd = cp.ring_emulate(blk(qc), blk(kc), blk(vc), pos, mask)
    lses = [fwd[r][1] for r in range(N)]
    deltas = [cp.backward_delta(fwd[r][0], blk(gc)[r].contiguous()) for r in range(N)]
    got = cp.ring_backward(blk(qv), blk(kv), blk(vv), pos, mask, lses, deltas, blk(gv))
    ref = cp.ring_backward(blk(qc), blk(kc), blk(vc), pos, mask, lses, deltas, [t.contiguous() for t in blk(gc)])
    torch.cuda.synchronize()
    for r in range(N):
        _equal(got[r], ref[r], "ring backward W %d rank %d" % (window, r))
    mask.free()
