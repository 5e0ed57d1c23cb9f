"""Seeded random configurations (GPU): the features of the partial call drawn
together, each case against the fp64 reference.

Every other test fixes most of the call and varies one or two features.  Here
each seed draws all of them at once: dtype, head dim, grouped-query heads,
a causal mask or a random preorder tree (nested segments, ragged lengths),
a sliding window or none, query and key position maps (contiguous or
strided, e.g. striped, at random offsets), ragged block sizes, head-major or
token-major tensors, sometimes a second key block merged in first
(accumulate), and the backward of the pair.  Tolerances as everywhere:
fp32 1e-5 on O and LSE, bf16 2e-2 on O and 1e-3 on LSE; gradients fp32 1e-4,
bf16 1e-2 of the gradient's largest magnitude (+1e-4).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from test_gpu_parity import _cmp, _preorder_tree

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def cp():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import context_blockwise_attention_amd as cpattn
    cpattn.lib()
    return cpattn


def _posmap(rng, n_pos, n_max):
    """(base, stride, n) with every position base + stride * i inside [0, n_pos)."""
    stride = int(rng.choice([1, 1, 1, 2, 3]))
    n = int(rng.integers(1, min(n_max, (n_pos - 1) // stride + 1) + 1))
    base = int(rng.integers(0, n_pos - stride * (n - 1)))
    return base, stride, n


def _place(t, token_major):
    """Device copy of [H, n, d] ``t``, head-major or as a token-major view."""
    if token_major:
        return t.permute(1, 0, 2).contiguous().cuda().permute(1, 0, 2)
    return t.cuda()


def _case(seed):
    rng = np.random.default_rng(5000 + seed)
    c = {"dtype": str(rng.choice(["bf16", "f32"])), "d": int(rng.choice([64, 128]))}
    c["hkv"] = int(rng.choice([1, 2, 3]))
    c["H"] = c["hkv"] * int(rng.choice([1, 2, 4]))
    c["kind"] = str(rng.choice(["causal", "tree"]))
    if c["kind"] == "causal":
        c["n_pos"] = int(rng.integers(64, 1500))
    else:
        c["tree"] = _preorder_tree(rng, int(rng.integers(2, 13)), 1, 200)
        c["n_pos"] = len(c["tree"][0])
    c["window"] = int(rng.integers(1, 400)) if rng.random() < 0.4 else 0
    c["q"] = _posmap(rng, c["n_pos"], 600)
    c["k"] = _posmap(rng, c["n_pos"], 600)
    c["k2"] = _posmap(rng, c["n_pos"], 300) if rng.random() < 0.3 else None
    c["token_major"] = bool(rng.random() < 0.5)
    c["backward"] = c["k2"] is None and rng.random() < 0.6
    return c


@pytest.mark.parametrize("seed", range(150))
def test_random_config(cp, seed):
    c = _case(seed)
    what = "seed %d: %s" % (seed, {k: v for k, v in c.items() if k != "tree"})
    print(what, flush=True)
    H, hkv, d, dtype = c["H"], c["hkv"], c["d"], c["dtype"]
    g = H // hkv
    (qb, qs, nq), (kb, ks, nk) = c["q"], c["k"]
    q, _, _ = workloads.qkv(3 * seed, H, nq, d, dtype)
    _, k, v = workloads.qkv(3 * seed + 1, hkv, nk, d, dtype)
    if c["kind"] == "causal":
        mask = cp.Mask.causal(c["n_pos"])
        omask = oracle.Causal(window=c["window"])
    else:
        seg, parent = c["tree"]
        mask = cp.Mask.tree(seg, parent)
        omask = oracle.Tree(seg, parent, window=c["window"])
    base = mask
    if c["window"]:
        mask = base.with_window(c["window"])
    tm = c["token_major"]
    qd, kd, vd = _place(q, tm), _place(k, tm), _place(v, tm)
    qpos, kpos = qb + qs * np.arange(nq), kb + ks * np.arange(nk)
    kr, vr = k.repeat_interleave(g, 0), v.repeat_interleave(g, 0)
    if c["k2"] is None:
        o, l = cp.partial(qd, kd, vd, mask, (qb, qs), (kb, ks))
        torch.cuda.synchronize()
        O, L = oracle.attention(q, kr, vr, qpos, kpos, omask)
    else:
        # a second key block first, then the main one merged into it
        kb2, ks2, nk2 = c["k2"]
        _, k2, v2 = workloads.qkv(3 * seed + 2, hkv, nk2, d, dtype)
        run = cp.partial(qd, _place(k2, tm), _place(v2, tm), mask, (qb, qs), (kb2, ks2))
        o, l = cp.partial(qd, kd, vd, mask, (qb, qs), (kb, ks), out=run, accumulate=True)
        torch.cuda.synchronize()
        O, L = oracle.attention(q, torch.cat([k2.repeat_interleave(g, 0), kr], 1),
                                torch.cat([v2.repeat_interleave(g, 0), vr], 1), qpos,
                                np.concatenate([kb2 + ks2 * np.arange(nk2), kpos]), omask)
    _cmp(o, l, O, L, dtype, what)
    if c["backward"]:
        gen = torch.Generator().manual_seed(seed)
        G = torch.randn((H, nq, d), generator=gen)
        G = G.to(torch.bfloat16) if dtype == "bf16" else G
        Gd = _place(G, tm)
        delta = cp.backward_delta(o, Gd)
        grads = cp.partial_backward(qd, kd, vd, mask, l, delta, Gd, (qb, qs), (kb, ks))
        torch.cuda.synchronize()
        rq, rk, rv = oracle.attention_backward(q, kr, vr, qpos, kpos, O, L, G.double().numpy(), omask)
        refs = (rq, rk.reshape(hkv, g, nk, d).sum(1), rv.reshape(hkv, g, nk, d).sum(1))
        for got, ref, name in zip(grads, refs, ("dq", "dk", "dv")):
            err = float(np.abs(got.double().cpu().numpy() - ref).max()) if ref.size else 0.0
            tol = 1e-4 if dtype == "f32" else 1e-2 * float(np.abs(ref).max()) + 1e-4
            assert err <= tol, "%s: %s max|err| %.2e > %.2e" % (what, name, err, tol)
    if mask is not base:
        mask.free()
    base.free()
