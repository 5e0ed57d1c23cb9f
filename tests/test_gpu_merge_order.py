"""The merge in any order, on the GPU.

The lesson's ring-attention section notes that the log-sum-exp merge is
associative and commutative, so a ring may visit the key blocks in any order
("Context Parallelism in ART", section 03, says the same of the merge's
composition).  Here each rank's rounds are run through the kernel's fused
merge (cpattn_partial with accumulate) in the ring order, in reversed order
and in seeded random orders, and the materialised partials are merged by
cpattn_merge in permuted orders; every result must match the unpartitioned
fp64 reference at the usual bounds (fp32 inputs 1e-5 on every row; bf16
inputs 2e-2 on O and 1e-3 on LSE), and the orders must agree with each other
to within the same bounds.
"""
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


def _cmp(o, l, O_ref, L_ref, dtype, what):
    tol_o, tol_l = TOL[dtype]
    o = o.detach().double().cpu().numpy()
    l = l.detach().double().cpu().numpy()
    fin = np.isfinite(L_ref)
    assert np.array_equal(np.isfinite(l), fin), "%s: empty-row pattern differs" % what
    assert np.all(o[~fin] == 0), "%s: empty rows must be zero" % what
    do = float(np.abs(o - O_ref).max())
    dl = float(np.abs(l[fin] - L_ref[fin]).max()) if fin.any() else 0.0
    print("  %s: max|dO| %.2e max|dLSE| %.2e" % (what, do, dl), flush=True)
    assert do <= tol_o and dl <= tol_l, what


def _orders(N, r, seed):
    ring = [((r - kk) % N + N) % N for kk in range(N)]
    rng = np.random.default_rng(seed)
    return {"ring": ring, "reversed": ring[::-1],
            "random_a": [int(x) for x in rng.permutation(N)], "random_b": [int(x) for x in rng.permutation(N)]}


def _run_orders(cp, q, k, v, n, N, mask, omask, dtype, seed):
    c = n // N
    sl = [slice(b * c, (b + 1) * c) for b in range(N)]
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    pos = np.arange(n)
    O, L = oracle.attention(q, k, v, pos, pos, omask)
    for r in range(N):
        results = {}
        for name, order in _orders(N, r, seed + r).items():
            run = None
            for b in order:
                if run is None:
                    run = cp.partial(qd[:, sl[r]], kd[:, sl[b]], vd[:, sl[b]], mask, (r * c, 1), (b * c, 1))
                    run = (run[0].clone(), run[1].clone())
                else:
                    cp.partial(qd[:, sl[r]], kd[:, sl[b]], vd[:, sl[b]], mask, (r * c, 1), (b * c, 1), out=run,
                               accumulate=True)
            _cmp(run[0], run[1], O[:, sl[r]], L[:, sl[r]], dtype, "rank %d, fused merge, %s order" % (r, name))
            results[name] = run
        # materialised partials (empty ones included) merged in permuted orders
        parts = [cp.partial(qd[:, sl[r]], kd[:, sl[b]], vd[:, sl[b]], mask, (r * c, 1), (b * c, 1))
                 for b in range(N)]
        for name, order in _orders(N, r, 100 + seed + r).items():
            o, l = cp.merge([parts[b] for b in order])
            _cmp(o, l, O[:, sl[r]], L[:, sl[r]], dtype, "rank %d, cpattn_merge, %s order" % (r, name))
        # the orders against one another
        tol_o, tol_l = TOL[dtype]
        ref = results["ring"]
        fin = torch.isfinite(ref[1])
        for name, (o, l) in results.items():
            assert torch.equal(torch.isfinite(l), fin)
            assert float((o - ref[0]).abs().max()) <= tol_o
            assert float((l[fin] - ref[1][fin]).abs().max()) <= tol_l if bool(fin.any()) else True


def test_any_order_tiny_causal_fp32(cp):
    """The tiny causal workload: 1 head, d 64, 256 tokens in 4 blocks, fp32."""
    w = workloads.WORKLOADS["tiny_causal"]
    q, k, v = workloads.qkv(0, w.heads, w.n_tok, w.d, "f32")
    _run_orders(cp, q, k, v, w.n_tok, w.n_blocks, cp.Mask.causal(w.n_tok), oracle.Causal(), "f32", 0)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("N", [4, 8])
def test_any_order_packed_tree(cp, dtype, N):
    seg, parent = workloads.tree_prompt_completions(384, (128, 200, 96, 160))
    n = len(seg) // N * N
    seg = seg[:n]
    H, d = 2, 128
    q, k, v = workloads.qkv(7, H, n, d, dtype)
    _run_orders(cp, q, k, v, n, N, cp.Mask.tree(seg, parent), oracle.Tree(seg, parent), dtype, 10 * N)
