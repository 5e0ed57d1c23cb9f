"""Adjoints of the merge and of the sink step on the GPU (cpattn_merge_backward,
cpattn_sink_backward) against the fp64 reference's merge_backward and
sink_backward ("Context Parallelism in ART", sections 04 and 06), which are
pinned by finite differences in test_oracle_pins.py.

Inputs are fp32 on the GPU; the reference gets the same fp32 values widened
to fp64.  The kernels compute in fp32: a weight exp(L_p - L) carries a
relative error of a few ulp and a dot product over d terms of unit size an
absolute error of about d * 2^-24, so the bound is 2e-5 times the largest
reference magnitude (at least 1) for the per-row outputs, and 1e-4 for the
sink gradient, a sum over every row of a head.
"""
import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu

TOL_ROW = 2e-5
TOL_SUM = 1e-4


@pytest.fixture(scope="module")
def cp():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import context_blockwise_attention_amd as cpattn
    cpattn.lib()
    return cpattn


def _close(got, ref, tol, what):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, what
    fin = np.isfinite(ref)
    assert np.array_equal(np.isfinite(got), fin), "%s: non-finite entries differ" % what
    err = np.abs(got[fin] - ref[fin]).max(initial=0.0)
    bound = tol * max(1.0, np.abs(ref[fin]).max(initial=0.0))
    assert err <= bound, "%s: max error %.3e > %.3e" % (what, err, bound)


def _parts(rng, n_parts, H, n, d):
    """Partials (O_p, L_p) in fp32 with empty rows: some rows empty in some
    parts, the first rows empty in every part."""
    parts = []
    for p in range(n_parts):
        o = rng.standard_normal((H, n, d)).astype(np.float32)
        l = (2.0 * rng.standard_normal((H, n))).astype(np.float32)
        drop = rng.random((H, n)) < 0.2
        l[drop] = -np.inf
        o[drop] = 0.0
        l[:, :3] = -np.inf
        o[:, :3] = 0.0
        parts.append((o, l))
    return parts


@pytest.mark.parametrize("with_gl", [False, True])
@pytest.mark.parametrize("n_parts", [1, 3, 6])
@pytest.mark.parametrize("d", [64, 128])
def test_merge_backward(cp, d, n_parts, with_gl):
    rng = np.random.default_rng(100 * d + 10 * n_parts + with_gl)
    H, n = 4, 301
    parts = _parts(rng, n_parts, H, n, d)
    O, L = oracle.merge([(o.astype(np.float64), l.astype(np.float64)) for o, l in parts])
    O32, L32 = O.astype(np.float32), L.astype(np.float32)
    G = rng.standard_normal((H, n, d)).astype(np.float32)
    gL = rng.standard_normal((H, n)).astype(np.float32) if with_gl else None
    ref = oracle.merge_backward([(o.astype(np.float64), l.astype(np.float64)) for o, l in parts],
                                O32.astype(np.float64), L32.astype(np.float64), G.astype(np.float64),
                                None if gL is None else gL.astype(np.float64))
    dev = torch.device("cuda:0")
    tparts = [(torch.from_numpy(o).to(dev), torch.from_numpy(l).to(dev)) for o, l in parts]
    outs = cp.merge_backward(tparts, (torch.from_numpy(O32).to(dev), torch.from_numpy(L32).to(dev)),
                             torch.from_numpy(G).to(dev), None if gL is None else torch.from_numpy(gL).to(dev))
    torch.cuda.synchronize()
    for p, ((go, gl), (ro, rl)) in enumerate(zip(outs, ref)):
        _close(go.cpu().numpy(), ro, TOL_ROW, "dO part %d" % p)
        _close(gl.cpu().numpy(), rl, TOL_ROW, "dL part %d" % p)
    # rows empty in every part get zero gradients
    assert float(torch.stack([x[0][:, :3].abs().max() for x in outs]).max()) == 0.0


@pytest.mark.parametrize("d", [64, 128])
def test_sink_backward(cp, d):
    rng = np.random.default_rng(7 + d)
    H, n = 5, 403
    O = rng.standard_normal((H, n, d))
    L = 3.0 * rng.standard_normal((H, n))
    L[:, :4] = -np.inf          # rows with no visible key
    O[:, :4] = 0.0
    a = 2.0 * rng.standard_normal(H)
    Y, Lt = oracle.apply_sink(O, L, a)
    Y32, Lt32, a32 = Y.astype(np.float32), Lt.astype(np.float32), a.astype(np.float32)
    G = rng.standard_normal((H, n, d)).astype(np.float32)
    # the reference takes the result before the sink: recover it from the
    # same fp32 values the GPU gets (w = 1 - exp(a - L'), O = y / w)
    u = np.exp(a32.astype(np.float64)[:, None] - Lt32.astype(np.float64))
    w = 1.0 - u
    O_ref = np.where(w[..., None] > 0, Y32.astype(np.float64) / np.where(w > 0, w, 1.0)[..., None], 0.0)
    L_ref = np.where(w > 0, Lt32.astype(np.float64) + np.log(np.where(w > 0, w, 1.0)), -np.inf)
    rO, rL, ra = oracle.sink_backward(O_ref, L_ref, a32.astype(np.float64), G.astype(np.float64))
    dev = torch.device("cuda:0")
    gO, gL, ga = cp.sink_backward(torch.from_numpy(Y32).to(dev), torch.from_numpy(Lt32).to(dev),
                                  torch.from_numpy(a32).to(dev), torch.from_numpy(G).to(dev))
    torch.cuda.synchronize()
    _close(gO.cpu().numpy(), rO, TOL_ROW, "dO")
    _close(gL.cpu().numpy(), rL, TOL_ROW, "dL")
    _close(ga.cpu().numpy(), ra, TOL_SUM, "da")
    assert float(gO[:, :4].abs().max()) == 0.0 and float(gL[:, :4].abs().max()) == 0.0


def test_sink_backward_no_rows(cp):
    dev = torch.device("cuda:0")
    o = torch.zeros((3, 0, 64), device=dev)
    l = torch.zeros((3, 0), device=dev)
    a = torch.ones(3, device=dev)
    gO, gL, ga = cp.sink_backward(o, l, a, o.clone())
    torch.cuda.synchronize()
    assert ga.cpu().tolist() == [0.0, 0.0, 0.0]


def test_merge_backward_of_gpu_merge(cp):
    """The adjoint applied to the GPU's own merge of GPU partials (the path a
    training step takes), d 128, 4 parts, against the reference on the same
    fp32 values."""
    rng = np.random.default_rng(5)
    H, n, d = 8, 1000, 128
    parts = _parts(rng, 4, H, n, d)
    dev = torch.device("cuda:0")
    tparts = [(torch.from_numpy(o).to(dev), torch.from_numpy(l).to(dev)) for o, l in parts]
    Om, Lm = cp.merge(tparts)
    G = rng.standard_normal((H, n, d)).astype(np.float32)
    outs = cp.merge_backward(tparts, (Om, Lm), torch.from_numpy(G).to(dev))
    torch.cuda.synchronize()
    ref = oracle.merge_backward([(o.astype(np.float64), l.astype(np.float64)) for o, l in parts],
                                Om.cpu().numpy().astype(np.float64), Lm.cpu().numpy().astype(np.float64),
                                G.astype(np.float64))
    for p, ((go, gl), (ro, rl)) in enumerate(zip(outs, ref)):
        _close(go.cpu().numpy(), ro, TOL_ROW, "dO part %d" % p)
        _close(gl.cpu().numpy(), rl, TOL_ROW, "dL part %d" % p)
