"""GPU parity where the online softmax's reference maximum has to move, and
for large scores ("Context Parallelism in ART", section 02: the summary is
kept in log space so that exp(s) does not overflow when scores are large).

Both forward kernels walk a query tile's key tiles from the highest key index
down (own run first, then the ancestor runs root-ward: still descending) and
keep, per query row, a reference m in base-2 units:

* fp32 inputs: m is raised to a tile's maximum whenever that maximum exceeds
  m by more than 8, and the accumulated output and denominator are rescaled;
* bf16 inputs: once a row has a reference, a tile's probabilities are taken
  against it without the tile's maximum and kept if every lane's sum of them
  stays within 2^16; otherwise the tile is redone with the maximum (the
  reference raised by the fp32 rule, accumulated state rescaled).

Inputs here make those raises happen after state has been accumulated:

* "staircase" scores: Q[:, :, 0] = 8 and K[:, j, 0] a step function that
  rises toward lower key indices (by about `step` base-2 units every `period`
  keys), on top of N(0, 1) in the other dimensions; the test computes on the
  host, from the fp64 scores and the kernels' tile walk, how many rows per
  head meet a tile whose maximum lies more than 16 above their running
  reference after keys were accumulated (both kernels must raise there) and
  requires at least 8 per head;
* Q and K scaled by 4 (bf16/fp32 rounding of 4 z) and by 30 (integers
  round(30 z): every product and partial sum of q.k is then an exact fp32
  integer, so the scores themselves carry no rounding);
* softmax scales other than 1/sqrt(d);
* the backward on the same inputs.

Tolerances.  The base bounds are the ones used throughout (fp32 inputs 1e-5,
bf16 inputs 2e-2 on O and 1e-3 on LSE).  With scores of magnitude |s| the fp32
arithmetic itself (the scale multiplication, the subtraction of the
reference, LSE = ln2 (m + log2 l)) rounds at about 2^-24 |s|, so each row's
bound adds delta = 16 * 2^-24 * max(|L|, max_j |s_j|) + scale * e_dot, where
e_dot = d * 2^-24 * max_j sum_c |q_c k_jc| bounds the fp32 accumulation of the
dot products (0 for the integer inputs).  LSE gets base + delta (LSE is
1-Lipschitz in the scores); O gets base + (exp(2 delta) - 1) * 2 max|V| (each
softmax weight moves by at most a factor exp(+-2 delta)).
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu

BASE = {"f32": (1e-5, 1e-5), "bf16": (2e-2, 1e-3)}
U = 2.0 ** -24
LOG2E = 1.0 / math.log(2.0)
# key tile of each forward kernel (bf16: ping-pong kernel; fp32: register-staged kernel)
BN = {"bf16": 64, "f32": 32}
TAU = 8.0          # reference raise threshold (base 2) of the exact path
SUM_CAP = 16.0     # bf16 fast path: log2 of the largest per-lane tile sum kept


@pytest.fixture(scope="module")
def cp():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import context_blockwise_attention_amd as cpattn
    cpattn.lib()
    return cpattn


def _cast(x, dtype):
    return x.to(torch.bfloat16) if dtype == "bf16" else x.float()


# ----------------------------------------------------------------------------
# inputs
# ----------------------------------------------------------------------------
def _staircase(seed, H, nq, nk, d, dtype, step, period, scale):
    """N(0, 1) inputs with q[..., 0] = 8 and k[j, 0] rising by `step` base-2
    units of score every `period` keys toward lower key indices."""
    q, _, _ = workloads.qkv(seed, H, nq, d, "f32")
    _, k, v = workloads.qkv(seed + 1, H, nk, d, "f32")
    q[:, :, 0] = 8.0
    level = ((nk - 1 - np.arange(nk)) // period).astype(np.float32)
    k[:, :, 0] = torch.from_numpy(level * (step / (8.0 * scale * LOG2E)))[None, :]
    return _cast(q, dtype), _cast(k, dtype), _cast(v, dtype)


def _scaled(seed, H, nq, nk, d, dtype, factor):
    q, _, _ = workloads.qkv(seed, H, nq, d, "f32")
    _, k, v = workloads.qkv(seed + 1, H, nk, d, "f32")
    if factor == 30:
        q, k = torch.round(q * 30), torch.round(k * 30)   # integers of magnitude < 256: exact in bf16
    else:
        q, k = q * factor, k * factor
    return _cast(q, dtype), _cast(k, dtype), _cast(v, dtype)


# ----------------------------------------------------------------------------
# host-side visibility and scores (fp64, for bounds and walk emulation)
# ----------------------------------------------------------------------------
def _visible(qpos, kpos, tree=None, window=0):
    qpos = np.asarray(qpos)[:, None]
    kpos = np.asarray(kpos)[None, :]
    if tree is None:
        vis = kpos <= qpos
        if window:
            vis &= qpos - kpos < window
        return vis
    seg, parent = np.asarray(tree[0]), np.asarray(tree[1])
    n_seg = len(parent)
    anc = np.zeros((n_seg, n_seg), bool)   # anc[s, a]: a is a strict ancestor of s
    for s in range(n_seg):
        a = parent[s]
        while a >= 0:
            anc[s, a] = True
            a = parent[a]
    sq, sk = seg[qpos[:, 0]][:, None], seg[kpos[0]][None, :]
    return ((sq == sk) & (kpos <= qpos)) | anc[sq, sk]


def _scores(q, k, h, scale):
    qh = q[h].double().numpy()
    kh = k[h].double().numpy()
    return scale * (qh @ kh.T), scale * (np.abs(qh) @ np.abs(kh).T)


def _row_delta(q, k, v, vis, scale, L_ref, exact_dots):
    """delta per (head, row): see the module docstring."""
    H, nq, d = q.shape
    out = np.zeros((H, nq))
    for h in range(H):
        s, sabs = _scores(q, k, h, scale)
        smax = np.where(vis, np.abs(s), 0.0).max(axis=1)
        e_dot = 0.0 if exact_dots else d * U * np.where(vis, sabs, 0.0).max(axis=1)
        lh = np.where(np.isfinite(L_ref[h]), np.abs(L_ref[h]), 0.0)
        out[h] = 16 * U * np.maximum(lh, smax) + e_dot
    return out


def _compare(o, l, O_ref, L_ref, dtype, delta, vmax, what):
    bo, bl = BASE[dtype]
    o = o.detach().double().cpu().numpy()
    l = l.detach().double().cpu().numpy()
    fin = np.isfinite(L_ref)
    assert np.array_equal(np.isfinite(l), fin), "%s: empty-row pattern differs" % what
    assert np.all(np.isfinite(o)), "%s: non-finite output" % what
    tol_l = bl + delta
    tol_o = bo + np.expm1(2 * delta) * 2 * vmax
    el = np.where(fin, np.abs(l - np.where(fin, L_ref, 0.0)), 0.0)
    eo = np.abs(o - O_ref).max(axis=2)
    print("  %s: max|dO| %.2e (tol <= %.2e), max|dLSE| %.2e (tol <= %.2e), max|L| %.1f" % (
        what, eo.max(), tol_o.max(), el.max(), tol_l.max(), np.abs(L_ref[fin]).max() if fin.any() else 0.0),
        flush=True)
    assert np.all(el <= tol_l), "%s: LSE out of bound (worst excess %.2e)" % (what, (el - tol_l).max())
    assert np.all(eo <= tol_o), "%s: O out of bound (worst excess %.2e)" % (what, (eo - tol_o).max())


# ----------------------------------------------------------------------------
# emulation of the reference raises along the tile walk
# ----------------------------------------------------------------------------
def _raises_with_state(s_log2, vis, bn, jump=SUM_CAP):
    """Rows whose running reference (raised by more than TAU) meets, after
    keys were accumulated, a tile whose maximum exceeds it by more than
    `jump`; the walk visits key tiles of `bn` keys from the last one down."""
    nq, nk = s_log2.shape
    m = np.full(nq, -np.inf)
    acc = np.zeros(nq, bool)
    hit = np.zeros(nq, bool)
    for t in range((nk - 1) // bn, -1, -1):
        sl = slice(t * bn, min(nk, (t + 1) * bn))
        st = np.where(vis[:, sl], s_log2[:, sl], -np.inf)
        mt = st.max(axis=1)
        hit |= acc & (mt > m + jump)
        raise_ = mt > m + TAU
        m = np.where(raise_, mt, m)
        acc |= np.isfinite(mt)
    return hit


def _require_raises(q, k, vis, scale, dtype, what, need=8):
    for h in range(q.shape[0]):
        s, _ = _scores(q, k, h, scale)
        n = int(_raises_with_state(s * LOG2E, vis, BN[dtype]).sum())
        print("  %s head %d: %d rows raise their reference with state" % (what, h, n), flush=True)
        assert n >= need, "%s: the inputs do not exercise the raise (head %d: %d rows)" % (what, h, n)


# ----------------------------------------------------------------------------
# partials
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("step", [10.0, 24.0])
def test_staircase_causal(cp, dtype, d, step):
    H, n = 2, 1536
    scale = 1.0 / math.sqrt(d)
    q, k, v = _staircase(100, H, n, n, d, dtype, step, 3 * BN[dtype], scale)
    pos = np.arange(n)
    vis = _visible(pos, pos)
    if step > SUM_CAP:
        _require_raises(q, k, vis, scale, dtype, "causal staircase")
    mask = cp.Mask.causal(n)
    o, l = cp.partial(q.cuda(), k.cuda(), v.cuda(), mask)
    O, L = oracle.attention(q, k, v, pos, pos, oracle.Causal())
    delta = _row_delta(q, k, v, vis, scale, L, exact_dots=False)
    _compare(o, l, O, L, dtype, delta, float(v.abs().max()), "causal staircase step %g" % step)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_staircase_offsets_window(cp, dtype):
    """Ragged block sizes, offset positions and a sliding window."""
    H, d, nq, nk, qbase, kbase, window = 2, 128, 900, 1300, 700, 100, 1000
    scale = 1.0 / math.sqrt(d)
    q, k, v = _staircase(110, H, nq, nk, d, dtype, 24.0, 2 * BN[dtype], scale)
    qpos, kpos = qbase + np.arange(nq), kbase + np.arange(nk)
    vis = _visible(qpos, kpos, window=window)
    _require_raises(q, k, vis, scale, dtype, "windowed staircase")
    mask = cp.Mask.causal(qbase + nq).with_window(window)
    o, l = cp.partial(q.cuda(), k.cuda(), v.cuda(), mask, (qbase, 1), (kbase, 1))
    O, L = oracle.attention(q, k, v, qpos, kpos, oracle.Causal(window=window))
    delta = _row_delta(q, k, v, vis, scale, L, exact_dots=False)
    _compare(o, l, O, L, dtype, delta, float(v.abs().max()), "windowed staircase")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_staircase_striped(cp, dtype):
    H, d, P, n = 2, 128, 4, 800
    scale = 1.0 / math.sqrt(d)
    q, k, v = _staircase(120, H, n * P, n * P, d, dtype, 24.0, 2 * BN[dtype], scale)
    lay = workloads.striped(n * P, P)
    mask = cp.Mask.causal(n * P)
    for b in (0, 1, 3):
        qq, kk, vv = q[:, lay[0]], k[:, lay[b]], v[:, lay[b]]
        vis = _visible(lay[0], lay[b])
        _require_raises(qq, kk, vis, scale, dtype, "striped staircase %d" % b)
        o, l = cp.partial(qq.contiguous().cuda(), kk.contiguous().cuda(), vv.contiguous().cuda(), mask, (0, P),
                          (b, P))
        O, L = oracle.attention(qq, kk, vv, lay[0], lay[b], oracle.Causal())
        delta = _row_delta(qq, kk, vv, vis, scale, L, exact_dots=False)
        _compare(o, l, O, L, dtype, delta, float(v.abs().max()), "striped staircase, stripe %d" % b)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_staircase_tree(cp, dtype):
    seg, parent = workloads.tree_prompt_completions(700, (300, 450, 200, 350))
    n = len(seg)
    H, d = 2, 128
    scale = 1.0 / math.sqrt(d)
    q, k, v = _staircase(130, H, n, n, d, dtype, 24.0, 2 * BN[dtype], scale)
    pos = np.arange(n)
    vis = _visible(pos, pos, tree=(seg, parent))
    _require_raises(q, k, vis, scale, dtype, "tree staircase")
    mask = cp.Mask.tree(seg, parent)
    o, l = cp.partial(q.cuda(), k.cuda(), v.cuda(), mask)
    O, L = oracle.attention(q, k, v, pos, pos, oracle.Tree(seg, parent))
    delta = _row_delta(q, k, v, vis, scale, L, exact_dots=False)
    _compare(o, l, O, L, dtype, delta, float(v.abs().max()), "tree staircase")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_staircase_tree_ring(cp, dtype):
    """Ring of 4 over a packed tree: every round's partial merged into the
    running result by the kernel epilogue, at large LSE values."""
    seg, parent = workloads.tree_prompt_completions(640, (384, 512, 256, 256))
    n = len(seg)
    N, H, d = 4, 2, 128
    c = n // N
    scale = 1.0 / math.sqrt(d)
    q, k, v = _staircase(140, H, n, n, d, dtype, 24.0, 3 * BN[dtype], scale)
    mask = cp.Mask.tree(seg, parent)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    sl = [slice(r * c, (r + 1) * c) for r in range(N)]
    out = cp.ring_emulate([qd[:, s] for s in sl], [kd[:, s] for s in sl], [vd[:, s] for s in sl],
                          [(r * c, 1) for r in range(N)], mask)
    pos = np.arange(n)
    O, L = oracle.attention(q, k, v, pos, pos, oracle.Tree(seg, parent))
    vis = _visible(pos, pos, tree=(seg, parent))
    delta = _row_delta(q, k, v, vis, scale, L, exact_dots=False)
    # raises inside each round's key block
    for r in range(N):
        for b in range(r + 1):
            vb = vis[sl[r], sl[b]]
            if vb.any() and b == r:
                _require_raises(q[:, sl[r]], k[:, sl[b]], vb, scale, dtype, "ring rank %d block %d" % (r, b))
    for r in range(N):
        _compare(out[r][0], out[r][1], O[:, sl[r]], L[:, sl[r]], dtype, delta[:, sl[r]], float(v.abs().max()),
                 "tree staircase ring, rank %d" % r)


# ----------------------------------------------------------------------------
# Q and K scaled by 4 and by 30; non-default softmax scales
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("factor", [4, 30])
@pytest.mark.parametrize("maskname", ["causal", "tree"])
def test_scaled_qk(cp, dtype, factor, maskname):
    H, d = 2, 128
    if maskname == "causal":
        n = 1100
        mask, omask, tree = cp.Mask.causal(n), oracle.Causal(), None
    else:
        seg, parent = workloads.tree_prompt_completions(400, (250, 180, 300))
        n = len(seg)
        mask, omask, tree = cp.Mask.tree(seg, parent), oracle.Tree(seg, parent), (seg, parent)
    scale = 1.0 / math.sqrt(d)
    q, k, v = _scaled(150 + factor, H, n, n, d, dtype, factor)
    pos = np.arange(n)
    o, l = cp.partial(q.cuda(), k.cuda(), v.cuda(), mask)
    O, L = oracle.attention(q, k, v, pos, pos, omask)
    assert np.all(np.isfinite(L)), "every row sees its own key"
    vis = _visible(pos, pos, tree=tree)
    delta = _row_delta(q, k, v, vis, scale, L, exact_dots=(factor == 30))
    _compare(o, l, O, L, dtype, delta, float(v.abs().max()), "%s x%d" % (maskname, factor))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("factor", [4, 30])
def test_scaled_qk_ring(cp, dtype, factor):
    seg, parent = workloads.tree_prompt_completions(384, (128, 200, 96, 160))
    n = len(seg) // 4 * 4
    seg = seg[:n]
    N, H, d = 4, 2, 64
    c = n // N
    scale = 1.0 / math.sqrt(d)
    q, k, v = _scaled(170 + factor, H, n, n, d, dtype, factor)
    mask = cp.Mask.tree(seg, parent)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    sl = [slice(r * c, (r + 1) * c) for r in range(N)]
    out = cp.ring_emulate([qd[:, s] for s in sl], [kd[:, s] for s in sl], [vd[:, s] for s in sl],
                          [(r * c, 1) for r in range(N)], mask)
    pos = np.arange(n)
    O, L = oracle.attention(q, k, v, pos, pos, oracle.Tree(seg, parent))
    delta = _row_delta(q, k, v, _visible(pos, pos, tree=(seg, parent)), scale, L, exact_dots=(factor == 30))
    for r in range(N):
        _compare(out[r][0], out[r][1], O[:, sl[r]], L[:, sl[r]], dtype, delta[:, sl[r]], float(v.abs().max()),
                 "ring x%d rank %d" % (factor, r))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("mult", [0.3, 3.0])
@pytest.mark.parametrize("maskname", ["causal", "tree"])
def test_nondefault_scale(cp, dtype, mult, maskname):
    H, d = 2, 128
    if maskname == "causal":
        n, qbase = 700, 0
        mask, omask, tree = cp.Mask.causal(n), oracle.Causal(), None
    else:
        seg, parent = workloads.tree_prompt_completions(300, (200, 150, 250))
        n = len(seg)
        mask, omask, tree = cp.Mask.tree(seg, parent), oracle.Tree(seg, parent), (seg, parent)
    scale = mult / math.sqrt(d)
    q, k, v = workloads.qkv(190, H, n, d, dtype)
    pos = np.arange(n)
    o, l = cp.partial(q.cuda(), k.cuda(), v.cuda(), mask, scale=scale)
    O, L = oracle.attention(q, k, v, pos, pos, omask, scale=scale)
    delta = _row_delta(q, k, v, _visible(pos, pos, tree=tree), scale, L, exact_dots=False)
    _compare(o, l, O, L, dtype, delta, float(v.abs().max()), "%s scale x%g" % (maskname, mult))
    # the same scale through the ring (fused merge)
    N = 4
    c = n // N
    sl = [slice(r * c, (r + 1) * c) for r in range(N)]
    qd, kd, vd = q[:, :N * c].cuda(), k[:, :N * c].cuda(), v[:, :N * c].cuda()
    if tree is not None:
        mask2 = cp.Mask.tree(seg[:N * c], parent)
    else:
        mask2 = cp.Mask.causal(N * c)
    out = cp.ring_emulate([qd[:, s] for s in sl], [kd[:, s] for s in sl], [vd[:, s] for s in sl],
                          [(r * c, 1) for r in range(N)], mask2, scale=scale)
    p2 = np.arange(N * c)
    om2 = oracle.Tree(seg[:N * c], parent) if tree is not None else oracle.Causal()
    O2, L2 = oracle.attention(q[:, :N * c], k[:, :N * c], v[:, :N * c], p2, p2, om2, scale=scale)
    for r in range(N):
        _compare(out[r][0], out[r][1], O2[:, sl[r]], L2[:, sl[r]], dtype, delta[:, sl[r]], float(v.abs().max()),
                 "%s scale x%g ring rank %d" % (maskname, mult, r))


# ----------------------------------------------------------------------------
# the backward on the same inputs
# ----------------------------------------------------------------------------
U_BF16 = 2.0 ** -8   # unit roundoff of bf16 (8 significant bits)
UF = 2.0 ** -125     # largest probability that may underflow to zero in fp32


def _grad_bounds(q, k, v, G, L, D, vis, scale, dtype):
    """Per-element worst-case bounds for the backward from the magnitudes of
    each gradient's terms, dS = P (dP - D) with P = exp(s - L):
      dQ[i, c] = scale sum_j dS[i, j] K[j, c],  dK[j, c] = scale sum_i dS[i, j] Q[i, c],
      dV[j, c] = sum_i P[i, j] G[i, c].
    * P[i, j] moves by a relative rho = exp(e) - 1, where e bounds the score's
      error: the fp32 dot product ((d + 2) 2^-24 scale sum_c |q_c k_c|) plus
      the exponent's rounding (16 * 2^-24 max(|s|, |L|));
    * dP = dot(dO, v) carries (d + 2) 2^-24 sum_c |dO_c v_c|, D its fp32
      rounding 2^-24 |D|;
    * bf16 inputs: P and dS are rounded to bf16 (2^-8) for the MFMAs;
    * the gradient sums accumulate in fp32: n 2^-24 sum |terms| over n terms;
    * a probability below fp32's normal range (2^-126) may become zero: at
      most 2^-125 of absolute error per probability (the reference's tiniest
      gradients, ~1e-46 here, are then zero on the GPU)."""
    H, n, d = q.shape
    ust = U_BF16 if dtype == "bf16" else 0.0
    bq, bk, bv = [], [], []
    for h in range(H):
        s, sabs = _scores(q, k, h, scale)
        Lh = L[h][:, None]
        P = np.where(vis, np.exp(np.minimum(np.where(vis, s, 0.0) - Lh, 0.0)), 0.0)
        gh, vh = G[h].double().numpy(), v[h].double().numpy()
        qh, kh = q[h].double().numpy(), k[h].double().numpy()
        dP = gh @ vh.T
        e_dp = (d + 2) * U * (np.abs(gh) @ np.abs(vh).T)
        rho = np.expm1((d + 2) * U * sabs + 16 * U * np.maximum(np.abs(s), np.abs(Lh)))
        dS = P * (dP - D[h][:, None])
        e_ds = P * (rho * np.abs(dP - D[h][:, None]) + e_dp + U * np.abs(D[h][:, None])) + ust * np.abs(dS)
        e_ds = np.where(vis, e_ds + UF * (np.abs(dP - D[h][:, None]) + e_dp + 1.0), 0.0)
        aq, ak = np.abs(qh), np.abs(kh)
        acc_q = n * U * scale * (np.abs(dS) @ ak)
        acc_k = n * U * scale * (np.abs(dS).T @ aq)
        bq.append(scale * (e_ds @ ak) + acc_q)
        bk.append(scale * (e_ds.T @ aq) + acc_k)
        bv.append(((P * (rho + ust) + np.where(vis, UF, 0.0)).T @ np.abs(gh)) + n * U * (P.T @ np.abs(gh)))
    return np.stack(bq), np.stack(bk), np.stack(bv)


def _check_grad(name, got, ref, bound):
    got = got.double().cpu().numpy()
    err = np.abs(got - ref)
    ratio = np.where(err > 0, err / np.where(bound > 0, bound, 1.0), 0.0)
    print("  %s: max|err| %.2e, max err/bound %.3f, max|ref| %.2e" % (
        name, float(err.max()), float(ratio.max()), float(np.abs(ref).max())), flush=True)
    assert np.all(err <= bound), name


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("inputs", ["staircase", "x4", "x30"])
def test_backward_large_scores(cp, dtype, inputs):
    """Gradients with the global softmax derivative, p = exp(s - L), on the
    inputs above.  The backward kernels get the reference's L and
    D = dot(dO, O) (rounded to fp32), so only their own arithmetic is
    compared.  Bounds: the per-element worst-case bounds of _grad_bounds
    (plus 1e-5 for fp32 inputs).  The staircase makes dQ's first dimension a
    sum of large, cancelling terms (the visible keys of a stair share
    K[j, 0] ~ 1e2), so there the score and probability roundings dominate."""
    seg, parent = workloads.tree_prompt_completions(300, (180, 240, 150))
    n = len(seg)
    H, d = 2, 128
    scale = 1.0 / math.sqrt(d)
    if inputs == "staircase":
        q, k, v = _staircase(200, H, n, n, d, dtype, 24.0, 2 * BN[dtype], scale)
    else:
        q, k, v = _scaled(210, H, n, n, d, dtype, 4 if inputs == "x4" else 30)
    g = torch.Generator().manual_seed(211)
    G = _cast(torch.randn((H, n, d), generator=g), dtype)
    mask, omask = cp.Mask.tree(seg, parent), oracle.Tree(seg, parent)
    pos = np.arange(n)
    O, L = oracle.attention(q, k, v, pos, pos, omask)
    D = np.einsum("hnd,hnd->hn", G.double().numpy(), O)
    qd, kd, vd, gd = q.cuda(), k.cuda(), v.cuda(), G.cuda()
    Ld = torch.from_numpy(L.astype(np.float32)).cuda()
    Dd = torch.from_numpy(D.astype(np.float32)).cuda()
    dq, dk, dv = cp.partial_backward(qd, kd, vd, mask, Ld, Dd, gd)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.attention_backward(q, k, v, pos, pos, O, L, G.double().numpy(), omask)
    vis = _visible(pos, pos, tree=(seg, parent))
    bounds = [b + (1e-5 if dtype == "f32" else 0.0)
              for b in _grad_bounds(q, k, v, G, L, D, vis, scale, dtype)]
    _check_grad("dq " + inputs, dq, rq, bounds[0])
    _check_grad("dk " + inputs, dk, rk, bounds[1])
    _check_grad("dv " + inputs, dv, rv, bounds[2])
