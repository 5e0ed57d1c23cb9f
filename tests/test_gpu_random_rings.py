"""Seeded random rings (GPU): the ring entry points with their features
drawn together, every rank's result against the fp64 reference.

Each seed draws a ring of N ranks (1 to 40: rings past 16 ranks need more
than one launch per round, since a launch holds at most 16 jobs) holding one
block or two chunks each, laid out contiguously, striped (rank r holds the
positions x with x mod N = r) or zig-zag (rank r holds chunks r and 2N-1-r),
a causal mask or a random preorder tree with or without a sliding window,
grouped-query heads, bf16 or fp32, d 64 or 128, sometimes only some ranks
run, and sometimes the ring backward.  In round k rank r visits the keys of
rank (r - k) mod N (ML-systems lesson on sequence/context parallelism, the
ring-attention section), so every rank ends with attention over all keys.
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


def _tree_with_total(rng, n):
    """A random preorder tree whose segments hold n tokens in all."""
    n_seg = int(rng.integers(1, min(12, n) + 1))
    cuts = np.sort(rng.choice(np.arange(1, n), size=n_seg - 1, replace=False)) if n_seg > 1 else np.array([], int)
    lens = np.diff(np.concatenate([[0], cuts, [n]])).tolist()
    parent = [-1] + [int(rng.integers(-1, s)) for s in range(1, n_seg)]
    kids = {s: [] for s in range(-1, n_seg)}
    for s, p in enumerate(parent):
        kids[p].append(s)
    order, stack = [], list(reversed(kids[-1]))
    while stack:
        s = stack.pop()
        order.append(s)
        stack.extend(reversed(kids[s]))
    new = {s: i for i, s in enumerate(order)}
    par = [-1 if parent[s] < 0 else new[parent[s]] for s in order]
    return workloads.tree_from_lengths(lens, par)


def _case(seed):
    rng = np.random.default_rng(7000 + seed)
    c = {"N": int(rng.choice([1, 2, 3, 4, 5, 8, 12, 17, 24, 40]))}
    c["layout"] = str(rng.choice(["contiguous", "striped", "zigzag", "chunks"]))
    c["C"] = 2 if c["layout"] in ("zigzag", "chunks") else 1
    c["c"] = int(rng.integers(1, max(1, 800 // (c["N"] * c["C"])) + 1))
    c["n"] = c["N"] * c["C"] * c["c"]
    c["kind"] = str(rng.choice(["causal", "tree"]))
    if c["kind"] == "tree":
        c["tree"] = _tree_with_total(rng, c["n"])
    c["window"] = int(rng.integers(1, 300)) if rng.random() < 0.4 else 0
    c["dtype"] = str(rng.choice(["bf16", "f32"]))
    c["d"] = int(rng.choice([64, 128]))
    c["hkv"] = int(rng.choice([1, 2]))
    c["H"] = c["hkv"] * int(rng.choice([1, 2]))
    c["ranks"] = None
    if c["N"] > 1 and rng.random() < 0.25:
        c["ranks"] = sorted(rng.choice(c["N"], size=int(rng.integers(1, c["N"] + 1)), replace=False).tolist())
    c["backward"] = c["ranks"] is None and rng.random() < 0.5
    return c


def _chunk_positions(c):
    """Global positions of each chunk (chunk i = r * C + j) and its posmap."""
    N, C, cc = c["N"], c["C"], c["c"]
    ar = np.arange(cc)
    if c["layout"] == "contiguous" or c["layout"] == "chunks":
        return [(i * cc + ar, (i * cc, 1)) for i in range(N * C)]
    if c["layout"] == "striped":
        return [(r + N * ar, (r, N)) for r in range(N)]
    out = []
    for r in range(N):
        for blk in (r, 2 * N - 1 - r):
            out.append((blk * cc + ar, (blk * cc, 1)))
    return out


@pytest.mark.parametrize("seed", range(120))
def test_random_ring(cp, seed):
    c = _case(seed)
    what = "seed %d: %s" % (seed, {k: v for k, v in c.items() if k != "tree"})
    print(what, flush=True)
    N, C, n, H, hkv, d, dtype = c["N"], c["C"], c["n"], c["H"], c["hkv"], c["d"], c["dtype"]
    g = H // hkv
    q, _, _ = workloads.qkv(5 * seed, H, n, d, dtype)
    _, k, v = workloads.qkv(5 * seed + 1, hkv, n, d, dtype)
    if c["kind"] == "causal":
        base, omask = cp.Mask.causal(n), oracle.Causal(window=c["window"])
    else:
        seg, parent = c["tree"]
        base, omask = cp.Mask.tree(seg, parent), oracle.Tree(seg, parent, window=c["window"])
    mask = base.with_window(c["window"]) if c["window"] else base
    chunks = _chunk_positions(c)
    take = lambda t, p: t[:, torch.from_numpy(p)].contiguous().cuda()
    Q = [take(q, p) for p, _ in chunks]
    K = [take(k, p) for p, _ in chunks]
    V = [take(v, p) for p, _ in chunks]
    pos = [pm for _, pm in chunks]
    if C == 1:
        out = cp.ring_emulate(Q, K, V, pos, mask, ranks=c["ranks"])
        units = {r: r for r in (c["ranks"] if c["ranks"] is not None else range(N))}
    else:
        out = cp.ring_emulate_chunks(Q, K, V, pos, mask, chunks_per_rank=C, ranks=c["ranks"])
        run = c["ranks"] if c["ranks"] is not None else range(N)
        units = {r * C + j: r * C + j for r in run for j in range(C)}
    torch.cuda.synchronize()
    allpos = np.arange(n)
    kr, vr = k.repeat_interleave(g, 0), v.repeat_interleave(g, 0)
    O, L = oracle.attention(q, kr, vr, allpos, allpos, omask)
    assert sorted(out.keys()) == sorted(units.keys())
    for i in units:
        p = chunks[i][0]
        _cmp(out[i][0], out[i][1], O[:, p], L[:, p], dtype, "%s, chunk %d" % (what, i))
    if c["backward"]:
        G = torch.randn((H, n, d), generator=torch.Generator().manual_seed(seed))
        G = G.to(torch.bfloat16) if dtype == "bf16" else G
        Gs = [take(G, p) for p, _ in chunks]
        deltas = [cp.backward_delta(out[i][0], Gs[i]) for i in range(N * C)]
        lses = [out[i][1] for i in range(N * C)]
        if C == 1:
            grads = cp.ring_backward(Q, K, V, pos, mask, lses, deltas, Gs)
        else:
            grads = cp.ring_backward_chunks(Q, K, V, pos, mask, lses, deltas, Gs, chunks_per_rank=C)
        torch.cuda.synchronize()
        rq, rk, rv = oracle.attention_backward(q, kr, vr, allpos, allpos, O, L, G.double().numpy(), omask)
        refs = (rq, rk.reshape(hkv, g, n, d).sum(1), rv.reshape(hkv, g, n, d).sum(1))
        for j, name in enumerate(("dq", "dk", "dv")):
            got = np.zeros(refs[j].shape)
            for i, (p, _) in enumerate(chunks):
                got[:, p] = grads[i][j].double().cpu().numpy()
            err = float(np.abs(got - refs[j]).max())
            tol = 1e-4 if dtype == "f32" else 1e-2 * float(np.abs(refs[j]).max()) + 1e-4
            assert err <= tol, "%s: %s max|err| %.2e > %.2e" % (what, name, err, tol)
    if mask is not base:
        mask.free()
    base.free()
