"""Pins for the fp64 CPU reference (``oracle/``), each against something other
than the reference itself: values the pages print (``tests/golden``), closed
forms, invariants the pages state, library routines for special cases, and a
dense brute force whose mask is built a different way (from trajectories).
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rand(rng, *shape):
    return rng.standard_normal(shape)


# ----------------------------------------------------------------------------
# helpers that do not go through the reference's predicate
# ----------------------------------------------------------------------------
def _trajectory_mask(seg, parent, window=0):
    """Dense visibility built from root-to-leaf trajectories: a packed tree
    must behave as every trajectory run separately as a causal sequence
    (Context Parallelism in ART, section 01).  M[q, k] is True iff some
    trajectory contains both and k comes no later than q in it (and, with a
    window, fewer than `window` tokens before it in that trajectory:
    section 06, sliding windows on the root-to-leaf path)."""
    seg = np.asarray(seg)
    parent = np.asarray(parent)
    n_seg = len(parent)
    children = {s: [] for s in range(n_seg)}
    for s, p in enumerate(parent):
        if p >= 0:
            children[int(p)].append(s)
    leaves = [s for s in range(n_seg) if not children[s]]
    n = len(seg)
    M = np.zeros((n, n), dtype=bool)
    for leaf in leaves:
        path = []
        s = leaf
        while s >= 0:
            path.append(s)
            s = int(parent[s])
        path.reverse()
        toks = np.concatenate([np.flatnonzero(seg == s) for s in path])
        for a in range(len(toks)):
            lo = 0 if window <= 0 else max(0, a - window + 1)
            M[toks[a], toks[lo: a + 1]] = True
    return M


def _dense_attention(Q, K, V, M, scale):
    """Dense fp64 softmax attention over a boolean mask (one head)."""
    S = (Q @ K.T) * scale
    S = np.where(M, S, -np.inf)
    m = S.max(axis=1, keepdims=True)
    m_safe = np.where(np.isfinite(m), m, 0.0)
    P = np.exp(S - m_safe)
    Z = P.sum(axis=1, keepdims=True)
    with np.errstate(divide="ignore", invalid="ignore"):
        L = (m_safe + np.log(Z))[:, 0]
        O = np.where(Z > 0, (P / Z) @ V, 0.0)
    L = np.where(Z[:, 0] > 0, L, -np.inf)
    return O, L


def _random_tree(rng, n_seg, min_len=1, max_len=9):
    """A random tree laid out in depth-first preorder."""
    parent = [-1]
    for s in range(1, n_seg):
        parent.append(int(rng.integers(-1, s)))   # -1 starts a new family
    # reorder into DFS preorder so that subtrees are contiguous
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
    new_id = {s: i for i, s in enumerate(order)}
    par2 = [(-1 if parent[s] < 0 else new_id[parent[s]]) for s in order]
    lengths = rng.integers(min_len, max_len + 1, size=n_seg).tolist()
    return workloads.tree_from_lengths(lengths, par2)


def _visible_sets_via_oracle(n, mask):
    """Ask the reference which keys each query sees, using only its outputs:
    with Q = 0 every visible key gets the same weight 1/n_visible, so with
    one-hot values O[q, k] > 0 exactly on the visible keys and L = ln n_vis."""
    Q = np.zeros((1, n, 4))
    K = np.ones((1, n, 4))
    V = np.eye(n)[None]
    pos = np.arange(n)
    O, L = oracle.attention(Q, K, V, pos, pos, mask)
    return O[0], L[0]


# ----------------------------------------------------------------------------
# values printed on the pages
# ----------------------------------------------------------------------------
def test_tiny_tree_visible_sets():
    g = _golden("tiny_tree.json")
    seg, parent = workloads.tiny_tree()
    O, L = _visible_sets_via_oracle(len(seg), oracle.Tree(seg, parent))
    for q, expect in g["visible"].items():
        q = int(q)
        got = np.flatnonzero(O[q] > 0).tolist()
        assert got == expect
        assert L[q] == pytest.approx(math.log(len(expect)), abs=1e-15)
        np.testing.assert_allclose(O[q][expect], 1.0 / len(expect), rtol=0, atol=1e-15)


def _pair_count_table(layout_tokens, n_ranks):
    """Per-round, per-rank visible (query, key) pair counts from the
    reference's ring: with Q = 0, exp(L) of a partial is its visible count."""
    table = np.zeros((n_ranks, n_ranks), dtype=np.int64)   # [round, rank]
    for r in range(n_ranks):
        qpos = np.asarray(layout_tokens[r], dtype=np.int64)
        Kb = [np.ones((1, len(t), 2)) for t in layout_tokens]
        Vb = [np.ones((1, len(t), 2)) for t in layout_tokens]
        Q = np.zeros((1, len(qpos), 2))
        _, _, rounds = oracle.ring(Q, qpos, Kb, Vb, [np.asarray(t) for t in layout_tokens], r,
                                   oracle.Causal(), keep_rounds=True)
        for k, (b, (Op, Lp), _) in enumerate(rounds):
            assert b == (r - k) % n_ranks
            table[k, r] = int(round(np.exp(Lp[np.isfinite(Lp)]).sum()))
    return table


def test_ring_pair_tables_from_page():
    g = _golden("causal_ring_n4_s8.json")
    N = g["n_ranks"]
    for name in ("zigzag", "contiguous"):
        lay = g[name]
        table = _pair_count_table(lay["tokens"], N)
        assert table.sum(axis=0).tolist() == lay["per_rank"]
        assert table.max(axis=1).tolist() == lay["round_max"]
        assert int(table.max(axis=1).sum()) == lay["ring_time"]
        assert int(table.sum()) == g["total_pairs"]
    # the zig-zag table lists every visible pair; check the reference's sets
    lay = g["zigzag"]
    for k, per_rank in enumerate(lay["pairs"]):
        for r, pairs in enumerate(per_rank):
            b = (r - k) % N
            qtok, ktok = lay["tokens"][r], lay["tokens"][b]
            Q = np.zeros((1, 2, 2))
            K = np.ones((1, 2, 2))
            V = np.zeros((1, 2, 2))
            V[0, :, 0] = ktok        # value = key position, to read out which keys are seen
            V[0, :, 1] = 1.0
            O, L = oracle.attention(Q, K, V, qtok, ktok, oracle.Causal())
            seen = set()
            for i, q in enumerate(qtok):
                if np.isfinite(L[0, i]):
                    n = int(round(np.exp(L[0, i])))
                    keys = [x for x in ktok if x <= q]
                    assert n == len(keys)
                    assert O[0, i, 0] == pytest.approx(np.mean(keys), abs=1e-14)
                    seen |= {(q, x) for x in keys}
            assert seen == {tuple(p) for p in pairs}


def test_fold_example_from_page():
    g = _golden("fold_8_tokens.json")
    _, L = _visible_sets_via_oracle(8, oracle.Causal())
    per_q = np.rint(np.exp(L)).astype(int)
    assert per_q.tolist() == g["per_query_visible"]
    assert [per_q[:4].sum(), per_q[4:].sum()] == g["two_rank_contiguous"]
    blocks = [per_q[2 * i:2 * i + 2].sum() for i in range(4)]
    assert blocks == g["four_blocks_of_two"]
    assert [blocks[0] + blocks[3], blocks[1] + blocks[2]] == g["fold_first_last_vs_middle"]


# ----------------------------------------------------------------------------
# closed forms
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("P,C", [(7, [3, 5, 2]), (13, [1, 9, 4, 6, 2]), (20, [20])])
def test_tree_pair_count_closed_form(P, C):
    """A_tree = P(P+1)/2 + sum[C_i P + C_i(C_i+1)/2], and the flattened
    layout costs (m-1)P(P+1)/2 more (Context Parallelism in ART, section 01)."""
    seg, parent = workloads.tree_prompt_completions(P, C)
    _, L = _visible_sets_via_oracle(len(seg), oracle.Tree(seg, parent))
    a_tree = int(np.rint(np.exp(L)).sum())
    assert a_tree == P * (P + 1) // 2 + sum(c * P + c * (c + 1) // 2 for c in C)
    a_flat = 0
    for c in C:   # each trajectory run alone as a causal sequence
        _, Lc = _visible_sets_via_oracle(P + c, oracle.Causal())
        a_flat += int(np.rint(np.exp(Lc)).sum())
    assert a_flat - a_tree == (len(C) - 1) * P * (P + 1) // 2


def test_stripe_pair_count_closed_form():
    """Rank 0 of P=4 stripes: its n queries (positions 4i) see stripe 0 up to
    and including themselves and stripes 1..3 strictly before themselves."""
    n, P = 37, 4
    lay = workloads.striped(n * P, P)
    total = 0
    for b in range(P):
        Q = np.zeros((1, n, 2))
        K = np.ones((1, n, 2))
        V = np.ones((1, n, 2))
        _, L = oracle.attention(Q, K, V, lay[0], lay[b], oracle.Causal())
        total += int(np.rint(np.exp(L[np.isfinite(L)])).sum())
    assert total == n * (n + 1) // 2 + (P - 1) * n * (n - 1) // 2


# ----------------------------------------------------------------------------
# brute force and library routines
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_tree_vs_trajectory_bruteforce(seed):
    rng = np.random.default_rng(seed)
    seg, parent = _random_tree(rng, n_seg=7)
    n = len(seg)
    d = 16
    Q, K, V = _rand(rng, 1, n, d), _rand(rng, 1, n, d), _rand(rng, 1, n, d)
    scale = 0.37
    pos = np.arange(n)
    O, L = oracle.attention(Q, K, V, pos, pos, oracle.Tree(seg, parent), scale)
    M = _trajectory_mask(seg, parent)
    Ob, Lb = _dense_attention(Q[0], K[0], V[0], M, scale)
    np.testing.assert_allclose(O[0], Ob, rtol=0, atol=1e-12)
    np.testing.assert_allclose(L[0], Lb, rtol=0, atol=1e-12)


@pytest.mark.parametrize("n,d", [(1, 8), (33, 64), (200, 128)])
def test_causal_vs_torch_sdpa(n, d):
    import torch
    rng = np.random.default_rng(n)
    H = 2
    Q, K, V = _rand(rng, H, n, d), _rand(rng, H, n, d), _rand(rng, H, n, d)
    pos = np.arange(n)
    O, L = oracle.attention(Q, K, V, pos, pos, oracle.Causal())
    t = lambda a: torch.from_numpy(a)[None]
    ref = torch.nn.functional.scaled_dot_product_attention(t(Q), t(K), t(V), is_causal=True)[0]
    np.testing.assert_allclose(O, ref.numpy(), rtol=0, atol=1e-12)
    # the LSE against torch.logsumexp over the causal scores
    S = torch.from_numpy(Q) @ torch.from_numpy(K).transpose(1, 2) / math.sqrt(d)
    S = S.masked_fill(~torch.ones(n, n, dtype=torch.bool).tril(), float("-inf"))
    np.testing.assert_allclose(L, torch.logsumexp(S, dim=-1).numpy(), rtol=0, atol=1e-12)


def test_full_vs_torch_sdpa():
    import torch
    rng = np.random.default_rng(5)
    Q, K, V = _rand(rng, 3, 17, 32), _rand(rng, 3, 29, 32), _rand(rng, 3, 29, 48)
    O, L = oracle.attention(Q, K, V, np.arange(17), np.arange(29), oracle.Full(), 0.21)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(Q), torch.from_numpy(K), torch.from_numpy(V), scale=0.21)
    np.testing.assert_allclose(O, ref.numpy(), rtol=0, atol=1e-12)


# ----------------------------------------------------------------------------
# invariants the pages state
# ----------------------------------------------------------------------------
def _partitions(rng, nk):
    idx = np.arange(nk)
    yield [idx[: nk // 3], idx[nk // 3: 2 * nk // 3], idx[2 * nk // 3:]]          # contiguous
    yield [idx[i::4] for i in range(4)]                                            # strided
    lab = rng.integers(0, 5, size=nk)
    yield [np.flatnonzero(lab == i) for i in range(5)]                              # random
    yield [idx[:0], idx, idx[:0]]                                                   # with empties


@pytest.mark.parametrize("maskname", ["causal", "tree", "full"])
def test_merge_over_any_partition_equals_unpartitioned(maskname):
    """A merge of partials over disjoint key sets equals attention over their
    union, in any order (Context Parallelism in ART, section 03; the lesson's
    ring-attention section)."""
    rng = np.random.default_rng(11)
    if maskname == "tree":
        seg, parent = _random_tree(rng, 6)
        mask = oracle.Tree(seg, parent)
        n = len(seg)
    else:
        n = 41
        mask = oracle.Causal() if maskname == "causal" else oracle.Full()
    d = 24
    Q, K, V = _rand(rng, 2, n, d), _rand(rng, 2, n, d), _rand(rng, 2, n, d)
    pos = np.arange(n)
    O, L = oracle.attention(Q, K, V, pos, pos, mask)
    for parts in _partitions(rng, n):
        partials = [oracle.attention(Q, K[:, p], V[:, p], pos, pos[p], mask) for p in parts]
        for order in (list(range(len(parts))), list(reversed(range(len(parts)))),
                      list(rng.permutation(len(parts)))):
            Om, Lm = oracle.merge([partials[i] for i in order])
            np.testing.assert_allclose(Om, O, rtol=0, atol=1e-12)
            np.testing.assert_allclose(Lm, L, rtol=0, atol=1e-12)


@pytest.mark.parametrize("layout", ["contiguous", "striped", "zigzag"])
def test_ring_equals_unpartitioned(layout):
    rng = np.random.default_rng(3)
    n, N, d = 64, 4, 16
    lay = {"contiguous": workloads.contiguous, "striped": workloads.striped,
           "zigzag": workloads.zigzag}[layout](n, N)
    Q, K, V = _rand(rng, 2, n, d), _rand(rng, 2, n, d), _rand(rng, 2, n, d)
    pos = np.arange(n)
    O, L = oracle.attention(Q, K, V, pos, pos, oracle.Causal())
    for r in range(N):
        Or, Lr = oracle.ring(Q[:, lay[r]], lay[r], [K[:, p] for p in lay], [V[:, p] for p in lay],
                             lay, r, oracle.Causal())
        np.testing.assert_allclose(Or, O[:, lay[r]], rtol=0, atol=1e-12)
        np.testing.assert_allclose(Lr, L[:, lay[r]], rtol=0, atol=1e-12)


def test_packed_tree_equals_separate_trajectories():
    """A packed row gives exactly the outputs of each trajectory run alone
    (Context Parallelism in ART, sections 01 and 12).  In fp64 the keys and
    their order coincide, so the comparison is bitwise."""
    rng = np.random.default_rng(7)
    P, C = 23, [5, 11, 8]
    seg, parent = workloads.tree_prompt_completions(P, C)
    n, d = len(seg), 32
    Q, K, V = _rand(rng, 2, n, d), _rand(rng, 2, n, d), _rand(rng, 2, n, d)
    pos = np.arange(n)
    O, L = oracle.attention(Q, K, V, pos, pos, oracle.Tree(seg, parent))
    start = P
    for c in C:
        traj = np.concatenate([np.arange(P), np.arange(start, start + c)])
        lp = np.arange(P + c)                      # logical positions of the trajectory
        Ot, Lt = oracle.attention(Q[:, traj], K[:, traj], V[:, traj], lp, lp, oracle.Causal())
        assert np.array_equal(Ot, O[:, traj]) and np.array_equal(Lt, L[:, traj])
        start += c


# ----------------------------------------------------------------------------
# special cases
# ----------------------------------------------------------------------------
def test_single_visible_key():
    rng = np.random.default_rng(1)
    Q, K, V = _rand(rng, 1, 1, 8), _rand(rng, 1, 5, 8), _rand(rng, 1, 5, 8)
    O, L = oracle.attention(Q, K, V, [2], [2, 3, 4, 5, 6], oracle.Causal(), 0.5)
    assert np.array_equal(O[0, 0], V[0, 0])
    assert L[0, 0] == pytest.approx(0.5 * float(Q[0, 0] @ K[0, 0]), abs=1e-14)


def test_large_scores_stay_finite():
    from scipy.special import logsumexp
    rng = np.random.default_rng(2)
    Q, K, V = 30 * _rand(rng, 1, 9, 16), 30 * _rand(rng, 1, 9, 16), _rand(rng, 1, 9, 16)
    pos = np.arange(9)
    O, L = oracle.attention(Q, K, V, pos, pos, oracle.Causal())
    assert np.isfinite(L).all() and np.isfinite(O).all()
    S = Q[0] @ K[0].T / 4.0
    for i in range(9):
        assert L[0, i] == pytest.approx(logsumexp(S[i, : i + 1]), rel=1e-14)


def test_empty_visible_set_and_merge_identity():
    Q = np.ones((1, 2, 4))
    K = np.ones((1, 3, 4))
    V = np.full((1, 3, 4), 7.0)
    O, L = oracle.attention(Q, K, V, [0, 1], [5, 6, 7], oracle.Causal())
    assert np.all(O == 0) and np.all(L == -np.inf)
    rng = np.random.default_rng(0)
    Ob, Lb = rng.standard_normal((1, 2, 4)), rng.standard_normal((1, 2))
    Om, Lm = oracle.merge2((O, L), (Ob, Lb))
    assert np.array_equal(Om, Ob) and np.array_equal(Lm, Lb)
    Om, Lm = oracle.merge2((Ob, Lb), (O, L))
    assert np.array_equal(Om, Ob) and np.array_equal(Lm, Lb)
    Om, Lm = oracle.merge2((O, L), (O, L))
    assert np.all(Om == 0) and np.all(Lm == -np.inf)


def test_merge_of_equal_mass_is_average():
    """L_A = L_B: both weights are 1/2 and L = L_A + ln 2."""
    rng = np.random.default_rng(4)
    Oa, Ob = rng.standard_normal((3, 5)), rng.standard_normal((3, 5))
    La = rng.standard_normal(3)
    Om, Lm = oracle.merge2((Oa, La), (Ob, La.copy()))
    np.testing.assert_allclose(Om, (Oa + Ob) / 2, rtol=0, atol=1e-15)
    np.testing.assert_allclose(Lm, La + math.log(2), rtol=0, atol=1e-15)


def test_merge_weights_follow_mass_not_counts():
    """Two stages holding 30% and 70% of the exponential mass get those
    weights (Context Parallelism in ART, section 03)."""
    Oa, Ob = np.array([[1.0, 0.0]]), np.array([[0.0, 1.0]])
    La, Lb = np.array([math.log(0.3)]), np.array([math.log(0.7)])
    Om, Lm = oracle.merge2((Oa, La), (Ob, Lb))
    np.testing.assert_allclose(Om, [[0.3, 0.7]], rtol=0, atol=1e-15)
    assert Lm[0] == pytest.approx(0.0, abs=1e-15)


def test_bf16_inputs_are_widened_exactly():
    import torch
    q, k, v = workloads.qkv(3, 2, 19, 16, "bf16")
    pos = np.arange(19)
    O1, L1 = oracle.attention(q, k, v, pos, pos, oracle.Causal())
    O2, L2 = oracle.attention(q.double().numpy(), k.double().numpy(), v.double().numpy(),
                              pos, pos, oracle.Causal())
    assert np.array_equal(O1, O2) and np.array_equal(L1, L2)


def test_row_subset_matches_full():
    rng = np.random.default_rng(9)
    Q, K, V = _rand(rng, 2, 30, 8), _rand(rng, 2, 30, 8), _rand(rng, 2, 30, 8)
    pos = np.arange(30)
    O, L = oracle.attention(Q, K, V, pos, pos, oracle.Causal())
    rows = [0, 7, 29, 13]
    Os, Ls = oracle.attention(Q, K, V, pos, pos, oracle.Causal(), rows=rows)
    assert np.array_equal(Os, O[:, rows]) and np.array_equal(Ls, L[:, rows])


def test_uniform_weights_count_pin_on_tree():
    """With Q = 0 every visible key has probability 1/n exactly, so for a
    value equal to a bit of the key position the output is the fraction of
    visible keys with that bit set (an integer count over n)."""
    seg, parent = workloads.tree_prompt_completions(50, [20, 31, 17])
    n = len(seg)
    bits = 7
    pos = np.arange(n)
    V = ((pos[:, None] >> np.arange(bits)[None, :]) & 1).astype(np.float64)[None]
    Q = np.zeros((1, n, 4))
    K = np.ones((1, n, 4))
    O, L = oracle.attention(Q, K, V, pos, pos, oracle.Tree(seg, parent))
    M = _trajectory_mask(seg, parent)
    for q in range(n):
        vis = np.flatnonzero(M[q])
        assert L[0, q] == pytest.approx(math.log(len(vis)), abs=1e-14)
        np.testing.assert_allclose(O[0, q], V[0, vis].sum(axis=0) / len(vis), rtol=0, atol=1e-14)


def test_bad_arguments_are_rejected():
    seg, parent = workloads.tiny_tree()
    Q = np.zeros((1, 2, 4))
    with pytest.raises(ValueError):
        oracle.attention(Q, Q, Q, [0, 1], [0, 99], oracle.Tree(seg, parent))
    with pytest.raises(ValueError):
        oracle.attention(Q, Q, Q, [0], [0, 1], oracle.Causal())


# ----------------------------------------------------------------------------
# learned attention sink ("Context Parallelism in ART", section 06): extra
# probability mass with zero value, applied once to the complete result
# ----------------------------------------------------------------------------
def _sink_by_extra_key(Q, K, V, qpos, kpos, mask, scale, a):
    """Brute force: for each query row, attention over its visible keys plus
    one extra key whose score is exactly a_h (k* = a_h / (scale |q|^2) q) and
    whose value is zero, under the all-visible mask."""
    H, nq, d = Q.shape
    O = np.zeros((H, nq, V.shape[2]))
    L = np.zeros((H, nq))
    vis_O, vis_L = oracle.attention(Q, K, V, qpos, kpos, mask, scale)   # only to learn the visible sets
    for h in range(H):
        for i in range(nq):
            # visible keys of row i: those whose removal changes nothing is not
            # testable; take the predicate from a one-hot value probe instead
            onehot = np.eye(K.shape[1])[None]
            P, _ = oracle.attention(np.zeros((1, 1, d)), K[h:h + 1], onehot, [qpos[i]], kpos, mask, scale)
            vis = np.flatnonzero(P[0, 0] > 0)
            q = Q[h, i]
            kstar = a[h] / (scale * float(q @ q)) * q
            Ka = np.concatenate([K[h, vis], kstar[None]], 0)[None]
            Va = np.concatenate([V[h, vis], np.zeros((1, V.shape[2]))], 0)[None]
            o, l = oracle.attention(q[None, None], Ka, Va, [0], np.arange(Ka.shape[1]), oracle.Full(), scale)
            O[h, i], L[h, i] = o[0, 0], l[0, 0]
    return O, L


@pytest.mark.parametrize("maskname", ["causal", "tree"])
def test_sink_equals_zero_value_extra_key(maskname):
    rng = np.random.default_rng(21)
    H, n, d = 2, 24, 8
    Q, K, V = _rand(rng, H, n, d), _rand(rng, H, n, d), _rand(rng, H, n, d)
    if maskname == "causal":
        mask = oracle.Causal()
    else:
        seg, parent = _random_tree(rng, 5)
        n = len(seg)
        Q, K, V = _rand(rng, H, n, d), _rand(rng, H, n, d), _rand(rng, H, n, d)
        mask = oracle.Tree(seg, parent)
    pos = np.arange(n)
    a = np.array([0.7, -1.3])
    O, L = oracle.attention(Q, K, V, pos, pos, mask, 0.35)
    Os, Ls = oracle.apply_sink(O, L, a)
    Ob, Lb = _sink_by_extra_key(Q, K, V, pos, pos, mask, 0.35, a)
    assert np.abs(Os - Ob).max() <= 1e-12 and np.abs(Ls - Lb).max() <= 1e-12


def test_sink_once_not_per_stage():
    """Applying the sink inside each of N stage partials and then merging
    counts its mass N times (the page's warning): the merged LSE equals
    logaddexp(L, a + ln N), not logaddexp(L, a)."""
    rng = np.random.default_rng(22)
    H, n, d, N = 1, 32, 8, 4
    Q, K, V = _rand(rng, H, n, d), _rand(rng, H, n, d), _rand(rng, H, n, d)
    pos = np.arange(n)
    a = np.array([0.4])
    blocks = workloads.contiguous(n, N)
    parts = [oracle.attention(Q, K[:, b], V[:, b], pos, pos[b], oracle.Full()) for b in blocks]
    once = oracle.apply_sink(*oracle.merge(parts), a)
    per_stage = oracle.merge([oracle.apply_sink(o, l, a) for o, l in parts])
    O, L = oracle.attention(Q, K, V, pos, pos, oracle.Full())
    assert np.abs(once[1] - np.logaddexp(L, a[0])).max() <= 1e-12
    assert np.abs(per_stage[1] - np.logaddexp(L, a[0] + math.log(N))).max() <= 1e-12
    assert np.abs(once[1] - per_stage[1]).min() > 0.01


def test_sink_special_cases():
    O = np.arange(12, dtype=np.float64).reshape(1, 3, 4)
    O[0, 1] = 0.0                                                 # a row with no visible key is (0, -inf)
    L = np.array([[1.5, -np.inf, 0.0]])
    Os, Ls = oracle.apply_sink(O, L, np.array([-np.inf]))        # no sink: identity
    assert np.array_equal(Os, O) and np.array_equal(Ls, L)
    Os, Ls = oracle.apply_sink(O, L, np.array([1.5]))            # equal mass: half the weight
    assert Ls[0, 0] == pytest.approx(1.5 + math.log(2.0), abs=1e-15)
    assert np.allclose(Os[0, 0], 0.5 * O[0, 0], atol=1e-15)
    assert Ls[0, 1] == 1.5 and np.all(Os[0, 1] == 0)              # no visible key: all mass is the sink's



# ----------------------------------------------------------------------------
# sliding window on logical (root-to-leaf) positions ("Context Parallelism in
# ART", section 06)
# ----------------------------------------------------------------------------
def test_tiny_tree_window_from_page():
    g = _golden("tiny_tree.json")
    seg, parent = workloads.tiny_tree()
    n = len(seg)
    O, L = _visible_sets_via_oracle(n, oracle.Tree(seg, parent, window=3))
    for q, keys in g["window3_visible"].items():
        assert np.flatnonzero(O[int(q)] > 0).tolist() == keys
    # without a window a query sees its logical position + 1 keys
    O, L = _visible_sets_via_oracle(n, oracle.Tree(seg, parent))
    for q, lpos in g["logical_position"].items():
        assert round(math.exp(L[int(q)])) == lpos + 1


@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("window", [1, 2, 5, 20])
def test_window_vs_trajectory_bruteforce(seed, window):
    rng = np.random.default_rng(100 + seed)
    seg, parent = _random_tree(rng, 7)
    n = len(seg)
    M = _trajectory_mask(seg, parent, window)
    Q, K, V = _rand(rng, 1, n, 8), _rand(rng, 1, n, 8), _rand(rng, 1, n, 8)
    pos = np.arange(n)
    O, L = oracle.attention(Q, K, V, pos, pos, oracle.Tree(seg, parent, window=window), 0.3)
    Od, Ld = _dense_attention(Q[0], K[0], V[0], M, 0.3)
    assert np.abs(O[0] - Od).max() <= 1e-12 and np.abs(L[0] - Ld).max() <= 1e-12


@pytest.mark.parametrize("window", [1, 7, 64])
def test_causal_window_vs_torch_sdpa(window):
    import torch
    rng = np.random.default_rng(7)
    n, d = 96, 16
    Q, K, V = _rand(rng, 1, n, d), _rand(rng, 1, n, d), _rand(rng, 1, n, d)
    pos = np.arange(n)
    O, L = oracle.attention(Q, K, V, pos, pos, oracle.Causal(window=window))
    i, j = np.meshgrid(pos, pos, indexing="ij")
    band = torch.from_numpy((j <= i) & (i - j < window))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(Q), torch.from_numpy(K), torch.from_numpy(V), attn_mask=band)
    S = torch.from_numpy(Q[0] @ K[0].T / math.sqrt(d)).masked_fill(~band, -float("inf"))
    assert np.abs(O[0] - ref[0].numpy()).max() <= 1e-12
    assert np.abs(L[0] - torch.logsumexp(S, dim=1).numpy()).max() <= 1e-12


def test_window_covering_everything_is_no_window():
    rng = np.random.default_rng(8)
    seg, parent = _random_tree(rng, 6)
    n = len(seg)
    Q, K, V = _rand(rng, 1, n, 8), _rand(rng, 1, n, 8), _rand(rng, 1, n, 8)
    pos = np.arange(n)
    a = oracle.attention(Q, K, V, pos, pos, oracle.Tree(seg, parent))
    b = oracle.attention(Q, K, V, pos, pos, oracle.Tree(seg, parent, window=n))
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


# ----------------------------------------------------------------------------
# backward ("Context Parallelism in ART", section 04: the global softmax
# derivative and the merge adjoints; section 06: the sink adjoints)
# ----------------------------------------------------------------------------
def _fd(f, X, eps=1e-6):
    """Central finite differences of the scalar f at X (all entries)."""
    g = np.zeros_like(X)
    for idx in np.ndindex(X.shape):
        Xp = X.copy()
        Xp[idx] += eps
        Xm = X.copy()
        Xm[idx] -= eps
        g[idx] = (f(Xp) - f(Xm)) / (2 * eps)
    return g


@pytest.mark.parametrize("maskname", ["causal", "tree", "full", "tree_window"])
def test_attention_backward_vs_finite_differences(maskname):
    rng = np.random.default_rng(31)
    H, d = 2, 4
    if maskname.startswith("tree"):
        seg, parent = _random_tree(rng, 4, 1, 4)
        n = len(seg)
        mask = oracle.Tree(seg, parent, window=3 if maskname == "tree_window" else 0)
    else:
        n = 10
        mask = oracle.Causal() if maskname == "causal" else oracle.Full()
    Q, K, V, G = (_rand(rng, H, n, d) for _ in range(4))
    pos = np.arange(n)

    def J(Q_, K_, V_):
        O, L = oracle.attention(Q_, K_, V_, pos, pos, mask, 0.7)
        return float((O * G).sum())

    O, L = oracle.attention(Q, K, V, pos, pos, mask, 0.7)
    dQ, dK, dV = oracle.attention_backward(Q, K, V, pos, pos, O, L, G, mask, 0.7)
    assert np.abs(dQ - _fd(lambda X: J(X, K, V), Q)).max() <= 1e-7
    assert np.abs(dK - _fd(lambda X: J(Q, X, V), K)).max() <= 1e-7
    assert np.abs(dV - _fd(lambda X: J(Q, K, X), V)).max() <= 1e-7


def test_staged_backward_with_global_softmax_sums_to_full():
    """Every stage uses the complete O and LSE: the stages' dQ add up and
    each key block gets exactly its share of dK, dV."""
    rng = np.random.default_rng(32)
    H, n, d, N = 2, 48, 8, 4
    Q, K, V, G = (_rand(rng, H, n, d) for _ in range(4))
    pos = np.arange(n)
    O, L = oracle.attention(Q, K, V, pos, pos, oracle.Causal())
    dQ, dK, dV = oracle.attention_backward(Q, K, V, pos, pos, O, L, G, oracle.Causal())
    dQs = np.zeros_like(dQ)
    for b in workloads.zigzag(n, N):
        q_, k_, v_ = oracle.attention_backward(Q, K[:, b], V[:, b], pos, pos[b], O, L, G, oracle.Causal())
        dQs += q_
        assert np.abs(k_ - dK[:, b]).max() <= 1e-12 and np.abs(v_ - dV[:, b]).max() <= 1e-12
    assert np.abs(dQs - dQ).max() <= 1e-12


def test_local_denominators_are_wrong():
    """The page's warning: running each stage's softmax backward with its own
    (local) O and LSE and the original output gradient is not the gradient."""
    rng = np.random.default_rng(33)
    H, n, d, N = 1, 32, 8, 2
    Q, K, V, G = (_rand(rng, H, n, d) for _ in range(4))
    pos = np.arange(n)
    O, L = oracle.attention(Q, K, V, pos, pos, oracle.Full())
    dQ, _, _ = oracle.attention_backward(Q, K, V, pos, pos, O, L, G, oracle.Full())
    wrong = np.zeros_like(dQ)
    for b in workloads.contiguous(n, N):
        Ol, Ll = oracle.attention(Q, K[:, b], V[:, b], pos, pos[b], oracle.Full())
        wrong += oracle.attention_backward(Q, K[:, b], V[:, b], pos, pos[b], Ol, Ll, G, oracle.Full())[0]
    assert np.abs(wrong - dQ).max() > 1e-2


def test_merge_backward_vs_finite_differences():
    rng = np.random.default_rng(34)
    rows, dv, n_parts = 5, 3, 3
    parts = [(_rand(rng, rows, dv), 2 * _rand(rng, rows)) for _ in range(n_parts)]
    parts[1][1][2] = -np.inf
    parts[1][0][2] = 0.0
    G, gL = _rand(rng, rows, dv), _rand(rng, rows)

    def J(ps):
        O, L = oracle.merge(ps)
        return float((O * G).sum() + (L * gL).sum())

    O, L = oracle.merge(parts)
    adj = oracle.merge_backward(parts, O, L, G, gL)
    for p in range(n_parts):
        fo = _fd(lambda X: J([(X if i == p else parts[i][0], parts[i][1]) for i in range(n_parts)]), parts[p][0])
        L_p = parts[p][1].copy()
        fin = np.isfinite(L_p)
        L_p[~fin] = 0.0   # the empty row carries no mass: perturb only finite entries
        fl = _fd(lambda X: J([(parts[i][0], np.where(fin, X, -np.inf) if i == p else parts[i][1])
                              for i in range(n_parts)]), L_p)
        assert np.abs(adj[p][0] - fo).max() <= 1e-7
        assert np.abs(adj[p][1][fin] - fl[fin]).max() <= 1e-7


def test_sink_backward_vs_finite_differences():
    rng = np.random.default_rng(35)
    H, n, dv = 2, 4, 3
    O, L, a, G = _rand(rng, H, n, dv), 2 * _rand(rng, H, n), _rand(rng, H), _rand(rng, H, n, dv)

    def J(O_, L_, a_):
        y, _ = oracle.apply_sink(O_, L_, a_)
        return float((y * G).sum())

    dO, dL, da = oracle.sink_backward(O, L, a, G)
    assert np.abs(dO - _fd(lambda X: J(X, L, a), O)).max() <= 1e-7
    assert np.abs(dL - _fd(lambda X: J(O, X, a), L)).max() <= 1e-7
    assert np.abs(da - _fd(lambda X: J(O, L, X), a)).max() <= 1e-7
