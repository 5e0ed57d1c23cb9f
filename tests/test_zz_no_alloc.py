"""cpattn_mask_tree_static -- the prefix-tree descriptor built without device
allocation, in the library's static per-GPU buffer -- against
cpattn_mask_tree, through the C ABI.

Two calls in a row on one GPU, the second with a smaller tree (the buffer
keeps the first call's contents beyond the second's end).  Each descriptor
drives the ring of 4 (every rank, fused merge): the outputs must be
identical to those of the allocated descriptor (same kernels, same
descriptor contents), and match the fp64 reference (bf16 inputs: 2e-2 on O,
1e-3 on LSE) on sampled rows.  The static descriptor also goes through
cpattn_mask_with_window, and rejects malformed trees like cpattn_mask_tree.
"""
import ctypes

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


def _ring(cp, q, k, v, N, mask):
    n = k.shape[1]
    c = n // N
    sl = [slice(r * c, (r + 1) * c) for r in range(N)]
    out = cp.ring_emulate([q[:, s] for s in sl], [k[:, s] for s in sl], [v[:, s] for s in sl],
                          [(r * c, 1) for r in range(N)], mask)
    torch.cuda.synchronize()
    return torch.cat([out[r][0] for r in range(N)], 1), torch.cat([out[r][1] for r in range(N)], 1)


def _check_case(cp, seg, parent, seed, rows_per_head):
    n = len(seg)
    H, d, N = 4, 128, 4
    q, k, v = workloads.qkv(seed, H, n, d, "bf16")
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    ref_mask = cp.Mask.tree(seg, parent)
    o_ref, l_ref = _ring(cp, qd, kd, vd, N, ref_mask)
    st_mask = cp.Mask.tree_static(seg, parent)
    assert st_mask.n_pos == n
    o_st, l_st = _ring(cp, qd, kd, vd, N, st_mask)
    assert torch.equal(o_st, o_ref) and torch.equal(l_st, l_ref), "static descriptor gives other outputs"
    # against the fp64 reference on sampled rows
    pos = np.arange(n)
    worst_o = worst_l = 0.0
    bounds = [b for ab in workloads.segment_bounds(seg) for b in ab]
    for h in range(H):
        rows = workloads.sample_rows(seed, h, n, forced=bounds)[:rows_per_head]
        O, L = oracle.attention(q[h:h + 1], k[h:h + 1], v[h:h + 1], pos, pos, oracle.Tree(seg, parent), rows=rows)
        idx = torch.from_numpy(rows).cuda()
        worst_o = max(worst_o, float(np.abs(o_st[h].index_select(0, idx).double().cpu().numpy() - O[0]).max()))
        worst_l = max(worst_l, float(np.abs(l_st[h].index_select(0, idx).double().cpu().numpy() - L[0]).max()))
    print("  n=%d: static == allocated; sampled rows max|dO| %.2e max|dLSE| %.2e" % (n, worst_o, worst_l),
          flush=True)
    assert worst_o <= 2e-2 and worst_l <= 1e-3
    # a window over the static descriptor (an ordinary, allocated copy)
    w_ref, w_st = ref_mask.with_window(700), st_mask.with_window(700)
    a = _ring(cp, qd, kd, vd, N, w_ref)
    b = _ring(cp, qd, kd, vd, N, w_st)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    w_ref.free()
    w_st.free()
    st_mask.free()   # a no-op for the static descriptor
    ref_mask.free()


def test_static_descriptor_two_calls(cp):
    # first call: 24576 + 4 x 6144 tokens; second: a smaller random-shaped tree
    seg, parent = workloads.tree_prompt_completions(24576, (6144,) * 4)
    _check_case(cp, seg, parent, 0, 64)
    seg2, parent2 = workloads.tree_prompt_completions(700, (300, 450, 200, 350))
    _check_case(cp, seg2, parent2, 1, 256)


def _random_preorder_tree(seed, n_seg, seg_len):
    """A random rooted tree of n_seg segments (each segment's parent drawn
    uniformly from the earlier ones), relabelled in depth-first preorder and
    packed with seg_len tokens per segment."""
    rng = np.random.default_rng(seed)
    parent = np.concatenate([[-1], rng.integers(0, np.arange(1, n_seg))])
    kids = [[] for _ in range(n_seg)]
    for s_, p_ in enumerate(parent[1:], 1):
        kids[p_].append(s_)
    order, stack = [], [0]
    while stack:
        s_ = stack.pop()
        order.append(s_)
        stack.extend(reversed(kids[s_]))
    new = np.empty(n_seg, dtype=np.int64)
    new[np.asarray(order)] = np.arange(n_seg)
    par = [-1 if parent[s_] < 0 else int(new[parent[s_]]) for s_ in order]
    return workloads.tree_from_lengths([seg_len] * n_seg, par)


def test_static_descriptor_at_its_limits(cp):
    """The largest tree the static buffer holds: CPATTN_STATIC_MAX_TOK tokens
    in CPATTN_STATIC_MAX_SEG segments (a random preorder tree of 65536
    segments of 16 tokens, depth about 25).  The ring of 4 over it (2 heads,
    d 64, bf16) gives the allocated descriptor's outputs bit for bit, and
    sampled rows (every head, the first and last row of some segments among
    them) match the fp64 reference."""
    n_seg, seg_len = 1 << 16, 16
    seg, parent = _random_preorder_tree(5, n_seg, seg_len)
    n = len(seg)
    assert n == 1 << 20
    H, d, N = 2, 64, 4
    q, k, v = workloads.qkv(7, H, n, d, "bf16")
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    ref_mask = cp.Mask.tree(seg, parent)
    o_ref, l_ref = _ring(cp, qd, kd, vd, N, ref_mask)
    st_mask = cp.Mask.tree_static(seg, parent)
    assert st_mask.n_pos == n
    o_st, l_st = _ring(cp, qd, kd, vd, N, st_mask)
    assert torch.equal(o_st, o_ref) and torch.equal(l_st, l_ref), "static descriptor gives other outputs"
    pos = np.arange(n)
    firsts = np.arange(0, n, seg_len)
    for h in range(H):
        forced = np.concatenate([firsts[::4096], firsts[::4096] + seg_len - 1, [n - 1]])
        rows = workloads.sample_rows(11, h, n, forced=forced, count=96)
        O, L = oracle.attention(q[h:h + 1], k[h:h + 1], v[h:h + 1], pos, pos, oracle.Tree(seg, parent), rows=rows)
        idx = torch.from_numpy(rows).cuda()
        do = float(np.abs(o_st[h].index_select(0, idx).double().cpu().numpy() - O[0]).max())
        dl = float(np.abs(l_st[h].index_select(0, idx).double().cpu().numpy() - L[0]).max())
        print("  head %d: %d rows, max|dO| %.2e max|dLSE| %.2e" % (h, len(rows), do, dl), flush=True)
        assert do <= 2e-2 and dl <= 1e-3
    st_mask.free()
    ref_mask.free()


@pytest.mark.parametrize("seg,parent,code", [
    ([0, 0, 1, 1, 2, 2], [-1, -1, 0], -2),   # child stored outside its parent's subtree
    ([0, 1, 0], [-1, 0], -1),                # segment 0 split into two runs
    ([0, 1], [1, 0], -1),                    # parent cycle
])
def test_static_descriptor_rejections(cp, seg, parent, code):
    L = cp.lib()
    s = np.asarray(seg, dtype=np.int32)
    p = np.asarray(parent, dtype=np.int32)
    h = ctypes.c_void_p()
    rc = L.cpattn_mask_tree_static(s.ctypes.data, len(s), p.ctypes.data, len(p), None, ctypes.byref(h))
    assert rc == code, L.cpattn_last_error()
    assert L.cpattn_last_error().startswith(b"cpattn_mask_tree_static")
