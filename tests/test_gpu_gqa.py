"""Grouped-query attention (query head h reads K/V head h // g): GPU parity
through the C ABI.  The pages' measured model has 32 query heads and 4 KV
heads ("Context Parallelism in ART", section 02 and the weak-scaling runs).
The reference reduces GQA to multi-head attention with every K/V head
repeated g times (brute force), so the fp64 oracle needs no GQA code.

* partial attention, H = 8 query heads over 2 and 1 K/V heads, causal and
  tree, bf16 and fp32, every row (tolerances as for multi-head), also with a
  sliding window;
* the 64K tree row, ring of 4, 32 query / 4 KV heads: bitwise equal to the
  same ring with the K/V heads materialised 8 times (the kernels do the same
  arithmetic on the same values), and sampled rows of 8 heads against the
  reference.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from test_gpu_parity import TOL, _cmp

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def cp():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import context_blockwise_attention_amd as cpattn
    cpattn.lib()
    return cpattn


def _repeat_heads(t, g):
    return t.repeat_interleave(g, dim=0)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("hkv", [2, 1])
@pytest.mark.parametrize("maskname", ["causal", "tree"])
def test_partial_gqa(cp, dtype, hkv, maskname):
    H, n, d = 8, 300, 128
    g = H // hkv
    q, _, _ = workloads.qkv(5, H, n, d, dtype)
    _, k, v = workloads.qkv(6, hkv, n, d, dtype)
    if maskname == "causal":
        mask, omask = cp.Mask.causal(n), oracle.Causal()
    else:
        seg, parent = workloads.tree_prompt_completions(100, (80, 70, 50))
        mask, omask = cp.Mask.tree(seg, parent), oracle.Tree(seg, parent)
    o, l = cp.partial(q.cuda(), k.cuda(), v.cuda(), mask)
    torch.cuda.synchronize()
    pos = np.arange(n)
    O_ref, L_ref = oracle.attention(q, _repeat_heads(k, g), _repeat_heads(v, g), pos, pos, omask)
    _cmp(o, l, O_ref, L_ref, dtype, "gqa %s %s hkv=%d" % (dtype, maskname, hkv))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("maskname,window", [("causal", 45), ("tree", 30), ("tree", 120)])
def test_partial_gqa_window(cp, dtype, maskname, window):
    """Grouped-query heads with a sliding window (on logical positions for
    the tree): the K/V head index and the window mask are independent parts
    of the kernel, checked together."""
    H, hkv, n, d = 8, 2, 300, 128
    g = H // hkv
    q, _, _ = workloads.qkv(7, H, n, d, dtype)
    _, k, v = workloads.qkv(8, hkv, n, d, dtype)
    if maskname == "causal":
        mask, omask = cp.Mask.causal(n).with_window(window), oracle.Causal(window=window)
    else:
        seg, parent = workloads.tree_prompt_completions(100, (80, 70, 50))
        mask, omask = cp.Mask.tree(seg, parent).with_window(window), oracle.Tree(seg, parent, window=window)
    o, l = cp.partial(q.cuda(), k.cuda(), v.cuda(), mask)
    torch.cuda.synchronize()
    pos = np.arange(n)
    O_ref, L_ref = oracle.attention(q, _repeat_heads(k, g), _repeat_heads(v, g), pos, pos, omask)
    _cmp(o, l, O_ref, L_ref, dtype, "gqa window %s %s W=%d" % (dtype, maskname, window))


@pytest.mark.parametrize("b", [0, 1])
def test_partial_striped_gqa(cp, b):
    """Striped positions (P = 2, rank 0's queries against stripe b) with 8
    query heads over 2 K/V heads."""
    H, hkv, n, d, P = 8, 2, 400, 128, 2
    g = H // hkv
    q, _, _ = workloads.qkv(11, H, n * P, d, "bf16")
    _, k, v = workloads.qkv(12, hkv, n * P, d, "bf16")
    lay = workloads.striped(n * P, P)
    mask = cp.Mask.causal(n * P)
    qq, kk, vv = q[:, lay[0]], k[:, lay[b]], v[:, lay[b]]
    o, l = cp.partial(qq.cuda(), kk.cuda(), vv.cuda(), mask, (0, P), (b, P))
    torch.cuda.synchronize()
    O_ref, L_ref = oracle.attention(qq, _repeat_heads(kk, g), _repeat_heads(vv, g), lay[0], lay[b], oracle.Causal())
    _cmp(o, l, O_ref, L_ref, "bf16", "striped gqa stripe %d" % b)


def test_tree64k_ring_gqa_32q_4kv(cp):
    H, hkv, d, N = 32, 4, 128, 4
    g = H // hkv
    seg, parent = workloads.tree_prompt_completions(24576, (8192,) * 5)
    n = len(seg)
    c = n // N
    print("tree64k gqa: generating inputs", flush=True)
    q, _, _ = workloads.qkv(7, H, n, d, "bf16")
    _, k, v = workloads.qkv(8, hkv, n, d, "bf16")
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    kr, vr = _repeat_heads(kd, g).contiguous(), _repeat_heads(vd, g).contiguous()
    mask = cp.Mask.tree(seg, parent)
    blk = lambda t: [t[:, r * c:(r + 1) * c] for r in range(N)]
    pos = [(r * c, 1) for r in range(N)]
    out_g = cp.ring_emulate(blk(qd), blk(kd), blk(vd), pos, mask)
    out_m = cp.ring_emulate(blk(qd), blk(kr), blk(vr), pos, mask)
    torch.cuda.synchronize()
    for r in range(N):
        assert torch.equal(out_g[r][0], out_m[r][0]) and torch.equal(out_g[r][1], out_m[r][1]), r
    O = torch.cat([out_g[r][0] for r in range(N)], 1)
    L = torch.cat([out_g[r][1] for r in range(N)], 1)
    worst_o = worst_l = 0.0
    allpos = np.arange(n)
    for h in range(0, H, 4):   # 8 heads, two per K/V head
        rows = workloads.sample_rows(0, h, n, forced=(0, n - 1, 24575, 24576, n - 8192))
        O_ref, L_ref = oracle.attention(q[h:h + 1], k[h // g:h // g + 1], v[h // g:h // g + 1], allpos, allpos,
                                        oracle.Tree(seg, parent), rows=rows)
        idx = torch.from_numpy(rows).cuda()
        worst_o = max(worst_o, float(np.abs(O[h].index_select(0, idx).double().cpu().numpy() - O_ref[0]).max()))
        worst_l = max(worst_l, float(np.abs(L[h].index_select(0, idx).double().cpu().numpy() - L_ref[0]).max()))
    print("tree64k gqa: sampled rows max|dO| %.2e max|dLSE| %.2e" % (worst_o, worst_l), flush=True)
    assert worst_o <= TOL["bf16"][0] and worst_l <= TOL["bf16"][1]
    mask.free()
