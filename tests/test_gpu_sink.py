"""Learned attention sink (cpattn_apply_sink) on the GPU against the fp64
reference's sink step, which is pinned to a zero-value extra key
("Context Parallelism in ART", section 06: the sink belongs to the whole
query and is applied once, after the last merge).

* composed with the ring: a packed tree ring of 4 ranks then the sink, bf16
  and fp32, d 64 and 128, every row against reference attention + sink;
* rows with no visible key become (0, a);
* full size: the sink on 32 heads x 65536 rows x 128 of arbitrary (O, LSE),
  256 sampled rows per head against the reference's sink on the same input.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from test_gpu_parity import TOL

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def cp():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import context_blockwise_attention_amd as cpattn
    cpattn.lib()
    return cpattn


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
def test_ring_then_sink(cp, dtype, d):
    H, N = 3, 4
    seg, parent = workloads.tree_prompt_completions(160, (96, 64, 80))
    n = len(seg)
    c = n // N
    q, k, v = workloads.qkv(11, H, n, d, dtype)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    mask = cp.Mask.tree(seg, parent)
    blk = lambda t: [t[:, r * c:(r + 1) * c] for r in range(N)]
    out = cp.ring_emulate(blk(qd), blk(kd), blk(vd), [(r * c, 1) for r in range(N)], mask)
    a = np.array([0.5, -2.0, 3.0])
    sink = torch.tensor(a, dtype=torch.float32, device="cuda")
    O = torch.cat([out[r][0] for r in range(N)], 1).contiguous()
    L = torch.cat([out[r][1] for r in range(N)], 1).contiguous()
    cp.apply_sink(O, L, sink)
    torch.cuda.synchronize()
    pos = np.arange(n)
    O_ref, L_ref = oracle.apply_sink(*oracle.attention(q, k, v, pos, pos, oracle.Tree(seg, parent)),
                                     a.astype(np.float32).astype(np.float64))
    do = float(np.abs(O.double().cpu().numpy() - O_ref).max())
    dl = float(np.abs(L.double().cpu().numpy() - L_ref).max())
    print("ring + sink %s d=%d: max|dO| %.2e max|dLSE| %.2e" % (dtype, d, do, dl), flush=True)
    assert do <= TOL[dtype][0] and dl <= TOL[dtype][1]
    mask.free()


def test_sink_on_rows_without_keys(cp):
    H, n, d = 2, 40, 64
    q, k, v = workloads.qkv(12, H, n, d, "f32")
    mask = cp.Mask.causal(2 * n)
    # queries at positions 0..39, keys at 40..79: nothing visible
    o, l = cp.partial(q.cuda(), k.cuda(), v.cuda(), mask, q_pos=(0, 1), k_pos=(n, 1))
    cp.apply_sink(o, l, torch.tensor([0.25, -1.0], device="cuda"))
    torch.cuda.synchronize()
    assert torch.all(o == 0)
    assert torch.equal(l.cpu(), torch.tensor([[0.25] * n, [-1.0] * n]))


def test_sink_full_size_sampled(cp):
    H, n, d = 32, 65536, 128
    g = torch.Generator(device="cpu").manual_seed(13)
    O = torch.randn((H, n, d), generator=g).cuda()
    L = (4.0 * torch.randn((H, n), generator=g)).cuda()
    L[:, ::997] = -float("inf")
    O[:, ::997] = 0.0
    a = 4.0 * torch.randn((H,), generator=g)
    O0, L0 = O.cpu(), L.cpu()
    cp.apply_sink(O, L, a.cuda())
    torch.cuda.synchronize()
    worst_o = worst_l = 0.0
    for h in range(H):
        rows = workloads.sample_rows(13, h, n, forced=(0, 997, n - 1))
        Or, Lr = oracle.apply_sink(O0[h:h + 1, rows].double().numpy(), L0[h:h + 1, rows].double().numpy(),
                                   a[h:h + 1].double().numpy())
        worst_o = max(worst_o, float(np.abs(O[h, rows].double().cpu().numpy() - Or[0]).max()))
        fin = np.isfinite(Lr[0])
        worst_l = max(worst_l, float(np.abs(L[h, rows].double().cpu().numpy()[fin] - Lr[0][fin]).max()))
    print("sink full size: max|dO| %.2e max|dLSE| %.2e" % (worst_o, worst_l), flush=True)
    assert worst_o <= 1e-5 and worst_l <= 1e-5
