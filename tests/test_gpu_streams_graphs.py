"""Stream and graph use of the compute calls (GPU).

* Two independent rings (different trees, heads and sizes) enqueued on two
  streams at once, three times over, give bit for bit what each gives alone
  on one stream: the calls keep no state that concurrent calls share.
* A ring call captured in a HIP graph (torch.cuda.graph) and replayed three
  times, with eager work between the replays (the outputs overwritten by
  fill kernels), gives the eager result bit for bit on every replay: the
  calls enqueue only kernels, no allocation, copy or memset.

The forward kernels are deterministic (fixed reduction order, no atomics), so
equal inputs give equal bits.
"""
import pytest
import torch

import workloads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def cp():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import context_blockwise_attention_amd as cpattn
    cpattn.lib()
    return cpattn


def _problem(cp, seed, H, prompt, completions, N):
    seg, parent = workloads.tree_prompt_completions(prompt, completions)
    n = len(seg) // N * N
    seg, c = seg[:n], n // N
    dev = torch.device("cuda:0")
    q, k, v = workloads.qkv(seed, H, n, 128, "bf16")
    q, k, v = q.to(dev), k.to(dev), v.to(dev)
    blk = lambda t: [t[:, r * c:(r + 1) * c] for r in range(N)]
    mask = cp.Mask.tree(seg, parent)
    pos = [(r * c, 1) for r in range(N)]
    outs = lambda: {r: (torch.empty((H, c, 128), dtype=torch.float32, device=dev),
                        torch.empty((H, c), dtype=torch.float32, device=dev)) for r in range(N)}
    return blk(q), blk(k), blk(v), pos, mask, outs


def _same(a, b, what):
    for r in a:
        for x, y, name in ((a[r][0], b[r][0], "O"), (a[r][1], b[r][1], "LSE")):
            assert torch.equal(x, y), "%s: rank %d %s differs (max |diff| %.3g)" % (
                what, r, name, float((x - y).abs().nan_to_num(0.0).max()))


def test_two_streams_at_once(cp):
    A = _problem(cp, 11, 8, 2048, (1024,) * 3, 4)
    B = _problem(cp, 12, 12, 1024, (512,) * 6, 3)
    cur = torch.cuda.current_stream()
    ref_a = cp.ring_emulate(*A[:5], outs=A[5](), stream=cur)
    ref_b = cp.ring_emulate(*B[:5], outs=B[5](), stream=cur)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    out_a, out_b = A[5](), B[5]()
    s1.wait_stream(cur)
    s2.wait_stream(cur)
    for _ in range(3):
        cp.ring_emulate(*A[:5], outs=out_a, stream=s1)
        cp.ring_emulate(*B[:5], outs=out_b, stream=s2)
    torch.cuda.synchronize()
    _same(out_a, ref_a, "stream 1")
    _same(out_b, ref_b, "stream 2")
    A[4].free()
    B[4].free()


def test_graph_capture_replay(cp):
    Q, K, V, pos, mask, outs = _problem(cp, 13, 8, 2048, (1024,) * 3, 4)
    cur = torch.cuda.current_stream()
    ref = cp.ring_emulate(Q, K, V, pos, mask, outs=outs(), stream=cur)
    out_g = outs()
    # warm-up on a side stream before capture (as torch.cuda.graph asks)
    side = torch.cuda.Stream()
    side.wait_stream(cur)
    with torch.cuda.stream(side):
        cp.ring_emulate(Q, K, V, pos, mask, outs=out_g)
    cur.wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        cp.ring_emulate(Q, K, V, pos, mask, outs=out_g)
    for rep in range(3):
        for o, l in out_g.values():
            o.fill_(7.0)
            l.fill_(-7.0)
        g.replay()
        torch.cuda.synchronize()
        _same(out_g, ref, "replay %d" % rep)
    del g
    mask.free()
