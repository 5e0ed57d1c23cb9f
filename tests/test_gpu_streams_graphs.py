"""Stream and graph use of the compute calls (GPU).

* Two independent rings (different trees, heads and sizes) enqueued on two
  streams at once, three times over, give bit for bit what each gives alone
  on one stream: the calls keep no state that concurrent calls share.
* A ring call captured in a HIP graph (torch.cuda.graph) and replayed three
  times, with eager work between the replays (the outputs overwritten by
  fill kernels), gives the eager result bit for bit on every replay: the
  calls enqueue only kernels, no allocation, copy or memset.
* The same for the ring backward (dQ, dK, dV added into the caller's
  buffers, which are zeroed before each replay).

The kernels are deterministic (fixed reduction order and launch order, no
atomics), so equal inputs give equal bits.
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


def _backward_inputs(cp, Q, K, V, pos, mask, outs, seed):
    cur = torch.cuda.current_stream()
    fwd = cp.ring_emulate(Q, K, V, pos, mask, outs=outs(), stream=cur)
    g = torch.Generator(device="cpu").manual_seed(seed)
    douts = [torch.randn(q.shape, generator=g).to(torch.bfloat16).to(q.device) for q in Q]
    deltas = [cp.backward_delta(fwd[r][0], douts[r]) for r in range(len(Q))]
    lses = [fwd[r][1] for r in range(len(Q))]
    zeros = lambda: [tuple(torch.zeros(t.shape, dtype=torch.float32, device=t.device) for t in (Q[r], K[r], V[r]))
                     for r in range(len(Q))]
    return lses, deltas, douts, zeros


def _same_grads(a, b, what):
    for r, (ga, gb) in enumerate(zip(a, b)):
        for x, y, name in zip(ga, gb, ("dQ", "dK", "dV")):
            assert torch.equal(x, y), "%s: rank %d %s differs (max |diff| %.3g)" % (
                what, r, name, float((x - y).abs().max()))


def test_backward_two_streams_and_graph_replay(cp):
    """The ring backward (dQ, dK, dV added into the caller's buffers) on two
    streams at once next to a second problem's, and captured in a graph and
    replayed (buffers zeroed by eager fill kernels before each replay): bit
    for bit the eager result every time."""
    A = _problem(cp, 21, 8, 2048, (1024,) * 3, 4)
    B = _problem(cp, 22, 4, 1024, (512,) * 6, 3)
    la, da, ga, za = _backward_inputs(cp, *A, seed=5)
    lb, db, gb, zb = _backward_inputs(cp, *B, seed=6)
    cur = torch.cuda.current_stream()
    ref_a = cp.ring_backward(*A[:5], la, da, ga, grads=za(), stream=cur)
    ref_b = cp.ring_backward(*B[:5], lb, db, gb, grads=zb(), stream=cur)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    out_a, out_b = za(), zb()   # zero-filled on cur, before the side streams wait for it
    s1.wait_stream(cur)
    s2.wait_stream(cur)
    cp.ring_backward(*A[:5], la, da, ga, grads=out_a, stream=s1)
    cp.ring_backward(*B[:5], lb, db, gb, grads=out_b, stream=s2)
    torch.cuda.synchronize()
    _same_grads(out_a, ref_a, "stream 1")
    _same_grads(out_b, ref_b, "stream 2")

    grads = za()
    side = torch.cuda.Stream()
    side.wait_stream(cur)
    with torch.cuda.stream(side):
        cp.ring_backward(*A[:5], la, da, ga, grads=grads)   # warm-up before capture
    cur.wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        cp.ring_backward(*A[:5], la, da, ga, grads=grads)
    for rep in range(3):
        for trio in grads:
            for t in trio:
                t.zero_()
        graph.replay()
        torch.cuda.synchronize()
        _same_grads(grads, ref_a, "replay %d" % rep)
    del graph
    A[4].free()
    B[4].free()


def test_two_host_threads_share_a_descriptor(cp):
    """Two host threads (the binding's foreign calls release the interpreter
    lock, so the library's host code runs in both at once) drive the forward
    and backward rings of two problems through one windowed tree
    descriptor, created just before, so that both fill its cached pair
    counts together, each thread on its own stream, three times over: bit
    for bit what each gives alone."""
    import threading
    seg, parent = workloads.tree_prompt_completions(2048, (1024,) * 3)
    N = 4
    n = len(seg)
    c = n // N
    dev = torch.device("cuda:0")
    pos = [(r * c, 1) for r in range(N)]
    blk = lambda t: [t[:, r * c:(r + 1) * c] for r in range(N)]
    probs = []
    for seed in (41, 42):
        q, k, v = workloads.qkv(seed, 8, n, 128, "bf16")
        G = torch.randn((8, n, 128), generator=torch.Generator().manual_seed(seed)).to(torch.bfloat16)
        probs.append(tuple(blk(t.to(dev)) for t in (q, k, v)) + ([x.contiguous() for x in blk(G.to(dev))],))

    def run(p, mask, stream):
        Q, K, V, Gs = p
        out = cp.ring_emulate(Q, K, V, pos, mask, stream=stream)
        deltas = [cp.backward_delta(out[r][0], Gs[r], stream=stream) for r in range(N)]
        grads = cp.ring_backward(Q, K, V, pos, mask, [out[r][1] for r in range(N)], deltas, Gs, stream=stream)
        return out, grads

    base = cp.Mask.tree(seg, parent)
    ref_mask = base.with_window(700)
    cur = torch.cuda.current_stream()
    refs = [run(p, ref_mask, cur) for p in probs]
    torch.cuda.synchronize()
    for rep in range(3):
        mask = base.with_window(700)   # fresh: no cached pair counts yet
        streams = [torch.cuda.Stream(), torch.cuda.Stream()]
        for s in streams:
            s.wait_stream(cur)
        results, errors = [None, None], []

        def worker(i):
            try:
                results[i] = run(probs[i], mask, streams[i])
            except Exception as e:   # reported in the main thread
                errors.append(e)

        threads = [threading.Thread(target=worker, args=(i,)) for i in range(2)]
        for t in threads:
            t.start()
        for t in threads:
            t.join()
        torch.cuda.synchronize()
        assert not errors, errors
        for i in range(2):
            _same(results[i][0], refs[i][0], "thread %d forward, round %d" % (i, rep))
            _same_grads(results[i][1], refs[i][1], "thread %d backward, round %d" % (i, rep))
        mask.free()
    ref_mask.free()
    base.free()


def test_descriptors_made_in_several_threads(cp):
    """Four host threads each build tree descriptors (and windowed copies of
    them), run a ring through them on their own stream and free them, five
    times over, all at once: every result bit for bit the one made alone."""
    import threading
    dev = torch.device("cuda:0")
    shapes = [(700, (300, 450, 200)), (1024, (512,) * 4), (300, (900, 60)), (2048, (256,) * 6)]
    windows = [0, 90, 400, 0]
    N = 2
    jobs = []
    for i, (prompt, comps) in enumerate(shapes):
        seg, parent = workloads.tree_prompt_completions(prompt, comps)
        n = len(seg) // N * N
        c = n // N
        q, k, v = (t.to(dev) for t in workloads.qkv(50 + i, 4, n, 128, "bf16"))
        blk = lambda t, c=c: [t[:, r * c:(r + 1) * c] for r in range(N)]
        jobs.append((seg[:n], parent, windows[i], blk(q), blk(k), blk(v), [(r * c, 1) for r in range(N)]))

    def run(job, stream):
        seg, parent, w, Q, K, V, pos = job
        base = cp.Mask.tree(seg, parent)
        mask = base.with_window(w) if w else base
        out = cp.ring_emulate(Q, K, V, pos, mask, stream=stream)
        stream_sync = stream.synchronize if stream is not None else torch.cuda.synchronize
        stream_sync()
        if mask is not base:
            mask.free()
        base.free()
        return out

    refs = [run(j, None) for j in jobs]
    results = [[None] * 5 for _ in jobs]
    errors = []

    def worker(i):
        try:
            s = torch.cuda.Stream()
            for rep in range(5):
                results[i][rep] = run(jobs[i], s)
        except Exception as e:   # reported in the main thread
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(jobs))]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for i in range(len(jobs)):
        for rep in range(5):
            _same(results[i][rep], refs[i], "thread %d, round %d" % (i, rep))
