"""The C ABI without a GPU: the library loads, exports every function that
include/cpattn.h declares, and rejects malformed or unsupported arguments
with the documented status codes before any device work (no compute call is
made here).  Pointers below are dummies that validation rejects first."""
import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "cpattn.h")

OK, EINVAL, EUNSUPPORTED = 0, -1, -2


@pytest.fixture(scope="module")
def L():
    from context_blockwise_attention_amd import build as b
    if not b.up_to_date():
        b.build()
    import context_blockwise_attention_amd as cp
    return cp.lib()


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(cpattn_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_function(L):
    names = _declared()
    assert "cpattn_partial" in names and "cpattn_ring_emulate" in names and "cpattn_merge" in names
    for n in names:
        assert hasattr(L, n), "libcpattn.so does not export %s" % n


def test_version_and_error_string(L):
    import context_blockwise_attention_amd as cp
    assert cp.version() == (0, 9)
    assert isinstance(L.cpattn_last_error(), bytes)


def _tensor(cp, data=0x1000, dtype=0, H=2, n=16, d=128, sh=None, st=None):
    st = d if st is None else st
    sh = n * st if sh is None else sh
    return cp._Tensor(data, dtype, 0, H, n, d, sh, st)


def test_causal_mask_is_host_only(L):
    h = ctypes.c_void_p()
    assert L.cpattn_mask_causal(100, ctypes.byref(h)) == OK
    assert L.cpattn_mask_npos(h) == 100
    assert L.cpattn_mask_free(h) == OK
    assert L.cpattn_mask_causal(-1, ctypes.byref(h)) == EINVAL
    assert L.cpattn_mask_causal(5, None) == EINVAL


@pytest.mark.parametrize("seg,parent,code", [
    ([0, 0, 1, 1, 2, 2], [-1, -1, 0], EUNSUPPORTED),   # child stored outside its parent's subtree
    ([0, 1, 0], [-1, 0], EINVAL),                      # segment 0 split into two runs
    ([0, 0, 3], [-1, 0], EINVAL),                      # segment id out of range
    ([0, 1], [1, 0], EINVAL),                          # parent cycle
    ([0, 1], [-1, 5], EINVAL),                         # parent out of range
    ([0, 0], [-1, 0], EINVAL),                         # segment 1 has no token
    ([0, 0, 1, 1], [1, -1], EUNSUPPORTED),             # parent stored after its child
])
def test_tree_descriptor_rejections(L, seg, parent, code):
    s = np.asarray(seg, dtype=np.int32)
    p = np.asarray(parent, dtype=np.int32)
    h = ctypes.c_void_p()
    rc = L.cpattn_mask_tree(s.ctypes.data, len(s), p.ctypes.data, len(p), None, ctypes.byref(h))
    assert rc == code, L.cpattn_last_error()
    assert L.cpattn_last_error().startswith(b"cpattn_mask_tree")


def test_static_tree_descriptor_limits(L):
    """The no-allocation tree descriptor rejects trees beyond its static
    buffer (2^20 tokens, 2^16 segments) before any device work."""
    h = ctypes.c_void_p()
    n = (1 << 20) + 1
    seg = np.zeros(n, dtype=np.int32)
    par = np.full(1, -1, dtype=np.int32)
    assert L.cpattn_mask_tree_static(seg.ctypes.data, n, par.ctypes.data, 1, None, ctypes.byref(h)) == EUNSUPPORTED
    assert b"capacity" in L.cpattn_last_error()
    par = np.full((1 << 16) + 1, -1, dtype=np.int32)
    assert L.cpattn_mask_tree_static(seg.ctypes.data, 10, par.ctypes.data, len(par), None,
                                     ctypes.byref(h)) == EUNSUPPORTED
    assert L.cpattn_mask_tree_static(seg.ctypes.data, 10, par.ctypes.data, 1, None, None) == EINVAL


def _partial(L, cp, q, k, v, mask, qpos=(0, 1), kpos=(0, 1), scale=0.1, o=0x2000, lse=0x3000, acc=0):
    return L.cpattn_partial(ctypes.byref(q), ctypes.byref(k), ctypes.byref(v), mask, cp._PosMap(*qpos),
                            cp._PosMap(*kpos), scale, o, lse, acc, None)


def test_partial_validation(L):
    import context_blockwise_attention_amd as cp
    h = ctypes.c_void_p()
    assert L.cpattn_mask_causal(64, ctypes.byref(h)) == OK
    t = _tensor(cp)
    assert _partial(L, cp, _tensor(cp, dtype=7), t, t, h) == EUNSUPPORTED          # dtype
    assert _partial(L, cp, _tensor(cp, d=96), t, t, h) == EUNSUPPORTED             # head dim
    assert _partial(L, cp, t, _tensor(cp, dtype=1), t, h) == EUNSUPPORTED          # mixed dtypes
    assert _partial(L, cp, t, _tensor(cp, H=3), t, h) == EINVAL                    # head counts differ
    assert _partial(L, cp, t, _tensor(cp, H=1), t, h) == EINVAL                    # k and v heads differ
    assert _partial(L, cp, t, _tensor(cp, H=4), _tensor(cp, H=4), h) == EINVAL     # K/V heads do not divide q heads
    assert _partial(L, cp, t, t, _tensor(cp, n=15), h) == EINVAL                   # k/v lengths differ
    assert _partial(L, cp, _tensor(cp, data=0x1008), t, t, h) == EUNSUPPORTED      # alignment
    assert _partial(L, cp, _tensor(cp, st=132), t, t, h) == EUNSUPPORTED           # stride not x8
    assert _partial(L, cp, t, t, t, None) == EINVAL                                # no mask
    assert _partial(L, cp, t, t, t, h, scale=0.0) == EUNSUPPORTED                  # scale
    assert _partial(L, cp, t, t, t, h, scale=float("nan")) == EUNSUPPORTED
    assert _partial(L, cp, t, t, t, h, acc=2) == EINVAL                            # accumulate flag
    assert _partial(L, cp, t, t, t, h, o=0) == EINVAL                              # no output
    assert _partial(L, cp, t, t, t, h, o=0x2004) == EUNSUPPORTED                   # output alignment
    assert _partial(L, cp, t, t, t, h, qpos=(60, 1)) == EINVAL                     # beyond the mask
    assert _partial(L, cp, t, t, t, h, kpos=(0, 0)) == EINVAL                      # stride 0
    assert _partial(L, cp, _tensor(cp, n=0), t, t, h) == OK                        # empty query block
    huge = _tensor(cp, n=(1 << 23), st=256)
    assert _partial(L, cp, huge, huge, huge, h) == EUNSUPPORTED                    # > 2 GiB per head
    assert L.cpattn_mask_free(h) == OK


def test_stream_probe_validation(L):
    """The bandwidth probe checks its arguments before any device work."""
    assert L.cpattn_stream_probe(2, 0x1000, 0x2000, 1024, 0, None) == EINVAL      # kind
    assert L.cpattn_stream_probe(0, 0x1000, 0x2000, 1000, 0, None) == EINVAL      # not a multiple of 16
    assert L.cpattn_stream_probe(1, 0x1000, 0x2000, -16, 0, None) == EINVAL       # negative size
    assert L.cpattn_stream_probe(1, 0x1000, 0x2000, 1024, 1 << 21, None) == EINVAL  # grid
    assert L.cpattn_stream_probe(1, 0, 0x2000, 1024, 0, None) == EINVAL           # NULL
    assert L.cpattn_stream_probe(1, 0x1008, 0x2000, 1024, 0, None) == EUNSUPPORTED  # alignment
    assert L.cpattn_stream_probe(1, 0x1000, 0x2000, 0, 0, None) == OK             # nothing to stream


def test_merge_and_ring_validation(L):
    import context_blockwise_attention_amd as cp
    P = ctypes.c_void_p
    parts = (P * 65)(*([0x1000] * 65))
    assert L.cpattn_merge(0, parts, parts, 10, 128, 0x2000, 0x3000, None) == EINVAL
    assert L.cpattn_merge(65, parts, parts, 10, 128, 0x2000, 0x3000, None) == EINVAL
    assert L.cpattn_merge(2, parts, parts, 10, 0, 0x2000, 0x3000, None) == EINVAL
    assert L.cpattn_merge(2, parts, parts, 0, 128, 0x2000, 0x3000, None) == OK     # no rows: no-op
    h = ctypes.c_void_p()
    assert L.cpattn_mask_causal(64, ctypes.byref(h)) == OK
    N = 2
    ts = (cp._Tensor * N)(*[_tensor(cp) for _ in range(N)])
    pos = (cp._PosMap * N)(cp._PosMap(0, 1), cp._PosMap(16, 1))
    outs = (P * N)(0x2000, 0x2000)
    assert L.cpattn_ring_emulate(0, ts, ts, ts, pos, None, 0, h, 0.1, outs, outs, None) == EINVAL
    assert L.cpattn_ring_emulate(65, ts, ts, ts, pos, None, 65, h, 0.1, outs, outs, None) == EINVAL
    bad = (ctypes.c_int * 1)(5)
    assert L.cpattn_ring_emulate(N, ts, ts, ts, pos, bad, 1, h, 0.1, outs, outs, None) == EINVAL
    dup = (ctypes.c_int * 2)(1, 1)
    assert L.cpattn_ring_emulate(N, ts, ts, ts, pos, dup, 2, h, 0.1, outs, outs, None) == EINVAL
    assert L.cpattn_ring_emulate(N, ts, ts, ts, pos, None, 1, h, 0.1, outs, outs, None) == EINVAL
    far = (cp._PosMap * N)(cp._PosMap(0, 1), cp._PosMap(60, 1))
    assert L.cpattn_ring_emulate(N, ts, ts, ts, far, None, N, h, 0.1, outs, outs, None) == EINVAL
    assert L.cpattn_mask_free(h) == OK


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    import context_blockwise_attention_amd as cp
    monkeypatch.setattr(cp, "_lib", None)
    monkeypatch.setattr(cp, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(ImportError):
        cp.lib()


def test_merge_and_sink_backward_validation(L):
    P = ctypes.c_void_p
    parts = (P * 65)(*([0x1000] * 65))
    bad = (P * 2)(0x1000, 0x1004)
    a = (0x2000, 0x3000, 0x4000)   # o, lse, g_o
    assert L.cpattn_merge_backward(0, parts, parts, 10, 128, *a, None, parts, parts, None) == EINVAL
    assert L.cpattn_merge_backward(65, parts, parts, 10, 128, *a, None, parts, parts, None) == EINVAL
    assert L.cpattn_merge_backward(2, parts, parts, 10, 0, *a, None, parts, parts, None) == EINVAL
    assert L.cpattn_merge_backward(2, parts, parts, 10, 6, *a, None, parts, parts, None) == EUNSUPPORTED
    assert L.cpattn_merge_backward(2, parts, parts, 10, 128, *a, None, None, parts, None) == EINVAL
    assert L.cpattn_merge_backward(2, parts, parts, 0, 128, *a, None, parts, parts, None) == OK     # no rows
    assert L.cpattn_merge_backward(2, bad, parts, 10, 128, *a, None, parts, parts, None) == EUNSUPPORTED
    assert L.cpattn_merge_backward(2, parts, parts, 10, 128, 0, 0x3000, 0x4000, None, parts, parts, None) == EINVAL
    assert L.cpattn_last_error().startswith(b"cpattn_merge_backward")
    s = (0x2000, 0x3000, 0x5000)   # o, lse, sink
    assert L.cpattn_sink_backward(*s, 0, 10, 128, 0x4000, 0x6000, 0x7000, 0x8000, None) == EINVAL
    assert L.cpattn_sink_backward(*s, 2, 10, 6, 0x4000, 0x6000, 0x7000, 0x8000, None) == EUNSUPPORTED
    assert L.cpattn_sink_backward(0x2000, 0x3000, 0, 2, 10, 128, 0x4000, 0x6000, 0x7000, 0x8000, None) == EINVAL
    assert L.cpattn_sink_backward(*s, 2, 10, 128, 0x4000, 0x6004, 0x7000, 0x8000, None) == EUNSUPPORTED
    assert L.cpattn_sink_backward(*s, 2, 10, 128, 0x4000, 0x6000, 0, 0x8000, None) == EINVAL
    assert L.cpattn_last_error().startswith(b"cpattn_sink_backward")


def test_backward_validation(L):
    import context_blockwise_attention_amd as cp
    P = ctypes.c_void_p
    h = ctypes.c_void_p()
    assert L.cpattn_mask_causal(64, ctypes.byref(h)) == OK
    N, C = 2, 2
    ts = (cp._Tensor * (N * C))(*[_tensor(cp) for _ in range(N * C)])
    pos = (cp._PosMap * (N * C))(*[cp._PosMap(16 * i, 1) for i in range(N * C)])
    ptrs = (P * (N * C))(*([0x2000] * (N * C)))
    args = lambda n, c, t=ts, p=pos: (n, c, t, t, t, p, h, 0.1, ptrs, ptrs, t, ptrs, ptrs, ptrs, None)
    assert L.cpattn_ring_backward_chunks(*args(0, C)) == EINVAL                      # N out of range
    assert L.cpattn_ring_backward_chunks(*args(N, 0)) == EINVAL                      # C out of range
    assert L.cpattn_ring_backward_chunks(*args(N, 9)) == EINVAL
    far = (cp._PosMap * (N * C))(*[cp._PosMap(60, 1) for _ in range(N * C)])
    assert L.cpattn_ring_backward_chunks(*args(N, C, p=far)) == EINVAL               # positions past the mask
    bad = (cp._Tensor * (N * C))(*([_tensor(cp)] * 3 + [_tensor(cp, d=64)]))
    assert L.cpattn_ring_backward_chunks(*args(N, C, t=bad)) == EUNSUPPORTED         # mixed head dims
    assert L.cpattn_last_error().startswith(b"cpattn_ring_backward_chunks")
    assert L.cpattn_ring_backward(0, ts, ts, ts, pos, h, 0.1, ptrs, ptrs, ts, ptrs, ptrs, ptrs, None) == EINVAL
    t = _tensor(cp)
    assert L.cpattn_partial_backward(ctypes.byref(t), ctypes.byref(t), ctypes.byref(t), None, cp._PosMap(0, 1),
                                     cp._PosMap(0, 1), 0.1, 0x3000, 0x3000, ctypes.byref(t), 0x2000, 0x2000,
                                     0x2000, None) == EINVAL                          # no mask
    t7 = _tensor(cp, dtype=7)
    assert L.cpattn_backward_delta(0x2000, ctypes.byref(t7), 0x3000, None) == EUNSUPPORTED
    assert L.cpattn_backward_delta(0x2004, ctypes.byref(t), 0x3000, None) == EUNSUPPORTED   # o misaligned
    assert L.cpattn_backward_delta(0x2000, ctypes.byref(t), 0x3002, None) == EUNSUPPORTED   # delta misaligned
    assert L.cpattn_backward_delta(0, ctypes.byref(t), 0x3000, None) == EINVAL              # no o
    assert L.cpattn_mask_free(h) == OK


def test_last_error_is_per_thread(L):
    """cpattn_last_error() is the calling thread's own: eight host threads
    fail validation at once, each in its own way, many times over, and each
    reads back the message of its own failure (the binding's foreign calls
    release the interpreter lock, so the calls do overlap)."""
    import threading
    import context_blockwise_attention_amd as cp
    h = ctypes.c_void_p()
    assert L.cpattn_mask_causal(64, ctypes.byref(h)) == OK
    t = _tensor(cp)
    cases = [
        (lambda: _partial(L, cp, _tensor(cp, d=96), t, t, h), EUNSUPPORTED, b"head dim"),
        (lambda: _partial(L, cp, t, t, t, h, scale=0.0), EUNSUPPORTED, b"scale"),
        (lambda: _partial(L, cp, t, t, t, h, acc=2), EINVAL, b"accumulate"),
        (lambda: _partial(L, cp, t, t, t, h, qpos=(60, 1)), EINVAL, b"q_pos"),
        (lambda: _partial(L, cp, t, t, _tensor(cp, n=15), h), EINVAL, b"token counts"),
        (lambda: _partial(L, cp, _tensor(cp, st=132), t, t, h), EUNSUPPORTED, b"strides"),
        (lambda: _partial(L, cp, t, t, t, None), EINVAL, b"mask is NULL"),
        (lambda: _partial(L, cp, t, t, t, h, o=0x2004), EUNSUPPORTED, b"aligned"),
    ]
    bad = []
    start = threading.Barrier(len(cases))

    def worker(call, code, word):
        start.wait()
        for _ in range(2000):
            rc = call()
            msg = L.cpattn_last_error()
            if rc != code or word not in msg:
                bad.append((word, rc, msg))
                return

    threads = [threading.Thread(target=worker, args=c) for c in cases]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    assert L.cpattn_mask_free(h) == OK
    assert not bad, bad[:4]
