"""Blockwise (ring / context-parallel) attention on AMD gfx950.

A thin ctypes binding over ``libcpattn.so`` (C ABI in ``include/cpattn.h``).
Every step of the computation runs in the library's HIP kernels; this module
only marshals arguments: it turns torch tensors into (pointer, sizes, strides)
descriptors and passes the current HIP stream.  PyTorch supplies device
memory and streams, nothing else.  There is no fallback: if the library is
missing or a call is rejected, an exception says why.

Entry points (same names as the C ABI):

* :class:`Mask` -- ``Mask.causal(n_pos)`` / ``Mask.tree(seg_id, parent)``:
  visibility descriptors.
* :func:`partial` -- (O, LSE) of a query block against one K/V block,
  optionally merged into a running (O, LSE).
* :func:`merge` -- merge of several partials.
* :func:`ring_emulate` -- every round of a ring of N ranks on one GPU.
* :func:`ring_emulate_chunks` -- the same for ranks that hold several chunks
  (the zig-zag layout).
* :func:`ring_plan` -- per-rank, per-round visible-pair counts (host only).
* :func:`apply_sink` -- learned attention-sink logits applied once to a
  complete result.
* :func:`backward_delta`, :func:`partial_backward`, :func:`ring_backward` --
  gradients with the global softmax derivative.
"""
from __future__ import annotations

import contextlib
import ctypes
import math
import os
from typing import List, Optional, Sequence, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libcpattn.so")

OK, EINVAL, EUNSUPPORTED, EDEVICE, ENOMEM = 0, -1, -2, -3, -4
BF16, F32 = 0, 1


class CpattnError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__("cpattn error %d: %s" % (code, msg))
        self.code = code


class _Tensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("n_heads", ctypes.c_int64), ("n_tok", ctypes.c_int64), ("d", ctypes.c_int64),
                ("stride_head", ctypes.c_int64), ("stride_tok", ctypes.c_int64)]


class _PosMap(ctypes.Structure):
    _fields_ = [("base", ctypes.c_int64), ("stride", ctypes.c_int64)]


_lib = None


def lib():
    """The loaded C library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("libcpattn.so is not built: run `python -m context_blockwise_attention_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        L.cpattn_last_error.restype = ctypes.c_char_p
        L.cpattn_version.restype = ctypes.c_int
        L.cpattn_mask_causal.argtypes = [ctypes.c_int64, ctypes.POINTER(P)]
        L.cpattn_mask_tree.argtypes = [P, ctypes.c_int64, P, ctypes.c_int32, P, ctypes.POINTER(P)]
        L.cpattn_mask_tree_static.argtypes = [P, ctypes.c_int64, P, ctypes.c_int32, P, ctypes.POINTER(P)]
        L.cpattn_mask_free.argtypes = [P]
        L.cpattn_mask_with_window.argtypes = [P, ctypes.c_int64, P, ctypes.POINTER(P)]
        L.cpattn_mask_npos.argtypes = [P]
        L.cpattn_mask_npos.restype = ctypes.c_int64
        L.cpattn_partial.argtypes = [ctypes.POINTER(_Tensor)] * 3 + [P, _PosMap, _PosMap, ctypes.c_float,
                                                                      P, P, ctypes.c_int, P]
        L.cpattn_merge.argtypes = [ctypes.c_int, P, P, ctypes.c_int64, ctypes.c_int64, P, P, P]
        L.cpattn_ring_emulate.argtypes = [ctypes.c_int, P, P, P, P, P, ctypes.c_int, P, ctypes.c_float,
                                          P, P, P]
        L.cpattn_ring_emulate_chunks.argtypes = [ctypes.c_int, ctypes.c_int, P, P, P, P, P, ctypes.c_int, P,
                                                 ctypes.c_float, P, P, P]
        L.cpattn_ring_plan.argtypes = [ctypes.c_int, ctypes.c_int, P, P, P, P]
        L.cpattn_apply_sink.argtypes = [P, P, P, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, P]
        L.cpattn_backward_delta.argtypes = [P, ctypes.POINTER(_Tensor), P, P]
        L.cpattn_partial_backward.argtypes = [ctypes.POINTER(_Tensor)] * 3 + [P, _PosMap, _PosMap, ctypes.c_float,
                                                                               P, P, ctypes.POINTER(_Tensor), P, P, P,
                                                                               P]
        L.cpattn_ring_backward.argtypes = [ctypes.c_int, P, P, P, P, P, ctypes.c_float, P, P, P, P, P, P, P]
        L.cpattn_merge_backward.argtypes = [ctypes.c_int, P, P, ctypes.c_int64, ctypes.c_int64, P, P, P, P, P, P, P]
        L.cpattn_ring_backward_chunks.argtypes = [ctypes.c_int, ctypes.c_int, P, P, P, P, P, ctypes.c_float, P, P, P,
                                                  P, P, P, P]
        L.cpattn_sink_backward.argtypes = [P, P, P, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, P, P, P, P, P]
        L.cpattn_stream_probe.argtypes = [ctypes.c_int, P, P, ctypes.c_int64, ctypes.c_int, P]
        for f in ("cpattn_mask_causal", "cpattn_mask_tree", "cpattn_mask_tree_static", "cpattn_mask_free",
                  "cpattn_partial",
                  "cpattn_merge", "cpattn_ring_emulate", "cpattn_ring_emulate_chunks", "cpattn_ring_plan",
                  "cpattn_apply_sink", "cpattn_mask_with_window", "cpattn_backward_delta",
                  "cpattn_partial_backward", "cpattn_ring_backward", "cpattn_ring_backward_chunks",
                  "cpattn_merge_backward",
                  "cpattn_sink_backward", "cpattn_stream_probe"):
            getattr(L, f).restype = ctypes.c_int
        _lib = L
    return _lib


def _check(rc: int):
    if rc != OK:
        raise CpattnError(rc, lib().cpattn_last_error().decode())


def version() -> Tuple[int, int]:
    v = lib().cpattn_version()
    return v >> 16, v & 0xFFFF


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def _on(stream):
    """Context for the tensors a call allocates itself (outputs, zero-filled
    gradient buffers): made on the stream the call enqueues on.  torch's
    caching allocator ties a block to the stream it is made on, and a zero
    fill runs on that stream, so both are then ordered with the call's
    kernels; made on another stream, a fill could still be running when the
    kernels add into the buffer."""
    if stream is None:
        return contextlib.nullcontext()
    if not isinstance(stream, torch.cuda.Stream):
        handle = int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)
        stream = torch.cuda.default_stream() if handle == 0 else torch.cuda.ExternalStream(handle)
    return torch.cuda.stream(stream)


def _desc(t: Optional[torch.Tensor], name: str) -> _Tensor:
    if t is None:
        return _Tensor(None, BF16, 0, 1, 0, 64, 64, 64)
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    if t.dim() != 3:
        raise ValueError("%s must be [heads, tokens, d]" % name)
    if t.dtype == torch.bfloat16:
        dt = BF16
    elif t.dtype == torch.float32:
        dt = F32
    else:
        raise CpattnError(EUNSUPPORTED, "%s dtype %s unsupported (bf16 or f32)" % (name, t.dtype))
    if t.stride(2) != 1:
        raise CpattnError(EUNSUPPORTED, "%s: the last dimension must be contiguous" % name)
    H, n, d = t.shape
    return _Tensor(t.data_ptr(), dt, 0, H, n, d, t.stride(0), t.stride(1))


def _posmap(p) -> _PosMap:
    if p is None:
        return _PosMap(0, 1)
    base, stride = p
    return _PosMap(int(base), int(stride))


class Mask:
    """Visibility descriptor.  Key position x is visible to query position y
    iff x <= y < end[x]; end[x] = +inf for a causal mask, and the end of the
    subtree of x's segment for a prefix tree stored in depth-first preorder."""

    def __init__(self, handle: int, n_pos: int, kind: str):
        self._h = ctypes.c_void_p(handle)
        self.n_pos = n_pos
        self.kind = kind

    @classmethod
    def causal(cls, n_pos: int) -> "Mask":
        h = ctypes.c_void_p()
        _check(lib().cpattn_mask_causal(int(n_pos), ctypes.byref(h)))
        return cls(h.value, int(n_pos), "causal")

    @classmethod
    def tree(cls, seg_id, parent, stream=None) -> "Mask":
        import numpy as np
        seg = np.ascontiguousarray(seg_id, dtype=np.int32)
        par = np.ascontiguousarray(parent, dtype=np.int32)
        h = ctypes.c_void_p()
        _check(lib().cpattn_mask_tree(seg.ctypes.data, seg.shape[0], par.ctypes.data, par.shape[0],
                                      _stream(stream), ctypes.byref(h)))
        return cls(h.value, int(seg.shape[0]), "tree")

    @classmethod
    def tree_static(cls, seg_id, parent, stream=None) -> "Mask":
        """The same descriptor as :meth:`tree`, built without device
        allocation into the library's static per-GPU buffer (at most 2^20
        tokens and 2^16 segments).  Every call on a GPU returns the same
        descriptor, replacing its previous contents."""
        import numpy as np
        seg = np.ascontiguousarray(seg_id, dtype=np.int32)
        par = np.ascontiguousarray(parent, dtype=np.int32)
        h = ctypes.c_void_p()
        _check(lib().cpattn_mask_tree_static(seg.ctypes.data, seg.shape[0], par.ctypes.data, par.shape[0],
                                             _stream(stream), ctypes.byref(h)))
        return cls(h.value, int(seg.shape[0]), "tree-static")

    def with_window(self, window: int, stream=None) -> "Mask":
        """A new descriptor: this visibility restricted to keys within
        ``window`` logical (root-to-leaf) positions of the query, itself
        included."""
        h = ctypes.c_void_p()
        # a causal descriptor has no device arrays: no stream needed (host only)
        st = 0 if (stream is None and not self.kind.startswith("tree")) else _stream(stream)
        _check(lib().cpattn_mask_with_window(self.handle, int(window), st, ctypes.byref(h)))
        return Mask(h.value, self.n_pos, self.kind + "+window%d" % int(window))

    @property
    def handle(self):
        if self._h is None or not self._h.value:
            raise ValueError("mask already freed")
        return self._h

    def free(self):
        if self._h is not None and self._h.value:
            _check(lib().cpattn_mask_free(self._h))
        self._h = None

    def __del__(self):
        try:
            if _lib is not None and self._h is not None and self._h.value:
                _lib.cpattn_mask_free(self._h)
        except Exception:
            pass


def _default_scale(d: int) -> float:
    return 1.0 / math.sqrt(d)


def partial(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, mask: Mask, q_pos=(0, 1), k_pos=(0, 1),
            scale: Optional[float] = None, out: Optional[Tuple[torch.Tensor, torch.Tensor]] = None,
            accumulate: bool = False, stream=None):
    """(O [H, n_q, d] fp32, LSE [H, n_q] fp32) of ``q`` against the block
    ``k``/``v`` (which may have H / g heads: grouped-query attention, query
    head h reads K/V head h // g).  Positions: row i of the query block sits at
    ``q_pos[0] + q_pos[1] * i`` (likewise ``k_pos``).  With ``accumulate``
    the result is merged into ``out`` (which must hold a running result)."""
    H, nq, d = q.shape
    if out is None:
        if accumulate:
            raise ValueError("accumulate needs out=")
        with _on(stream):
            out = (torch.empty((H, nq, d), dtype=torch.float32, device=q.device),
                   torch.empty((H, nq), dtype=torch.float32, device=q.device))
    o, lse = out
    if o.shape != (H, nq, d) or lse.shape != (H, nq) or o.dtype != torch.float32 or lse.dtype != torch.float32 \
            or not o.is_contiguous() or not lse.is_contiguous():
        raise ValueError("out must be contiguous fp32 ([H, n_q, d], [H, n_q])")
    qd, kd, vd = _desc(q, "q"), _desc(k, "k"), _desc(v, "v")
    _check(lib().cpattn_partial(ctypes.byref(qd), ctypes.byref(kd), ctypes.byref(vd), mask.handle,
                                _posmap(q_pos), _posmap(k_pos),
                                float(_default_scale(d) if scale is None else scale),
                                o.data_ptr(), lse.data_ptr(), 1 if accumulate else 0, _stream(stream)))
    return o, lse


def merge(parts: Sequence[Tuple[torch.Tensor, torch.Tensor]], out=None, stream=None):
    """Merge of partials ``[(O_p, LSE_p), ...]`` (fp32, O_p [..., d],
    LSE_p [...]) into one (O, LSE)."""
    parts = list(parts)
    if not parts:
        raise ValueError("nothing to merge")
    o0, l0 = parts[0]
    d = o0.shape[-1]
    rows = l0.numel()
    for o, l in parts:
        if o.shape != o0.shape or l.shape != l0.shape or o.dtype != torch.float32 or l.dtype != torch.float32 \
                or not o.is_contiguous() or not l.is_contiguous() or not o.is_cuda:
            raise ValueError("parts must be contiguous fp32 device tensors of one shape")
        if o.numel() != rows * d:
            raise ValueError("O and LSE shapes disagree")
    if out is None:
        with _on(stream):
            out = (torch.empty_like(o0), torch.empty_like(l0))
    n = len(parts)
    optrs = (ctypes.c_void_p * n)(*[p[0].data_ptr() for p in parts])
    lptrs = (ctypes.c_void_p * n)(*[p[1].data_ptr() for p in parts])
    _check(lib().cpattn_merge(n, optrs, lptrs, rows, d, out[0].data_ptr(), out[1].data_ptr(), _stream(stream)))
    return out


def ring_emulate(q_blocks: Sequence[Optional[torch.Tensor]], k_blocks: Sequence[torch.Tensor],
                 v_blocks: Sequence[torch.Tensor], pos: Sequence[Tuple[int, int]], mask: Mask,
                 scale: Optional[float] = None, ranks: Optional[Sequence[int]] = None, outs=None, stream=None):
    """Ring attention of N emulated ranks on one GPU.  Rank r holds
    ``q_blocks[r]``, ``k_blocks[r]``, ``v_blocks[r]`` at positions
    ``pos[r] = (base, stride)``; in round k it visits the K/V of rank
    ``(r - k) mod N``.  Returns ``{rank: (O, LSE)}`` for the ranks run."""
    N = len(k_blocks)
    if not (len(v_blocks) == len(pos) == len(q_blocks) == N):
        raise ValueError("every rank needs a q/k/v block and positions")
    run = list(range(N)) if ranks is None else [int(r) for r in ranks]
    d = k_blocks[0].shape[2]
    H = q_blocks[run[0]].shape[0] if run else k_blocks[0].shape[0]   # query heads (K/V may have fewer)
    if outs is None:
        outs = {}
        for r in run:
            nq = q_blocks[r].shape[1]
            with _on(stream):
                outs[r] = (torch.empty((H, nq, d), dtype=torch.float32, device=k_blocks[0].device),
                           torch.empty((H, nq), dtype=torch.float32, device=k_blocks[0].device))
    for r in run:
        o, l = outs[r]
        nq = q_blocks[r].shape[1]
        if o.shape != (H, nq, d) or l.shape != (H, nq) or o.dtype != torch.float32 or l.dtype != torch.float32 \
                or not o.is_contiguous() or not l.is_contiguous():
            raise ValueError("outs[%d] must be contiguous fp32 ([H, n_q, d], [H, n_q])" % r)
    qd = (_Tensor * N)(*[_desc(q_blocks[r] if r in run else None, "q") for r in range(N)])
    kd = (_Tensor * N)(*[_desc(k, "k") for k in k_blocks])
    vd = (_Tensor * N)(*[_desc(v, "v") for v in v_blocks])
    pd = (_PosMap * N)(*[_posmap(p) for p in pos])
    rk = (ctypes.c_int * len(run))(*run)
    op = (ctypes.c_void_p * N)(*[(outs[r][0].data_ptr() if r in outs else None) for r in range(N)])
    lp = (ctypes.c_void_p * N)(*[(outs[r][1].data_ptr() if r in outs else None) for r in range(N)])
    _check(lib().cpattn_ring_emulate(N, qd, kd, vd, pd, rk, len(run), mask.handle,
                                     float(_default_scale(d) if scale is None else scale), op, lp,
                                     _stream(stream)))
    return {r: outs[r] for r in run}


def ring_emulate_chunks(q_chunks: Sequence[Optional[torch.Tensor]], k_chunks: Sequence[torch.Tensor],
                        v_chunks: Sequence[torch.Tensor], pos: Sequence[Tuple[int, int]], mask: Mask,
                        chunks_per_rank: int, scale: Optional[float] = None, ranks: Optional[Sequence[int]] = None,
                        outs=None, stream=None):
    """Ring of N ranks holding ``chunks_per_rank`` (C) chunks each: chunk
    ``r * C + c`` of rank r has queries ``q_chunks[i]``, keys/values
    ``k_chunks[i]``/``v_chunks[i]`` at positions ``pos[i] = (base, stride)``.
    In round k every chunk of rank r meets every key chunk of rank
    ``(r - k) mod N``.  Returns ``{chunk index: (O, LSE)}`` for the chunks of
    the ranks run."""
    C = int(chunks_per_rank)
    NC = len(k_chunks)
    if C < 1 or NC % C != 0:
        raise ValueError("the number of chunks must be a multiple of chunks_per_rank")
    N = NC // C
    if not (len(v_chunks) == len(pos) == len(q_chunks) == NC):
        raise ValueError("every chunk needs q/k/v and positions")
    run = list(range(N)) if ranks is None else [int(r) for r in ranks]
    units = [r * C + c for r in run for c in range(C)]
    d = k_chunks[0].shape[2]
    H = q_chunks[units[0]].shape[0] if units else k_chunks[0].shape[0]   # query heads (K/V may have fewer)
    if outs is None:
        outs = {}
        for i in units:
            nq = q_chunks[i].shape[1]
            with _on(stream):
                outs[i] = (torch.empty((H, nq, d), dtype=torch.float32, device=k_chunks[0].device),
                           torch.empty((H, nq), dtype=torch.float32, device=k_chunks[0].device))
    for i in units:
        o, l = outs[i]
        nq = q_chunks[i].shape[1]
        if o.shape != (H, nq, d) or l.shape != (H, nq) or o.dtype != torch.float32 or l.dtype != torch.float32 \
                or not o.is_contiguous() or not l.is_contiguous():
            raise ValueError("outs[%d] must be contiguous fp32 ([H, n_q, d], [H, n_q])" % i)
    qd = (_Tensor * NC)(*[_desc(q_chunks[i] if i in outs else None, "q") for i in range(NC)])
    kd = (_Tensor * NC)(*[_desc(k, "k") for k in k_chunks])
    vd = (_Tensor * NC)(*[_desc(v, "v") for v in v_chunks])
    pd = (_PosMap * NC)(*[_posmap(p) for p in pos])
    rk = (ctypes.c_int * len(run))(*run)
    op = (ctypes.c_void_p * NC)(*[(outs[i][0].data_ptr() if i in outs else None) for i in range(NC)])
    lp = (ctypes.c_void_p * NC)(*[(outs[i][1].data_ptr() if i in outs else None) for i in range(NC)])
    _check(lib().cpattn_ring_emulate_chunks(N, C, qd, kd, vd, pd, rk, len(run), mask.handle,
                                            float(_default_scale(d) if scale is None else scale), op, lp,
                                            _stream(stream)))
    return {i: outs[i] for i in units}


def ring_plan(n_tok: Sequence[int], pos: Sequence[Tuple[int, int]], mask: Mask, chunks_per_rank: int = 1):
    """Visible (query, key) pairs per head of every rank in every round, as an
    ``[N, N]`` int64 array: ``work[r, k]`` = rank r's pairs against the keys
    of rank ``(r - k) mod N``.  Host-only; chunk i has ``n_tok[i]`` tokens at
    ``pos[i]``."""
    import numpy as np
    C = int(chunks_per_rank)
    NC = len(n_tok)
    if C < 1 or NC % C != 0 or len(pos) != NC:
        raise ValueError("n_tok and pos need N * chunks_per_rank entries")
    N = NC // C
    nt = (ctypes.c_int64 * NC)(*[int(x) for x in n_tok])
    pd = (_PosMap * NC)(*[_posmap(p) for p in pos])
    work = np.zeros(N * N, dtype=np.int64)
    _check(lib().cpattn_ring_plan(N, C, nt, pd, mask.handle, work.ctypes.data))
    return work.reshape(N, N)


def apply_sink(o: torch.Tensor, lse: torch.Tensor, sink_logits: torch.Tensor, stream=None):
    """Applies per-head sink logits ``sink_logits`` [H] (fp32, natural log)
    once to a complete result ``(o [H, n, d], lse [H, n])``, in place:
    ``lse <- logaddexp(lse, a)``, ``o <- o * exp(lse_old - lse)``."""
    H, n, d = o.shape
    if lse.shape != (H, n) or sink_logits.shape != (H,):
        raise ValueError("apply_sink expects o [H, n, d], lse [H, n], sink_logits [H]")
    for t, name in ((o, "o"), (lse, "lse"), (sink_logits, "sink_logits")):
        if not t.is_cuda or t.dtype != torch.float32 or not t.is_contiguous():
            raise ValueError("%s must be a contiguous fp32 device tensor" % name)
    _check(lib().cpattn_apply_sink(o.data_ptr(), lse.data_ptr(), sink_logits.data_ptr(), H, n, d,
                                   _stream(stream)))
    return o, lse


def ring_backward_chunks(q_chunks, k_chunks, v_chunks, pos, mask: Mask, lses, deltas, douts,
                         chunks_per_rank: int, scale=None, grads=None, stream=None):
    """Backward of :func:`ring_emulate_chunks` (all ranks): C =
    ``chunks_per_rank`` chunks per rank, chunk c of rank r at index r*C + c.
    ``grads[i]`` = (dq, dk, dv) fp32 per chunk (zero-filled new tensors if
    None); returns it."""
    NC = len(q_chunks)
    C = int(chunks_per_rank)
    if C < 1 or NC % C:
        raise ValueError("the number of chunks must be a multiple of chunks_per_rank")
    n_ranks = NC // C
    d = q_chunks[0].shape[2]
    if grads is None:
        with _on(stream):
            grads = [(torch.zeros(q_chunks[i].shape, dtype=torch.float32, device=q_chunks[i].device),
                      torch.zeros(k_chunks[i].shape, dtype=torch.float32, device=k_chunks[i].device),
                      torch.zeros(v_chunks[i].shape, dtype=torch.float32, device=v_chunks[i].device)) for i in range(NC)]
    qd = (_Tensor * NC)(*[_desc(t, "q") for t in q_chunks])
    kd = (_Tensor * NC)(*[_desc(t, "k") for t in k_chunks])
    vd = (_Tensor * NC)(*[_desc(t, "v") for t in v_chunks])
    od = (_Tensor * NC)(*[_desc(t, "dout") for t in douts])
    pd = (_PosMap * NC)(*[_posmap(p) for p in pos])
    P = ctypes.c_void_p
    arr = lambda ts, name: (P * NC)(*[_f32_dev(t, name) for t in ts])
    _check(lib().cpattn_ring_backward_chunks(n_ranks, C, qd, kd, vd, pd, mask.handle,
                                             float(_default_scale(d) if scale is None else scale),
                                             arr(lses, "lse"), arr(deltas, "delta"), od,
                                             arr([g[0] for g in grads], "dq"), arr([g[1] for g in grads], "dk"),
                                             arr([g[2] for g in grads], "dv"), _stream(stream)))
    return grads


def merge_backward(parts, merged, g_o, g_lse=None, outs=None, stream=None):
    """Adjoints of :func:`merge`: for parts ``[(O_p, LSE_p)]`` merged into
    ``merged = (O, LSE)``, output gradient ``g_o`` and optional LSE gradient
    ``g_lse``, returns ``[(dO_p, dLSE_p)]`` (fp32, shapes of the parts)."""
    parts = list(parts)
    if not parts:
        raise ValueError("no parts")
    o, lse = merged
    d = o.shape[-1]
    rows = lse.numel()
    for t, name in [(o, "o"), (lse, "lse"), (g_o, "g_o")] + [(g_lse, "g_lse")] * (g_lse is not None):
        _f32_dev(t, name)
    if g_o.shape != o.shape or (g_lse is not None and g_lse.shape != lse.shape):
        raise ValueError("gradient shapes differ from the merged result")
    for po, pl in parts:
        if po.shape != o.shape or pl.shape != lse.shape:
            raise ValueError("parts must have the merged result's shapes")
        _f32_dev(po, "o_p")
        _f32_dev(pl, "lse_p")
    if outs is None:
        with _on(stream):
            outs = [(torch.empty_like(o), torch.empty_like(lse)) for _ in parts]
    n = len(parts)
    P = ctypes.c_void_p
    arr = lambda ts: (P * n)(*[t.data_ptr() for t in ts])
    _check(lib().cpattn_merge_backward(n, arr([p[0] for p in parts]), arr([p[1] for p in parts]), rows, d,
                                       o.data_ptr(), lse.data_ptr(), g_o.data_ptr(),
                                       None if g_lse is None else g_lse.data_ptr(),
                                       arr([x[0] for x in outs]), arr([x[1] for x in outs]), _stream(stream)))
    return outs


def sink_backward(o: torch.Tensor, lse: torch.Tensor, sink_logits: torch.Tensor, g_o: torch.Tensor, stream=None):
    """Adjoints of :func:`apply_sink` from the result it left (``o`` [H, n, d]
    and ``lse`` [H, n] after the sink) and the output gradient ``g_o``:
    returns (dO, dLSE, d sink_logits) for the result before the sink."""
    H, n, d = o.shape
    if lse.shape != (H, n) or sink_logits.shape != (H,) or g_o.shape != o.shape:
        raise ValueError("sink_backward expects o [H, n, d], lse [H, n], sink_logits [H], g_o [H, n, d]")
    for t, name in ((o, "o"), (lse, "lse"), (sink_logits, "sink_logits"), (g_o, "g_o")):
        _f32_dev(t, name)
    with _on(stream):
        g_in = torch.empty_like(o)
        gl_in = torch.empty_like(lse)
        ga = torch.empty_like(sink_logits)
    _check(lib().cpattn_sink_backward(o.data_ptr(), lse.data_ptr(), sink_logits.data_ptr(), H, n, d,
                                      g_o.data_ptr(), g_in.data_ptr(), gl_in.data_ptr(), ga.data_ptr(),
                                      _stream(stream)))
    return g_in, gl_in, ga


def _f32_dev(t, name):
    if not t.is_cuda or t.dtype != torch.float32 or not t.is_contiguous():
        raise ValueError("%s must be a contiguous fp32 device tensor" % name)
    return t.data_ptr()


def backward_delta(o: torch.Tensor, dout: torch.Tensor, delta: Optional[torch.Tensor] = None, stream=None):
    """D = rowsum(dO * O) per query row ([H, n]) from the complete output O
    (fp32 [H, n, d]) and the output gradient dout (bf16 or fp32)."""
    H, n, d = dout.shape
    if o.shape != (H, n, d):
        raise ValueError("o and dout shapes differ")
    if delta is None:
        with _on(stream):
            delta = torch.empty((H, n), dtype=torch.float32, device=dout.device)
    dd = _desc(dout, "dout")
    _check(lib().cpattn_backward_delta(_f32_dev(o, "o"), ctypes.byref(dd), _f32_dev(delta, "delta"),
                                       _stream(stream)))
    return delta


def partial_backward(q, k, v, mask: Mask, lse, delta, dout, q_pos=(0, 1), k_pos=(0, 1), scale=None, grads=None,
                     stream=None):
    """Adds this (query block, K/V block) pair's gradients into ``grads`` =
    (dq [H, n_q, d], dk [H_kv, n_k, d], dv [H_kv, n_k, d]) fp32 (zero-filled
    new tensors if None), using the queries' complete ``lse`` and ``delta``."""
    H, nq, d = q.shape
    Hk, nk, _ = k.shape
    if grads is None:
        with _on(stream):
            grads = (torch.zeros((H, nq, d), dtype=torch.float32, device=q.device),
                     torch.zeros((Hk, nk, d), dtype=torch.float32, device=q.device),
                     torch.zeros((Hk, nk, d), dtype=torch.float32, device=q.device))
    dq, dk, dv = grads
    qd, kd, vd, dd = _desc(q, "q"), _desc(k, "k"), _desc(v, "v"), _desc(dout, "dout")
    _check(lib().cpattn_partial_backward(ctypes.byref(qd), ctypes.byref(kd), ctypes.byref(vd), mask.handle,
                                         _posmap(q_pos), _posmap(k_pos),
                                         float(_default_scale(d) if scale is None else scale),
                                         _f32_dev(lse, "lse"), _f32_dev(delta, "delta"), ctypes.byref(dd),
                                         _f32_dev(dq, "dq"), _f32_dev(dk, "dk"), _f32_dev(dv, "dv"),
                                         _stream(stream)))
    return grads


def ring_backward(q_blocks, k_blocks, v_blocks, pos, mask: Mask, lses, deltas, douts, scale=None, grads=None,
                  stream=None):
    """Backward of the ring of N ranks: in round k rank r's queries meet the
    keys of rank (r - k) mod N; dQ stays with rank r, dK and dV are added to
    the key owner's buffers.  ``grads[r]`` = (dq, dk, dv) fp32 per rank
    (zero-filled new tensors if None); returns it."""
    N = len(k_blocks)
    d = q_blocks[0].shape[2]
    if grads is None:
        with _on(stream):
            grads = [(torch.zeros(q_blocks[r].shape, dtype=torch.float32, device=q_blocks[r].device),
                      torch.zeros(k_blocks[r].shape, dtype=torch.float32, device=k_blocks[r].device),
                      torch.zeros(v_blocks[r].shape, dtype=torch.float32, device=v_blocks[r].device)) for r in range(N)]
    qd = (_Tensor * N)(*[_desc(t, "q") for t in q_blocks])
    kd = (_Tensor * N)(*[_desc(t, "k") for t in k_blocks])
    vd = (_Tensor * N)(*[_desc(t, "v") for t in v_blocks])
    od = (_Tensor * N)(*[_desc(t, "dout") for t in douts])
    pd = (_PosMap * N)(*[_posmap(p) for p in pos])
    P = ctypes.c_void_p
    lp = (P * N)(*[_f32_dev(t, "lse") for t in lses])
    dp = (P * N)(*[_f32_dev(t, "delta") for t in deltas])
    gq = (P * N)(*[_f32_dev(g[0], "dq") for g in grads])
    gk = (P * N)(*[_f32_dev(g[1], "dk") for g in grads])
    gv = (P * N)(*[_f32_dev(g[2], "dv") for g in grads])
    _check(lib().cpattn_ring_backward(N, qd, kd, vd, pd, mask.handle,
                                      float(_default_scale(d) if scale is None else scale), lp, dp, od, gq, gk, gv,
                                      _stream(stream)))
    return grads


def stream_probe(kind: str, src: torch.Tensor, dst: torch.Tensor, grid: int = 0, stream=None):
    """Measurement helper (not part of the attention path): one streaming
    ``"read"`` of ``src`` or ``"copy"`` of ``src`` into ``dst`` by the
    library's plain grid-stride kernel, ``grid`` workgroups (0: one lane per
    16 bytes)."""
    if kind not in ("read", "copy"):
        raise ValueError("kind must be 'read' or 'copy'")
    if not (src.is_cuda and dst.is_cuda and src.is_contiguous() and dst.is_contiguous()):
        raise ValueError("src and dst must be contiguous device tensors")
    nbytes = src.numel() * src.element_size()
    need = nbytes if kind == "copy" else 16
    if dst.numel() * dst.element_size() < need:
        raise ValueError("dst is too small")
    _check(lib().cpattn_stream_probe(0 if kind == "read" else 1, src.data_ptr(), dst.data_ptr(), nbytes, int(grid),
                                     _stream(stream)))
