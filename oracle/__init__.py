"""fp64 CPU reference for blockwise attention, its merge and the ring loop.

TEST INFRASTRUCTURE ONLY.  The product package never imports this module; only
``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` do.  It shares no code with the HIP path: the arithmetic lives in
``cpattn_oracle.c`` (plain C, fp64, OpenMP over rows), compiled here with gcc.

What each function follows:

* :func:`attention` -- "Context Parallelism in ART", section 02: the attention
  definition (scores ``q.k/sqrt(d)``, softmax over the visible keys, weighted
  sum of values) and the log-sum-exp summary ``(o_A, L_A)`` of a key subset.
  Visibility (same section and the tiny tree of section 03): causal = key
  position <= query position; tree = own segment up to and including the
  query, plus all tokens of strict ancestor segments.
* :func:`merge` -- same page, section 03: the stable two-way merge with the
  max shift, folded left over the parts (the page states the merge composes).
* :func:`ring` -- the ML-systems lesson on sequence/context parallelism, ring
  attention: in round ``k`` rank ``r`` computes against the K/V block of rank
  ``(r - k) mod N`` and merges the result into its running answer.

Readings of points the pages leave open that change results here: an empty visible set gives ``O = 0, L = -inf``; LSE is a
natural logarithm; bf16 inputs are widened exactly to fp64.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "cpattn_oracle.c")
_LIB_DIR = os.path.join(_HERE, "_build")
_LIB = os.path.join(_LIB_DIR, "libcpattn_oracle.so")
# A test may point the loader at a separately compiled copy (used to check that
# deliberately broken copies of the reference fail its pins).
_LIB_OVERRIDE = os.environ.get("CPATTN_ORACLE_LIB")

F64, F32, BF16 = 0, 1, 2
CAUSAL, TREE, FULL = 0, 1, 2


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (plain -O2, IEEE arithmetic, OpenMP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        os.makedirs(_LIB_DIR, exist_ok=True)
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fno-fast-math", "-fopenmp", "-shared", "-fPIC",
                               "-std=c99", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        if _LIB_OVERRIDE:
            lib = ctypes.CDLL(_LIB_OVERRIDE)
        else:
            build(force=False)
            lib = ctypes.CDLL(_LIB)
        i64, p = ctypes.c_int64, ctypes.c_void_p
        lib.oracle_attention.restype = ctypes.c_int
        lib.oracle_attention.argtypes = [i64, i64, i64, i64, i64, ctypes.c_int,
                                         p, i64, i64, p, i64, i64, p, i64, i64,
                                         p, p, ctypes.c_int, p, i64, p, ctypes.c_int32,
                                         i64, ctypes.c_double, p, i64, p, p, ctypes.c_int]
        lib.oracle_merge2.restype = None
        lib.oracle_merge2.argtypes = [i64, i64, p, p, p, p]
        lib.oracle_attention_backward.restype = ctypes.c_int
        lib.oracle_attention_backward.argtypes = [i64, i64, i64, i64, i64, ctypes.c_int,
                                                  p, i64, i64, p, i64, i64, p, i64, i64,
                                                  p, p, ctypes.c_int, p, i64, p, ctypes.c_int32,
                                                  i64, ctypes.c_double, p, i64, p, p, p, p, p, p]
        lib.oracle_merge_backward.restype = None
        lib.oracle_merge_backward.argtypes = [ctypes.c_int, p, p, i64, i64, p, p, p, p, p, p]
        lib.oracle_sink_backward.restype = None
        lib.oracle_sink_backward.argtypes = [i64, i64, i64, p, p, p, p, p, p, p]
        lib.oracle_apply_sink.restype = None
        lib.oracle_apply_sink.argtypes = [i64, i64, i64, p, p, p]
        lib.oracle_max_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def max_threads() -> int:
    return int(_load().oracle_max_threads())


# ----------------------------------------------------------------------------
# visibility descriptions (plain data; the predicate itself is in C)
# ----------------------------------------------------------------------------
@dataclass(frozen=True)
class Causal:
    """Key visible iff its global position <= the query's; with ``window``
    > 0 also within ``window`` positions of it, the query itself included."""
    window: int = 0


@dataclass(frozen=True)
class Full:
    """Every key visible (the non-causal case)."""


@dataclass(frozen=True)
class Tree:
    """Prefix tree: ``seg[x]`` = segment of global position x, ``parent[s]`` =
    parent segment of s (-1 for a root).  With ``window`` > 0 a query sees
    only the visible keys whose logical (root-to-leaf path) position is
    within ``window`` of its own ("Context Parallelism in ART", section 06)."""
    seg: np.ndarray
    parent: np.ndarray
    window: int = 0


def _as_array(x):
    """numpy view of a numpy array or CPU torch tensor; returns (array, dtype code)."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            if x.device.type != "cpu":
                raise ValueError("oracle inputs must live on the CPU")
            if x.dtype == torch.bfloat16:
                return x.contiguous().view(torch.int16).numpy().view(np.uint16), BF16
            x = x.contiguous().numpy()
    except ImportError:  # pragma: no cover
        pass
    x = np.ascontiguousarray(x)
    if x.dtype == np.float64:
        return x, F64
    if x.dtype == np.float32:
        return x, F32
    if x.dtype == np.uint16:
        return x, BF16
    raise TypeError("unsupported oracle input dtype %s" % x.dtype)


def attention(Q, K, V, qpos, kpos, mask=Causal(), scale: Optional[float] = None,
              rows: Optional[Sequence[int]] = None, n_threads: int = 0):
    """fp64 attention of queries ``Q[H, nq, d]`` over keys ``K[H, nk, d]`` /
    values ``V[H, nk, dv]`` (numpy or CPU torch; fp64, fp32 or bf16).

    ``qpos``/``kpos`` are the global positions of the query and key rows.
    ``rows`` restricts the computation to those query rows.  Returns
    ``(O[H, n_rows, dv], L[H, n_rows])`` in fp64; ``L`` is the natural-log LSE.
    """
    lib = _load()
    q, dt = _as_array(Q)
    k, dk = _as_array(K)
    v, dv_ = _as_array(V)
    if not (dt == dk == dv_):
        raise TypeError("Q, K and V must share one dtype")
    if q.ndim != 3 or k.ndim != 3 or v.ndim != 3:
        raise ValueError("Q, K, V must be [H, n, d]")
    H, nq, d = q.shape
    nk = k.shape[1]
    dv = v.shape[2]
    if k.shape != (H, nk, d) or v.shape[:2] != (H, nk):
        raise ValueError("shape mismatch")
    qpos = np.ascontiguousarray(qpos, dtype=np.int64)
    kpos = np.ascontiguousarray(kpos, dtype=np.int64)
    if qpos.shape != (nq,) or kpos.shape != (nk,):
        raise ValueError("position arrays must match the row counts")
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    rows_arr = None
    n_rows = nq
    if rows is not None:
        rows_arr = np.ascontiguousarray(rows, dtype=np.int64)
        n_rows = rows_arr.shape[0]
    O = np.zeros((H, n_rows, dv), dtype=np.float64)
    L = np.zeros((H, n_rows), dtype=np.float64)
    seg_p = par_p = None
    n_pos = 0
    n_seg = 0
    if isinstance(mask, Causal):
        kind = CAUSAL
    elif isinstance(mask, Full):
        kind = FULL
    elif isinstance(mask, Tree):
        kind = TREE
        seg = np.ascontiguousarray(mask.seg, dtype=np.int32)
        par = np.ascontiguousarray(mask.parent, dtype=np.int32)
        n_pos, n_seg = seg.shape[0], par.shape[0]
        seg_p, par_p = seg.ctypes.data, par.ctypes.data
    else:
        raise TypeError("unknown mask %r" % (mask,))
    rc = lib.oracle_attention(H, nq, nk, d, dv, dt,
                              q.ctypes.data, nq * d, d, k.ctypes.data, nk * d, d,
                              v.ctypes.data, nk * dv, dv,
                              qpos.ctypes.data, kpos.ctypes.data, kind, seg_p, n_pos,
                              par_p, n_seg, int(getattr(mask, "window", 0)), float(scale),
                              rows_arr.ctypes.data if rows_arr is not None else None, n_rows,
                              O.ctypes.data, L.ctypes.data, int(n_threads))
    if rc != 0:
        raise ValueError("oracle_attention rejected its arguments")
    return O, L


def merge2(a, b):
    """Stable two-way merge of partials ``(O, L)``; returns a new pair."""
    lib = _load()
    Oa = np.array(a[0], dtype=np.float64, copy=True, order="C")
    La = np.array(a[1], dtype=np.float64, copy=True, order="C")
    Ob = np.ascontiguousarray(b[0], dtype=np.float64)
    Lb = np.ascontiguousarray(b[1], dtype=np.float64)
    if Oa.shape != Ob.shape or La.shape != Lb.shape or Oa.shape[:-1] != La.shape:
        raise ValueError("partials must have matching shapes")
    dv = Oa.shape[-1]
    n = La.size
    lib.oracle_merge2(n, dv, Oa.ctypes.data, La.ctypes.data, Ob.ctypes.data, Lb.ctypes.data)
    return Oa, La


def merge(parts):
    """Merge of any number of partials, as a left fold of :func:`merge2`."""
    parts = list(parts)
    if not parts:
        raise ValueError("nothing to merge")
    acc = (np.array(parts[0][0], dtype=np.float64), np.array(parts[0][1], dtype=np.float64))
    for p in parts[1:]:
        acc = merge2(acc, p)
    return acc


def apply_sink(O, L, a):
    """Learned sink logits ``a`` [H] applied once to a complete result
    ``(O [H, n, d], L [H, n])`` ("Context Parallelism in ART", section 06):
    ``L_total = logaddexp(L, a)``, ``O * exp(L - L_total)``.  Returns new
    fp64 arrays."""
    lib = _load()
    Oc = np.array(O, dtype=np.float64, copy=True, order="C")
    Lc = np.array(L, dtype=np.float64, copy=True, order="C")
    ac = np.ascontiguousarray(a, dtype=np.float64)
    if Oc.ndim != 3 or Lc.shape != Oc.shape[:2] or ac.shape != (Oc.shape[0],):
        raise ValueError("apply_sink expects O [H, n, d], L [H, n], a [H]")
    lib.oracle_apply_sink(Oc.shape[0], Oc.shape[1], Oc.shape[2], Oc.ctypes.data, Lc.ctypes.data, ac.ctypes.data)
    return Oc, Lc


def ring(Q_r, q_pos, K_blocks, V_blocks, kv_pos, rank: int, mask=Causal(), scale=None,
         rows=None, n_threads: int = 0, keep_rounds: bool = False):
    """One rank's share of ring attention: round ``k`` visits K/V block
    ``(rank - k) mod N`` and merges into the running result.

    Returns ``(O, L)``, or ``(O, L, rounds)`` with ``keep_rounds`` where
    ``rounds`` is a list of ``(block, partial, running)`` per round.
    """
    N = len(K_blocks)
    if not (len(V_blocks) == len(kv_pos) == N) or not (0 <= rank < N):
        raise ValueError("bad ring arguments")
    run = None
    rounds = []
    for k in range(N):
        b = (rank - k) % N
        part = attention(Q_r, K_blocks[b], V_blocks[b], q_pos, kv_pos[b], mask, scale, rows,
                         n_threads)
        run = part if run is None else merge2(run, part)
        if keep_rounds:
            rounds.append((b, part, run))
    return (run[0], run[1], rounds) if keep_rounds else run



def _mask_fields(mask):
    """(kind, seg array or None, parent array or None, window) of a mask."""
    if isinstance(mask, Causal):
        return CAUSAL, None, None, mask.window
    if isinstance(mask, Full):
        return FULL, None, None, 0
    if isinstance(mask, Tree):
        return (TREE, np.ascontiguousarray(mask.seg, dtype=np.int32),
                np.ascontiguousarray(mask.parent, dtype=np.int32), mask.window)
    raise TypeError("unknown mask %r" % (mask,))


def attention_backward(Q, K, V, qpos, kpos, O, L, G, mask=Causal(), scale: Optional[float] = None, rows=None):
    """Gradients (dQ [H, n_rows, d], dK [H, nk, d], dV [H, nk, dv]) of
    attention over the keys of this call, given the rows' complete outputs
    O [H, n_rows, dv] and LSE L [H, n_rows] (over all their visible keys) and
    the output gradient G ("Context Parallelism in ART", section 04).
    Summing over any partition of the keys gives the full gradients."""
    lib = _load()
    q, dt = _as_array(Q)
    k, dk_ = _as_array(K)
    v, dv_ = _as_array(V)
    if not (dt == dk_ == dv_):
        raise TypeError("Q, K and V must share one dtype")
    H, nq, d = q.shape
    nk = k.shape[1]
    dv = v.shape[2]
    qpos = np.ascontiguousarray(qpos, dtype=np.int64)
    kpos = np.ascontiguousarray(kpos, dtype=np.int64)
    rows_arr = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    n_rows = nq if rows_arr is None else rows_arr.shape[0]
    O = np.ascontiguousarray(O, dtype=np.float64)
    L = np.ascontiguousarray(L, dtype=np.float64)
    G = np.ascontiguousarray(G, dtype=np.float64)
    if O.shape != (H, n_rows, dv) or G.shape != O.shape or L.shape != (H, n_rows):
        raise ValueError("O, G must be [H, n_rows, dv] and L [H, n_rows]")
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    kind, seg, par, window = _mask_fields(mask)
    dQ = np.zeros((H, n_rows, d))
    dK = np.zeros((H, nk, d))
    dV = np.zeros((H, nk, dv))
    rc = lib.oracle_attention_backward(
        H, nq, nk, d, dv, dt, q.ctypes.data, nq * d, d, k.ctypes.data, nk * d, d, v.ctypes.data, nk * dv, dv,
        qpos.ctypes.data, kpos.ctypes.data, kind, None if seg is None else seg.ctypes.data,
        0 if seg is None else seg.shape[0], None if par is None else par.ctypes.data,
        0 if par is None else par.shape[0], int(window), float(scale),
        None if rows_arr is None else rows_arr.ctypes.data, n_rows,
        O.ctypes.data, L.ctypes.data, G.ctypes.data, dQ.ctypes.data, dK.ctypes.data, dV.ctypes.data)
    if rc != 0:
        raise ValueError("oracle_attention_backward rejected its arguments")
    return dQ, dK, dV


def merge_backward(parts, O, L, G, gL=None):
    """Adjoints [(dO_r, dL_r)] of the merge of ``parts`` = [(O_r, L_r)] into
    (O, L), for output gradient G and optional LSE gradient gL ("Context
    Parallelism in ART", section 04)."""
    lib = _load()
    parts = [(np.ascontiguousarray(o, dtype=np.float64), np.ascontiguousarray(l, dtype=np.float64))
             for o, l in parts]
    O = np.ascontiguousarray(O, dtype=np.float64)
    L = np.ascontiguousarray(L, dtype=np.float64)
    G = np.ascontiguousarray(G, dtype=np.float64)
    dv = O.shape[-1]
    n_rows = L.size
    gl = None if gL is None else np.ascontiguousarray(gL, dtype=np.float64)
    outs = [(np.zeros_like(o), np.zeros_like(l)) for o, l in parts]
    n = len(parts)
    P = ctypes.c_void_p
    op = (P * n)(*[o.ctypes.data for o, _ in parts])
    lp = (P * n)(*[l.ctypes.data for _, l in parts])
    dop = (P * n)(*[o.ctypes.data for o, _ in outs])
    dlp = (P * n)(*[l.ctypes.data for _, l in outs])
    lib.oracle_merge_backward(n, op, lp, n_rows, dv, O.ctypes.data, L.ctypes.data, G.ctypes.data,
                              None if gl is None else gl.ctypes.data, dop, dlp)
    return outs


def sink_backward(O, L, a, G):
    """Adjoints (dO, dL, da) of the sink step y = w O, w = exp(L -
    logaddexp(L, a)) for output gradient G ("Context Parallelism in ART",
    section 06).  O is the output before the sink."""
    lib = _load()
    O = np.ascontiguousarray(O, dtype=np.float64)
    L = np.ascontiguousarray(L, dtype=np.float64)
    a = np.ascontiguousarray(a, dtype=np.float64)
    G = np.ascontiguousarray(G, dtype=np.float64)
    H, n, dv = O.shape
    dO = np.zeros_like(O)
    dL = np.zeros_like(L)
    da = np.zeros_like(a)
    lib.oracle_sink_backward(H, n, dv, O.ctypes.data, L.ctypes.data, a.ctypes.data, G.ctypes.data,
                             dO.ctypes.data, dL.ctypes.data, da.ctypes.data)
    return dO, dL, da
