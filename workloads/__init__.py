"""Seeded synthetic workloads for blockwise attention.

This module serves both the HIP path's tests/benchmark and the CPU reference.
It holds no attention arithmetic: only random tensors, packed-tree layouts,
position lists for block/stripe/zig-zag sharding, and sampled query rows.

Workloads (all inputs synthetic and seeded):

* ``tiny_causal``   -- 1 head, d=64, 256 tokens in 4 blocks of 64, fp32.
* ``causal_ring``   -- 32 heads, d=128, 32768 tokens in 8 contiguous blocks
  of 4096, bf16 (a Llama-2-7B-like attention layer: 32 heads x 128).
* ``striped``       -- P=4 stripes over 65536 positions: rank 0 owns positions
  ``x % 4 == 0`` (16384 queries) and visits the 4 stripes of K/V, bf16.
* ``tree64k``       -- prefix-tree packed row: a 24576-token prompt and five
  8192-token completions (65536 physical tokens, 32768 logical per
  trajectory), 4 contiguous blocks of 16384, bf16.
* ``tree128k_share`` -- 131072 tokens packed from seeded prompt/completion
  families, one GPU's share of a 4-way split: 32768 local queries against 4
  K/V blocks of 32768, bf16.

Tensors are drawn as float32 N(0, 1) with ``torch.Generator().manual_seed``
in the order Q, K, V, each ``[H, n, d]``, then rounded to bf16 (round to
nearest even) where the workload is bf16.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional, Tuple

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    heads: int
    d: int
    n_tok: int          # physical tokens in the packed row / sequence
    n_blocks: int       # ring size (number of K/V blocks)
    dtype: str          # "f32" or "bf16"
    layout: str         # "contiguous" or "striped"
    mask: str           # "causal" or "tree"
    ranks: Tuple[int, ...] = ()   # ranks whose queries are computed (empty = all)
    description: str = ""


WORKLOADS = {
    "tiny_causal": Workload("tiny_causal", 1, 64, 256, 4, "f32", "contiguous", "causal",
                            description="1 head, d=64, 256 tokens, 4 blocks of 64, fp32"),
    "causal_ring": Workload("causal_ring", 32, 128, 32768, 8, "bf16", "contiguous", "causal",
                            description="32 heads, d=128, 32768 tokens, 8 blocks of 4096"),
    "striped": Workload("striped", 32, 128, 65536, 4, "bf16", "striped", "causal", ranks=(0,),
                        description="P=4 stripes of 65536 positions, rank 0's 16384 queries"),
    "tree64k": Workload("tree64k", 32, 128, 65536, 4, "bf16", "contiguous", "tree",
                        description="24576-token prompt + 5 x 8192 completions, 4 blocks"),
    "tree128k_share": Workload("tree128k_share", 32, 128, 131072, 4, "bf16", "contiguous",
                               "tree", ranks=(0,),
                               description="131072 tokens of seeded families, rank 0 of 4"),
}


# ----------------------------------------------------------------------------
# random tensors
# ----------------------------------------------------------------------------
def qkv(seed: int, heads: int, n: int, d: int, dtype: str = "bf16", n_kv: Optional[int] = None):
    """Q [heads, n, d] and K, V [heads, n_kv, d] as CPU torch tensors."""
    import torch
    g = torch.Generator(device="cpu").manual_seed(int(seed))
    n_kv = n if n_kv is None else n_kv
    q = torch.randn((heads, n, d), generator=g, dtype=torch.float32)
    k = torch.randn((heads, n_kv, d), generator=g, dtype=torch.float32)
    v = torch.randn((heads, n_kv, d), generator=g, dtype=torch.float32)
    if dtype == "bf16":
        q, k, v = q.to(torch.bfloat16), k.to(torch.bfloat16), v.to(torch.bfloat16)
    elif dtype != "f32":
        raise ValueError(dtype)
    return q, k, v


# ----------------------------------------------------------------------------
# packed prefix trees: per-token segment ids and per-segment parents
# ----------------------------------------------------------------------------
def tree_from_lengths(lengths: List[int], parents: List[int]):
    """Segments laid out in the given order; returns (seg_id[int32], parent[int32])."""
    seg = np.repeat(np.arange(len(lengths), dtype=np.int32), np.asarray(lengths, dtype=np.int64))
    return seg.astype(np.int32), np.asarray(parents, dtype=np.int32)


def tree_prompt_completions(prompt: int = 24576, completions=(8192,) * 5):
    """One prompt followed by its completions, each a child of the prompt."""
    lengths = [prompt] + list(completions)
    parents = [-1] + [0] * len(completions)
    return tree_from_lengths(lengths, parents)


def tree_families(seed: int, total: int = 131072, prompt_range=(2048, 16384), m_range=(2, 8),
                  completion_range=(1024, 8192)):
    """Seeded families packed until ``total`` tokens: per family draw (in this
    order, with ``numpy.random.default_rng(seed)``) the prompt length, the
    number of completions and their lengths, all uniform with inclusive ends.
    The segment that crosses ``total`` is clipped and packing stops there.
    Returns (seg_id, parent, segments) with segments = list of (start, len, parent)."""
    rng = np.random.default_rng(seed)
    lengths: List[int] = []
    parents: List[int] = []
    used = 0
    while used < total:
        P = int(rng.integers(prompt_range[0], prompt_range[1], endpoint=True))
        m = int(rng.integers(m_range[0], m_range[1], endpoint=True))
        C = rng.integers(completion_range[0], completion_range[1], size=m, endpoint=True)
        root = len(lengths)
        for i, L in enumerate([P] + [int(c) for c in C]):
            take = min(L, total - used)
            lengths.append(take)
            parents.append(-1 if i == 0 else root)
            used += take
            if used >= total:
                break
    return tree_from_lengths(lengths, parents)


def tiny_tree():
    """The tiny tree used to explain tree masks: root at 0..3, completion A at
    4..6 and completion B at 7..8, both children of the root."""
    return tree_from_lengths([4, 3, 2], [-1, 0, 0])


# ----------------------------------------------------------------------------
# sharding layouts (global positions owned by each rank)
# ----------------------------------------------------------------------------
def contiguous(n: int, n_ranks: int) -> List[np.ndarray]:
    c = n // n_ranks
    return [np.arange(r * c, (r + 1) * c, dtype=np.int64) for r in range(n_ranks)]


def striped(n: int, P: int) -> List[np.ndarray]:
    """Rank r owns the positions x with x % P == r."""
    return [np.arange(r, n, P, dtype=np.int64) for r in range(P)]


def zigzag(n: int, n_ranks: int) -> List[np.ndarray]:
    """2N chunks; rank r owns chunk r and chunk 2N-1-r."""
    c = n // (2 * n_ranks)
    return [np.concatenate([np.arange(r * c, (r + 1) * c),
                            np.arange((2 * n_ranks - 1 - r) * c, (2 * n_ranks - r) * c)]).astype(np.int64)
            for r in range(n_ranks)]


# ----------------------------------------------------------------------------
# sampled query rows for large-size checks
# ----------------------------------------------------------------------------
def sample_rows(seed: int, head: int, n_rows: int, forced=(), count: int = 256) -> np.ndarray:
    """Up to ``count`` distinct rows: the forced ones (clipped to range, at
    most 64) then seeded uniform draws without replacement."""
    forced = sorted({int(f) for f in forced if 0 <= int(f) < n_rows})[:64]
    count = min(count, n_rows)
    rest = np.setdiff1d(np.arange(n_rows), np.asarray(forced, dtype=np.int64))
    rng = np.random.default_rng(1000 * seed + head)
    extra = rng.choice(rest, size=max(0, count - len(forced)), replace=False) if len(rest) else []
    return np.sort(np.concatenate([np.asarray(forced, dtype=np.int64),
                                   np.asarray(extra, dtype=np.int64)])).astype(np.int64)


def segment_bounds(seg: np.ndarray) -> List[Tuple[int, int]]:
    """(first, last) position of each contiguous run of equal segment ids."""
    change = np.flatnonzero(np.diff(seg)) + 1
    starts = np.concatenate([[0], change])
    ends = np.concatenate([change, [len(seg)]]) - 1
    return list(zip(starts.tolist(), ends.tolist()))
