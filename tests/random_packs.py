"""Seeded random packs for parity tests: shapes and segment lists only, no attention arithmetic.

Each pack holds 1-3 sequences (lengths drawn at and around the tile sizes, and query and key
lengths that may differ) with 1-4 stored heads. A sequence's heads are cut into 1-3 contiguous
subsets; each subset is covered by one segment kind:
  * whole: every query against every key;
  * query range: a random query sub-range against every key (the other query rows stay
    uncovered);
  * ring group: 2-4 parts over uneven key ranges, numbered in a random order (the key-block
    chain of the group then does not follow key order), over all queries or a sub-range.
Distinct head subsets never share O or K/V rows, so every pack is a valid segment list.
"""
from __future__ import annotations

import numpy as np

import workloads as W

_EDGE_LENGTHS = (1, 2, 63, 64, 65, 127, 128, 129)


def _length(rng) -> int:
    if rng.random() < 0.4:
        return int(rng.choice(_EDGE_LENGTHS))
    return int(rng.integers(1, 2500))


def random_pack(seed: int) -> W.Pack:
    rng = np.random.default_rng(seed)
    d = int(rng.choice((64, 128)))
    seq_q, seq_kv, heads, segs = [], [], [], []
    for s in range(int(rng.integers(1, 4))):
        lq = _length(rng)
        lkv = lq if rng.random() < 0.6 else _length(rng)
        nh = int(rng.integers(1, 5))
        seq_q.append(lq)
        seq_kv.append(lkv)
        heads.append(nh)
        n_sub = int(rng.integers(1, min(3, nh) + 1))
        cuts = sorted(int(c) for c in rng.choice(np.arange(1, nh), n_sub - 1, replace=False)) if n_sub > 1 else []
        bounds = [0, *cuts, nh]
        for h0, h1 in zip(bounds[:-1], bounds[1:]):
            kind = rng.choice(("whole", "qrange", "ring"))
            q0, q1 = 0, lq
            if kind != "whole" and lq > 1 and rng.random() < 0.5:
                q0 = int(rng.integers(0, lq))
                q1 = int(rng.integers(q0 + 1, lq + 1))
            if kind == "ring" and lkv >= 2:
                k = min(int(rng.integers(2, 5)), lkv)
                inner = sorted(int(c) for c in rng.choice(np.arange(1, lkv), k - 1, replace=False))
                kvb = [0, *inner, lkv]
                order = rng.permutation(k)
                for b in range(k):
                    segs.append((s, h0, h1, q0, q1, kvb[b], kvb[b + 1], int(order[b])))
            else:
                segs.append((s, h0, h1, q0, q1, 0, lkv, -1))
    return W.Pack(f"random{seed}", tuple(seq_q), tuple(seq_kv), tuple(heads), tuple(segs), d, 1000 + seed)


SEEDS = tuple(range(32))
