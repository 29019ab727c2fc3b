"""Seeded synthetic packs for the coalesced attention engine.

A *pack* is one GPU's share of a mixed image-video batch, described the way the
Zellige page (Moldable Sequence Placement for Mixed Image-Video DiT Training,
§IV-D "Coalesced Attention Engine") describes a rank-local schedule: a list of
sequences, each stored as ``[tokens, heads, d]`` rows, and a list of segments that
say which query rows of a sequence attend to which of its key/value rows, over
which stored heads, and whether the result is final or one ring part of a
KV-split group (Table II: all-gather ``(q,1,1)``, Ulysses ``(1,h,1)``, ring
``(1,1,k)``).

This module holds shapes, segment lists and random draws only: no attention
arithmetic. Both the fp64 oracle tests and the HIP-path tests draw their inputs
here, so the two sides see identical bf16 values.
"""
from __future__ import annotations

import dataclasses
import hashlib
from typing import List, Optional, Sequence, Tuple

import torch

# (seq, head_begin, head_end, q_begin, q_end, kv_begin, kv_end, part)
Segment = Tuple[int, int, int, int, int, int, int, int]


@dataclasses.dataclass(frozen=True)
class Pack:
    """A rank-local pack: per-sequence lengths and stored heads, plus segments."""

    name: str
    seq_q: Tuple[int, ...]        # query tokens stored per sequence
    seq_kv: Tuple[int, ...]       # key/value tokens stored per sequence
    heads: Tuple[int, ...]        # heads stored per token, per sequence
    segments: Tuple[Segment, ...]
    d: int
    seed: int
    scale: Optional[float] = None  # None -> 1/sqrt(d)

    @property
    def n_seq(self) -> int:
        return len(self.seq_q)

    def q_rows(self) -> int:
        return sum(l * h for l, h in zip(self.seq_q, self.heads))

    def kv_rows(self) -> int:
        return sum(l * h for l, h in zip(self.seq_kv, self.heads))

    def softmax_scale(self) -> float:
        return self.scale if self.scale is not None else self.d ** -0.5

    def flops_fwd(self) -> float:
        """4*Lq*Lkv*d per (segment, head): the forward FLOP convention of the metric."""
        tot = 0
        for (s, h0, h1, q0, q1, k0, k1, part) in self.segments:
            tot += 4 * (q1 - q0) * (k1 - k0) * self.d * (h1 - h0)
        return float(tot)

    def flops_fwd_bwd(self) -> float:
        """Forward plus backward at 2.5x forward."""
        return 3.5 * self.flops_fwd()


def whole_pack(name: str, lengths: Sequence[int], heads: Sequence[int], d: int, seed: int) -> Pack:
    """Every sequence kept whole: one segment per sequence over all stored heads."""
    segs = tuple((i, 0, h, 0, l, 0, l, -1) for i, (l, h) in enumerate(zip(lengths, heads)))
    return Pack(name, tuple(lengths), tuple(lengths), tuple(heads), segs, d, seed)


def ring_pack(name: str, lq: int, lkv: int, n_parts: int, heads: int, d: int, seed: int) -> Pack:
    """One query chunk against the full K/V split into ``n_parts`` equal ring blocks."""
    blk = lkv // n_parts
    assert blk * n_parts == lkv
    segs = tuple((0, 0, heads, 0, lq, b * blk, (b + 1) * blk, b) for b in range(n_parts))
    return Pack(name, (lq,), (lkv,), (heads,), segs, d, seed)


def tiny() -> Pack:
    """3 whole sequences of 64, 256, 1024 tokens, 4 heads, d_head 64, seed 1."""
    return whole_pack("tiny", [64, 256, 1024], [4] * 3, 64, 1)


def image() -> Pack:
    """Image-only pack: 24 x 1024 then 8 x 4096 tokens, 24 heads, d_head 128, seed 2."""
    lens = [1024] * 24 + [4096] * 8
    return whole_pack("image", lens, [24] * len(lens), 128, 2)


def mixed() -> Pack:
    """Mixed image-video pack: 16 x 1024, 4 x 4096, 2 x 32760 tokens at 40 heads, then the
    5-head Ulysses shard of a 75600-token video (full length, 5 stored heads), d_head 128, seed 3."""
    lens = [1024] * 16 + [4096] * 4 + [32760] * 2 + [75600]
    heads = [40] * 22 + [5]
    return whole_pack("mixed", lens, heads, 128, 3)


def ring() -> Pack:
    """Ring KV-split shard: 9450 query tokens against 75600 K/V tokens in 8 blocks, 40 heads."""
    return ring_pack("ring", 9450, 75600, 8, 40, 128, 4)


def long() -> Pack:
    """Long-video share: 5 stored heads of a 497760-token sequence plus 8 x 4096 at 40 heads."""
    lens = [497760] + [4096] * 8
    heads = [5] + [40] * 8
    return whole_pack("long", lens, heads, 128, 5)


def shard() -> Pack:
    """One GPU's Ulysses share of a single 32760-token video: 5 of its 40 heads (8-way head
    split), full length, d_head 128, seed 6. 1280 forward items, 2.5 per resident workgroup."""
    return whole_pack("shard", [32760], [5], 128, 6)


def head1() -> Pack:
    """One stored head of a 32760-token video, full length, d_head 128, seed 7: 256 forward
    items, fewer than the resident workgroups, so the forward is split over keys."""
    return whole_pack("head1", [32760], [1], 128, 7)


CONFIGS = {"tiny": tiny, "image": image, "mixed": mixed, "ring": ring, "long": long, "shard": shard,
           "head1": head1}


def config(name: str) -> Pack:
    return CONFIGS[name]()


def draw(pack: Pack, seed: Optional[int] = None) -> dict:
    """Draw Q, K, V, dO (in that order) as fp32 N(0,1), each rounded once to bf16 (RNE).

    Shapes are ``[rows, d]`` over the packed row count of each tensor (Q and dO: query
    rows; K and V: key/value rows), all on the CPU.
    """
    g = torch.Generator(device="cpu")
    g.manual_seed(pack.seed if seed is None else seed)
    out = {}
    for name, rows in (("q", pack.q_rows()), ("k", pack.kv_rows()), ("v", pack.kv_rows()), ("do", pack.q_rows())):
        out[name] = torch.randn(rows, pack.d, generator=g, dtype=torch.float32).to(torch.bfloat16)
    return out


def sha256(t: torch.Tensor) -> str:
    return hashlib.sha256(t.contiguous().view(torch.uint8).numpy().tobytes()).hexdigest()


def draw_partials(n_parts: int, n_rows: int, d: int, seed: int, empty_frac: float = 0.0,
                  empty_rows: int = 0) -> dict:
    """A synthetic ring partial slab: ``o_part`` fp32 ``[n_parts, n_rows, d]`` and ``lse_part``
    fp32 ``[n_parts, n_rows]``, shaped like what ring parts of long sequences emit.

    Values: normalised partial outputs of a long block are averages of many unit-variance value
    rows, so ``o_part`` is N(0, 0.05^2); a part's log-sum-exp is about ln(block keys) plus a
    spread, so ``lse_part`` is 9 + 2 N(0, 1). ``empty_frac`` of the (part, row) entries get
    ``lse = -inf`` (a part that contributed no keys to the row), and the last ``empty_rows``
    rows are -inf in every part. Draw order: o_part, lse_part, then the empty mask.
    """
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    o = 0.05 * torch.randn(n_parts, n_rows, d, generator=g, dtype=torch.float32)
    lse = 9.0 + 2.0 * torch.randn(n_parts, n_rows, generator=g, dtype=torch.float32)
    if empty_frac > 0:
        lse[torch.rand(n_parts, n_rows, generator=g) < empty_frac] = float("-inf")
    if empty_rows > 0:
        lse[:, n_rows - empty_rows:] = float("-inf")
    return {"o_part": o, "lse_part": lse}
