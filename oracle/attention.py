"""Plain fp64 CPU oracle for coalesced varlen attention.

TEST INFRASTRUCTURE, NOT PRODUCT CODE. Only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import or call anything here. The
library under ``coalesced_varlen_attention_amd`` never does, and this module never
imports it: the two share no code.

What is computed, and where the pages fix it (all on the Zellige page, "Moldable
Sequence Placement for Mixed Image-Video DiT Training"):

* §II-A: DiT attention is dense, bidirectional self-attention over one sequence's
  tokens. There is no causal mask and nothing inside a sequence is masked.
* §II-B: context parallelism computes *exact* attention by exchanging K/V; Ulysses
  turns sequence shards into head shards, so a head shard is ordinary attention on
  a subset of heads at full length; ring attention circulates K/V blocks while
  accumulating the output, which is an exact merge of per-block partial results.
* §IV-A and Table II: the query, head and key/value axes ``(q, h, k)`` of a
  placement option; a rank holds a query range, a head range and a K/V range.
* §IV-D: whole sequences are packed into one block-diagonal attention call that
  keeps sequences separate and returns outputs in the rank-local input order.
* §V-A: the training baselines use an exact backward.

Readings where the pages are silent (each is listed with its reason in the design
notes of the repository):

* softmax scale ``tau``: a parameter, ``1/sqrt(d)`` by default;
* log-sum-exp in natural log;
* a KV-split part emits a *normalised* partial output and its log-sum-exp; the
  merge is ``LSE = M + ln sum_b exp(LSE_b - M)``, ``O = sum_b exp(LSE_b - LSE) O_b``;
  parts with ``LSE_b = -inf`` have weight 0, and if every part is ``-inf`` the merge
  gives ``O = 0`` and ``LSE = -inf``;
* the backward of a KV-split group uses the merged (global) O and LSE, sums dQ over
  the parts, and gives each part's K/V rows the contribution of this query chunk;
* the backward gradients are those of ``f = sum_i dO_i . O_i`` over the rows that
  segments cover.

Everything is float64 numpy. The caller converts bf16 inputs to float64 first.
"""
from __future__ import annotations

import math
from typing import Dict, List, Sequence, Tuple

import numpy as np

# Largest number of score-matrix entries one query block may hold (float64): 256 MiB.
# Blocks are evaluated in preallocated buffers with in-place operations; each query row
# is still computed on its own, exactly as the definition states.
_BLOCK_ELEMS = 1 << 25
_MAX_ROWS = 256


def default_scale(d: int) -> float:
    """Softmax scale 1/sqrt(d) (the pages do not state one)."""
    return 1.0 / math.sqrt(d)


def _row_block(n_keys: int) -> int:
    return max(1, min(_MAX_ROWS, _BLOCK_ELEMS // max(1, n_keys)))


def head_scores(q: np.ndarray, k: np.ndarray, scale: float) -> np.ndarray:
    """s_ij = tau * q_i . k_j for every query row i and key row j (Zellige §II-A)."""
    return scale * (q @ k.T)


def head_probs(q: np.ndarray, k: np.ndarray, scale: float) -> np.ndarray:
    """Row-wise softmax of the scores: the full P matrix (small inputs only)."""
    s = head_scores(q, k, scale)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    return e / e.sum(axis=1, keepdims=True)


def head_forward(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float) -> Tuple[np.ndarray, np.ndarray]:
    """Softmax attention of one head: O = softmax(tau Q K^T) V and LSE per query row.

    Dense and bidirectional (Zellige §II-A): every query row sees every key row given.
    ``LSE_i = m_i + ln l_i`` with ``m_i = max_j s_ij`` and ``l_i = sum_j exp(s_ij - m_i)``;
    ``O_i = sum_j p_ij v_j`` with ``p_ij = exp(s_ij - LSE_i) = exp(s_ij - m_i) / l_i``.
    Query rows are processed in blocks only to bound memory.
    """
    lq = q.shape[0]
    nk = k.shape[0]
    o = np.empty((lq, v.shape[1]), dtype=np.float64)
    lse = np.empty(lq, dtype=np.float64)
    blk = _row_block(nk)
    buf = np.empty((min(blk, lq), nk), dtype=np.float64)
    kt = np.ascontiguousarray(k.T)
    for i0 in range(0, lq, blk):
        i1 = min(lq, i0 + blk)
        s = buf[: i1 - i0]
        np.matmul(q[i0:i1], kt, out=s)
        s *= scale                      # s_ij
        m = s.max(axis=1)
        s -= m[:, None]
        np.exp(s, out=s)                # exp(s_ij - m_i)
        l_sum = s.sum(axis=1)
        lse[i0:i1] = m + np.log(l_sum)
        s /= l_sum[:, None]             # p_ij
        o[i0:i1] = s @ v
    return o, lse


def head_delta(o: np.ndarray, do: np.ndarray) -> np.ndarray:
    """D_i = sum_c dO_ic O_ic for every query row: the row term of the exact softmax
    backward (§V-A), taken from the final output rows O_i."""
    return (do * o).sum(axis=1)


def head_backward(q: np.ndarray, k: np.ndarray, v: np.ndarray, o: np.ndarray, lse: np.ndarray,
                  do: np.ndarray, scale: float) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Exact gradients of f = sum_i dO_i . O_i for one head (the exact backward of §V-A).

    ``o`` and ``lse`` are the final output rows and log-sum-exps of these query rows
    (for a KV-split group: the merged ones), so ``p_ij = exp(s_ij - LSE_i)`` is the
    global softmax restricted to the keys given here.
      D_i   = sum_c dO_ic O_ic
      dp_ij = dO_i . v_j
      ds_ij = p_ij (dp_ij - D_i)
      dQ_i  = tau sum_j ds_ij k_j
      dK_j  = tau sum_i ds_ij q_i
      dV_j  = sum_i p_ij dO_i
    Passing a subset of the keys gives exact dK/dV rows for that subset; passing a
    subset of the queries (with their own O and LSE) gives exact dQ rows for them.
    """
    return head_backward_delta(q, k, v, lse, head_delta(o, do), do, scale)


def head_backward_delta(q: np.ndarray, k: np.ndarray, v: np.ndarray, lse: np.ndarray, dd: np.ndarray,
                        do: np.ndarray, scale: float) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """``head_backward`` given each query row's ``D_i`` (``dd``) instead of its output row.

    dK/dV of a key need every query row's LSE and D; this form lets a caller keep those two
    numbers per row instead of whole output rows.
    """
    lq = q.shape[0]
    nk = k.shape[0]
    dq = np.empty((lq, k.shape[1]), dtype=np.float64)
    dk = np.zeros(k.shape, dtype=np.float64)
    dv = np.zeros(v.shape, dtype=np.float64)
    blk = _row_block(nk)
    buf_p = np.empty((min(blk, lq), nk), dtype=np.float64)
    buf_s = np.empty((min(blk, lq), nk), dtype=np.float64)
    kt = np.ascontiguousarray(k.T)
    vt = np.ascontiguousarray(v.T)
    for i0 in range(0, lq, blk):
        i1 = min(lq, i0 + blk)
        p = buf_p[: i1 - i0]
        np.matmul(q[i0:i1], kt, out=p)
        p *= scale                      # s_ij
        p -= lse[i0:i1, None]
        np.exp(p, out=p)                # p_ij
        ds = buf_s[: i1 - i0]
        np.matmul(do[i0:i1], vt, out=ds)  # dp_ij
        ds -= dd[i0:i1, None]
        ds *= p                         # ds_ij
        dq[i0:i1] = scale * (ds @ k)
        dk += scale * (ds.T @ q[i0:i1])
        dv += p.T @ do[i0:i1]
    return dq, dk, dv


def lse_merge(o_parts: np.ndarray, lse_parts: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Exact merge of normalised partial outputs over disjoint key blocks (ring, §II-B).

    ``o_parts``: ``[n_parts, rows, d]``, ``lse_parts``: ``[n_parts, rows]``.
    ``LSE = M + ln sum_b exp(LSE_b - M)`` with ``M = max_b LSE_b``;
    ``O = sum_b exp(LSE_b - LSE) O_b``. A part with ``LSE_b = -inf`` has weight 0; a row
    whose parts are all ``-inf`` gets ``O = 0`` and ``LSE = -inf``.
    """
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    o_parts = np.asarray(o_parts, dtype=np.float64)
    m = lse_parts.max(axis=0)
    finite = np.isfinite(m)
    m_safe = np.where(finite, m, 0.0)
    w_un = np.where(np.isfinite(lse_parts), np.exp(lse_parts - m_safe[None, :]), 0.0)
    tot = w_un.sum(axis=0)
    lse = np.where(finite, m_safe + np.log(np.where(finite, tot, 1.0)), -np.inf)
    w = np.where(finite[None, :], w_un / np.where(finite, tot, 1.0)[None, :], 0.0)
    o = (w[:, :, None] * o_parts).sum(axis=0)
    return o, lse


def running_merge(o_acc: np.ndarray, lse_acc: np.ndarray, o_b: np.ndarray,
                  lse_b: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Fold one more normalised partial into a running (O, LSE) pair (ring, §II-B).

    The ring step that receives key block b updates the accumulated result in place:
    ``LSE' = ln(exp LSE + exp LSE_b)`` and ``O' = exp(LSE - LSE') O + exp(LSE_b - LSE') O_b``.
    A side with LSE = -inf carries no keys and has weight 0, so folding a part into the
    empty pair ``(anything, -inf)`` returns the part. Rows: ``o_*`` is ``[rows, d]``, ``lse_*`` is
    ``[rows]``.
    """
    o_acc = np.asarray(o_acc, dtype=np.float64)
    o_b = np.asarray(o_b, dtype=np.float64)
    lse_acc = np.asarray(lse_acc, dtype=np.float64)
    lse_b = np.asarray(lse_b, dtype=np.float64)
    m = np.maximum(lse_acc, lse_b)
    live = np.isfinite(m)
    m_safe = np.where(live, m, 0.0)
    ea = np.where(np.isfinite(lse_acc), np.exp(lse_acc - m_safe), 0.0)
    eb = np.where(np.isfinite(lse_b), np.exp(lse_b - m_safe), 0.0)
    tot = np.where(live, ea + eb, 1.0)
    lse = np.where(live, m_safe + np.log(tot), -np.inf)
    # a side of weight 0 is not read at all: its O may hold anything, NaN included
    wa, wb = (ea / tot)[:, None], (eb / tot)[:, None]
    o = np.where(wa > 0, wa * o_acc, 0.0) + np.where(wb > 0, wb * o_b, 0.0)
    return o, lse


class PackLayout:
    """Row layout of a packed batch: sequence s stores its tokens as ``[tokens, heads_s, d]``.

    Row index of (sequence s, token t, stored head h) is ``off[s] + t * heads_s + h``;
    the query side (Q, O, dO, dQ, LSE) and the key side (K, V, dK, dV) each have their
    own offsets. This is the plain reading of "materialise the assigned tokens from
    their global token ranges" (§IV-D) with a per-sequence head count (Table II: a
    Ulysses shard holds fewer heads).
    """

    def __init__(self, seq_q: Sequence[int], seq_kv: Sequence[int], heads: Sequence[int]):
        self.seq_q = list(seq_q)
        self.seq_kv = list(seq_kv)
        self.heads = list(heads)
        self.q_off = [0]
        self.kv_off = [0]
        for lq, lk, h in zip(self.seq_q, self.seq_kv, self.heads):
            self.q_off.append(self.q_off[-1] + lq * h)
            self.kv_off.append(self.kv_off[-1] + lk * h)

    @property
    def q_rows(self) -> int:
        return self.q_off[-1]

    @property
    def kv_rows(self) -> int:
        return self.kv_off[-1]

    def q_index(self, s: int, t0: int, t1: int, h: int) -> np.ndarray:
        return self.q_off[s] + np.arange(t0, t1, dtype=np.int64) * self.heads[s] + h

    def kv_index(self, s: int, t0: int, t1: int, h: int) -> np.ndarray:
        return self.kv_off[s] + np.arange(t0, t1, dtype=np.int64) * self.heads[s] + h


def _groups(segments) -> Dict[tuple, List[tuple]]:
    """KV-split groups: parts sharing (sequence, query range, head range)."""
    groups: Dict[tuple, List[tuple]] = {}
    for seg in segments:
        s, h0, h1, q0, q1, k0, k1, part = seg
        if part >= 0:
            groups.setdefault((s, q0, q1, h0, h1), []).append(seg)
    for key in groups:
        groups[key].sort(key=lambda x: x[7])
    return groups


def pack_forward(seq_q, seq_kv, heads, segments, d: int, scale: float,
                 q: np.ndarray, k: np.ndarray, v: np.ndarray) -> dict:
    """Forward of a whole pack: block-diagonal attention, segment by segment (§IV-D).

    ``q``: ``[q_rows, d]``, ``k``/``v``: ``[kv_rows, d]`` in the packed layout. Segments
    are ``(seq, head_begin, head_end, q_begin, q_end, kv_begin, kv_end, part)``; a
    segment only ever reads K/V rows of its own sequence, so sequences never mix.
    Returns ``o`` ``[q_rows, d]`` and ``lse`` ``[q_rows]`` (NaN where no segment writes),
    and ``parts``: for each KV-split group key and part index, that part's normalised
    partial output ``[tokens, heads, d]`` and log-sum-exp ``[tokens, heads]``.
    """
    lay = PackLayout(seq_q, seq_kv, heads)
    o = np.full((lay.q_rows, d), np.nan)
    lse = np.full(lay.q_rows, np.nan)
    parts = {}
    for (s, h0, h1, q0, q1, k0, k1, part) in segments:
        if part >= 0:
            continue
        for h in range(h0, h1):
            qi = lay.q_index(s, q0, q1, h)
            ki = lay.kv_index(s, k0, k1, h)
            o[qi], lse[qi] = head_forward(q[qi], k[ki], v[ki], scale)
    for key, segs in _groups(segments).items():
        s, q0, q1, h0, h1 = key
        nt, nh = q1 - q0, h1 - h0
        po = np.empty((len(segs), nt, nh, d))
        pl = np.empty((len(segs), nt, nh))
        for b, (_, _, _, _, _, k0, k1, part) in enumerate(segs):
            for hh, h in enumerate(range(h0, h1)):
                qi = lay.q_index(s, q0, q1, h)
                ki = lay.kv_index(s, k0, k1, h)
                po[b, :, hh], pl[b, :, hh] = head_forward(q[qi], k[ki], v[ki], scale)
            parts[(key, part)] = (po[b].copy(), pl[b].copy())
        mo, ml = lse_merge(po.reshape(len(segs), nt * nh, d), pl.reshape(len(segs), nt * nh))
        mo = mo.reshape(nt, nh, d)
        ml = ml.reshape(nt, nh)
        for hh, h in enumerate(range(h0, h1)):
            qi = lay.q_index(s, q0, q1, h)
            o[qi] = mo[:, hh]
            lse[qi] = ml[:, hh]
    return {"o": o, "lse": lse, "parts": parts}


def pack_backward(seq_q, seq_kv, heads, segments, d: int, scale: float,
                  q: np.ndarray, k: np.ndarray, v: np.ndarray, o: np.ndarray, lse: np.ndarray,
                  do: np.ndarray) -> dict:
    """Backward of a whole pack: the exact gradients of f = sum over covered rows of dO . O.

    Every segment adds its contribution; for a KV-split group each part uses the merged
    O and LSE of the group's rows, so dQ sums over parts and each part's K/V rows get this
    query chunk's share. Rows no segment touches are NaN.
    """
    lay = PackLayout(seq_q, seq_kv, heads)
    dq = np.full((lay.q_rows, d), np.nan)
    dk = np.full((lay.kv_rows, d), np.nan)
    dv = np.full((lay.kv_rows, d), np.nan)
    for (s, h0, h1, q0, q1, k0, k1, part) in segments:
        for h in range(h0, h1):
            qi = lay.q_index(s, q0, q1, h)
            ki = lay.kv_index(s, k0, k1, h)
            for arr, idx in ((dq, qi), (dk, ki), (dv, ki)):
                sel = np.isnan(arr[idx, 0])
                arr[idx[sel]] = 0.0
            g_q, g_k, g_v = head_backward(q[qi], k[ki], v[ki], o[qi], lse[qi], do[qi], scale)
            dq[qi] += g_q
            dk[ki] += g_k
            dv[ki] += g_v
    return {"dq": dq, "dk": dk, "dv": dv}
