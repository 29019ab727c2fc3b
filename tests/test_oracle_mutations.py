"""Plant plausible mistakes in the oracle (on the CPU) and check that some pin catches each.

Every mutant below is a copy of one oracle function with one deliberate error: a
dropped term, a wrong sign, a wrong index, a transposed operand, a wrong log base.
If a mutant passed every pin, the pins would not be strong enough to trust the
oracle with; so each test asserts that at least one pin fails under its mutant.
"""
import math

import numpy as np
import pytest

import oracle.attention as A
from tests import oracle_pins as pins

_orig_forward = A.head_forward
_orig_backward = A.head_backward
_orig_merge = A.lse_merge
_orig_pack_backward = A.pack_backward


def fwd_log2_lse(q, k, v, scale):
    o, lse = _orig_forward(q, k, v, scale)
    return o, lse / math.log(2.0)


def fwd_no_scale(q, k, v, scale):
    return _orig_forward(q, k, v, 1.0)


def fwd_unnormalised(q, k, v, scale):
    s = scale * (q @ k.T)
    m = s.max(axis=1)
    e = np.exp(s - m[:, None])
    return e @ v, m + np.log(e.sum(axis=1))


def fwd_drop_max_in_lse(q, k, v, scale):
    s = scale * (q @ k.T)
    m = s.max(axis=1)
    e = np.exp(s - m[:, None])
    lse = np.log(e.sum(axis=1))
    p = e / e.sum(axis=1, keepdims=True)
    return p @ v, lse


def _bwd_variant(kind):
    def bwd(q, k, v, o, lse, do, scale):
        dd = (do * o).sum(axis=1)
        if kind == "D_without_o":
            dd = do.sum(axis=1)
        s = scale * (q @ k.T)
        p = np.exp(s - lse[:, None])
        dp = do @ v.T
        ds = p * (dp - dd[:, None])
        if kind == "ds_sign":
            ds = -ds
        dq = scale * (ds @ k)
        dk = scale * (ds.T @ q)
        dv = p.T @ do
        if kind == "dk_no_scale":
            dk = ds.T @ q
        if kind == "dv_uses_ds":
            dv = ds.T @ do
        if kind == "dq_uses_v":
            dq = scale * (ds @ v)
        if kind == "dq_drop_scale":
            dq = ds @ k
        if kind == "p_without_lse":
            p2 = np.exp(s)
            dv = p2.T @ do
        return dq, dk, dv
    return bwd


def merge_unnormalised(o_parts, lse_parts):
    m = lse_parts.max(axis=0)
    w = np.exp(lse_parts - m[None, :])
    return (w[:, :, None] * o_parts).sum(axis=0), m + np.log(w.sum(axis=0))


def merge_wrong_shift(o_parts, lse_parts):
    m = lse_parts.min(axis=0)
    w = np.exp(lse_parts - m[None, :])
    lse = m + np.log(w.sum(axis=0))
    w = w / w.sum(axis=0)[None, :]
    return (w[:, :, None] * o_parts).sum(axis=0), lse - 1e-3


def running_merge_weights_swapped(o_acc, lse_acc, o_b, lse_b):
    m = np.maximum(lse_acc, lse_b)
    ea = np.where(np.isfinite(lse_acc), np.exp(lse_acc - m), 0.0)
    eb = np.where(np.isfinite(lse_b), np.exp(lse_b - m), 0.0)
    tot = ea + eb
    o = np.nan_to_num((eb / tot)[:, None] * np.nan_to_num(o_acc)) + np.nan_to_num((ea / tot)[:, None] * o_b)
    return o, m + np.log(tot)


def running_merge_lse_max_only(o_acc, lse_acc, o_b, lse_b):
    m = np.maximum(lse_acc, lse_b)
    ea = np.where(np.isfinite(lse_acc), np.exp(lse_acc - m), 0.0)
    eb = np.where(np.isfinite(lse_b), np.exp(lse_b - m), 0.0)
    tot = ea + eb
    wa, wb = (ea / tot)[:, None], (eb / tot)[:, None]
    o = np.where(wa > 0, wa * o_acc, 0.0) + np.where(wb > 0, wb * o_b, 0.0)
    return o, m


class _WrongHeadLayout(A.PackLayout):
    """Reads K/V of the neighbouring head: a wrong index in the row layout."""

    def kv_index(self, s, t0, t1, h):
        return super().kv_index(s, t0, t1, (h + 1) % self.heads[s])


class _TransposedLayout(A.PackLayout):
    """Token and head strides swapped: rows read as [heads, tokens] instead of [tokens, heads]."""

    def q_index(self, s, t0, t1, h):
        return self.q_off[s] + h * self.seq_q[s] + np.arange(t0, t1, dtype=np.int64)


def pack_backward_overwrites_parts(seq_q, seq_kv, heads, segments, d, scale, q, k, v, o, lse, do):
    out = None
    for seg in segments:
        one = _orig_pack_backward(seq_q, seq_kv, heads, [seg], d, scale, q, k, v, o, lse, do)
        if out is None:
            out = one
        else:
            for n in out:
                sel = ~np.isnan(one[n][:, 0])
                out[n][sel] = one[n][sel]
    return out


MUTANTS = {
    "lse_in_log2": ("head_forward", fwd_log2_lse),
    "scale_dropped_in_scores": ("head_forward", fwd_no_scale),
    "output_not_normalised": ("head_forward", fwd_unnormalised),
    "max_dropped_from_lse": ("head_forward", fwd_drop_max_in_lse),
    "D_without_o": ("head_backward", _bwd_variant("D_without_o")),
    "ds_sign_flipped": ("head_backward", _bwd_variant("ds_sign")),
    "dk_scale_dropped": ("head_backward", _bwd_variant("dk_no_scale")),
    "dv_uses_ds": ("head_backward", _bwd_variant("dv_uses_ds")),
    "dq_uses_v_for_k": ("head_backward", _bwd_variant("dq_uses_v")),
    "dq_scale_dropped": ("head_backward", _bwd_variant("dq_drop_scale")),
    "p_without_lse": ("head_backward", _bwd_variant("p_without_lse")),
    "merge_unnormalised": ("lse_merge", merge_unnormalised),
    "merge_wrong_shift": ("lse_merge", merge_wrong_shift),
    "running_merge_weights_swapped": ("running_merge", running_merge_weights_swapped),
    "running_merge_lse_is_max": ("running_merge", running_merge_lse_max_only),
    "kv_rows_of_wrong_head": ("PackLayout", _WrongHeadLayout),
    "token_head_strides_swapped": ("PackLayout", _TransposedLayout),
    "parts_overwrite_dq": ("pack_backward", pack_backward_overwrites_parts),
}


def _failing_pins():
    failed = []
    for pin in pins.ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin()
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            failed.append(pin.__name__)
    return failed


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    attr, repl = MUTANTS[name]
    monkeypatch.setattr(A, attr, repl)
    failed = _failing_pins()
    assert failed, f"mutant {name} passed every pin"
