"""Pins for the fp64 oracle: checks that tie it to something other than itself.

Each ``pin_*`` function raises ``AssertionError`` when the oracle is wrong. The pins
reach the oracle through the module object ``oracle.attention`` at call time, so the
mutation tests can plant a mistake in one oracle function and show that some pin
catches it. Sources of truth used here:

* brute force: pure-Python loops over the full score matrix with ``math.fsum`` and
  no max-subtraction (a different evaluation of the softmax definition);
* closed forms derived by hand (zero queries, one key, two keys in one dimension,
  constant values, a dominant key, zero upstream gradient);
* invariants the definition implies (rows of P sum to 1, key permutation, block
  diagonal separation, head and query-range slicing, exact merge of any split,
  gradient sums, LSE bounds);
* central finite differences of ``f = sum dO . O`` through the whole pack forward,
  merge included.
"""
from __future__ import annotations

import math

import numpy as np

import oracle.attention as A


def _rng(seed):
    return np.random.default_rng(seed)


def _close(a, b, tol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    err = np.max(np.abs(a - b)) if a.size else 0.0
    assert err <= tol, f"{what}: max abs err {err:.3e} > {tol:.1e}"


# ---------------------------------------------------------------- brute force

def brute_attention(q, k, v, scale):
    """Softmax attention with explicit loops: p_ij = e^{s_ij} / sum_j e^{s_ij}."""
    lq, d = len(q), len(q[0])
    lk = len(k)
    o, lse = [], []
    for i in range(lq):
        s = [scale * math.fsum(q[i][c] * k[j][c] for c in range(d)) for j in range(lk)]
        e = [math.exp(x) for x in s]
        z = math.fsum(e)
        lse.append(math.log(z))
        o.append([math.fsum(e[j] * v[j][c] for j in range(lk)) / z for c in range(len(v[0]))])
    return np.array(o), np.array(lse)


def pin_brute_force_forward():
    r = _rng(11)
    for (lq, lk, d, scale) in [(5, 7, 4, 0.5), (1, 1, 3, 1.0), (9, 3, 8, 8 ** -0.5), (4, 12, 2, 1.7)]:
        q, k, v = r.normal(size=(lq, d)), r.normal(size=(lk, d)), r.normal(size=(lk, d))
        o, lse = A.head_forward(q, k, v, scale)
        bo, bl = brute_attention(q.tolist(), k.tolist(), v.tolist(), scale)
        _close(o, bo, 1e-12, "O vs brute force")
        _close(lse, bl, 1e-12, "LSE vs brute force")
        p = A.head_probs(q, k, scale)
        bp = np.array([[math.exp(scale * float(q[i] @ k[j]) - bl[i]) for j in range(lk)] for i in range(lq)])
        _close(p, bp, 1e-12, "P vs brute force")


# ---------------------------------------------------------------- closed forms

def pin_zero_query():
    """Q = 0: every score is 0, so O_i = mean_j V_j and LSE_i = ln Lkv."""
    r = _rng(12)
    for lk in (1, 2, 7, 300):
        k, v = r.normal(size=(lk, 6)), r.normal(size=(lk, 6))
        o, lse = A.head_forward(np.zeros((4, 6)), k, v, 0.3)
        _close(o, np.repeat(v.mean(axis=0, keepdims=True), 4, axis=0), 1e-12, "O for Q=0")
        _close(lse, np.full(4, math.log(lk)), 1e-12, "LSE for Q=0")


def pin_single_key():
    """One key: O_i = v_0, LSE_i = tau q_i . k_0; gradients dQ = dK = 0, dV_0 = sum_i dO_i."""
    r = _rng(13)
    for scale in (0.25, 1.0, 3.0):
        q, k, v, do = r.normal(size=(6, 5)), r.normal(size=(1, 5)), r.normal(size=(1, 5)), r.normal(size=(6, 5))
        o, lse = A.head_forward(q, k, v, scale)
        _close(o, np.repeat(v, 6, axis=0), 1e-12, "O for one key")
        _close(lse, scale * (q @ k[0]), 1e-12, "LSE for one key")
        dq, dk, dv = A.head_backward(q, k, v, o, lse, do, scale)
        _close(dq, np.zeros_like(dq), 1e-12, "dQ for one key")
        _close(dk, np.zeros_like(dk), 1e-12, "dK for one key")
        _close(dv, do.sum(axis=0, keepdims=True), 1e-12, "dV for one key")


def pin_two_keys_scalar():
    """d = 1, one query, two keys, derived by hand.

    s_j = tau q k_j, p_0 = 1 / (1 + e^{s_1 - s_0}), p_1 = 1 - p_0,
    O = p_0 v_0 + p_1 v_1, LSE = s_0 + ln(1 + e^{s_1 - s_0}).
    For f = g O: df/dq = g (v_0 - v_1) p_0 p_1 tau (k_0 - k_1),
    df/dk_0 = g (v_0 - v_1) p_0 p_1 tau q = -df/dk_1, df/dv_j = g p_j.
    """
    for (qq, k0, k1, v0, v1, g, tau) in [(0.7, 1.3, -0.4, 2.0, -1.0, 0.5, 0.9), (-1.1, 0.2, 0.9, -0.3, 0.8, -1.7, 1.4)]:
        s0, s1 = tau * qq * k0, tau * qq * k1
        p0 = 1.0 / (1.0 + math.exp(s1 - s0))
        p1 = 1.0 - p0
        o_ref = p0 * v0 + p1 * v1
        lse_ref = s0 + math.log1p(math.exp(s1 - s0))
        q = np.array([[qq]])
        k = np.array([[k0], [k1]])
        v = np.array([[v0], [v1]])
        do = np.array([[g]])
        o, lse = A.head_forward(q, k, v, tau)
        _close(o, [[o_ref]], 1e-13, "two-key O")
        _close(lse, [lse_ref], 1e-13, "two-key LSE")
        dq, dk, dv = A.head_backward(q, k, v, o, lse, do, tau)
        common = g * (v0 - v1) * p0 * p1
        _close(dq, [[common * tau * (k0 - k1)]], 1e-13, "two-key dQ")
        _close(dk, [[common * tau * qq], [-common * tau * qq]], 1e-13, "two-key dK")
        _close(dv, [[g * p0], [g * p1]], 1e-13, "two-key dV")


def pin_constant_v():
    """V = c in every row: O = c, dQ = dK = 0, sum_j dV_j = sum_i dO_i."""
    r = _rng(14)
    q, k, do = r.normal(size=(11, 4)), r.normal(size=(17, 4)), r.normal(size=(11, 4))
    c = r.normal(size=4)
    v = np.repeat(c[None, :], 17, axis=0)
    o, lse = A.head_forward(q, k, v, 0.6)
    _close(o, np.repeat(c[None, :], 11, axis=0), 1e-12, "O for constant V")
    dq, dk, dv = A.head_backward(q, k, v, o, lse, do, 0.6)
    _close(dq, np.zeros_like(dq), 1e-12, "dQ for constant V")
    _close(dk, np.zeros_like(dk), 1e-12, "dK for constant V")
    _close(dv.sum(axis=0), do.sum(axis=0), 1e-12, "sum dV for constant V")


def pin_dominant_key():
    """A query aligned with one key at large norm puts (almost) all weight on that key."""
    r = _rng(15)
    k = np.eye(6)[:5] * 4.0
    v = r.normal(size=(5, 3))
    q = 10.0 * k[[2, 0, 4]]
    o, lse = A.head_forward(q, k, v, 1.0)
    _close(o, v[[2, 0, 4]], 1e-12, "dominant key O")
    _close(lse, np.full(3, 160.0), 1e-12, "dominant key LSE")


def pin_zero_upstream():
    """dO = 0 gives zero gradients everywhere."""
    r = _rng(16)
    q, k, v = r.normal(size=(7, 4)), r.normal(size=(9, 4)), r.normal(size=(9, 4))
    o, lse = A.head_forward(q, k, v, 0.5)
    dq, dk, dv = A.head_backward(q, k, v, o, lse, np.zeros_like(q), 0.5)
    for t, n in ((dq, "dQ"), (dk, "dK"), (dv, "dV")):
        _close(t, np.zeros_like(t), 0.0, n + " for dO=0")


# ---------------------------------------------------------------- invariants

def pin_probs_rows_sum_to_one():
    r = _rng(17)
    q, k = 3.0 * r.normal(size=(20, 8)), r.normal(size=(33, 8))
    p = A.head_probs(q, k, 0.7)
    _close(p.sum(axis=1), np.ones(20), 1e-13, "rows of P")
    assert (p >= 0).all()


def pin_key_permutation():
    """Permuting K and V rows jointly leaves O and LSE unchanged and permutes dK, dV."""
    r = _rng(18)
    q, k, v, do = r.normal(size=(9, 5)), r.normal(size=(14, 5)), r.normal(size=(14, 5)), r.normal(size=(9, 5))
    perm = r.permutation(14)
    o, lse = A.head_forward(q, k, v, 0.4)
    o2, lse2 = A.head_forward(q, k[perm], v[perm], 0.4)
    _close(o2, o, 1e-13, "O under key permutation")
    _close(lse2, lse, 1e-13, "LSE under key permutation")
    _, dk, dv = A.head_backward(q, k, v, o, lse, do, 0.4)
    _, dk2, dv2 = A.head_backward(q, k[perm], v[perm], o2, lse2, do, 0.4)
    _close(dk2, dk[perm], 1e-13, "dK under key permutation")
    _close(dv2, dv[perm], 1e-13, "dV under key permutation")


def pin_lse_bounds():
    """max_j s_ij <= LSE_i <= max_j s_ij + ln Lkv."""
    r = _rng(19)
    q, k, v = 2.0 * r.normal(size=(30, 6)), r.normal(size=(40, 6)), r.normal(size=(40, 6))
    _, lse = A.head_forward(q, k, v, 0.8)
    smax = A.head_scores(q, k, 0.8).max(axis=1)
    assert (lse >= smax - 1e-12).all() and (lse <= smax + math.log(40) + 1e-12).all()


def pin_gradient_sums():
    """Per head: sum_j dK_j = 0 (softmax shift invariance) and sum_j dV_j = sum_i dO_i."""
    r = _rng(20)
    q, k, v, do = r.normal(size=(12, 6)), r.normal(size=(19, 6)), r.normal(size=(19, 6)), r.normal(size=(12, 6))
    o, lse = A.head_forward(q, k, v, 0.45)
    _, dk, dv = A.head_backward(q, k, v, o, lse, do, 0.45)
    _close(dk.sum(axis=0), np.zeros(6), 1e-12, "sum dK")
    _close(dv.sum(axis=0), do.sum(axis=0), 1e-12, "sum dV")


def pin_merge_equals_unsplit():
    """Merging normalised partials of any split of the keys equals unsplit attention."""
    r = _rng(21)
    q, k, v = r.normal(size=(8, 4)), r.normal(size=(23, 4)), r.normal(size=(23, 4))
    o, lse = A.head_forward(q, k, v, 0.9)
    for cuts in ([0, 23], [0, 1, 23], [0, 5, 6, 17, 23], [0, 22, 23], list(range(24))):
        po, pl = [], []
        for a, b in zip(cuts[:-1], cuts[1:]):
            x, y = A.head_forward(q, k[a:b], v[a:b], 0.9)
            po.append(x)
            pl.append(y)
        mo, ml = A.lse_merge(np.stack(po), np.stack(pl))
        _close(mo, o, 1e-13, f"merged O for cuts {cuts}")
        _close(ml, lse, 1e-13, f"merged LSE for cuts {cuts}")
    # associativity: merge(merge(a, b), c) == merge(a, b, c)
    parts = [A.head_forward(q, k[a:b], v[a:b], 0.9) for a, b in ((0, 4), (4, 15), (15, 23))]
    ab = A.lse_merge(np.stack([parts[0][0], parts[1][0]]), np.stack([parts[0][1], parts[1][1]]))
    abc = A.lse_merge(np.stack([ab[0], parts[2][0]]), np.stack([ab[1], parts[2][1]]))
    _close(abc[0], o, 1e-13, "nested merge O")
    _close(abc[1], lse, 1e-13, "nested merge LSE")


def pin_merge_empty_parts():
    """A part with LSE = -inf has weight 0; all parts -inf gives O = 0 and LSE = -inf."""
    r = _rng(22)
    po = r.normal(size=(3, 5, 2))
    pl = r.normal(size=(3, 5))
    pl_inf = pl.copy()
    pl_inf[1, :] = -np.inf
    mo, ml = A.lse_merge(po, pl_inf)
    ro, rl = A.lse_merge(po[[0, 2]], pl[[0, 2]])
    _close(mo, ro, 1e-14, "merge with an empty part")
    _close(ml, rl, 1e-14, "merge LSE with an empty part")
    mo, ml = A.lse_merge(po, np.full((3, 5), -np.inf))
    assert np.all(mo == 0.0) and np.all(np.isneginf(ml))


def pin_running_merge():
    """Folding the parts one at a time, in any order, into the empty pair equals the batch
    merge and unsplit attention; folding into the empty pair returns the part unchanged,
    whatever O the empty pair holds; folding an empty part changes nothing."""
    r = _rng(23)
    q, k, v = r.normal(size=(7, 5)), r.normal(size=(31, 5)), r.normal(size=(31, 5))
    o, lse = A.head_forward(q, k, v, 0.7)
    cuts = [0, 3, 4, 19, 31]
    parts = [A.head_forward(q, k[a:b], v[a:b], 0.7) for a, b in zip(cuts[:-1], cuts[1:])]
    for order in ([0, 1, 2, 3], [3, 1, 0, 2], [2, 3, 1, 0]):
        acc_o = np.full((7, 5), np.nan)
        acc_l = np.full(7, -np.inf)
        for i in order:
            acc_o, acc_l = A.running_merge(acc_o, acc_l, *parts[i])
        _close(acc_o, o, 1e-13, f"running merge O, order {order}")
        _close(acc_l, lse, 1e-13, f"running merge LSE, order {order}")
    bo, bl = A.lse_merge(np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]))
    _close(acc_o, bo, 1e-13, "running vs batch merge O")
    _close(acc_l, bl, 1e-13, "running vs batch merge LSE")
    # first fold: the part itself, bit for bit
    fo, fl = A.running_merge(np.full((7, 5), np.nan), np.full(7, -np.inf), *parts[2])
    assert np.array_equal(fo, parts[2][0]) and np.array_equal(fl, parts[2][1])
    # an empty part (LSE = -inf) leaves the running pair as it is
    eo, el = A.running_merge(parts[1][0], parts[1][1], np.full((7, 5), np.nan), np.full(7, -np.inf))
    assert np.array_equal(eo, parts[1][0]) and np.array_equal(el, parts[1][1])
    # two equal LSEs: the mean of the two outputs and LSE + ln 2
    a_o, b_o = r.normal(size=(3, 2)), r.normal(size=(3, 2))
    l = r.normal(size=3)
    mo, ml = A.running_merge(a_o, l, b_o, l)
    _close(mo, 0.5 * (a_o + b_o), 1e-15, "equal-weight fold O")
    _close(ml, l + np.log(2.0), 1e-15, "equal-weight fold LSE")


# ---------------------------------------------------------------- pack-level

def _rand_pack_inputs(r, seq_q, seq_kv, heads, d):
    lay = A.PackLayout(seq_q, seq_kv, heads)
    return (r.normal(size=(lay.q_rows, d)), r.normal(size=(lay.kv_rows, d)),
            r.normal(size=(lay.kv_rows, d)), r.normal(size=(lay.q_rows, d)))


def pin_block_diagonal_separation():
    """Changing one sequence's K/V changes only that sequence's outputs, bit for bit."""
    r = _rng(23)
    seq, heads, d = [5, 9, 4], [2, 3, 2], 4
    segs = [(i, 0, h, 0, l, 0, l, -1) for i, (l, h) in enumerate(zip(seq, heads))]
    q, k, v, _ = _rand_pack_inputs(r, seq, seq, heads, d)
    base = A.pack_forward(seq, seq, heads, segs, d, 0.5, q, k, v)
    lay = A.PackLayout(seq, seq, heads)
    k2, v2 = k.copy(), v.copy()
    k2[lay.kv_off[1]:lay.kv_off[2]] += 1.0
    v2[lay.kv_off[1]:lay.kv_off[2]] -= 2.0
    pert = A.pack_forward(seq, seq, heads, segs, d, 0.5, q, k2, v2)
    for s in (0, 2):
        sl = slice(lay.q_off[s], lay.q_off[s + 1])
        assert np.array_equal(pert["o"][sl], base["o"][sl]) and np.array_equal(pert["lse"][sl], base["lse"][sl])
    sl = slice(lay.q_off[1], lay.q_off[2])
    assert not np.allclose(pert["o"][sl], base["o"][sl])


def pin_head_and_query_slices():
    """A head-range segment equals those heads of whole-sequence attention; a query-range
    segment equals those rows (Ulysses head shards and query shards, Table II)."""
    r = _rng(24)
    seq, heads, d = [13], [4], 6
    q, k, v, _ = _rand_pack_inputs(r, seq, seq, heads, d)
    whole = A.pack_forward(seq, seq, heads, [(0, 0, 4, 0, 13, 0, 13, -1)], d, 0.3, q, k, v)
    sub = A.pack_forward(seq, seq, heads, [(0, 1, 3, 0, 13, 0, 13, -1)], d, 0.3, q, k, v)
    rows = A.PackLayout(seq, seq, heads)
    idx = np.concatenate([rows.q_index(0, 0, 13, h) for h in (1, 2)])
    _close(sub["o"][idx], whole["o"][idx], 0.0, "head subset O")
    other = np.concatenate([rows.q_index(0, 0, 13, h) for h in (0, 3)])
    assert np.isnan(sub["o"][other]).all()
    qs = A.pack_forward(seq, seq, heads, [(0, 0, 4, 3, 9, 0, 13, -1)], d, 0.3, q, k, v)
    idx = np.concatenate([rows.q_index(0, 3, 9, h) for h in range(4)])
    _close(qs["o"][idx], whole["o"][idx], 0.0, "query range O")


def pin_pack_kv_split_equals_whole():
    """A ring group (parts over disjoint K/V blocks) merges to whole-sequence attention."""
    r = _rng(25)
    seq, heads, d = [10], [3], 4
    q, k, v, do = _rand_pack_inputs(r, seq, seq, heads, d)
    whole = A.pack_forward(seq, seq, heads, [(0, 0, 3, 0, 10, 0, 10, -1)], d, 0.5, q, k, v)
    segs = [(0, 0, 3, 0, 10, 0, 3, 0), (0, 0, 3, 0, 10, 3, 4, 1), (0, 0, 3, 0, 10, 4, 10, 2)]
    split = A.pack_forward(seq, seq, heads, segs, d, 0.5, q, k, v)
    _close(split["o"], whole["o"], 1e-13, "ring-merged O")
    _close(split["lse"], whole["lse"], 1e-13, "ring-merged LSE")
    gw = A.pack_backward(seq, seq, heads, [(0, 0, 3, 0, 10, 0, 10, -1)], d, 0.5, q, k, v, whole["o"], whole["lse"], do)
    gs = A.pack_backward(seq, seq, heads, segs, d, 0.5, q, k, v, split["o"], split["lse"], do)
    for n in ("dq", "dk", "dv"):
        _close(gs[n], gw[n], 1e-13, "ring " + n)


FD_PACK = dict(
    seq_q=[3, 4, 5], seq_kv=[3, 4, 7], heads=[2, 3, 2], d=3, scale=0.7,
    segments=[(0, 0, 2, 0, 3, 0, 3, -1),          # whole sequence
              (1, 1, 3, 0, 4, 0, 4, -1),          # head subset [1, 3)
              (1, 0, 1, 1, 3, 0, 4, -1),          # query range of head 0
              (2, 0, 2, 0, 5, 0, 2, 0),           # ring part 0
              (2, 0, 2, 0, 5, 2, 3, 1),           # ring part 1 (one key)
              (2, 0, 2, 0, 5, 3, 7, 2)],          # ring part 2
)


def pin_finite_differences(step=1e-6, tol=1e-7):
    """Central differences of f = sum over covered rows of dO . O through pack_forward
    (merge included) agree with pack_backward for every entry of Q, K and V."""
    r = _rng(26)
    P = FD_PACK
    q, k, v, do = _rand_pack_inputs(r, P["seq_q"], P["seq_kv"], P["heads"], P["d"])
    args = (P["seq_q"], P["seq_kv"], P["heads"], P["segments"], P["d"], P["scale"])
    fwd = A.pack_forward(*args, q, k, v)
    cov = ~np.isnan(fwd["o"][:, 0])

    def f(qq, kk, vv):
        o = A.pack_forward(*args, qq, kk, vv)["o"]
        return float(np.sum(do[cov] * o[cov]))

    g = A.pack_backward(*args, q, k, v, fwd["o"], fwd["lse"], do)
    for name, x, grad in (("Q", q, g["dq"]), ("K", k, g["dk"]), ("V", v, g["dv"])):
        fd = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += step
            xm[idx] -= step
            ins_p = {"Q": (xp, k, v), "K": (q, xp, v), "V": (q, k, xp)}[name]
            ins_m = {"Q": (xm, k, v), "K": (q, xm, v), "V": (q, k, xm)}[name]
            fd[idx] = (f(*ins_p) - f(*ins_m)) / (2 * step)
        an = np.where(np.isnan(grad), 0.0, grad)
        err = np.max(np.abs(fd - an))
        scale = max(1.0, np.max(np.abs(an)))
        assert err <= tol * scale * 10, f"finite differences d{name}: max err {err:.3e}"
        rel = np.linalg.norm(fd - an) / max(np.linalg.norm(an), 1e-300)
        assert rel <= tol, f"finite differences d{name}: rel err {rel:.3e} > {tol:.0e}"


def pin_pack_layout():
    """Row (s, t, h) of the packed tensors is sequence s's block reshaped to [tokens, heads, d]:
    pack_forward on the pack equals head_forward on the per-head slices taken by reshape."""
    r = _rng(27)
    seq_q, seq_kv, heads, d = [4, 6], [5, 3], [3, 2], 4
    segs = [(0, 0, 3, 0, 4, 0, 5, -1), (1, 0, 2, 0, 6, 0, 3, -1)]
    q, k, v, _ = _rand_pack_inputs(r, seq_q, seq_kv, heads, d)
    out = A.pack_forward(seq_q, seq_kv, heads, segs, d, 0.6, q, k, v)
    qo = np.cumsum([0] + [l * h for l, h in zip(seq_q, heads)])
    ko = np.cumsum([0] + [l * h for l, h in zip(seq_kv, heads)])
    for s in range(2):
        qs = q[qo[s]:qo[s + 1]].reshape(seq_q[s], heads[s], d)
        ks = k[ko[s]:ko[s + 1]].reshape(seq_kv[s], heads[s], d)
        vs = v[ko[s]:ko[s + 1]].reshape(seq_kv[s], heads[s], d)
        os_ = out["o"][qo[s]:qo[s + 1]].reshape(seq_q[s], heads[s], d)
        ls_ = out["lse"][qo[s]:qo[s + 1]].reshape(seq_q[s], heads[s])
        for h in range(heads[s]):
            ro, rl = brute_attention(qs[:, h].tolist(), ks[:, h].tolist(), vs[:, h].tolist(), 0.6)
            _close(os_[:, h], ro, 1e-12, f"pack layout O seq {s} head {h}")
            _close(ls_[:, h], rl, 1e-12, f"pack layout LSE seq {s} head {h}")


ALL_PINS = [pin_brute_force_forward, pin_zero_query, pin_single_key, pin_two_keys_scalar, pin_constant_v,
            pin_dominant_key, pin_zero_upstream, pin_probs_rows_sum_to_one, pin_key_permutation,
            pin_lse_bounds, pin_gradient_sums, pin_merge_equals_unsplit, pin_merge_empty_parts,
            pin_running_merge,
            pin_block_diagonal_separation, pin_head_and_query_slices, pin_pack_kv_split_equals_whole,
            pin_finite_differences, pin_pack_layout]
