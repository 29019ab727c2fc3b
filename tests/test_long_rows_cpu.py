"""The cached per-row oracle values of the long heads (tests/golden/long_rows_<pack>.npz, written
by tests/golden/make_long_rows.py) against closed forms that hold for these inputs.

Q, K, V and dO are N(0,1) draws rounded to bf16, d = 128, tau = d^-1/2, so for query row i the
scores s_ij = tau q_i . k_j over L keys are close to N(0, sigma_i^2) with
sigma_i^2 = tau^2 |q_i|^2, |q_i|^2 ~ chi^2(d). Then:
  * LSE_i = ln sum_j e^{s_ij} = ln L + sigma_i^2 / 2 + O(L^-1/2): over the rows, LSE - ln L has
    mean 1/2 and standard deviation tau^2 sqrt(2 d) / 2 = (2 d)^-1/2 = 0.0625;
  * D_i = dO_i . O_i with dO independent of O has mean 0 and variance E|O_i|^2 =
    d E[sum_j p_ij^2] = d E[e^{sigma^2}] / L, about d e / L.
These pin the stored values without the oracle's code: a wrong scale, a dropped max shift, a
transposed operand or rows of the wrong head would move them far outside these bounds.
"""
import math
import os

import numpy as np
import pytest

import workloads as W
from tests.golden import make_long_rows as LR


@pytest.mark.parametrize("name", sorted(LR.TARGETS))
def test_cached_rows_match_closed_forms(name):
    path = LR.path_for(name)
    assert os.path.exists(path), f"{path} is missing: run tests/golden/make_long_rows.py {name}"
    pack = W.config(name)
    s, heads = LR.TARGETS[name]
    z = np.load(path, allow_pickle=False)
    assert str(z["pack"]) == name and int(z["seed"]) == pack.seed and int(z["seq"]) == s
    assert sorted(int(h) for h in z["heads"]) == sorted(heads)
    lq, lk, d = pack.seq_q[s], pack.seq_kv[s], pack.d
    assert d == 128 and abs(pack.softmax_scale() - d ** -0.5) < 1e-12
    for h in heads:
        lse = z[f"lse_{h}"].astype(np.float64)
        dd = z[f"d_{h}"].astype(np.float64)
        assert lse.shape == (lq,) and dd.shape == (lq,)
        assert np.isfinite(lse).all() and np.isfinite(dd).all()
        x = lse - math.log(lk)
        assert abs(x.mean() - 0.5) < 3e-3, (h, x.mean())
        assert abs(x.std() / (2 * d) ** -0.5 - 1) < 0.05, (h, x.std())
        sd = math.sqrt(d * math.e / lk)
        assert abs(dd.mean()) < 5 * sd / math.sqrt(lq), (h, dd.mean())
        assert abs(dd.std() / sd - 1) < 0.05, (h, dd.std(), sd)
