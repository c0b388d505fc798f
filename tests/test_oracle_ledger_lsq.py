"""Pins for the ledger (figures printed on the pages) and for the
gradient-mean equivalence (exact rationals on a least-squares model)."""
import json
import os
from fractions import Fraction

import numpy as np

from oracle import ledger, lsq
from oracle.bf16 import narrow
from oracle.reduce import reduce_mean
from synth import workloads as W

GOLD = os.path.join(os.path.dirname(__file__), "golden", "ledger_printed.json")


def test_ledger_matches_printed_figures():
    g = json.load(open(GOLD))
    for c in g["cases"]:
        got = ledger.model_state_bytes(c["psi"], c["P"], c["zero_stage"])
        assert abs(got - c["printed_bytes"]) <= c["rel_tol"] * c["printed_bytes"], c["cite"]
    pp = g["per_param_bytes"]
    assert (ledger.PARAM, ledger.GRAD, ledger.MASTER, ledger.EXP_AVG, ledger.EXP_AVG_SQ) == \
        (pp["param"], pp["grad"], pp["master"], pp["exp_avg"], pp["exp_avg_sq"])
    assert ledger.bytes_per_param(8, 0) == pp["total"]
    assert ledger.optimizer_share() == g["optimizer_share"]["value"]
    f = g["fits_70B_on_32x80GB"]
    assert (ledger.model_state_bytes(f["psi"], f["P"], 3) <= f["cap_bytes"]) == f["zero3_fits"]
    assert (ledger.model_state_bytes(f["psi"], f["P"], 0) <= f["cap_bytes"]) == f["ddp_fits"]
    s = g["smallest_P_70B_zero3_80GB"]
    P = next(P for P in range(1, 1000)
             if ledger.model_state_bytes(s["psi"], P, 3) <= s["cap_bytes"])
    assert P == s["value"]


def test_ledger_stage_formulas_at_P1_and_large_P():
    for st in range(4):
        assert ledger.bytes_per_param(1, st) == 16        # nothing to shard with one rank
    assert abs(ledger.bytes_per_param(10 ** 9, 1) - 4) < 1e-6
    assert abs(ledger.bytes_per_param(10 ** 9, 2) - 2) < 1e-6
    assert ledger.bytes_per_param(8, 1) == 5.5 and ledger.bytes_per_param(8, 2) == 3.75


def test_mean_of_shard_gradients_is_the_full_batch_gradient():
    X, theta, Y = W.lsq_problem()
    full = lsq.full_batch_grad(X, theta, Y)
    shards = lsq.shard_grads(X, theta, Y, 4)
    mean = [sum(gk[j] for gk in shards) / 4 for j in range(4)]
    assert mean == full
    assert any(gk != full for gk in shards)            # the shards really differ
    # summing instead of averaging scales the gradient by N
    assert [sum(gk[j] for gk in shards) for j in range(4)] == [4 * f for f in full]
    # each shard gradient is an integer over 16 with |numerator| <= 96: exact in bf16
    for gk in shards:
        for f in gk:
            assert (f * 16).denominator == 1 and abs(f * 16) <= 96
    contribs = [narrow(np.array([float(f) for f in gk], np.float32)) for gk in shards]
    for r in range(4):
        g = reduce_mean(contribs, r)
        assert [Fraction(float(x)) for x in g] == full

