"""Pins of oracle/speedup.py against numbers the pages print."""
import json
import os

import pytest

from oracle import speedup as S


@pytest.fixture(scope="module")
def pages(golden_dir):
    with open(os.path.join(golden_dir, "page_arithmetic.json")) as f:
        return json.load(f)


def test_implied_denominators(pages):
    g = pages["implied_denominators"]
    tol = g["tolerance_abs"]
    for row in g["rows"]:
        assert abs(S.implied_denominator(row["tau"], row["speedup"]) - row["denominator"]) < tol
        assert abs(1.0 / row["denominator"] - row["speedup_per_tau"]) < tol
    sub = g["rows"][1]
    eag = g["rows"][0]
    assert abs(sub["tau"] / g["small_draft_denominator"] - g["bound_if_small_draft_cost"]) < 0.01
    assert abs(1.0 / g["small_draft_denominator"] - g["small_draft_speedup_per_tau"]) < tol
    assert abs(sub["tau"] / eag["tau"] - g["tau_ratio_subspec_over_eagle"]) < 0.01
    assert abs(sub["speedup"] / eag["speedup"] - g["speedup_ratio_subspec_over_eagle"]) < 0.01
    assert abs(S.implied_denominator(sub["tau"], sub["speedup"])
               / S.implied_denominator(eag["tau"], eag["speedup"]) - g["denominator_growth"]) < 0.01


def test_subspec_speedup_formula_reproduces_denominator(pages):
    # speedup = tau / (D t_draft / t_target + g_v): with the implied denominator
    # split as any (draft, verify) pair the formula returns the printed speedup.
    row = pages["implied_denominators"]["rows"][1]
    den = row["tau"] / row["speedup"]
    g_v = 1.0
    t_ratio = (den - g_v) / 48
    assert abs(S.subspec_speedup(row["tau"], 48, t_ratio, 1.0, g_v) - row["speedup"]) < 1e-9


def test_table5_ratios(pages):
    t = pages["table5"]
    assert abs(100 * t["tau_subspec_T02"] / t["tau_self_T02"] - t["ratio_percent"]) < t["tolerance_abs"]
    assert abs(100 * t["tau_subspec_T02"] / t["depth"] - t["per_token_acceptance_percent"]) < t["tolerance_abs"]


def test_sparsespec_cost_ratio(pages):
    s = pages["sparsespec"]
    c = S.sparsespec_cost_ratio(s["alpha"], s["k"], s["speedup"])
    assert abs(c - s["cost_ratio_about"]) < s["tolerance_abs"]
    assert abs(S.sparsespec_speedup(s["alpha"], s["k"], c) - s["speedup"]) < 1e-12
    # efficiency inversion: dS/dk has the sign of alpha - c
    for alpha, cc in ((0.7, 0.2), (0.1, 0.3)):
        up = S.sparsespec_speedup(alpha, 5.0, cc) < S.sparsespec_speedup(alpha, 6.0, cc)
        assert up == (alpha > cc)


def test_kv_bytes(pages):
    k = pages["kv_bytes"]
    b = S.kv_bytes_per_token(k["n_layers"], k["n_kv_heads"], k["head_dim"])
    assert b == k["bytes_per_token"]
    assert abs(b * k["context_tokens_60k"] / 2 ** 30 - k["gib_at_60k"]) < 1e-9


def test_tau_bounds_and_limits():
    for gamma in (1, 4, 16, 48):
        assert S.tau_iid(0.0, gamma) == 1.0
        assert S.tau_iid(1.0, gamma) == gamma + 1
        for a in (0.1, 0.5, 0.9):
            t = S.tau_iid(a, gamma)
            assert 1.0 <= t <= gamma + 1
            assert abs(t - sum(a ** i for i in range(gamma + 1))) < 1e-12
            assert abs(S.expected_accepted([a] * gamma) + 1 - t) < 1e-12
