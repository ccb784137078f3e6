"""Pins for the contextual-penalty / temperature / top-p / min-p oracle."""

import json
import os

import numpy as np
import pytest
from scipy.special import softmax

from oracle import penalty_sample
from synth import penalty_inputs
from synth.inputs import TABLE11

F32 = np.float32


def _run(x, win, theta=1.2, tau=1.0, top_p=0.9, min_p=0.05, u=None):
    return penalty_sample(np.atleast_2d(x), win, float(F32(theta)), float(F32(tau)),
                          float(F32(top_p)), float(F32(min_p)), u)


def test_table11_defaults_match_golden():
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "table11_llama31_8b.json")))
    for key in ("k", "temperature", "top_p", "min_p", "penalty", "penalty_len"):
        assert TABLE11[key] == g[key]


def test_unit_penalty_and_empty_window_are_identity():
    x = penalty_inputs(1, 3, 500, 64)
    r1 = _run(x["logits"], x["window"], theta=1.0)
    np.testing.assert_array_equal(r1.z, x["logits"].astype(np.float64))
    r2 = _run(x["logits"], np.full((3, 5), -1, np.int32))
    np.testing.assert_array_equal(r2.z, x["logits"].astype(np.float64))


def test_penalty_lowers_exactly_the_window():
    x = penalty_inputs(2, 2, 400, 50)
    x["logits"][:, 7] = 0.0
    x["window"][:, 0] = 7
    r = _run(x["logits"], x["window"], theta=1.5)
    for row in range(2):
        w = set(int(i) for i in x["window"][row])
        for i in range(400):
            xi = float(x["logits"][row, i])
            if i in w and xi != 0.0:
                assert r.z[row, i] < xi
                want = xi / float(F32(1.5)) if xi > 0 else xi * float(F32(1.5))
                assert r.z[row, i] == want
            else:
                assert r.z[row, i] == xi


def test_window_duplicates_and_out_of_range_ids_are_ignored():
    x = penalty_inputs(3, 1, 300, 40)
    w = x["window"].copy()
    w_dup = np.concatenate([w, w[:, :10], np.array([[-5, 300, 1000, -1]], np.int32)], axis=1)
    a = _run(x["logits"], w)
    b = _run(x["logits"], w_dup)
    np.testing.assert_array_equal(a.z, b.z)


def test_temperature_and_softmax_match_scipy():
    x = penalty_inputs(4, 2, 1000, 100)
    r = _run(x["logits"], x["window"], tau=0.7)
    r1 = _run(x["logits"], x["window"], tau=1.0)
    np.testing.assert_allclose(r.z, r1.z / float(F32(0.7)), rtol=1e-15)
    np.testing.assert_allclose(r.p, softmax(r.z, axis=1), rtol=1e-12)


def test_two_token_closed_form():
    # one windowed positive logit a and an unwindowed b
    a, b, theta, tau = 1.75, 0.5, 1.25, 0.8
    r = _run(np.array([a, b], F32), np.array([0], np.int32), theta=theta, tau=tau, top_p=1.0, min_p=0.0)
    tau32 = float(F32(tau))
    p0 = 1.0 / (1.0 + np.exp((b - a / theta) / tau32))
    np.testing.assert_allclose(r.p[0], [p0, 1 - p0], rtol=1e-14)


def test_limits():
    x = penalty_inputs(5, 2, 800, 30)
    allk = _run(x["logits"], x["window"], top_p=1.0, min_p=0.0)
    assert allk.keep.all()
    for kw in (dict(top_p=0.0, min_p=0.0), dict(top_p=1.0, min_p=1.0)):
        r = _run(x["logits"], x["window"], **kw)
        for row in range(2):
            assert np.flatnonzero(r.keep[row]).tolist() == [int(np.argmax(r.p[row]))]


def test_min_p_exact_ties_survive():
    x = np.array([1.0, 3.0, 3.0, -2.0], F32)
    r = _run(x, np.array([-1], np.int32), top_p=1.0, min_p=1.0)
    assert r.keep[0].tolist() == [False, True, True, False]


@pytest.mark.parametrize("top_p", [0.1, 0.5, 0.9, 0.99])
def test_top_p_is_smallest_set_exceeding_p(top_p):
    x = penalty_inputs(6, 1, 2000, 100, sigma=1.0)
    r = _run(x["logits"], x["window"], top_p=top_p, min_p=0.0)
    p = r.p[0]
    ps = np.sort(p)[::-1]
    csum = np.cumsum(ps)
    k = int(np.searchsorted(csum, float(F32(top_p)), side="right")) + 1  # first prefix sum > p
    k = min(k, len(p))
    assert int(r.keep[0].sum()) == k
    assert p[r.keep[0]].min() >= ps[k - 1] and (k == len(p) or p[~r.keep[0]].max() <= ps[k])


@pytest.mark.parametrize("min_p", [0.01, 0.05, 0.5])
def test_min_p_closed_form_on_logits(min_p):
    x = penalty_inputs(7, 1, 3000, 100)
    r = _run(x["logits"], x["window"], top_p=1.0, min_p=min_p)
    z = r.z[0]
    np.testing.assert_array_equal(r.keep[0], z - z.max() >= np.log(float(F32(min_p))))


def test_renormalisation_and_inverse_cdf():
    x = penalty_inputs(8, 4, 1500, 200, sigma=1.0)
    u = np.array([0.0, 0.3, 0.77, 0.999], F32)
    r = _run(x["logits"], x["window"], u=u)
    for row in range(4):
        q = r.probs[row]
        np.testing.assert_allclose(q.sum(), 1.0, rtol=1e-12)
        kept = r.keep[row]
        np.testing.assert_allclose(q[kept], r.p[row][kept] / r.p[row][kept].sum(), rtol=1e-12)
        assert np.all(q[~kept] == 0)
        t = int(np.searchsorted(np.cumsum(q), float(u[row]), side="right"))
        assert r.token[row] == t and kept[t]


def test_shared_window_equals_per_row_window():
    x = penalty_inputs(9, 3, 700, 64, shared_window=True)
    a = _run(x["logits"], x["window"])
    b = _run(x["logits"], np.broadcast_to(x["window"], (3, 64)).copy())
    np.testing.assert_array_equal(a.z, b.z)
    np.testing.assert_array_equal(a.keep, b.keep)


# ---- eta-sampling variant ----

from oracle import eta_sample  # noqa: E402


def test_eta_entropy_matches_scipy():
    from scipy.stats import entropy
    x = penalty_inputs(31, 4, 5000, 64)
    r = eta_sample(x["logits"], x["window"], 1.2, 1.0, 3e-4, 0.0173, x["u"])
    for i in range(4):
        assert abs(r.entropy[i] - entropy(r.p[i])) <= 1e-9 * r.entropy[i]
        assert r.eta[i] == min(3e-4, 0.0173 * np.exp(-entropy(r.p[i]))) or \
            abs(r.eta[i] - min(3e-4, 0.0173 * np.exp(-entropy(r.p[i])))) <= 1e-12


@pytest.mark.parametrize("V", [10, 1000])
def test_eta_uniform_row_closed_form(V):
    # uniform probabilities: H = ln V, so eta = min(eps, alpha / V)
    logits = np.zeros((1, V), dtype=np.float32)
    r = eta_sample(logits, np.zeros(0, dtype=np.int32), 1.0, 1.0, 0.5, 0.9)
    assert abs(r.entropy[0] - np.log(V)) <= 1e-12
    assert abs(r.eta[0] - min(0.5, 0.9 / V)) <= 1e-15
    assert r.keep.all()                                   # every p = 1/V >= 0.9 / V
    np.testing.assert_allclose(r.probs[0], 1.0 / V, rtol=1e-12)


def test_eta_two_level_row_closed_form():
    # 4 tokens at logit ln 8 and 96 at 0: p_hi = 8/128, p_lo = 1/128
    logits = np.zeros((1, 100), dtype=np.float32)
    logits[0, :4] = np.log(8.0)
    r = eta_sample(logits, np.zeros(0, dtype=np.int32), 1.0, 1.0, 1.0, 1.0)
    z = 4 * 8 + 96
    H = -(4 * (8 / z) * np.log(8 / z) + 96 * (1 / z) * np.log(1 / z))
    assert abs(r.entropy[0] - H) <= 1e-6
    eta = np.exp(-H)                                      # epsilon = 1 does not bind
    assert abs(r.eta[0] - eta) <= 1e-8
    assert (r.keep[0, :4].all() and not r.keep[0, 4:].any()) == (1 / z < eta <= 8 / z)


def test_eta_keeps_the_top_token_when_eta_is_above_it():
    logits = np.zeros((1, 50), dtype=np.float32)
    logits[0, 7] = 0.5
    r = eta_sample(logits, np.zeros(0, dtype=np.int32), 1.0, 1.0, 1.0, 1e6)   # eta = epsilon = 1 > max p
    assert r.keep[0].sum() == 1 and r.keep[0, 7] and r.probs[0, 7] == 1.0


def test_eta_with_alpha_zero_keeps_only_the_maximum_set():
    x = penalty_inputs(32, 2, 3000, 32)
    r = eta_sample(x["logits"], x["window"], 1.2, 1.0, 0.01, 0.0, x["u"])   # eta = 0: every token reaches it
    assert r.keep.all()
    q = penalty_sample(x["logits"], x["window"], 1.2, 1.0, 1.0, 0.0, x["u"])  # same as no truncation
    np.testing.assert_allclose(r.probs, q.probs, rtol=0, atol=1e-15)
    np.testing.assert_array_equal(r.token, q.token)
