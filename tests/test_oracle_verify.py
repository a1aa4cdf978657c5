"""Pins for the oracle's verification (single-token rule, prefix rule, eq. (8) for c*)."""
import json
import os

import numpy as np
import pytest
from scipy import special, stats

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "appendix_a.json")))
AB = GOLD["two_token_vocab"]


def _verify_rows(ora, target_rows, draft_logits, x, ell, seed=0, cycle=0, bonus=None):
    """Verify with q_j = softmax(draft_logits_j) (U carries the logits, W2 = 0)."""
    R, g, V = draft_logits.shape
    target = np.zeros((R, g + 1, V), np.float32)
    target[:, :g] = target_rows
    if bonus is not None:
        target[:, g] = bonus
    W2 = np.zeros((1, V), np.float32)
    bias = np.zeros((R, g, 1))
    return ora.verify(target, draft_logits.astype(np.float32), W2, bias, x, ell, seed, cycle)


def test_two_token_example_c_star(ora):
    t = np.log(np.array(AB["p_target"]))[None, None, :]
    q = np.log(np.array(AB["p_draft"]))[None, None, :]
    out = _verify_rows(ora, t, q, np.zeros((1, 1), np.int32), np.ones(1, np.int32))
    assert out["c_star"][0, 0] == pytest.approx(AB["acceptance"], abs=1e-7)
    p, qq = np.array(AB["p_target"]), np.array(AB["p_draft"])
    assert np.minimum(p, qq).sum() == pytest.approx(AB["acceptance"])


def test_equal_distributions_always_accept(ora):
    rng = np.random.default_rng(0)
    R, g, V = 300, 3, 17
    l = rng.normal(0, 2, (R, g, V)).astype(np.float32)
    x = rng.integers(0, V, (R, g)).astype(np.int32)
    out = _verify_rows(ora, l, l, x, np.full(R, g, np.int32))
    np.testing.assert_allclose(out["c_star"], 1.0, atol=1e-12)
    assert np.all(out["n_acc"] == g)
    assert np.array_equal(out["y"][:, :g], x)


def test_disjoint_supports_always_reject(ora):
    R, V = 200, 4
    q = np.full((R, 1, V), -1e4, np.float32)
    q[:, 0, 0] = 0.0
    t = np.full((R, 1, V), -1e4, np.float32)
    t[:, 0, 1:] = 0.0
    out = _verify_rows(ora, t, q, np.zeros((R, 1), np.int32), np.ones(R, np.int32))
    np.testing.assert_allclose(out["c_star"], 0.0, atol=1e-12)
    assert np.all(out["n_acc"] == 0)
    assert np.all(out["y"][:, 0] >= 1)  # correction drawn from the residual (= p)


def test_c_star_is_overlap_mass(ora):
    rng = np.random.default_rng(1)
    R, g, V = 50, 4, 300
    t = rng.normal(0, 2, (R, g, V)).astype(np.float32)
    q = (t + rng.normal(0, 1, (R, g, V))).astype(np.float32)
    x = rng.integers(0, V, (R, g)).astype(np.int32)
    ell = rng.integers(0, g + 1, R).astype(np.int32)
    out = _verify_rows(ora, t, q, x, ell)
    P = special.softmax(t.astype(np.float64), axis=2)
    Q = special.softmax(q.astype(np.float64), axis=2)
    overlap = np.minimum(P, Q).sum(axis=2)
    for r in range(R):
        np.testing.assert_allclose(out["c_star"][r, : ell[r]], overlap[r, : ell[r]], atol=1e-12)
        assert np.all(np.isnan(out["c_star"][r, ell[r]:]))


def test_single_token_rule_recovers_target(ora):
    """[explainer] section 06: accept w.p. min(1,p/q), else residual => output ~ p."""
    V, R = 5, 1_000_000
    qv = np.array([0.40, 0.05, 0.25, 0.20, 0.10])
    pv = np.array([0.10, 0.30, 0.20, 0.15, 0.25])
    lq = np.log(qv)
    counts_x = ora.sample_trials(lq, 0, 0, ora.S_DRAFT_BLK, ora.S_DRAFT_IN, R)
    x = np.repeat(np.arange(V), counts_x).astype(np.int32)  # exactly q-distributed drafts
    x = np.random.default_rng(0).permutation(x).reshape(R, 1)
    t = np.broadcast_to(np.log(pv).astype(np.float32), (R, 1, V))
    dq = np.broadcast_to(lq.astype(np.float32), (R, 1, V))
    out = _verify_rows(ora, t, dq, x, np.ones(R, np.int32), seed=4, cycle=1)
    y0 = out["y"][:, 0]
    counts = np.bincount(y0, minlength=V)
    assert stats.chisquare(counts, pv * R).pvalue > 1e-4
    # acceptance frequency equals 1 - 1/2 |p - q|_1
    acc = (out["n_acc"] == 1).mean()
    cstar = 1 - 0.5 * np.abs(pv - qv).sum()
    assert out["c_star"][0, 0] == pytest.approx(cstar, abs=1e-7)
    z = (acc - cstar) / np.sqrt(cstar * (1 - cstar) / R)
    assert abs(z) < 4.5


def test_appendix_a_selection_bias(ora):
    """Pr(Y=A) is 0.7 when the schedule is fixed before x_1, 0.85 when it peeks at x_1."""
    R, g = 1_000_000, 2
    pt = np.log(np.array(AB["p_target"], np.float32))
    pd = np.log(np.array(AB["p_draft"], np.float32))
    counts_x = ora.sample_trials(pd.astype(np.float64), 1, 0, 0, 1, R)
    x1 = np.random.default_rng(1).permutation(np.repeat(np.arange(2), counts_x))
    x = np.stack([x1, np.zeros(R, np.int64)], axis=1).astype(np.int32)
    t = np.broadcast_to(pt, (R, g, 2))
    dq = np.broadcast_to(pd, (R, g, 2))
    # early stop: Theta_1 = 0.9 < Theta_0 = 1.0, so ell = 0 before x_1 exists
    sps = np.array([GOLD["sps"][k] for k in ("1", "2", "3")], np.float32)
    sched = ora.schedule(np.array([[GOLD["a1"], 0.9]], np.float32), sps, 1, 0)
    ell_sync = np.full(R, sched["ell"][0], np.int32)
    out = _verify_rows(ora, t, dq, x, ell_sync, seed=2, bonus=pt)
    pA = (out["y"][:, 0] == 0).mean()
    assert pA == pytest.approx(AB["pr_A_lossless"], abs=5 * np.sqrt(0.21 / R))
    # backtracking search: x_1 = A gives c_2 = 0.9 (ell = 2), x_1 = B gives c_2 = 0 (ell = 0)
    ell_peek = np.where(x1 == 0, 2, 0).astype(np.int32)
    out = _verify_rows(ora, t, dq, x, ell_peek, seed=2, bonus=pt)
    pA = (out["y"][:, 0] == 0).mean()
    assert pA == pytest.approx(AB["pr_A_anticipating"], abs=5 * np.sqrt(0.13 / R))


def test_toy_chain_decode_is_lossless(ora):
    """Multi-cycle decode on a 4-token Markov chain: draft with chain Q through the Markov
    head (W1 = I, W2 = log Q), schedule with Algorithm 1, verify against chain P; the
    emitted bigrams must follow P."""
    V, g, R, cycles = 4, 4, 4000, 60
    rng = np.random.default_rng(3)
    P = rng.dirichlet(np.ones(V) * 1.5, V)
    Q = 0.5 * P + 0.5 * rng.dirichlet(np.ones(V), V)
    W1 = np.eye(V, dtype=np.float32)
    W2 = np.log(Q).astype(np.float32)
    U = np.zeros((R, g, V), np.float32)
    h = np.zeros((R, g, 1), np.float32)
    w = np.concatenate([[0.0], np.linspace(-1, 2.5, V)]).astype(np.float32)
    sps = np.array([1.0 / (1.0 + 0.00005 * B) for B in range(R, R * (g + 1) + 1)], np.float32)
    anchors = rng.integers(0, V, R).astype(np.int32)
    big = np.zeros((V, V), np.int64)
    logP = np.log(P).astype(np.float32)
    for cyc in range(cycles):
        d = ora.draft_markov(U, h, W1, W2, w, anchors, seed=5, cycle=cyc)
        s = ora.schedule(d["c"].astype(np.float32), sps, R, 0)
        prevs = np.concatenate([anchors[:, None], d["x"]], axis=1)  # x_0 .. x_gamma
        target = logP[prevs]                                      # row j ~ P[x_{j-1}]
        v = ora.verify(target, U, W2, d["bias_rows"], d["x"], s["ell"],
                       seed=6, cycle=cyc)
        for r in range(R):
            n = v["n_acc"][r] + 1
            toks = v["y"][r, :n]
            prev = anchors[r]
            for t in toks:
                big[prev, t] += 1
                prev = t
            anchors[r] = prev
    for a in range(V):
        assert stats.chisquare(big[a], P[a] * big[a].sum()).pvalue > 1e-4, (a, big[a])
    assert big.sum() > 400_000


def test_verify_rejects_bad_length(ora):
    l = np.zeros((2, 2, 8), np.float32)
    with pytest.raises(ValueError):
        _verify_rows(ora, l, l, np.zeros((2, 2), np.int32), np.array([0, 3], np.int32))
