"""Pins of the oracle's multi-cycle decode driver on a toy chain (digest page, overall
cycle; explainer, section 06).

The chain is built so the answers are known: the drafter is the Markov head with W1 = I and
W2 = log Q (so q_k = Q[x_{k-1}] exactly), the target is the bigram chain P, and P and Q are
circulant, so every position's acceptance probability is the same constant
c* = sum_v min(pi(v), rho(v)).  Losslessness fixes the emitted bigram law to P whatever the
length policy; the counters must then show c* at every position."""
import numpy as np
import pytest
from scipy import stats

V, G = 4, 4
PI = np.array([0.55, 0.25, 0.15, 0.05])
RHO = np.array([0.30, 0.40, 0.20, 0.10])


def _circ(v):
    return np.stack([np.roll(v, a) for a in range(len(v))])


def _chain(R, seed=3):
    P, Q = _circ(PI), _circ(RHO)
    W1 = np.eye(V, dtype=np.float32)
    W2 = np.log(Q).astype(np.float32)
    Tb = np.log(P).astype(np.float32)
    Ub = np.zeros((V, G, V), np.float32)
    Hb = np.zeros((V, G, 0), np.float32)
    w = np.linspace(-1, 2.5, V).astype(np.float32)  # z = w[x_{k-1}]
    x0 = np.random.default_rng(seed).integers(0, V, R).astype(np.int32)
    return dict(Ub=Ub, Hb=Hb, W1=W1, W2=W2, w=w, Tb=Tb, x0=x0), P


def _sps(R, alpha):
    return np.array([1.0 / (1.0 + alpha * B) for B in range(1, R * (G + 1) + 1)], np.float32)


def _run(ora, T, ncycles, **kw):
    return ora.decode_run(T["Ub"], T["Hb"], T["W1"], T["W2"], T["w"], T["Tb"], T["x0"],
                          ncycles, seed=9, **kw)


def _bigrams(o, x0):
    big = np.zeros((V, V), np.int64)
    for q in range(len(x0)):
        prev = x0[q]
        for t in o["tokens"][q, :o["n_emitted"][q]]:
            big[prev, t] += 1
            prev = t
    return big


def _counts_consistent(o, R, ncycles):
    assert o["request_cycles"] == R * ncycles
    assert o["emitted"] == int(o["n_emitted"].sum())
    assert o["emitted"] == o["request_cycles"] + int(o["accepted"].sum())
    assert np.all(o["accepted"] <= o["tested"])
    assert np.all(o["tested"][1:] <= o["accepted"][:-1])
    assert np.all(o["tokens"][np.arange(o["tokens"].shape[1]) >= o["n_emitted"][:, None]] == -1)


def test_fixed_length_acceptance_is_cstar_and_lossless(ora):
    R, ncyc = 3000, 20
    T, P = _chain(R)
    o = _run(ora, T, ncyc, policy=ora.FIXED)
    _counts_consistent(o, R, ncyc)
    assert o["sum_ell"] == G * R * ncyc and o["tested"][0] == R * ncyc
    cstar = np.minimum(PI, RHO).sum()
    for k in range(G):
        n = o["tested"][k]
        rate = o["accepted"][k] / n
        assert abs(rate - cstar) < 5 * np.sqrt(cstar * (1 - cstar) / n), (k, rate, cstar)
    big = _bigrams(o, T["x0"])
    for a in range(V):
        assert stats.chisquare(big[a], P[a] * big[a].sum()).pvalue > 1e-4, (a, big[a])


def test_no_drafts_emits_target_samples(ora):
    # a threshold above 1 verifies nothing: every cycle emits one bonus token from P
    R, ncyc = 2000, 15
    T, P = _chain(R, seed=4)
    o = _run(ora, T, ncyc, policy=ora.THRESHOLD, threshold=1.5)
    _counts_consistent(o, R, ncyc)
    assert o["sum_ell"] == 0 and o["tested"].sum() == 0 and o["emitted"] == R * ncyc
    big = _bigrams(o, T["x0"])
    for a in range(V):
        assert stats.chisquare(big[a], P[a] * big[a].sum()).pvalue > 1e-4, (a, big[a])


def test_zero_threshold_is_fixed_length(ora):
    T, _ = _chain(50, seed=5)
    a = _run(ora, T, 6, policy=ora.FIXED)
    b = _run(ora, T, 6, policy=ora.THRESHOLD, threshold=0.0)
    assert np.array_equal(a["tokens"], b["tokens"]) and np.array_equal(a["tested"], b["tested"])


@pytest.mark.parametrize("policy", [0, 1, 2])
def test_scheduled_decode_is_lossless(ora, policy):
    R, ncyc = 3000, 15
    T, P = _chain(R, seed=6)
    o = _run(ora, T, ncyc, policy=policy, sps=_sps(R, 0.00005), sps_B0=1)
    _counts_consistent(o, R, ncyc)
    assert 0 < o["sum_ell"] < G * R * ncyc
    cstar = np.minimum(PI, RHO).sum()
    # scheduling picks which positions are tested, not how a tested position is accepted
    n = o["tested"][0]
    assert abs(o["accepted"][0] / n - cstar) < 5 * np.sqrt(cstar * (1 - cstar) / n)
    big = _bigrams(o, T["x0"])
    for a in range(V):
        assert stats.chisquare(big[a], P[a] * big[a].sum()).pvalue > 1e-4, (a, big[a])


def test_verification_budget_shrinks_with_batch(ora):
    # the Fig. 8 shape: with a throughput curve that falls with the batch, the mean verified
    # length per request is smaller for a larger batch
    means = []
    for R in (16, 512):
        T, _ = _chain(R, seed=7)
        o = _run(ora, T, 6, policy=0, sps=_sps(R, 0.002), sps_B0=1)
        means.append(o["sum_ell"] / o["request_cycles"])
    assert means[0] > means[1] + 0.3, means
