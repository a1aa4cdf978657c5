"""Pins of the oracle's training-objective forward (Module F, eqs. (8)-(12)).

Each pin is a case whose answer is fixed by the mathematics rather than by the oracle's
own loops: zero or disjoint supports for the total variation, uniform and W2 = 0 drafts
whose log-probabilities are a library log-sum-exp, z = 0 confidences, the closed form of
the position weights, and agreement with the separately pinned draft and verify oracles
when the reference tokens are the drafted ones."""
import math

import numpy as np
import pytest
from scipy.special import logsumexp

from draft_sampling_scheduling_amd import synth

NEG = -1.0e4  # exp(NEG - 0) is exactly 0 in double


def _wsum(gamma):
    # sum_{k=1..gamma} exp(-(k-1)/gamma), a geometric series
    return (1.0 - math.exp(-1.0)) / (1.0 - math.exp(-1.0 / gamma))


def _blank(R=3, gamma=4, V=64, r=16, d=8, seed=0):
    rng = np.random.default_rng(seed)
    return dict(
        U=rng.standard_normal((R, gamma, V)).astype(np.float32),
        h=rng.standard_normal((R, gamma, d)).astype(np.float32),
        W1=rng.standard_normal((V, r)).astype(np.float32),
        W2=np.zeros((r, V), np.float32),
        w=np.zeros(d + r, np.float32),
        x0=rng.integers(0, V, R).astype(np.int32),
        xs=rng.integers(0, V, (R, gamma)).astype(np.int32))


def _run(ora, I, target, alpha=(0.1, 0.9, 1.0)):
    return ora.train_forward(I["U"], I["h"], I["W1"], I["W2"], I["w"], target, I["x0"],
                             I["xs"], alpha)


def test_weights_sum_closed_form():
    for g in (1, 4, 8, 16):
        assert abs(sum(math.exp(-(k - 1) / g) for k in range(1, g + 1)) - _wsum(g)) < 1e-12


def test_identical_distributions(ora):
    # W2 = 0: q_k = softmax(U_k); the target equal to U makes p = q
    I = _blank()
    o = _run(ora, I, I["U"].copy())
    assert np.all(np.abs(o["tv"]) < 1e-12) and np.all(np.abs(o["c_star"] - 1.0) < 1e-12)
    R, gamma, _ = I["U"].shape
    # log q_k(x*_k) from a library log-sum-exp; L_ce weights position k by exp(-(k-1)/gamma)
    lq = np.take_along_axis(I["U"].astype(np.float64), I["xs"][..., None], 2)[..., 0] - \
        logsumexp(I["U"].astype(np.float64), axis=2)
    np.testing.assert_allclose(o["logq"], lq, rtol=0, atol=1e-12)
    wk = np.exp(-np.arange(gamma) / gamma)
    np.testing.assert_allclose(o["loss"][:, 0], -(lq * wk).sum(1), rtol=1e-12)
    assert np.all(np.abs(o["loss"][:, 1]) < 1e-12)
    # w = 0: c = 1/2 whatever the label, so L_conf = ln 2 * sum_k w_k
    np.testing.assert_allclose(o["c"], 0.5, rtol=0, atol=0)
    np.testing.assert_allclose(o["loss"][:, 2], math.log(2) * _wsum(gamma), rtol=1e-12)


def test_uniform_draft_cross_entropy(ora):
    I = _blank(gamma=8, V=100)
    I["U"][:] = 0.0
    o = _run(ora, I, np.random.default_rng(1).standard_normal(I["U"].shape).astype(np.float32))
    np.testing.assert_allclose(o["logq"], -math.log(100), rtol=0, atol=1e-12)
    np.testing.assert_allclose(o["loss"][:, 0], math.log(100) * _wsum(8), rtol=1e-12)


def test_total_variation_of_uniform_sets(ora):
    # p uniform on A, q uniform on B: ||p - q||_1 = |A\B|/|A| + |B\A|/|B| + |A&B| |1/|A| - 1/|B||
    R, gamma, V = 2, 3, 64
    I = _blank(R=R, gamma=gamma, V=V)
    target = np.full((R, gamma, V), NEG, np.float32)
    U = np.full((R, gamma, V), NEG, np.float32)
    expect = np.zeros((R, gamma))
    rng = np.random.default_rng(5)
    for q in range(R):
        for k in range(gamma):
            A = set(rng.choice(V, rng.integers(1, 20), replace=False).tolist())
            B = set(rng.choice(V, rng.integers(1, 20), replace=False).tolist())
            target[q, k, list(A)] = 0.0
            U[q, k, list(B)] = 0.0
            expect[q, k] = (len(A - B) / len(A) + len(B - A) / len(B)
                            + len(A & B) * abs(1 / len(A) - 1 / len(B)))
    I["U"] = U
    I["xs"] = np.array([[next(iter(sorted(np.flatnonzero(U[q, k] == 0)))) for k in range(gamma)]
                        for q in range(R)], np.int32)
    o = _run(ora, I, target)
    np.testing.assert_allclose(o["tv"], expect, rtol=0, atol=1e-12)
    np.testing.assert_allclose(o["c_star"], 1 - expect / 2, rtol=0, atol=1e-12)
    wk = np.exp(-np.arange(gamma) / gamma)
    np.testing.assert_allclose(o["loss"][:, 1], (expect * wk).sum(1), rtol=1e-12)


@pytest.mark.parametrize("same", [True, False])
def test_confidence_loss_at_saturation(ora, same):
    # one-hot p and q at the same token (c* = 1) or different tokens (c* = 0), z = 50 for
    # every position: L_conf = sum_k w_k log(1 + e^-50) or sum_k w_k log(1 + e^50)
    R, gamma, V, r, d = 2, 4, 32, 16, 8
    I = _blank(R=R, gamma=gamma, V=V, r=r, d=d)
    I["W1"][:] = 1.0
    I["w"][d:] = 50.0 / r
    target = np.full((R, gamma, V), NEG, np.float32)
    U = np.full((R, gamma, V), NEG, np.float32)
    target[..., 3] = 0.0
    U[..., 3 if same else 7] = 0.0
    I["U"] = U
    I["xs"][:] = 3 if same else 7
    o = _run(ora, I, target, alpha=(0.25, 0.5, 2.0))
    cs = 1.0 if same else 0.0
    np.testing.assert_allclose(o["c_star"], cs, rtol=0, atol=1e-12)
    sp = math.log1p(math.exp(-50.0)) if same else 50.0 + math.log1p(math.exp(-50.0))
    np.testing.assert_allclose(o["loss"][:, 2], sp * _wsum(gamma), rtol=1e-12)
    np.testing.assert_allclose(o["loss"][:, 3], 0.25 * o["loss"][:, 0] + 0.5 * o["loss"][:, 1]
                               + 2.0 * o["loss"][:, 2], rtol=1e-12)


def test_agrees_with_draft_and_verify_on_drafted_tokens(ora):
    # reference tokens = the drafted tokens: log q(x*_k) and c must be the draft's own
    # (logit_x - lse, c), and c* the verify oracle's, which read the same rows
    cfg = synth.scaled(synth.CONFIGS["c1"], R=3, gamma=4, V=256, r=16, d=32)
    I = synth.inputs(cfg)
    dr = ora.draft_markov(I["U"], I["h"], I["W1"], I["W2"], I["w"], I["x0"], 4, 2)
    noise, fresh = synth.target_parts(cfg, range(cfg.R), 2)
    tgt = (synth.decode(cfg, I["U"]) + noise[:, :cfg.gamma]).astype(np.float32)
    o = ora.train_forward(I["U"], I["h"], I["W1"], I["W2"], I["w"], tgt, I["x0"], dr["x"])
    np.testing.assert_allclose(o["logq"], dr["logit_x"] - dr["lse"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(o["c"], dr["c"], rtol=0, atol=1e-15)
    tg1 = np.concatenate([tgt, fresh[:, None, :]], axis=1)
    ell = np.full(cfg.R, cfg.gamma, np.int32)
    v = ora.verify(tg1, I["U"], I["W2"], dr["bias_rows"], dr["x"], ell, seed=4, cycle=2)
    np.testing.assert_allclose(o["c_star"], v["c_star"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(o["tv"], 2 * (1 - v["c_star"]), rtol=0, atol=1e-12)


def test_rejects_out_of_range_tokens(ora):
    I = _blank()
    I["xs"][1, 2] = 64
    with pytest.raises(ValueError):
        _run(ora, I, I["U"])
