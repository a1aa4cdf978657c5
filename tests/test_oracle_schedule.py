"""Pins for the oracle's prefix scheduler (Module E, Algorithm 1 and its variants)."""
import itertools
import json
import os
from fractions import Fraction

import numpy as np
import pytest

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "appendix_a.json")))
SYNC, GLOBAL, ASYNC = 0, 1, 2


def _sps_table(B0, B1, fn):
    return np.array([fn(B) for B in range(B0, B1 + 1)], np.float32)


def test_appendix_a_early_stop(ora):
    sps = np.array([GOLD["sps"][k] for k in ("1", "2", "3")], np.float32)
    c = np.array([[GOLD["a1"], GOLD["high_branch"]["c2"]]], np.float32)
    out = ora.schedule(c, sps, 1, SYNC, trace=True)
    assert out["ell"][0] == GOLD["sync_break_ell"]
    assert out["theta"][0] == pytest.approx(GOLD["theta0"], abs=1e-6)
    assert out["theta"][1] == pytest.approx(GOLD["theta1"], abs=1e-6)
    assert out["stats"][0] == 1 and out["stats"][3] == 0


def test_appendix_a_backtracking_branches(ora):
    sps = np.array([GOLD["sps"][k] for k in ("1", "2", "3")], np.float32)
    hb, lb = GOLD["high_branch"], GOLD["low_branch"]
    hi = ora.schedule(np.array([[GOLD["a1"], hb["c2"]]], np.float32), sps, 1, GLOBAL, trace=True)
    assert hi["ell"][0] == hb["global_ell"]
    assert hi["a"][0, 1] == pytest.approx(hb["a2"], abs=1e-6)
    assert hi["theta"][2] == pytest.approx(hb["theta2"], abs=1e-6)
    assert hi["stats"][2] == pytest.approx(hb["theta2"], abs=1e-6)
    lo = ora.schedule(np.array([[GOLD["a1"], lb["c2"]]], np.float32), sps, 1, GLOBAL, trace=True)
    assert lo["ell"][0] == lb["global_ell"]
    assert lo["a"][0, 1] == 0.0
    # a2 = 0 leaves the candidate set; the page's 0.81 counts it anyway: (1+0.8+0)*0.45
    assert (1 + GOLD["a1"] + lb["c2"]) * GOLD["sps"]["3"] == pytest.approx(lb["theta2_with_a2"])
    assert np.isnan(lo["theta"][2])


def test_prefix_survival_is_fp32_running_product(ora):
    rng = np.random.default_rng(0)
    c = rng.uniform(0, 1, (50, 12)).astype(np.float32)
    c[3, :] = 1e-20  # subnormal products must be kept, not flushed
    out = ora.schedule(c, np.ones(50 * 13, np.float32), 1, SYNC)
    ref = np.multiply.accumulate(c, axis=1, dtype=np.float32)
    assert np.array_equal(out["a"].view(np.uint32), ref.view(np.uint32))
    assert np.all(np.diff(out["a"].astype(np.float64), axis=1) <= 0)
    assert out["a"][3, 1] > 0 and out["a"][3, 1] < np.finfo(np.float32).tiny


def _admitted_set(a, n):
    """top-n candidates in (a desc, r asc, j asc), recomputed with numpy lexsort"""
    R, g = a.shape
    rr, jj = np.meshgrid(np.arange(R), np.arange(g), indexing="ij")
    m = a > 0
    av, rv, jv = a[m], rr[m], jj[m]
    order = np.lexsort((jv, rv, -av.astype(np.float64)))
    return rv[order[:n]], jv[order[:n]]


@pytest.mark.parametrize("mode", [SYNC, GLOBAL])
def test_contiguous_prefixes_with_exact_ties(ora, mode):
    rng = np.random.default_rng(5)
    c = rng.choice(np.array([1.0, 1.0, 0.5, 0.75, 0.25, 0.0], np.float32), (40, 8))
    sps = _sps_table(40, 40 * 9, lambda B: 1.0 / (1.0 + 0.001 * B))
    out = ora.schedule(c, sps, 40, mode)
    n = int(out["stats"][3])
    rv, jv = _admitted_set(out["a"], n)
    for q in range(40):
        js = np.sort(jv[rv == q])
        assert np.array_equal(js, np.arange(out["ell"][q])), (q, js)
    assert out["ell"].sum() == n


def _theta_exact(a, ell, sps, B0):
    R = a.shape[0]
    tau = Fraction(R)
    for q in range(R):
        for j in range(ell[q]):
            tau += Fraction(float(a[q, j]))
    B = R + int(sum(ell))
    return tau * Fraction(float(sps[B - B0]))


@pytest.mark.parametrize("seed", range(12))
def test_global_search_equals_brute_force(ora, seed):
    rng = np.random.default_rng(seed)
    R, g = int(rng.integers(1, 5)), int(rng.integers(1, 5))
    # dyadic confidences: every a is a multiple of 2^-32 and tau is exact
    c = (rng.integers(0, 9, (R, g)) / 8.0).astype(np.float32)
    B0, B1 = R, R * (g + 1)
    alpha = rng.uniform(0.01, 0.4)
    sps = _sps_table(B0, B1, lambda B: 1.0 / (1.0 + alpha * B + 0.3 * ((B * 7) % 3 == 0)))
    out = ora.schedule(c, sps, B0, GLOBAL)
    a = out["a"]
    best = max(_theta_exact(a, ell, sps, B0)
               for ell in itertools.product(range(g + 1), repeat=R))
    mine = _theta_exact(a, out["ell"], sps, B0)
    assert mine == best
    assert out["stats"][2] == pytest.approx(float(best), rel=1e-15)


@pytest.mark.parametrize("seed", range(6))
def test_early_stop_equals_global_when_unimodal(ora, seed):
    rng = np.random.default_rng(100 + seed)
    R, g = 30, 6
    c = rng.beta(5, 1.5, (R, g)).astype(np.float32)
    sps = _sps_table(R, R * (g + 1), lambda B: 1.0 / (1.0 + 0.01 * B))
    s = ora.schedule(c, sps, R, SYNC, trace=True)
    t = s["theta"][~np.isnan(s["theta"])]
    peak = int(np.argmax(t))
    unimodal = np.all(np.diff(t[: peak + 1]) > 0) and np.all(np.diff(t[peak:]) <= 0)
    assert unimodal
    gl = ora.schedule(c, sps, R, GLOBAL)
    assert np.array_equal(s["ell"], gl["ell"])
    assert int(s["stats"][3]) == peak


def test_early_stop_can_stop_short_of_global(ora):
    # a cliff in SPS: the break stops at the first drop, the no-break search crosses it
    R, g = 4, 4
    c = np.full((R, g), 0.99, np.float32)
    sps = _sps_table(R, R * (g + 1), lambda B: 1.0 if B < 6 else (0.5 if B < 8 else 0.45))
    s = ora.schedule(c, sps, R, SYNC)
    gl = ora.schedule(c, sps, R, GLOBAL)
    assert s["stats"][3] == 1
    assert gl["stats"][3] == R * g and gl["stats"][2] > s["stats"][2]


def test_constant_sps_admits_every_counted_candidate(ora):
    rng = np.random.default_rng(3)
    c = rng.uniform(0.05, 1.0, (20, 6)).astype(np.float32)
    c[0, 2] = 0.0
    sps = np.full(20 * 7, 0.25, np.float32)
    for mode in (SYNC, GLOBAL):
        out = ora.schedule(c, sps, 1, mode)
        expect = (out["a"].astype(np.float64) * 2**32 >= 1).sum(axis=1)
        assert np.array_equal(out["ell"], expect)
    assert out["ell"][0] == 2


def test_steep_sps_admits_nothing(ora):
    c = np.full((16, 5), 0.9, np.float32)
    sps = _sps_table(16, 96, lambda B: 1.0 / B**3)
    for mode in (SYNC, GLOBAL):
        out = ora.schedule(c, sps, 16, mode)
        assert np.all(out["ell"] == 0) and out["stats"][0] == 16


def test_async_lag2(ora):
    rng = np.random.default_rng(9)
    R, g = 25, 6
    c = rng.beta(4, 2, (R, g)).astype(np.float32)
    sps = _sps_table(1, 40 * (g + 1), lambda B: 1.0 / (1.0 + 0.004 * B + 0.05 * (B // 37)))
    gl = ora.schedule(c, sps, 1, GLOBAL)
    same = ora.schedule(c, sps, 1, ASYNC, c_lag=c)
    assert np.array_equal(gl["ell"], same["ell"])
    # capacity from a different, lagged batch; ranking from the current confidences
    c_lag = rng.beta(6, 1.5, (31, g)).astype(np.float32)
    lag = ora.schedule(c_lag, sps, 1, GLOBAL)
    K = max(int(lag["stats"][0]) - R, 0)
    out = ora.schedule(c, sps, 1, ASYNC, c_lag=c_lag)
    n_cand = int((out["a"] > 0).sum())
    n = min(K, n_cand)
    assert int(out["stats"][3]) == n
    rv, jv = _admitted_set(out["a"], n)
    assert np.array_equal(np.bincount(rv, minlength=R), out["ell"])


def test_error_codes(ora):
    c = np.full((4, 3), 0.5, np.float32)
    sps = np.ones(13, np.float32)                          # B = 4 .. 16 = R(1+gamma)
    assert ora.schedule_rc(c, sps, 4) == 0
    assert ora.schedule_rc(c, sps[:-1], 4) == -2           # does not reach R(1+gamma)=16
    assert ora.schedule_rc(c, sps, 5) == -2                # starts above R
    bad = c.copy()
    bad[1, 1] = np.nan
    assert ora.schedule_rc(bad, sps, 4) == -1
    bad[1, 1] = 1.5
    assert ora.schedule_rc(bad, sps, 4) == -1
    assert ora.schedule_rc(c, sps, 4, ASYNC) == -1         # no lagged confidences


@pytest.mark.parametrize("brk", [True, False], ids=["sync-break", "global"])
def test_literal_running_sum_differs_only_at_theta_near_ties(ora, brk):
    """Reading of Algorithm 1's precision (digest, Module E): the oracle keeps tau exactly
    (2^-32 fixed point) and Theta in double; the page's loop read literally keeps tau and
    Theta in single precision.  Wherever the two admit different counts, the decision that
    differs compares two Theta values closer than the single-precision summation error
    ((n + 2) 2^-24 relative after n additions).  The disagreement count is printed."""
    from tests.sched_sets import _conf_sets, _sps
    u = 2.0 ** -24
    differ = []
    sets = [(name, c, *_sps(kind, *c.shape)) for name, c, _, kind in _conf_sets()]
    # a flat Theta: every a = 0.7 and SPS(B) = 1 / (R + 0.7 (B - R)) rounded to float, so
    # Theta_n = 1 up to rounding and every decision is a near-tie
    Rf = 3000
    cf = np.tile(np.array([0.7, 1.0], np.float32), (Rf, 1))
    Bf = np.arange(Rf, 3 * Rf + 1, dtype=np.float64)
    sets.append(("flat-theta", cf, (1.0 / (Rf + 0.7 * (Bf - Rf))).astype(np.float32), Rf))
    for name, c, sps, B0 in sets:
        R, gamma = c.shape
        ex = ora.schedule(c, sps, B0, SYNC if brk else GLOBAL, trace=True)
        lit = ora.schedule_literal(c, sps, B0, brk=brk)
        th, thl = ex["theta"], lit["theta"]
        n_cand = int(np.sum(np.isfinite(th))) - 1
        tol = lambda m: (m + 2) * u * th[m] * 1.01  # noqa: E731
        n_ex, n_lit = int(ex["stats"][3]), int(lit["ell"].sum())
        # the single-precision Theta stays within its error bound of the exact one
        fin = np.isfinite(thl)
        m = np.nonzero(fin)[0]
        assert np.all(np.abs(thl[fin] - th[fin]) <= np.array([tol(k) for k in m])), name
        if n_ex == n_lit:
            assert np.array_equal(ex["ell"], lit["ell"]), name
            continue
        differ.append((name, n_ex, n_lit))
        if brk:
            # first step whose improve/stop decision differs
            k = 1
            while k <= n_cand and (th[k] > th[k - 1]) == (thl[k] > thl[k - 1]) and th[k] > th[k - 1]:
                k += 1
            assert abs(th[k] - th[k - 1]) <= tol(k) + tol(k - 1), (name, k, th[k], th[k - 1])
        else:
            assert th[n_ex] - th[n_lit] <= tol(n_ex) + tol(n_lit), (name, n_ex, n_lit)
    if not brk:  # without the break the flat case's argmax is decided by rounding alone
        assert any(d[0] == "flat-theta" for d in differ)
    print(f"literal single-precision sums: {len(differ)} of {len(sets)} confidence "
          f"sets admit a different count ({'break' if brk else 'no break'}): {differ}")
