"""Pins for the oracle's two-level Gumbel-max sampler: its draws follow softmax(l)."""
import numpy as np
import pytest
from scipy import special, stats


def _chi2_pvalue(counts, probs):
    n = counts.sum()
    exp = probs * n
    keep = exp > 0
    assert counts[~keep].sum() == 0, "drew an entry of zero probability"
    return stats.chisquare(counts[keep], exp[keep] * counts[keep].sum() / exp[keep].sum()).pvalue


@pytest.mark.parametrize("V,ntrials", [(4, 1_000_000), (64, 1_000_000), (1000, 300_000)])
def test_draws_follow_softmax(ora, V, ntrials):
    rng = np.random.default_rng(V)
    l = rng.normal(0.0, 1.5, V)
    if V == 1000:  # a peaked row spread over many blocks, last block short (1000 = 15*64+40)
        l[rng.integers(0, V, 20)] += 4.0
    counts = ora.sample_trials(l, 5, 0, ora.S_DRAFT_BLK, ora.S_DRAFT_IN, ntrials)
    p = special.softmax(l)
    if V == 1000:  # pool rare entries so every cell expects >= 5
        order = np.argsort(p)
        cum = np.cumsum(p[order]) * ntrials
        cut = np.searchsorted(cum, 50.0)
        pooled_c = np.concatenate([[counts[order[:cut]].sum()], counts[order[cut:]]])
        pooled_p = np.concatenate([[p[order[:cut]].sum()], p[order[cut:]]])
        counts, p = pooled_c, pooled_p
    assert _chi2_pvalue(counts, p) > 1e-4


def test_excluded_entries_never_drawn(ora):
    l = np.full(200, -np.inf)
    l[[3, 70, 71, 199]] = [0.0, 1.0, -0.5, 0.3]
    counts = ora.sample_trials(l, 1, 0, ora.S_RESID_BLK, ora.S_RESID_IN, 200_000)
    assert counts.sum() == 200_000
    p = special.softmax(l[[3, 70, 71, 199]])
    assert _chi2_pvalue(counts[[3, 70, 71, 199]], p) > 1e-4
    assert counts[np.isinf(l)].sum() == 0


def test_single_candidate_and_empty(ora):
    l = np.full(130, -np.inf)
    l[129] = -3.0
    x, gb, gi = ora.sample_two_level(l, 0, 0, 0, 1, 0, 1)
    assert x == 129 and np.isinf(gb) and np.isinf(gi)
    x, _, _ = ora.sample_two_level(np.full(10, -np.inf), 0, 0, 0, 1, 0, 1)
    assert x == -1


def test_one_block_is_plain_gumbel_argmax(ora):
    # with V <= 64 there is one block: the draw is argmax_v l(v) + g(stream_in, v)
    l = np.random.default_rng(0).normal(size=50)
    for r in range(200):
        x, _, _ = ora.sample_two_level(l, 9, 4, 0, 1, r, 2)
        g = np.array([ora.gumbel(9, 4, 1, r, 2, v) for v in range(50)])
        assert x == int(np.argmax(l + g))


def test_block_choice_uses_block_lse(ora):
    # the chosen block is argmax_b LSE_b + g(stream_blk, b)
    rng = np.random.default_rng(1)
    l = rng.normal(size=64 * 5)
    lse_b = special.logsumexp(l.reshape(5, 64), axis=1)
    for r in range(200):
        x, gap, _ = ora.sample_two_level(l, 2, 1, 0, 1, r, 3)
        G = lse_b + np.array([ora.gumbel(2, 1, 0, r, 3, b) for b in range(5)])
        assert x // 64 == int(np.argmax(G))
        s = np.sort(G)
        assert gap == pytest.approx(s[-1] - s[-2], abs=1e-12)
