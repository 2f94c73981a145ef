"""Pins of the oracle's sampler (temperature and nucleus filtering, inverse-CDF draw
with the uniform variate as an input).

The pins: hand-worked cases with exact probabilities (tests/golden/sampling.json);
greedy at temperature 0; exact counts over a stratified grid of u against scipy's
softmax (each token is drawn for a share of the grid equal to its probability, up to
one grid point); the nucleus against a brute-force enumeration of thresholds."""
import json
import os

import numpy as np
import pytest
import scipy.special

import oracle as O

HERE = os.path.dirname(os.path.abspath(__file__))


def test_hand_worked_cases():
    g = json.load(open(os.path.join(HERE, "golden", "sampling.json")))
    for c in g["cases"]:
        l = np.log(np.array(c["p"]))
        assert O.sample_top_p(l, 1.0, c["top_p"], c["u"]) == c["token"], c


def test_temperature_zero_is_greedy_lowest_index():
    l = np.array([0.1, 3.0, -2.0, 3.0, 1.0])
    for u in (0.0, 0.5, 0.99):
        assert O.sample_top_p(l, 0.0, 0.95, u) == 1


def _stratified_counts(l, T, top_p, M):
    counts = np.zeros(l.size, np.int64)
    for m in range(M):
        counts[O.sample_top_p(l, T, top_p, (m + 0.5) / M)] += 1
    return counts


@pytest.mark.parametrize("T", [1.0, 0.6])
def test_full_nucleus_draws_the_softmax(T):
    r = np.random.default_rng(1)
    l = r.standard_normal(40) * 1.4
    M = 4000
    counts = _stratified_counts(l, T, 1.0, M)
    p = scipy.special.softmax(l / T)
    assert np.all(np.abs(counts - M * p) <= 1.0 + 1e-9)


def _nucleus_brute(p, top_p):
    """Every threshold t over the distinct probabilities: the largest t whose set
    {p >= t} reaches top_p; that set."""
    best = None
    for t in sorted(set(p.tolist())):
        s = p[p >= t].sum()
        if s >= top_p * p.sum() * (1 - 1e-12):
            best = t
    return set(np.nonzero(p >= best)[0].tolist())


@pytest.mark.parametrize("seed,top_p,T", [(2, 0.95, 0.6), (3, 0.5, 1.0), (4, 0.8, 0.6), (5, 0.99, 1.0)])
def test_nucleus_matches_brute_force_and_draws_within_it(seed, top_p, T):
    r = np.random.default_rng(seed)
    l = r.standard_normal(60) * 1.4
    p = scipy.special.softmax(l / T)
    N = _nucleus_brute(p, top_p)
    M = 6000
    counts = _stratified_counts(l, T, top_p, M)
    drawn = set(np.nonzero(counts)[0].tolist())
    assert drawn <= N
    # inside the nucleus each token's share is its renormalised probability
    pn = np.array([p[i] if i in N else 0.0 for i in range(p.size)])
    pn /= pn.sum()
    assert np.all(np.abs(counts - M * pn) <= 1.0 + 1e-9)
    # minimal: dropping the least probable member falls below top_p
    mass = sum(p[i] for i in N)
    assert mass >= top_p - 1e-12 and mass - min(p[i] for i in N) < top_p
