"""Pins of the oracle sampler (CPU only)."""
import json
import os

import numpy as np
import pytest
from scipy import stats

from oracle import sampler as sm

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_splitmix64_reference_sequence():
    g = json.load(open(os.path.join(GOLDEN, "splitmix64.json")))
    state = g["seed"]
    for want in g["outputs"]:
        assert sm.splitmix64(state) == int(want, 16)
        state = (state + 0x9E3779B97F4A7C15) % 2 ** 64


def test_candidate_uniforms_in_open_interval():
    rng = np.random.default_rng(0)
    for u in rng.random(200).astype(np.float32):
        for j in range(64):
            x = sm.candidate_uniform(u, j)
            assert 0.0 < x < 1.0
            assert np.isfinite(sm.candidate_exponential(u, j)) and sm.candidate_exponential(u, j) > 0


def _logits(seed, V=4096, scale=1.0):
    return (np.random.default_rng(seed).standard_normal(V) * scale).astype(np.float32)


def test_greedy_is_argmax_lowest_index():
    l = _logits(1)
    for T in (0.0, -1.0, float("nan")):
        assert sm.sample(l, T, 0.8, 30, 0.5).code == int(np.argmax(l))
    t = np.zeros(16, np.float32)
    t[[3, 9]] = 2.0
    assert sm.sample(t, 0.0, 0.8, 30, 0.5).code == 3


def test_limits_reduce_to_argmax():
    for seed in range(20):
        l = _logits(10 + seed)
        a = int(np.argmax(l))
        u = np.float32(np.random.default_rng(seed).random())
        assert sm.sample(l, 1e-6, 0.8, 30, u).code == a        # temperature -> 0+
        assert sm.sample(l, 0.8, 0.8, 1, u).code == a          # top_k = 1
        assert sm.sample(l, 0.8, 1e-9, 30, u).code == a        # top_p -> 0+
        assert sm.sample(l, 0.8, 0.0, 30, u).code == a


def test_code_always_in_top_k_and_kept_set_minimal():
    rng = np.random.default_rng(3)
    for it in range(300):
        l = _logits(1000 + it, V=int(rng.integers(40, 600)), scale=float(rng.uniform(0.1, 4)))
        T = np.float32(rng.uniform(0.3, 1.5))
        tp = np.float32(rng.uniform(0.05, 1.0))
        k = int(rng.integers(1, 80))
        u = np.float32(rng.random())
        d = sm.sample(l, T, tp, k, u)
        n = min(max(k, 1), 64, l.size)
        top = set(np.argsort(-l, kind="stable")[:n].tolist())
        assert d.code in top
        assert 1 <= d.kept <= n
        # recompute the nucleus: the kept prefix is the smallest with mass >= top_p
        z = (l[d.ranks] / T).astype(np.float32)
        e = np.exp((z - z[0]).astype(np.float64)).astype(np.float32)
        p = e / np.float32(np.sum(e, dtype=np.float64))
        c = np.cumsum(p.astype(np.float64))
        m = d.kept - 1
        if m > 0:
            assert c[m - 1] < tp + 1e-6
        if d.kept < n:
            assert c[m] >= tp - 1e-6


def test_top_k_clamp():
    l = _logits(5, V=200)
    order = np.argsort(-l, kind="stable")
    d = sm.sample(l, 1.0, 1.0, 0, 0.25)       # top_k 0 -> 1
    assert d.code == order[0]
    d = sm.sample(l, 50.0, 1.0, 10 ** 6, 0.25)  # top_k capped at 64
    assert len(d.ranks) == 64


def test_exponential_race_frequencies():
    """argmax(p_j / E_j) picks candidate j with probability p_j / sum(kept)."""
    l = np.array([2.0, 1.7, 1.5, 1.0, 0.9, 0.2, -0.5, -1.0, -3.0], np.float32)
    T = np.float32(0.9)
    rng = np.random.default_rng(9)
    us = ((rng.integers(0, 1 << 23, size=20000) + 0.5) * 2.0 ** -23).astype(np.float32)
    for tp, kept_expected in ((1.0, 9), (0.8, None)):
        draws = [sm.sample(l, T, tp, 30, u) for u in us]
        kept = draws[0].kept
        if kept_expected:
            assert kept == kept_expected
        z = (l / T).astype(np.float64)
        p = np.exp(z - z.max())
        p = p[:kept] / p[:kept].sum()
        counts = np.bincount([d.code for d in draws], minlength=l.size)[:kept]
        assert counts.sum() == len(us)
        chi2, pval = stats.chisquare(counts, p * len(us))
        assert pval > 1e-4, (tp, counts, p * len(us))


def test_deterministic():
    l = _logits(77)
    a = [sm.sample(l, 0.8, 0.8, 30, np.float32(u)).code for u in (0.1, 0.5, 0.9)]
    b = [sm.sample(l, 0.8, 0.8, 30, np.float32(u)).code for u in (0.1, 0.5, 0.9)]
    assert a == b
