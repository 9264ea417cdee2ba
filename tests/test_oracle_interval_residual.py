"""Pins for two oracle outputs that the parity classifier relies on (CPU).

``oracle.cdf_interval(w, t)`` gives the range of uniforms for which the
inverse-CDF rule returns token t; the classifier uses it to decide whether a
GPU token that differs from the oracle's lies within 1e-5 of a CDF boundary.
It is pinned here against brute force over exact dyadic grids, where every
running sum divided by W is exact in float64: t is returned for u exactly
when lo <= u < hi, the intervals tile [0, 1) in token order, each has length
w_t / W (zero for zero-weight tokens), and random float weights keep u
inside the returned token's interval.

The residual sum W that the oracle reports at the rejected position is
pinned against the reject mass of "11.1 核心原理" 11.1.3: on the worked
example (p = (0.6, 0.4), q = (0.8, 0.2)) every rejection reports the
printed 0.2, and on random rows W equals 1 - sum_v min(p_n(v), q_n(v)) at
the position n where the round stopped, with p and q computed by
``torch.softmax`` (over ``torch.topk`` sets for top-k rows), and 0 when no
draft was rejected.

Each pin has a planted-mistake control: an interval shifted by one token,
and a residual sum taken at the wrong position, must both fail.
"""

import json
import os

import numpy as np
import pytest
import torch

import oracle
import oracle.verify as ov

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ---------------------------------------------------------------- cdf_interval
def _dyadic_weights(rng, V, log2_total):
    """Integer weights (zeros and ties included) summing to 2^log2_total."""
    total = 1 << log2_total
    cuts = np.sort(rng.integers(0, total + 1, size=V - 1))
    w = np.diff(np.concatenate([[0], cuts, [total]])).astype(np.float64)
    # force some zeros and ties
    if V >= 4:
        z = rng.integers(0, V)
        w[(z + 1) % V] += w[z]
        w[z] = 0.0
    return w


def _interval_violations(interval_fn, rng, trials=40):
    """Count the cases where interval_fn disagrees with inverse_cdf on an
    exact dyadic grid of uniforms."""
    bad = 0
    for _ in range(trials):
        V = int(rng.integers(1, 9))
        L = int(rng.integers(3, 9))
        w = _dyadic_weights(rng, V, L)
        W = w.sum()
        grid = np.arange(1 << (L + 2)) / float(1 << (L + 2))       # u = j / 2^(L+2), exact
        got = np.array([ov.inverse_cdf(w, u) for u in grid])
        prev_hi = 0.0
        for t in range(V):
            lo, hi = interval_fn(w, t)
            if lo != prev_hi:                                       # intervals tile [0, 1)
                bad += 1
            prev_hi = hi
            if hi - lo != w[t] / W:                                 # length w_t / W
                bad += 1
            inside = (grid >= lo) & (grid < hi)
            if w[t] > 0 and not np.array_equal(inside, got == t):    # t returned exactly there
                bad += 1
            if w[t] == 0 and (got == t).any():                       # never a zero-weight token
                bad += 1
        if prev_hi != 1.0:
            bad += 1
    return bad


def test_cdf_interval_exact_on_dyadic_grids():
    assert _interval_violations(oracle.cdf_interval, np.random.default_rng(0)) == 0


def test_cdf_interval_random_weights_contain_u():
    """Float weights (rounded sums): the token inverse_cdf returns for u has
    an interval that contains u, up to the rounding of the running sums."""
    rng = np.random.default_rng(1)
    for _ in range(300):
        V = int(rng.integers(1, 200))
        w = rng.exponential(size=V) * (rng.random(V) < 0.7)
        if not (w > 0).any():
            w[rng.integers(0, V)] = 1.0
        u = float(rng.random())
        t = ov.inverse_cdf(w, u)
        lo, hi = oracle.cdf_interval(w, t)
        assert w[t] > 0
        assert lo - 1e-12 <= u <= hi + 1e-12


def test_cdf_interval_planted_off_by_one_fails():
    def shifted(w, t):                      # the mistake: the next token's interval
        c = np.cumsum(np.asarray(w, np.float64))
        W = c[-1]
        lo = c[t]
        hi = c[t + 1] if t + 1 < len(c) else W
        return lo / W, hi / W

    assert _interval_violations(shifted, np.random.default_rng(0)) > 0


# ---------------------------------------------------------------- residual sum
def test_residual_sum_worked_example():
    """11.1.3: p = (0.6, 0.4), q = (0.8, 0.2) leave a reject mass of 0.2;
    every rejection of the worked example reports W = 0.2, every acceptance
    W = 0."""
    g = json.load(open(os.path.join(GOLDEN, "worked_example.json")))
    p, q = np.array(g["p"]), np.array(g["q"])
    R = 4000
    target = np.broadcast_to(np.log(np.stack([p, p]))[None], (R, 2, 2))
    draft = np.broadcast_to(np.log(q)[None, None], (R, 1, 2))
    toks = oracle.sample_draft_tokens(draft, 1.0, 0, 1.0, 3)
    r = oracle.verify_sample(target, draft, toks, 1.0, 0, 1.0, 0, seed=11)
    rejected = r["num_accepted"] == 0
    assert rejected.sum() > 100
    assert np.allclose(r["residual_sum"][rejected], g["reject_probability"], rtol=0, atol=1e-12)
    assert (r["residual_sum"][~rejected] == 0).all()


def _softmax(z, T, k=0):
    x = torch.as_tensor(np.asarray(z, np.float64)) / T
    if 0 < k < x.numel():
        keep = torch.zeros_like(x, dtype=torch.bool)
        keep[torch.topk(x, k).indices] = True
        x = torch.where(keep, x, torch.tensor(-np.inf, dtype=torch.float64))
    return torch.softmax(x, 0).numpy()


def _residual_mismatches(rng, rounds=6):
    """Rows where the oracle's residual sum differs from 1 - sum min(p_n, q_n)
    at the stopping position (or from 0 without a rejection)."""
    bad = 0
    rejections = 0
    for _ in range(rounds):
        B, gamma, V = 40, 4, int(rng.integers(5, 300))
        T = float(rng.uniform(0.5, 1.5))
        k = int(rng.choice([0, 3, 10]))
        t = rng.standard_normal((B, gamma + 1, V)) * 2.0     # float64: no ties
        d = t[:, :gamma] + rng.standard_normal((B, gamma, V)) * rng.uniform(0.2, 2.0)
        toks = oracle.sample_draft_tokens(d, T, k, 1.0, int(rng.integers(1 << 30)))
        r = oracle.verify_sample(t, d, toks, T, k, 1.0, 0, seed=int(rng.integers(1 << 30)))
        for b in range(B):
            n = int(r["num_accepted"][b])
            W = float(r["residual_sum"][b])
            if n == gamma:
                bad += W != 0.0
                continue
            rejections += 1
            P, Q = _softmax(t[b, n], T, k), _softmax(d[b, n], T, k)
            bad += not abs(W - (1.0 - np.minimum(P, Q).sum())) < 1e-12
    assert rejections > 50
    return bad


def test_residual_sum_is_reject_mass_at_stopping_position():
    assert _residual_mismatches(np.random.default_rng(5)) == 0


def test_residual_sum_planted_wrong_position_fails(monkeypatch):
    """The mistake: the correction weights (and so W) come from the previous
    position's distributions."""
    real = ov.process_row
    history = []

    def lagged(z, T, k=0, p=1.0):
        row = real(z, T, k, p)
        history.append(row)
        # calls alternate target / draft per position: two calls back is the
        # previous position's row of the same model
        return history[-3] if len(history) >= 3 else row

    monkeypatch.setattr(ov, "process_row", lagged)
    assert _residual_mismatches(np.random.default_rng(5)) > 0
