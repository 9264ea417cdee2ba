"""Pins for the oracle's per-distribution processing (CPU only).

* untruncated probabilities equal ``torch.softmax(z / T)`` in float64;
* the top-k set equals a brute force written from its definition by
  counting (keep v iff fewer than k tokens have a strictly larger logit);
* the top-p set equals a brute force that sums the mass of every candidate
  level directly and keeps the highest level whose mass reaches top_p;
* greedy argmax equals ``torch.argmax`` (first maximal index) including
  injected ties.
"""

import numpy as np
import pytest
import torch

from oracle import process_row, greedy_argmax


def _rows(seed, n, V, ties=True):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        z = (rng.standard_normal(V) * 3).astype(np.float32)
        if ties:
            # bf16-like coarse values produce many exact ties
            z = np.round(z * 4) / 4
        out.append(z)
    return out


@pytest.mark.parametrize("T", [1.0, 0.7, 2.5])
def test_softmax_matches_torch(T):
    for z in _rows(1, 20, 257, ties=False):
        P = process_row(z, np.float32(T))
        ref = torch.softmax(torch.from_numpy(z.astype(np.float64)) / float(np.float32(T)), 0).numpy()
        assert np.allclose(P.probs, ref, rtol=1e-13, atol=1e-300)
        assert abs(P.probs.sum() - 1.0) < 1e-13


def _brute_topk(z, k):
    V = len(z)
    if not (0 < k < V):
        return np.ones(V, bool)
    return np.array([(z > z[v]).sum() < k for v in range(V)])


def _brute_topp(z, T, keep, top_p):
    x = z.astype(np.float64) / T
    e = np.where(keep, np.exp(x - x[keep].max()), 0.0)
    pi = e / e.sum()
    best = None
    for lv in sorted(set(z[keep].tolist())):
        mass = sum(pi[v] for v in range(len(z)) if keep[v] and z[v] >= lv)
        if mass >= top_p:
            best = lv          # levels ascend, so the last one kept is the highest
    if best is None:
        best = min(z[keep])
    return keep & (z >= best)


@pytest.mark.parametrize("k", [1, 3, 10, 63, 64, 200])
def test_topk_brute_force(k):
    for z in _rows(2, 10, 64):
        P = process_row(z, 1.0, k, 1.0)
        want = _brute_topk(z, k)
        assert np.array_equal(P.kept, want)
        assert P.kept.sum() >= min(k, len(z))
        assert np.all(P.probs[~want] == 0)
        assert abs(P.probs.sum() - 1) < 1e-12


@pytest.mark.parametrize("k,top_p", [(0, 0.5), (0, 0.9), (10, 0.9), (5, 0.3), (64, 0.99), (3, 0.0)])
def test_topp_brute_force(k, top_p):
    for z in _rows(3, 10, 48):
        T = np.float32(0.8)
        P = process_row(z, T, k, top_p)
        keep_k = _brute_topk(z, k)
        want = _brute_topp(z, float(T), keep_k, top_p)
        assert np.array_equal(P.kept, want)
        assert P.kept[np.argmax(z)]           # the largest logit is always kept
        x = z.astype(np.float64) / float(T)
        e = np.where(want, np.exp(x - x.max()), 0.0)
        assert np.allclose(P.probs, e / e.sum(), rtol=1e-13, atol=0)


def test_truncation_off_switches():
    z = _rows(4, 1, 40)[0]
    base = process_row(z, 1.0)
    for k, p in [(0, 1.0), (40, 1.0), (1000, 1.0), (-1, 1.0), (0, 1.5)]:
        P = process_row(z, 1.0, k, p)
        assert np.array_equal(P.probs, base.probs)


def test_neg_inf_masked_and_nonfinite():
    z = np.array([0.0, -np.inf, 1.0, -np.inf], np.float32)
    P = process_row(z, 1.0)
    assert not P.nonfinite and P.probs[1] == 0 and P.probs[3] == 0
    assert process_row(np.array([0.0, np.nan]), 1.0).nonfinite
    assert process_row(np.array([0.0, np.inf]), 1.0).nonfinite
    assert process_row(np.array([-np.inf, -np.inf]), 1.0).nonfinite


def test_greedy_argmax_matches_torch():
    for z in _rows(5, 50, 33):
        z[7] = z.max()          # inject a tie with an earlier or later maximum
        assert greedy_argmax(z) == int(torch.argmax(torch.from_numpy(z)))
    assert greedy_argmax(np.array([1.0, np.nan])) is None
    assert greedy_argmax(np.array([-np.inf, -np.inf])) is None
    assert greedy_argmax(np.array([-np.inf, -3.0, -3.0])) == 1
