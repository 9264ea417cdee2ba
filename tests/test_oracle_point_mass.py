"""Pins of the oracle's verification against deterministic drafts (CPU).

A deterministic draft (n-gram or prompt lookup: "投机解码 Speculative
Decoding" tutorial sections 2.1 and 4.2) proposes d with probability one, so
the proposal distribution in the acceptance rule of "11.1 核心原理: Draft +
Verify 与 Rejection Sampling" (11.1.2, pseudo-code 10-1) is the point mass on
d.  What the pages fix, specialised to q = delta(d):

* the 11.1.3 identities: accepted mass min(p, q) = p(d) on d, rejection
  probability 1 - p(d), correction distribution norm(max(p - q, 0)) = p with
  d removed, and final law p (the proof of 11.1.3 holds for any q);
* lossless output: at every position the emitted token follows p_i;
* the acceptance rate at a position is sum_v min(p, q) = p(d);
* the general rule run with draft logits whose softmax is exactly delta(d)
  gives the same round, bit for bit (a special case of the pinned general
  oracle).

Each pin also runs against a planted mistake where that is cheap.
"""

import numpy as np
import pytest
import torch

import oracle
import oracle.verify as ov
from oracle import philox
from test_oracle_verify import GRID, Injected, _first_true, _chi2_pvalue, _softmax64


def _point_mass_law(inj, target, toks, pos, V, verify=None):
    """Exact law of the oracle at ``pos`` given it is reached: accept
    probability and token law after a rejection, per proposed token d."""
    verify = verify or ov.verify_point_mass
    acc = np.zeros(V)
    rej_law = np.zeros((V, V))
    for d in range(V):
        t = toks.copy()
        t[0, pos] = d

        def run(u_acc, u_res):
            inj.u = {(pos, philox.PURPOSE_ACCEPT): u_acc, (pos, philox.PURPOSE_RESIDUAL): u_res}
            return verify(target, t, 1.0, 0, 1.0, 0, seed=1)

        j_rej = _first_true(lambda j: run(j, 0)["num_accepted"][0] <= pos)
        acc[d] = j_rej / GRID
        if j_rej < GRID:
            prev = 0
            for v in range(V - 1):
                j = _first_true(lambda j: run(GRID - 1, j)["out_tokens"][0, pos] > v)
                rej_law[d, v] = (j - prev) / GRID
                prev = j
            rej_law[d, V - 1] = (GRID - prev) / GRID
    return acc, rej_law


def _identities(p, acc, rej, eps):
    """Check the 11.1.3 identities with q = delta(d) for every d."""
    V = len(p)
    for d in range(V):
        q = np.zeros(V)
        q[d] = 1.0
        assert abs(acc[d] - min(1.0, p[d])) < eps                       # min(1, p/q) at d
        accepted = q * acc[d]
        assert np.allclose(accepted, np.minimum(p, q), atol=eps)        # accepted mass min(p, q)
        reject = 1.0 - accepted.sum()
        assert abs(reject - (1.0 - p[d])) < eps
        if reject > eps:
            resid = np.maximum(p - q, 0.0)
            assert np.allclose(rej[d], resid / resid.sum(), atol=eps)   # norm(max(p - q, 0))
        final = accepted + reject * rej[d]
        assert np.allclose(final, p, atol=2 * eps)                      # final law p


def test_point_mass_worked_example_exact(monkeypatch):
    """p = (0.6, 0.4) of the 11.1.3 example, with a deterministic draft of
    either token: exact enumeration over all 2^24 uniforms."""
    p = np.array([0.6, 0.4])
    target = np.log(np.stack([p, p]))[None]
    toks = np.zeros((1, 1), np.int64)
    inj = Injected(monkeypatch)
    acc, rej = _point_mass_law(inj, target, toks, 0, 2)
    _identities(p, acc, rej, 2.0 / GRID)
    # concretely: d = 0 is kept with probability 0.6, and a rejection emits token 1
    assert abs(acc[0] - 0.6) < 2.0 / GRID and abs(rej[0, 1] - 1.0) < 2.0 / GRID


def test_point_mass_identities_exact_v4(monkeypatch):
    """A V = 4 row with unequal masses, at the second position of a chain
    (the first position always accepts: its uniform is 0 and p(d) > 0)."""
    p0 = np.array([0.1, 0.2, 0.3, 0.4])
    p1 = np.array([0.05, 0.5, 0.15, 0.3])
    target = np.log(np.stack([p0, p1, p1]))[None]
    toks = np.array([[3, 0]])
    inj = Injected(monkeypatch)
    acc, rej = _point_mass_law(inj, target, toks, 1, 4)
    _identities(p1, acc, rej, 2.0 / GRID)


def test_point_mass_negative_control(monkeypatch):
    """Keeping d in the correction distribution (resampling from p) breaks
    the final law, and the identity check catches it."""
    monkeypatch.setattr(ov, "residual_weights", lambda P, Q: P)
    p = np.array([0.6, 0.4])
    target = np.log(np.stack([p, p]))[None]
    toks = np.zeros((1, 1), np.int64)
    inj = Injected(monkeypatch)
    acc, rej = _point_mass_law(inj, target, toks, 0, 2)
    with pytest.raises(AssertionError):
        _identities(p, acc, rej, 2.0 / GRID)


def _tiny_deterministic(B, seed):
    """Tiny-recipe logits (V = 32, gamma = 4) with a deterministic draft per
    round: the argmax of a noisy copy of the target, as a lookup guess that
    is often but not always the target's favourite."""
    import synth
    rng = np.random.default_rng(seed)
    t, d = synth.make_logits(rng, B, 4, 32, 2.0, 1.0)
    toks = d.argmax(-1)
    return t, toks


def test_point_mass_lossless_chi2():
    """Fixed logits, 20,000 rounds with fresh uniforms: at every position the
    emitted token follows p_i (given the position is reached)."""
    t, toks = _tiny_deterministic(1, 5)
    B = 20000
    target = np.repeat(t, B, axis=0)
    tk = np.repeat(toks, B, axis=0)
    r = oracle.verify_point_mass(target, tk, 1.0, 0, 1.0, 0, seed=0x5EED0F2)
    for i in range(tk.shape[1] + 1):
        reach = r["num_emitted"] > i
        emitted = r["out_tokens"][reach, i]
        P = _softmax64(t[0, i].astype(np.float64))
        assert _chi2_pvalue(np.bincount(emitted, minlength=len(P)), P) > 1e-3, i


def test_point_mass_lossless_negative_control(monkeypatch):
    monkeypatch.setattr(ov, "residual_weights", lambda P, Q: P)
    p = np.array([[0.6, 0.4], [0.6, 0.4]])
    B = 20000
    target = np.repeat(np.log(p)[None], B, axis=0)
    toks = np.zeros((B, 1), np.int64)
    r = oracle.verify_point_mass(target, toks, 1.0, 0, 1.0, 0, seed=9)
    emitted = r["out_tokens"][:, 0]
    assert _chi2_pvalue(np.bincount(emitted, minlength=2), np.array([0.6, 0.4])) < 1e-6


def test_point_mass_acceptance_rate():
    """Fresh logits per round: the empirical acceptance at position 0
    matches the mean of p_0(d_0) (binomial, 4 sigma)."""
    t, toks = _tiny_deterministic(20000, 1003)
    r = oracle.verify_point_mass(t, toks, 1.0, 0, 1.0, 0, seed=78)
    P = torch.softmax(torch.from_numpy(t[:, 0].astype(np.float64)), -1).numpy()
    pd = P[np.arange(len(toks)), toks[:, 0]]
    acc0 = r["num_accepted"] > 0
    sd = np.sqrt((pd * (1 - pd)).sum()) / len(pd)
    assert abs(acc0.mean() - pd.mean()) < 4 * sd


@pytest.mark.parametrize("top_k,top_p", [(0, 1.0), (5, 1.0), (6, 0.8)])
def test_point_mass_equals_general_rule_with_delta_draft(top_k, top_p):
    """The general rule fed draft logits that are -inf everywhere but 0 at d
    (softmax exactly delta(d), under any temperature and truncation) gives
    the same round, bit for bit, including caps and EOS."""
    t, toks = _tiny_deterministic(400, 1004)
    B, g1, V = t.shape
    draft = np.full((B, g1 - 1, V), -np.inf)
    np.put_along_axis(draft, toks[..., None], 0.0, axis=-1)
    caps = np.random.default_rng(3).integers(0, 6, B)
    a = oracle.verify_point_mass(t, toks, 0.8, top_k, top_p, caps, seed=11, step=2, eos_id=7)
    b = oracle.verify_sample(t, draft, toks, 0.8, top_k, top_p, caps, seed=11, step=2, eos_id=7)
    for key in ("num_accepted", "out_tokens", "num_emitted", "row_flags", "residual_sum"):
        assert np.array_equal(a[key], b[key]), key
    assert np.array_equal(a["p_at_draft"], b["p_at_draft"], equal_nan=True)
    assert np.array_equal(a["q_at_draft"], b["q_at_draft"], equal_nan=True)


def test_point_mass_greedy_rows_match_greedy_rule():
    t, toks = _tiny_deterministic(64, 1005)
    temps = np.where(np.arange(64) % 2 == 0, 1.0, 0.0)
    r = oracle.verify_point_mass(t, toks, temps, 0, 1.0, 0, seed=12)
    g = oracle.verify_greedy(t, toks)
    odd = np.arange(64) % 2 == 1
    assert np.array_equal(r["out_tokens"][odd], g["out_tokens"][odd])
    assert np.array_equal(r["num_accepted"][odd], g["num_accepted"][odd])
