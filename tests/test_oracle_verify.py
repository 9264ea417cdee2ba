"""Pins for the oracle's verify step (CPU only).

What fixes the oracle here, independently of its own code:

* the worked example of "11.1 核心原理" section 11.1.3 (golden file
  ``worked_example.json``): accept probabilities, accepted mass, reject
  probability, residual and final law, obtained by exact enumeration of the
  oracle's decisions over all 2^24 possible uniforms;
* the identities of 11.1.3 (accepted mass min(p, q), reject mass
  sum max(p - q, 0), final law p) on random small rows, by the same
  enumeration, per position of a gamma = 2 chain;
* E[N] at alpha = 0.7 against the values the tutorial prints in section 2.3
  (golden file ``expected_tokens.json``), and the law of N implied by
  stopping at the first rejection (ICML summary);
* chi-square tests that emitted tokens follow p (lossless), with a negative
  control: planting the "resample from p" mistake in the oracle must fail;
* greedy verification against a ``torch.argmax`` path;
* special cases: q = p always accepts, gamma = 0 is plain sampling of p_0,
  a draft outside p's support is always rejected, V = 1, caps and EOS cut a
  prefix of the uncapped output, and the row flags.
"""

import json
import math
import os

import numpy as np
import pytest
import torch
from scipy import stats

import oracle
import oracle.verify as ov
from oracle import philox

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
GRID = 1 << 24


def _softmax64(z, T=1.0):
    return torch.softmax(torch.as_tensor(np.asarray(z, np.float64)) / T, 0).numpy()


class Injected:
    """Replace the oracle's uniforms: u[(i, purpose)] -> grid index / 2^24."""

    def __init__(self, monkeypatch):
        self.u = {}
        monkeypatch.setattr(ov, "uniform", self)

    def __call__(self, seed, b, i, purpose, step=0):
        return self.u.get((int(i), int(purpose)), 0) / GRID


def _first_true(pred):
    """Smallest j in [0, 2^24] with pred(j) true, pred monotone false->true."""
    lo, hi = 0, GRID
    while lo < hi:
        mid = (lo + hi) // 2
        if pred(mid):
            hi = mid
        else:
            lo = mid + 1
    return lo


def _exact_position_law(inj, target, draft, toks, pos, V):
    """Exact law of the oracle at position ``pos`` of a chain, given it is
    reached (earlier accept uniforms are 0, earlier drafts have p > 0).

    Returns (accept_prob[d], token_law_given_reject[d][v]) where d ranges
    over the draft token placed at ``pos``; both are counts / 2^24.
    """
    acc = np.zeros(V)
    rej_law = np.zeros((V, V))
    for d in range(V):
        t = toks.copy()
        t[0, pos] = d

        def run(u_acc, u_res):
            inj.u = {(pos, philox.PURPOSE_ACCEPT): u_acc, (pos, philox.PURPOSE_RESIDUAL): u_res}
            r = ov.verify_sample(target, draft, t, 1.0, 0, 1.0, 0, seed=1)
            return r

        # accepted iff num_accepted > pos; monotone in the uniform
        j_rej = _first_true(lambda j: run(j, 0)["num_accepted"][0] <= pos)
        acc[d] = j_rej / GRID
        if j_rej < GRID:
            # token after a rejection as a function of the residual uniform
            prev = 0
            for v in range(V - 1):
                j = _first_true(lambda j: run(GRID - 1, j)["out_tokens"][0, pos] > v)
                rej_law[d, v] = (j - prev) / GRID
                prev = j
            rej_law[d, V - 1] = (GRID - prev) / GRID
            # spot checks: the decision really is the bisected step function
            rng = np.random.default_rng(d)
            for j in rng.integers(0, GRID, 8):
                r = run(int(j), 0)
                assert (r["num_accepted"][0] > pos) == (j < j_rej)
    return acc, rej_law


def _worked_example_law(monkeypatch):
    g = json.load(open(os.path.join(GOLDEN, "worked_example.json")))
    p, q = np.array(g["p"]), np.array(g["q"])
    target = np.log(np.stack([p, p]))[None]           # [1, 2, 2]; row 1 = bonus
    draft = np.log(q)[None, None]                     # [1, 1, 2]
    toks = np.zeros((1, 1), np.int64)
    inj = Injected(monkeypatch)
    acc, rej = _exact_position_law(inj, target, draft, toks, 0, 2)
    return g, p, q, acc, rej


def test_worked_example_exact(monkeypatch):
    g, p, q, acc, rej = _worked_example_law(monkeypatch)
    eps = 2.0 / GRID
    assert np.allclose(acc, g["accept_probability"], atol=eps)
    accepted_mass = q * acc
    assert np.allclose(accepted_mass, g["accepted_mass"], atol=eps)
    reject = 1 - accepted_mass.sum()
    assert abs(reject - g["reject_probability"]) < eps
    # the first token is rejected with probability 0.25, and then always corrected to token 1
    assert np.allclose(rej[0], g["residual_distribution"], atol=eps)
    final = accepted_mass + (q * (1 - acc)) @ rej
    assert np.allclose(final, g["final_distribution"], atol=2 * eps)


def test_worked_example_negative_control(monkeypatch):
    """Planting the 'resample from p' mistake in the oracle reproduces the
    biased (0.72, 0.28) of 11.1.3 and fails the final-law pin."""
    monkeypatch.setattr(ov, "residual_weights", lambda P, Q: P)
    g, p, q, acc, rej = _worked_example_law(monkeypatch)
    final = q * acc + (q * (1 - acc)) @ rej
    assert np.allclose(final, g["biased_if_resampled_from_p"], atol=1e-6)
    assert not np.allclose(final, g["final_distribution"], atol=1e-3)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_identities_exact_small_chain(monkeypatch, seed):
    """gamma = 2, V = 3 or 4: at every position the accepted mass is
    min(p, q), the reject mass is sum max(p - q, 0), the final law is p, and
    P(reach i+1 | reach i) = alpha_i = sum min(p_i, q_i)."""
    rng = np.random.default_rng(seed)
    V = 3 + seed % 2
    gamma = 2
    P = rng.dirichlet(np.ones(V), size=gamma + 1)
    Q = rng.dirichlet(np.ones(V), size=gamma)
    target = np.log(P)[None]
    draft = np.log(Q)[None]
    toks = np.zeros((1, gamma), np.int64)
    inj = Injected(monkeypatch)
    eps = 4.0 / GRID
    for pos in range(gamma):
        # earlier positions carry a draft with p > 0 and uniform 0: always accepted
        acc, rej = _exact_position_law(inj, target, draft, toks, pos, V)
        p, q = P[pos], Q[pos]
        assert np.allclose(q * acc, np.minimum(p, q), atol=eps)
        reject_mass = (q * (1 - acc)).sum()
        assert abs(reject_mass - np.maximum(p - q, 0).sum()) < eps
        for d in range(V):
            if acc[d] < 1:
                assert np.allclose(reject_mass * rej[d], np.maximum(p - q, 0), atol=eps)
        final = q * acc + (q * (1 - acc)) @ rej
        assert np.allclose(final, p, atol=2 * eps)
        assert abs((q * acc).sum() - np.minimum(p, q).sum()) < eps


def _replicated_round(p_rows, q_rows, B, seed, step=0, cap=0, eos=-1):
    """B independent rounds (rows) sharing the same per-position logits."""
    target = np.broadcast_to(np.log(p_rows)[None], (B,) + p_rows.shape).copy()
    draft = np.broadcast_to(np.log(q_rows)[None], (B,) + q_rows.shape).copy()
    toks = oracle.sample_draft_tokens(draft, 1.0, 0, 1.0, seed, step)
    return oracle.verify_sample(target, draft, toks, 1.0, 0, 1.0, cap, seed, step, eos), toks


@pytest.mark.parametrize("gamma", [4, 8])
def test_expected_tokens_alpha_07(gamma):
    g = json.load(open(os.path.join(GOLDEN, "expected_tokens.json")))
    p, q = np.array([0.5, 0.5]), np.array([0.8, 0.2])
    alpha = np.minimum(p, q).sum()
    assert abs(alpha - g["alpha"]) < 1e-12
    B = 12000
    r, _ = _replicated_round(np.stack([p] * (gamma + 1)), np.stack([q] * gamma), B, seed=11 + gamma)
    N = r["num_emitted"].astype(np.float64)
    assert N.min() >= 1 and N.max() <= gamma + 1
    printed = g["printed"][str(gamma)]
    half_ulp = 0.5 * 10.0 ** -g["printed_decimals"]
    se = N.std() / math.sqrt(B)
    assert abs(N.mean() - printed) < half_ulp + 4 * se
    # law of N: P(N = n + 1) = alpha^n (1 - alpha) for n < gamma, alpha^gamma for n = gamma
    law = np.array([alpha ** n * (1 - alpha) for n in range(gamma)] + [alpha ** gamma])
    counts = np.bincount(N.astype(int) - 1, minlength=gamma + 1)
    assert stats.chisquare(counts, law * B).pvalue > 1e-3


def _chi2_pvalue(counts, probs):
    exp = probs * counts.sum()
    order = np.argsort(exp)
    c, e = counts[order].astype(float), exp[order]
    # pool the smallest expected counts until every bin expects >= 5
    cc, ee, acc_c, acc_e = [], [], 0.0, 0.0
    for ci, ei in zip(c, e):
        acc_c += ci
        acc_e += ei
        if acc_e >= 5:
            cc.append(acc_c)
            ee.append(acc_e)
            acc_c = acc_e = 0.0
    if acc_e > 0:
        if ee:
            cc[-1] += acc_c
            ee[-1] += acc_e
        else:
            cc.append(acc_c)
            ee.append(acc_e)
    if len(cc) < 2:
        return 1.0
    return stats.chisquare(cc, np.array(ee) * sum(cc) / sum(ee)).pvalue


def _lossless_pvalues(target_row, draft_row, B, seed):
    r, toks = _replicated_round(np.exp(target_row), np.exp(draft_row), B, seed)
    gamma = draft_row.shape[0]
    pv = []
    for i in range(gamma + 1):
        reach = r["num_emitted"] > i
        emitted = r["out_tokens"][reach, i]
        P = _softmax64(target_row[i])
        pv.append(_chi2_pvalue(np.bincount(emitted, minlength=len(P)), P))
    return pv, r


def _tiny_logits():
    import synth
    w = synth.tiny()
    return w.target_f32()[0].astype(np.float64), w.draft_f32()[0].astype(np.float64)


def test_lossless_chi2_tiny():
    """The tiny workload (V = 32, gamma = 4): 20,000 rounds on fixed logits;
    at every position the emitted token follows p_i."""
    t, d = _tiny_logits()
    pv, _ = _lossless_pvalues(t, d, 20000, seed=0x5EED0001)
    assert min(pv) > 1e-3, pv


def test_lossless_negative_control(monkeypatch):
    """With 'resample from p' planted in the oracle the chi-square test fails."""
    monkeypatch.setattr(ov, "residual_weights", lambda P, Q: P)
    p = np.array([[0.6, 0.4], [0.6, 0.4]])
    q = np.array([[0.8, 0.2]])
    pv, _ = _lossless_pvalues(np.log(p), np.log(q), 20000, seed=3)
    assert pv[0] < 1e-6
    monkeypatch.undo()
    pv, _ = _lossless_pvalues(np.log(p), np.log(q), 20000, seed=3)
    assert pv[0] > 1e-3


def test_acceptance_rate_matches_overlap():
    """Fresh tiny-recipe logits per round: the empirical acceptance at
    position 0 matches the mean overlap sum_v min(p, q) (binomial 4 sigma)."""
    import synth
    rng = np.random.default_rng(1001)
    B = 20000
    t, d = synth.make_logits(rng, B, 4, 32, 2.0, 1.0)
    toks = oracle.sample_draft_tokens(d, 1.0, 0, 1.0, 77)
    r = oracle.verify_sample(t, d, toks, 1.0, 0, 1.0, 0, 77)
    P = torch.softmax(torch.from_numpy(t[:, 0].astype(np.float64)), -1).numpy()
    Q = torch.softmax(torch.from_numpy(d[:, 0].astype(np.float64)), -1).numpy()
    alpha = np.minimum(P, Q).sum(-1)
    accepted0 = r["num_accepted"] > 0
    sd = math.sqrt((alpha * (1 - alpha)).sum()) / B
    assert abs(accepted0.mean() - alpha.mean()) < 4 * sd


def test_greedy_matches_torch_argmax():
    rng = np.random.default_rng(9)
    B, gamma, V = 200, 5, 50
    t = np.round(rng.standard_normal((B, gamma + 1, V)) * 4) / 4     # many ties
    am = torch.argmax(torch.from_numpy(t), -1).numpy()
    toks = am[:, :gamma].copy()
    # inject one mismatch at a random position in most rows
    for b in range(B):
        if b % 5:
            i = rng.integers(0, gamma)
            toks[b, i] = (am[b, i] + 1 + rng.integers(0, V - 1)) % V
    r = oracle.verify_greedy(t, toks)
    for b in range(B):
        want = []
        for i in range(gamma + 1):
            want.append(int(am[b, i]))
            if i == gamma or toks[b, i] != am[b, i]:
                break
        assert r["out_tokens"][b, :len(want)].tolist() == want
        assert r["num_emitted"][b] == len(want)
        assert r["num_accepted"][b] == len(want) - 1
    # the same rows with temperature 0 go through the greedy path of verify_sample
    r2 = oracle.verify_sample(t, t[:, :gamma], toks, 0.0, 0, 1.0, 0, 5)
    assert np.array_equal(r2["out_tokens"], r["out_tokens"])


def test_q_equals_p_always_accepts():
    t, _ = _tiny_logits()
    B = 4000
    r, _ = _replicated_round(np.exp(t), np.exp(t[:4]), B, seed=21)
    assert (r["num_accepted"] == 4).all() and (r["num_emitted"] == 5).all()
    P = _softmax64(t[4])
    assert _chi2_pvalue(np.bincount(r["out_tokens"][:, 4], minlength=32), P) > 1e-3


def test_gamma_zero_is_plain_sampling():
    t, _ = _tiny_logits()
    B = 20000
    target = np.broadcast_to(t[:1][None], (B, 1, 32)).copy()
    r = oracle.verify_sample(target, np.zeros((B, 0, 32)), np.zeros((B, 0), np.int32),
                             1.0, 0, 1.0, 0, 33)
    assert (r["num_emitted"] == 1).all() and (r["num_accepted"] == 0).all()
    assert _chi2_pvalue(np.bincount(r["out_tokens"][:, 0], minlength=32), _softmax64(t[0])) > 1e-3


def test_draft_outside_target_support_always_rejected():
    rng = np.random.default_rng(4)
    B, V = 500, 16
    t = rng.standard_normal((B, 2, V))
    t[:, 0, 3] = -np.inf
    d = rng.standard_normal((B, 1, V))
    toks = np.full((B, 1), 3)
    r = oracle.verify_sample(t, d, toks, 1.0, 0, 1.0, 0, 8)
    assert (r["num_accepted"] == 0).all()
    assert (r["out_tokens"][:, 0] != 3).all()


def test_vocab_of_one():
    B = 50
    r = oracle.verify_sample(np.zeros((B, 3, 1)), np.zeros((B, 2, 1)), np.zeros((B, 2), int),
                             1.0, 0, 1.0, 0, 1)
    assert (r["out_tokens"] == 0).all() and (r["num_emitted"] == 3).all()


def test_cap_and_eos_cut_a_prefix():
    import synth
    rng = np.random.default_rng(5)
    B, gamma, V = 400, 6, 40
    t, d = synth.make_logits(rng, B, gamma, V, 1.0, 0.3)
    toks = oracle.sample_draft_tokens(d, 1.0, 0, 1.0, 2)
    full = oracle.verify_sample(t, d, toks, 1.0, 0, 1.0, 0, 2)
    caps = rng.integers(1, gamma + 3, size=B)
    capped = oracle.verify_sample(t, d, toks, 1.0, 0, 1.0, caps, 2)
    eos = int(np.bincount(toks.ravel()).argmax())
    cut = oracle.verify_sample(t, d, toks, 1.0, 0, 1.0, 0, 2, eos_id=eos)
    for b in range(B):
        f = full["out_tokens"][b, :full["num_emitted"][b]].tolist()
        c = capped["out_tokens"][b, :capped["num_emitted"][b]].tolist()
        assert c == f[:caps[b]]
        assert capped["num_accepted"][b] == min(full["num_accepted"][b], len(c))
        e = cut["out_tokens"][b, :cut["num_emitted"][b]].tolist()
        want = f[:f.index(eos) + 1] if eos in f else f
        assert e == want
        assert (capped["out_tokens"][b, len(c):] == -1).all()


def test_row_flags():
    rng = np.random.default_rng(6)
    B, gamma, V = 6, 3, 20
    t = rng.standard_normal((B, gamma + 1, V))
    d = t[:, :gamma] + 0.5 * rng.standard_normal((B, gamma, V))
    toks = np.argmax(d, -1)
    toks[0, 1] = V                       # out of range
    t[1, 0, 4] = np.nan                  # consulted row with NaN
    t[2, gamma, 4] = np.nan              # NaN only in the bonus row
    toks[3, 0] = 7                       # draft token outside q's support, p > 0
    d[3, 0, 7] = -np.inf
    t[4, 0] = d[4, 0]                    # p == q, d outside both supports: W = 0
    t[4, 0, 2] = -np.inf
    d[4, 0, 2] = -np.inf
    toks[4, 0] = 2
    r = oracle.verify_sample(t, d, toks, 1.0, 0, 1.0, 0, 12)
    f = r["row_flags"]
    assert f[0] == oracle.FLAG_TOKEN_OOR and r["num_emitted"][0] == 0
    assert f[1] & oracle.FLAG_NONFINITE_ROW and r["num_emitted"][1] == 0
    # row 2 only hits the NaN if every draft is accepted
    if r["num_accepted"][2] == gamma:
        assert f[2] & oracle.FLAG_NONFINITE_ROW
    else:
        assert f[2] == 0 and r["num_emitted"][2] >= 1
    assert f[3] & oracle.FLAG_Q_ZERO and r["num_accepted"][3] >= 1    # accepted: p > 0 = q
    assert f[4] & oracle.FLAG_Q_ZERO and f[4] & oracle.FLAG_RESIDUAL_FALLBACK
    assert r["num_accepted"][4] == 0 and r["out_tokens"][4, 0] != 2
    assert f[5] == 0
