"""Pins of the oracle's drafter stand-in (CPU): the draw d_i ~ q_i and the
row statistics a drafter hands to the verifier.

What fixes them, independently of the oracle's own code:

* the law of the draw, by exact enumeration of its decisions over all 2^24
  uniforms, equals softmax(z / T) computed by ``torch.softmax`` (the
  temperature division of the tutorial's section 3.3), and with top-k, the
  softmax restricted to a brute-force top-k set ("11.1 核心原理", section
  11.1.2: q is the distribution actually sampled);
* greedy drafts equal ``torch.argmax`` (first maximal index);
* the statistics: m is the row maximum and m / T + log s equals
  ``torch.logsumexp(z / T)``, so exp((z - m) / T) / s is q; with top-k /
  top-p, [z >= t] exp((z - m) / T) / s equals ``torch.softmax`` over a
  brute-force kept set (the definitions written out with full sorts);
* a row with NaN / +inf or nothing finite gives token -1 and NaN statistics;
* drawing one column at a time with its position equals drawing them all.

Planted mistakes (temperature ignored, the uniform's position ignored) fail.
"""

import numpy as np
import pytest
import torch

import oracle
import oracle.verify as ov
from oracle import philox
from test_oracle_verify import GRID, _first_true

_orig_process_row = ov.process_row


class _DraftU:
    def __init__(self, monkeypatch):
        self.j = 0
        monkeypatch.setattr(ov, "uniform", self)

    def __call__(self, seed, b, i, purpose, step=0):
        assert purpose == philox.PURPOSE_DRAFT
        return self.j / GRID


def _exact_draw_law(monkeypatch, z, T, k=0, p=1.0):
    inj = _DraftU(monkeypatch)
    V = len(z)
    draft = np.asarray(z, np.float64)[None, None]

    def tok(j):
        inj.j = j
        return int(ov.sample_draft_tokens(draft, T, k, p, seed=1)[0, 0])

    law, prev = np.zeros(V), 0
    for v in range(V - 1):
        j = _first_true(lambda j: tok(j) > v)
        law[v] = (j - prev) / GRID
        prev = j
    law[V - 1] = (GRID - prev) / GRID
    return law


@pytest.mark.parametrize("T", [1.0, 0.7, 1.6])
def test_draw_law_is_softmax_over_temperature(monkeypatch, T):
    z = np.array([0.3, -1.2, 2.0, 0.9, -0.4])
    law = _exact_draw_law(monkeypatch, z, T)
    q = torch.softmax(torch.tensor(z, dtype=torch.float64) / T, 0).numpy()
    assert np.allclose(law, q, atol=2.0 / GRID)


def test_draw_law_top_k_brute_force(monkeypatch):
    z = np.array([0.3, -1.2, 2.0, 0.9, -0.4, 1.5])
    T, k = 0.8, 3
    law = _exact_draw_law(monkeypatch, z, T, k)
    keep = np.zeros(len(z), bool)
    keep[np.argsort(-z)[:k]] = True               # no ties in this row
    x = torch.tensor(np.where(keep, z / T, -np.inf), dtype=torch.float64)
    q = torch.softmax(x, 0).numpy()
    assert np.allclose(law, q, atol=2.0 / GRID)


def test_draw_law_negative_control(monkeypatch):
    """A drafter that ignores its temperature draws from the wrong law."""
    monkeypatch.setattr(ov, "process_row", lambda z, T, k, p: _orig_process_row(z, 1.0, k, p))
    z = np.array([0.3, -1.2, 2.0, 0.9, -0.4])
    law = _exact_draw_law(monkeypatch, z, 0.7)
    q = torch.softmax(torch.tensor(z, dtype=torch.float64) / 0.7, 0).numpy()
    assert not np.allclose(law, q, atol=2.0 / GRID)


def test_greedy_draft_is_torch_argmax():
    rng = np.random.default_rng(5)
    d = rng.standard_normal((6, 3, 50)).astype(np.float32)
    d[2, 1, [4, 9]] = 10.0                         # tie: the lower index
    toks = oracle.sample_draft_tokens(d, 0.0, 0, 1.0, seed=3)
    assert np.array_equal(toks, torch.argmax(torch.from_numpy(d), -1).numpy())
    assert toks[2, 1] == 4


def _lse_check(d, T, st):
    z = torch.from_numpy(np.asarray(d, np.float64))
    m = z.max(-1).values.numpy()
    lse = torch.logsumexp(z / T, -1).numpy()
    assert np.array_equal(st[..., 0], m)
    assert np.allclose(st[..., 0] / T + np.log(st[..., 1]), lse, rtol=0, atol=1e-12)
    assert np.all(st[..., 2] == -np.inf)


@pytest.mark.parametrize("T", [1.0, 0.7, 2.5])
def test_row_stats_logsumexp(T):
    rng = np.random.default_rng(int(T * 10))
    d = (3 * rng.standard_normal((4, 3, 1000))).astype(np.float32)
    st = oracle.draft_row_stats(d, T)
    _lse_check(d, T, st)
    # exp((z - m) / T) / s is the processed q
    q = np.exp((d[1, 2].astype(np.float64) - st[1, 2, 0]) / T) / st[1, 2, 1]
    assert np.allclose(q, ov.process_row(d[1, 2], T).probs, rtol=1e-12, atol=0)


def test_row_stats_negative_control(monkeypatch):
    """Statistics that leave out the temperature fail the logsumexp pin."""
    rng = np.random.default_rng(1)
    d = rng.standard_normal((2, 2, 300))
    st = oracle.draft_row_stats(d, 1.0)
    with pytest.raises(AssertionError):
        _lse_check(d, 0.6, st)


def test_bad_rows_and_greedy_rows():
    rng = np.random.default_rng(2)
    d = rng.standard_normal((4, 2, 40))
    d[0, 1, 3] = np.nan
    d[1, 0] = -np.inf
    d[2, 1, 7] = np.inf
    T = np.array([1.0, 1.0, 1.0, 0.0])
    toks = oracle.sample_draft_tokens(d, T, 0, 1.0, seed=4)
    st = oracle.draft_row_stats(d, T)
    assert toks[0, 1] == -1 and toks[1, 0] == -1 and toks[2, 1] == -1
    assert np.isnan(st[0, 1]).all() and np.isnan(st[1, 0]).all() and np.isnan(st[2, 1]).all()
    assert toks[0, 0] >= 0 and np.isfinite(st[0, 0, :2]).all() and st[0, 0, 2] == -np.inf
    assert np.isnan(st[3]).all()                    # greedy rows: no statistics
    assert toks[3].tolist() == d[3].argmax(-1).tolist()
    g = oracle.sample_draft_tokens(d[1:2], 0.0, 0, 1.0, seed=4)
    assert g[0, 0] == -1


def test_column_at_a_time_equals_all_at_once(monkeypatch):
    rng = np.random.default_rng(3)
    d = rng.standard_normal((8, 4, 64))
    full = oracle.sample_draft_tokens(d, 0.9, 0, 1.0, seed=77, step=5)
    for i in range(4):
        col = oracle.sample_draft_tokens(d[:, i:i + 1], 0.9, 0, 1.0, seed=77, step=5, pos0=i)
        assert np.array_equal(col[:, 0], full[:, i])
    # negative control: a drafter that forgets its position repeats column 0's uniforms
    wrong = [oracle.sample_draft_tokens(d[:, i:i + 1], 0.9, 0, 1.0, seed=77, step=5)[:, 0]
             for i in range(4)]
    assert not all(np.array_equal(wrong[i], full[:, i]) for i in range(4))


def _brute_kept(z, T, k, top_p):
    """Kept set from the definitions: top-k by counting larger values (ties
    kept), then the highest level whose value-ordered mass reaches top_p."""
    V = len(z)
    keep = np.array([(z > z[v]).sum() < k for v in range(V)]) if 0 < k < V else np.ones(V, bool)
    if top_p < 1.0:
        x = z / T
        e = np.where(keep, np.exp(x - x[keep].max()), 0.0)
        pi = e / e.sum()
        best = min(z[keep])
        for lv in sorted(set(z[keep].tolist())):
            if pi[keep & (z >= lv)].sum() >= top_p:
                best = lv
        keep = keep & (z >= best)
    return keep


@pytest.mark.parametrize("k,top_p", [(5, 1.0), (0, 0.8), (12, 0.9), (40, 0.5)])
def test_row_stats_truncated_brute_force(k, top_p):
    rng = np.random.default_rng(k + int(top_p * 100))
    d = np.round(rng.standard_normal((3, 2, 60)) * 8) / 4          # coarse values: ties
    T = 0.8
    st = oracle.draft_row_stats(d, T, k, top_p)
    for b in range(3):
        for i in range(2):
            z = d[b, i]
            keep = _brute_kept(z, T, k, top_p)
            q_bf = torch.softmax(torch.tensor(np.where(keep, z / T, -np.inf)), 0).numpy()
            m, s, t = st[b, i]
            q = np.where(z >= t, np.exp((z - m) / T), 0.0) / s
            assert np.allclose(q, q_bf, rtol=1e-12, atol=1e-300)
            assert t == z[keep].min() and m == z.max()


def test_row_stats_truncated_negative_control(monkeypatch):
    """Statistics that keep the whole row under top-k fail the pin."""
    d = np.round(np.random.default_rng(9).standard_normal((1, 1, 40)) * 8) / 4
    st = oracle.draft_row_stats(d, 0.8, 0, 1.0)                     # untruncated
    z = d[0, 0]
    keep = _brute_kept(z, 0.8, 5, 1.0)
    q_bf = torch.softmax(torch.tensor(np.where(keep, z / 0.8, -np.inf)), 0).numpy()
    m, s, t = st[0, 0]
    q = np.where(z >= t, np.exp((z - m) / 0.8), 0.0) / s
    assert not np.allclose(q, q_bf, rtol=1e-12, atol=1e-300)
