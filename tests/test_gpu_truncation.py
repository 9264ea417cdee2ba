"""GPU parity of truncated rows (top-k / top-p on both p and q) against the
oracle, to the bar in ``parity.py``.

The truncated workload: B=32, gamma=5, V=152064, bf16, T=0.7, top-k=50 and
top-p=0.9 on target and draft alike, draft tokens drawn from the truncated
draft distribution (Philox purpose DRAFT, by the oracle's sampler).  Plus
top-k alone, top-p alone, k=1, ties at the threshold, top_p=0, ragged float32
vocabularies; rows the candidate lists cannot settle (top-p alone on flat
rows, ties beyond every buffer, top_k above max_top_k), which take the exact
whole-row truncation; and a handle without truncation workspace.
"""

import numpy as np
import pytest
import torch

import oracle
import synth
import speculative_decoding_verification_sampling_amd as sv
from parity import compare

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    sv.load_library()
    return torch.device("cuda:0")


def _prm(B, T, k, p, cap=0):
    b = lambda x, dt: np.broadcast_to(np.asarray(x, dt), (B,)).copy()
    return {"temperature": b(T, np.float32), "top_k": b(k, np.int32), "top_p": b(p, np.float32),
            "max_new_tokens": b(cap, np.int32)}


def run_trunc(target, draft, prm, seed, max_top_k=1024, tokens=None, step=0, eos=-1):
    B, g1, V = target.shape
    gamma = g1 - 1
    tf, df = target.to(torch.float32).numpy(), draft.to(torch.float32).numpy()
    if tokens is None:
        tokens = oracle.sample_draft_tokens(df, prm["temperature"], prm["top_k"], prm["top_p"],
                                            seed ^ 0x1234)
    with sv.Verifier(B, gamma, V, max_top_k=max_top_k) as v:
        out = v.verify_sample(target.cuda(), draft.cuda(), torch.from_numpy(tokens).cuda(),
                              sv.make_row_params(B, prm["temperature"], prm["top_k"], prm["top_p"],
                                                 prm["max_new_tokens"]),
                              seed, step, eos, diag=True)
        torch.cuda.synchronize()
    orc = oracle.verify_sample(tf, df, tokens, prm["temperature"], prm["top_k"], prm["top_p"],
                               prm["max_new_tokens"], seed, step, eos)
    return out, orc, tokens, tf, df


def check(out, orc, tokens, tf, df, prm, max_tol=0.05, workload=None):
    rep = compare(out, orc, tokens, tf, df, prm, workload=workload)
    print(rep.summary())
    rep.assert_ok(max_tol)
    return rep


def test_truncated_workload_full_size(gpu):
    w = synth.truncated()
    prm = _prm(w.B, w.temperature, w.top_k, w.top_p)
    out, orc, toks, tf, df = run_trunc(w.target, w.draft, prm, w.seed, max_top_k=64)
    rep = check(out, orc, toks, tf, df, prm,
                workload="config 4: truncated B=32 gamma=5 V=152064 bf16 T=0.7 top-k 50 top-p 0.9")
    assert rep.value_checks > w.B
    f = out["row_flags"].cpu().numpy()
    assert not (f & (sv.FLAG_CAND_OVERFLOW | sv.FLAG_UNSUPPORTED)).any()


@pytest.mark.parametrize("k,p", [(50, 1.0), (0, 0.9), (1, 1.0), (5, 0.5), (200, 0.95), (20, 0.0)])
def test_truncation_variants(gpu, k, p):
    rng = np.random.default_rng(100 + k)
    B, gamma, V = 12, 4, 40000
    t, d = synth.make_logits(rng, B, gamma, V, 3.0, 1.0, boost_count=20)
    tt, dd = torch.from_numpy(t).to(torch.bfloat16), torch.from_numpy(d).to(torch.bfloat16)
    prm = _prm(B, 0.7, k, p)
    out, orc, toks, tf, df = run_trunc(tt, dd, prm, 77 + k)
    check(out, orc, toks, tf, df, prm, max_tol=0.1)


def test_truncation_ties_at_threshold(gpu):
    """Coarse values: many exact ties at the top-k threshold and at top-p levels."""
    rng = np.random.default_rng(5)
    B, gamma, V = 10, 3, 20000
    t = np.round(rng.standard_normal((B, gamma + 1, V)) * 2).astype(np.float32)
    d = np.round(t[:, :gamma] + rng.standard_normal((B, gamma, V))).astype(np.float32)
    prm = _prm(B, 1.0, 30, 0.8)
    out, orc, toks, tf, df = run_trunc(torch.from_numpy(t), torch.from_numpy(d), prm, 9)
    check(out, orc, toks, tf, df, prm, max_tol=0.2)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_signed_zeros_at_threshold(gpu, dtype):
    """-0.0 and +0.0 are the same logit: when the top-k threshold is 0, the
    kept set holds the zeros of both signs (ties kept)."""
    rng = np.random.default_rng(13)
    B, gamma, V = 8, 3, 9000
    t = np.full((B, gamma + 1, V), -6.0, np.float32)
    d = np.full((B, gamma, V), -6.0, np.float32)
    for arr in (t, d):
        for idx in np.ndindex(arr.shape[:2]):
            pos = rng.choice(V, 12, replace=False)
            arr[idx][pos] = rng.uniform(0.5, 3.0, 12)
            zeros = rng.choice(np.setdiff1d(np.arange(V), pos), 40, replace=False)
            arr[idx][zeros] = np.where(rng.random(40) < 0.5, -0.0, 0.0)
    tt, dd = torch.from_numpy(t).to(dtype), torch.from_numpy(d).to(dtype)
    assert (torch.signbit(tt) & (tt == 0)).any()
    for k, p in ((20, 1.0), (30, 0.97)):
        prm = _prm(B, 1.0, k, p)
        out, orc, toks, tf, df = run_trunc(tt, dd, prm, 21 + k)
        check(out, orc, toks, tf, df, prm, max_tol=0.2)


@pytest.mark.parametrize("V", [7, 300, 8193, 20001])
def test_truncation_ragged_f32(gpu, V):
    rng = np.random.default_rng(V)
    B, gamma = 6, 3
    t, d = synth.make_logits(rng, B, gamma, V, 2.0, 0.8, boost_count=min(20, V))
    prm = _prm(B, 0.9, min(10, V - 1) if V > 1 else 0, 0.9)
    out, orc, toks, tf, df = run_trunc(torch.from_numpy(t), torch.from_numpy(d), prm, 31)
    check(out, orc, toks, tf, df, prm, max_tol=0.2)


def test_truncation_with_caps_eos_and_greedy_rows(gpu):
    rng = np.random.default_rng(44)
    B, gamma, V = 16, 5, 30000
    t, d = synth.make_logits(rng, B, gamma, V, 3.0, 0.5, boost_count=20)
    T = np.where(np.arange(B) % 4 == 3, 0.0, 0.8).astype(np.float32)
    caps = rng.integers(0, gamma + 2, size=B).astype(np.int32)
    prm = _prm(B, T, 40, 0.9, caps)
    tf = t
    toks = oracle.sample_draft_tokens(d, T, 40, 0.9, 3)
    eos = int(np.bincount(toks.ravel()).argmax())
    for e in (-1, eos):
        out, orc, toks2, tf2, df2 = run_trunc(torch.from_numpy(t), torch.from_numpy(d), prm, 8,
                                              tokens=toks, eos=e)
        check(out, orc, toks2, tf2, df2, prm, max_tol=0.1)


def _no_overflow(out):
    f = out["row_flags"].cpu().numpy()
    assert not (f & (sv.FLAG_CAND_OVERFLOW | sv.FLAG_UNSUPPORTED)).any()


@pytest.mark.parametrize("top_p", [0.9, 0.95])
def test_top_p_alone_flat_rows_full_vocab(gpu, top_p):
    """Top-p without top-k on flat rows (sigma 0.1, V=152064, bf16, T=1): the
    kept set holds most of the vocabulary, far more than the candidates, and
    comes from the exact whole-row truncation; parity with the oracle."""
    rng = np.random.default_rng(int(top_p * 1000))
    B, gamma, V = 8, 3, 152064
    t, d = synth.make_logits(rng, B, gamma, V, 0.1, 0.05)
    tt, dd = torch.from_numpy(t).to(torch.bfloat16), torch.from_numpy(d).to(torch.bfloat16)
    prm = _prm(B, 1.0, 0, top_p)
    out, orc, toks, tf, df = run_trunc(tt, dd, prm, 0xF1A7, max_top_k=64)
    rep = check(out, orc, toks, tf, df, prm, max_tol=0.1,
                workload=f"top-p {top_p} alone, flat rows sigma 0.1, B=8 gamma=3 V=152064 bf16")
    assert rep.value_checks > 0
    _no_overflow(out)


def _tied_rows(rng, B, gamma, V):
    """Rows whose top-k threshold sits in a huge tie: b % 3 == 0 constant rows
    (every chunk's candidate list overflows), b % 3 == 1 thirty entries at 3
    and 3000 at 2 over N(0, 0.3) (more tied candidates than LDS holds),
    b % 3 == 2 ordinary rows; draft rows the target's with a few entries
    moved, so that the accept tests see p != q."""
    t = (rng.standard_normal((B, gamma + 1, V)) * 0.3).astype(np.float32)
    for b in range(B):
        for i in range(gamma + 1):
            if b % 3 == 0:
                t[b, i] = 0.5
            elif b % 3 == 1:
                ids = rng.choice(V, size=3030, replace=False)
                t[b, i, ids[:30]] = 3.0
                t[b, i, ids[30:]] = 2.0
            else:
                t[b, i, rng.choice(V, size=20, replace=False)] += 4.0
    d = t[:, :gamma].copy()
    for b in range(B):
        for i in range(gamma):
            d[b, i, rng.choice(V, size=200, replace=False)] += 1.0
    return t, d


@pytest.mark.parametrize("k,p", [(50, 1.0), (50, 0.8), (0, 0.5)])
def test_heavy_ties_full_vocab(gpu, k, p):
    """Ties at the threshold beyond every candidate buffer (V=152064, bf16):
    constant rows, a 3000-way tie, ordinary rows in one batch."""
    rng = np.random.default_rng(17 + k)
    B, gamma, V = 6, 2, 152064
    t, d = _tied_rows(rng, B, gamma, V)
    tt, dd = torch.from_numpy(t).to(torch.bfloat16), torch.from_numpy(d).to(torch.bfloat16)
    prm = _prm(B, 1.0, k, p)
    out, orc, toks, tf, df = run_trunc(tt, dd, prm, 0x71E5 + k, max_top_k=64)
    check(out, orc, toks, tf, df, prm, max_tol=0.2,
          workload=f"heavy ties top-k {k} top-p {p}, B=6 gamma=2 V=152064 bf16")
    _no_overflow(out)


@pytest.mark.parametrize("k,p", [(100, 1.0), (2000, 0.9), (5000, 1.0), (17, 0.95)])
def test_top_k_beyond_max_top_k(gpu, k, p):
    """top_k above the handle's max_top_k (16): the rows are truncated
    exactly over the whole row instead of being refused."""
    rng = np.random.default_rng(300 + k)
    B, gamma, V = 8, 3, 40000
    t, d = synth.make_logits(rng, B, gamma, V, 2.0, 0.5, boost_count=20)
    tt, dd = torch.from_numpy(t).to(torch.bfloat16), torch.from_numpy(d).to(torch.bfloat16)
    prm = _prm(B, 0.8, k, p)
    out, orc, toks, tf, df = run_trunc(tt, dd, prm, 0xB16 + k, max_top_k=16)
    check(out, orc, toks, tf, df, prm, max_tol=0.2,
          workload=f"top-k {k} > max_top_k 16, top-p {p}, B=8 gamma=3 V=40000 bf16")
    _no_overflow(out)


def test_exact_truncation_f32_rows(gpu):
    """The exact truncation on float32 keys (four radix passes): top-p alone on
    flat rows and a constant row, ragged V."""
    rng = np.random.default_rng(404)
    B, gamma, V = 6, 2, 50001
    t, d = synth.make_logits(rng, B, gamma, V, 0.2, 0.1)
    t[0] = 1.25
    prm = _prm(B, 0.9, 0, 0.9)
    out, orc, toks, tf, df = run_trunc(torch.from_numpy(t), torch.from_numpy(d), prm, 0xF32, max_top_k=32)
    check(out, orc, toks, tf, df, prm, max_tol=0.2)
    _no_overflow(out)


def test_handle_without_truncation_workspace(gpu):
    rng = np.random.default_rng(3)
    B, gamma, V = 4, 2, 1000
    t, d = synth.make_logits(rng, B, gamma, V, 2.0, 0.5)
    toks = d.argmax(-1).astype(np.int32)
    T = np.array([1.0, 1.0, 0.0, 1.0], np.float32)
    k = np.array([10, 0, 10, 0], np.int32)
    with sv.Verifier(B, gamma, V, max_top_k=0) as v:
        out = v.verify_sample(torch.from_numpy(t).cuda(), torch.from_numpy(d).cuda(),
                              torch.from_numpy(toks).cuda(), sv.make_row_params(B, T, k, 1.0), 3)
        torch.cuda.synchronize()
    f = out["row_flags"].cpu().numpy()
    assert f[0] & sv.FLAG_UNSUPPORTED and out["num_emitted"][0].item() == 0
    assert not f[1] & sv.FLAG_UNSUPPORTED and out["num_emitted"][1].item() >= 1
    assert not f[2] & sv.FLAG_UNSUPPORTED                    # greedy ignores top-k
    assert not f[3] & sv.FLAG_UNSUPPORTED


def test_truncated_draft_sampling_distribution(gpu):
    """Emitted tokens follow the truncated target distribution (chi-square),
    on 20,000 broadcast rounds of one small truncated pair."""
    from scipy import stats
    rng = np.random.default_rng(12)
    V = 64
    t = (rng.standard_normal((1, 2, V)) * 2).astype(np.float32)
    d = (t[:, :1] + rng.standard_normal((1, 1, V))).astype(np.float32)
    R = 20000
    tt = torch.from_numpy(t).expand(R, -1, -1)
    dd = torch.from_numpy(d).expand(R, -1, -1)
    prm = _prm(R, 1.0, 12, 0.85)
    toks = oracle.sample_draft_tokens(dd.numpy(), 1.0, 12, 0.85, 5)
    with sv.Verifier(R, 1, V, max_top_k=16) as v:
        out = v.verify_sample(torch.from_numpy(t).cuda().expand(R, -1, -1),
                              torch.from_numpy(d).cuda().expand(R, -1, -1),
                              torch.from_numpy(toks).cuda(), sv.make_row_params(R, 1.0, 12, 0.85), 6)
        torch.cuda.synchronize()
    first = out["out_tokens"][:, 0].cpu().numpy()
    P = oracle.process_row(t[0, 0], 1.0, 12, 0.85).probs
    keep = P > 0
    assert set(np.unique(first)) <= set(np.nonzero(keep)[0])
    counts = np.bincount(first, minlength=V)[keep]
    assert stats.chisquare(counts, P[keep] * R).pvalue > 1e-3
