"""GPU parity of verification against deterministic drafts
(``specv_verify_point_mass``: q_i is the point mass on d_i, no draft logits)
with the oracle's ``verify_point_mass``, to the bar of ``parity.py``.

The drafts stand in for n-gram / prompt-lookup proposals: the argmax of a
noisy copy of the target (the workloads' draft logits), a guess that is
often but not always the target's favourite.  Covered: the tiny workload
over 20,000 rounds with a chi-square test of the emitted tokens, the
serving batch at full size, the truncated workload at full size, greedy
rows with caps and EOS, ragged vocabularies, and the degenerate rows.
"""

import numpy as np
import pytest
import torch
from scipy import stats

import oracle
import synth
import speculative_decoding_verification_sampling_amd as sv
from parity import compare

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    sv.load_library()          # raises loudly when the HIP library is missing
    return torch.device("cuda:0")


def _prm(B, T, k=0, p=1.0, cap=0):
    b = lambda x, dt: np.broadcast_to(np.asarray(x, dt), (B,)).copy()
    return {"temperature": b(T, np.float32), "top_k": b(k, np.int32), "top_p": b(p, np.float32),
            "max_new_tokens": b(cap, np.int32)}


def run_pm(v, target, tokens, prm, seed, step=0, eos=-1, target_dev=None):
    """target: CPU tensor (float32 or bfloat16); tokens: int numpy [B, gamma]."""
    B = target.shape[0]
    tdev = target_dev if target_dev is not None else target.cuda()
    tok = torch.from_numpy(np.ascontiguousarray(tokens, np.int32)).cuda()
    rp = sv.make_row_params(B, prm["temperature"], prm["top_k"], prm["top_p"],
                            prm["max_new_tokens"])
    out = v.verify_point_mass(tdev, tok, rp, seed, step, eos, diag=True)
    torch.cuda.synchronize()
    tf = target.to(torch.float32).numpy()
    orc = oracle.verify_point_mass(tf, tokens, prm["temperature"], prm["top_k"], prm["top_p"],
                                   prm["max_new_tokens"], seed, step, eos, keep_weights=True)
    return out, orc, tf


def check(out, orc, tokens, tf, prm, max_tol=0.02):
    rep = compare(out, orc, tokens, tf, None, prm)
    print(rep.summary())
    rep.assert_ok(max_tol)
    return rep


def _lookup_tokens(w):
    return w.draft.to(torch.float32).numpy().argmax(-1).astype(np.int32)


def test_point_mass_tiny_rounds(gpu):
    """Tiny workload (V=32, gamma=4, fp32), 20,000 broadcast rounds with one
    fixed deterministic draft: parity, q_at_draft == 1, and at every
    position the emitted token follows p_i (chi-square)."""
    w = synth.tiny()
    R = 20000
    toks1 = _lookup_tokens(w)
    toks = np.repeat(toks1, R, axis=0)
    tgt = w.target.expand(R, -1, -1)
    prm = _prm(R, 1.0)
    with sv.Verifier(R, 4, 32) as v:
        out, orc, tf = run_pm(v, tgt, toks, prm, w.seed, target_dev=w.target.cuda().expand(R, -1, -1))
    check(out, orc, toks, tf, prm)
    qa = out["q_at_draft"].cpu().numpy()
    tested = ~np.isnan(qa)
    assert tested.any() and (qa[tested] == 1.0).all()
    em = out["num_emitted"].cpu().numpy()
    ot = out["out_tokens"].cpu().numpy()
    z = w.target_f32()[0].astype(np.float64)
    for i in range(5):
        P = np.exp(z[i] - z[i].max())
        P /= P.sum()
        reach = em > i
        counts = np.bincount(ot[reach, i], minlength=32)
        keep = P * reach.sum() >= 5
        obs, exp = counts[keep], P[keep] * reach.sum()
        if (~keep).any():
            obs = np.append(obs, counts[~keep].sum())
            exp = np.append(exp, P[~keep].sum() * reach.sum())
        assert stats.chisquare(obs, exp * obs.sum() / exp.sum()).pvalue > 1e-3


def test_point_mass_serving_batch_full_size(gpu):
    """B=64, gamma=5, V=128256, bf16, T=0.7 at full size, two steps."""
    w = synth.serving_batch()
    toks = _lookup_tokens(w)
    prm = _prm(w.B, w.temperature)
    with sv.Verifier(w.B, w.gamma, w.V) as v:
        out, orc, tf = run_pm(v, w.target, toks, prm, w.seed)
        rep = check(out, orc, toks, tf, prm)
        out2, orc2, _ = run_pm(v, w.target, toks, prm, w.seed, step=1)
        check(out2, orc2, toks, tf, prm)
    assert rep.value_checks > w.B


def test_point_mass_truncated_full_size(gpu):
    """B=32, gamma=5, V=152064, bf16, T=0.7, top-k 50, top-p 0.9 on p (the
    truncation-capable kernel); some drafts fall outside p's kept set."""
    w = synth.truncated()
    toks = _lookup_tokens(w)
    prm = _prm(w.B, w.temperature, w.top_k, w.top_p)
    with sv.Verifier(w.B, w.gamma, w.V, max_top_k=64) as v:
        out, orc, tf = run_pm(v, w.target, toks, prm, w.seed)
    check(out, orc, toks, tf, prm, max_tol=0.05)


def test_point_mass_greedy_rows_caps_eos(gpu):
    """Even rows stochastic, odd rows greedy; caps U{0..6}, an EOS id that
    some drafts hit; V=32000 fp32."""
    rng = np.random.default_rng(21)
    B, gamma, V = 48, 6, 32000
    t, d = synth.make_logits(rng, B, gamma, V, 3.0, 1.0, boost_count=20)
    toks = d.argmax(-1).astype(np.int32)
    eos = int(toks[3, 2])
    T = np.where(np.arange(B) % 2 == 0, 1.0, 0.0)
    cap = rng.integers(0, 7, B)
    prm = _prm(B, T, 0, 1.0, cap)
    with sv.Verifier(B, gamma, V) as v:
        out, orc, tf = run_pm(v, torch.from_numpy(t), toks, prm, 99, eos=eos)
    check(out, orc, toks, tf, prm, max_tol=0.1)
    em = out["num_emitted"].cpu().numpy()
    assert (em[cap >= 1] <= cap[cap >= 1]).all()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("V,gamma", [(2, 1), (7, 3), (8193, 2), (16385, 4), (40000, 0)])
def test_point_mass_ragged_vocab(gpu, dtype, V, gamma):
    rng = np.random.default_rng(V * 7 + gamma)
    B = 6
    t, d = synth.make_logits(rng, B, gamma, V, 2.0, 0.7, boost_count=min(20, V))
    tt = torch.from_numpy(t)
    if dtype == "bf16":
        tt = tt.to(torch.bfloat16)
    toks = d.argmax(-1).astype(np.int32) if gamma > 0 else np.zeros((B, 0), np.int32)
    prm = _prm(B, 0.9)
    with sv.Verifier(B, max(gamma, 1), V) as v:
        out, orc, tf = run_pm(v, tt, toks, prm, 4321)
    check(out, orc, toks, tf, prm, max_tol=0.2)


def test_point_mass_degenerate_rows(gpu):
    """Token out of range, NaN and all -inf rows, a draft with p(d) = 0
    (always rejected; the correction is then p itself), p(d) = 1 (always
    accepted)."""
    rng = np.random.default_rng(31)
    B, gamma, V = 8, 3, 9000
    t = rng.standard_normal((B, gamma + 1, V)).astype(np.float32)
    toks = t[:, :gamma].argmax(-1).astype(np.int32)
    toks[0, 1] = V                       # out of range
    t[1, 0, 4] = np.nan                  # NaN in a consulted row
    t[2, 0] = -np.inf                    # no finite value
    toks[3, 0] = 5
    t[3, 0, 5] = -np.inf                 # p(d) = 0: always rejected
    t[4, :gamma] = -np.inf               # p(d) = 1 at every test: all accepted
    for i in range(gamma):
        t[4, i, toks[4, i]] = 0.0
    prm = _prm(B, 1.0)
    with sv.Verifier(B, gamma, V) as v:
        out, orc, tf = run_pm(v, torch.from_numpy(t), toks, prm, 8)
    check(out, orc, toks, tf, prm, max_tol=0.2)
    f = out["row_flags"].cpu().numpy()
    acc = out["num_accepted"].cpu().numpy()
    assert f[0] & sv.FLAG_TOKEN_OOR
    assert f[1] & sv.FLAG_NONFINITE_ROW and f[2] & sv.FLAG_NONFINITE_ROW
    assert acc[3] == 0 and out["out_tokens"][3, 0].item() != 5
    assert acc[4] == gamma
