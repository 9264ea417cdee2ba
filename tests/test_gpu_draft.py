"""GPU parity of the draft-side sampler (``specv_sample_draft``) with the
oracle's draw and row statistics, and of verification that reuses those
statistics (``specv_verify_sample_qstats``) with ``specv_verify_sample``
(bit for bit) and the oracle.

Covered: the tiny workload over 20,000 rows with a chi-square test of the
draws, the serving batch at full size (all positions in one call, and one
position per call), greedy rows, ragged vocabularies and unaligned rows,
gamma at its maximum, rows that define no draw, truncated rows (including
rows only the exact whole-row truncation settles, verified from their draft
rows), and statistics that mark a row non-finite.
"""

import numpy as np
import pytest
import torch
from scipy import stats

import oracle
import synth
import speculative_decoding_verification_sampling_amd as sv
from parity import compare, compare_draft

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


def _rp(prm):
    return sv.make_row_params(len(prm["temperature"]), prm["temperature"], prm["top_k"], prm["top_p"],
                              prm["max_new_tokens"])


def _draw(v, draft_dev, prm, seed, step=0, pos0=0, out=None):
    o = v.sample_draft(draft_dev, _rp(prm), seed, step, pos0, out=out)
    torch.cuda.synchronize()
    return o


def _check_draft(o, draft_f32, prm, seed, step=0, pos0=0, max_tol=0.02, skip_rows=()):
    n = draft_f32.shape[1]
    sl = slice(pos0, pos0 + n)
    rep = compare_draft(o["tokens"][:, sl], o["stats"][:, sl], draft_f32, prm["temperature"], seed,
                        step, pos0, prm["top_k"], prm["top_p"], skip_rows=skip_rows)
    print(rep.summary())
    rep.assert_ok(max_tol)
    return rep


def test_draft_tiny_rows_chi2(gpu):
    """Tiny draft rows (V=32, fp32, T=1), 20,000 broadcast rows: parity with
    the oracle and, per position, the draws follow softmax(z) (chi-square)."""
    w = synth.tiny()
    R = 20000
    d = w.draft.expand(R, -1, -1)
    prm = _prm(R, 1.0)
    with sv.Verifier(R, 4, 32) as v:
        o = _draw(v, w.draft.cuda().expand(R, -1, -1), prm, 0xD1A)
    _check_draft(o, d.numpy(), prm, 0xD1A)
    toks = o["tokens"].cpu().numpy()
    for i in range(4):
        P = torch.softmax(torch.from_numpy(w.draft_f32()[0, i].astype(np.float64)), 0).numpy()
        counts = np.bincount(toks[:, i], minlength=32)
        keep = P * R >= 5
        obs, exp = counts[keep], P[keep] * R
        if (~keep).any():
            obs = np.append(obs, counts[~keep].sum())
            exp = np.append(exp, P[~keep].sum() * R)
        assert stats.chisquare(obs, exp * obs.sum() / exp.sum()).pvalue > 1e-3, i


def test_draft_serving_batch_full_size(gpu):
    """B=64, 5 positions, V=128256, bf16, T=0.7: one call for all positions,
    then one position per call into the same outputs: identical."""
    w = synth.serving_batch()
    prm = _prm(w.B, w.temperature)
    dd = w.draft.cuda()
    with sv.Verifier(w.B, w.gamma, w.V) as v:
        o = _draw(v, dd, prm, w.seed, step=3)
        _check_draft(o, w.draft_f32(), prm, w.seed, step=3)
        o2 = {"tokens": torch.full((w.B, w.gamma), -7, dtype=torch.int32, device=gpu),
              "stats": torch.zeros(w.B, w.gamma, 4, device=gpu)}
        for i in range(w.gamma):
            _draw(v, dd[:, i:i + 1], prm, w.seed, step=3, pos0=i, out=o2)
    assert torch.equal(o["tokens"], o2["tokens"])
    assert torch.equal(o["stats"].view(torch.int32), o2["stats"].view(torch.int32))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("V,n,aligned", [(1, 2, True), (7, 3, True), (8193, 2, True),
                                         (16385, 4, False), (40000, 3, False), (300, 31, True)])
def test_draft_greedy_ragged(gpu, dtype, V, n, aligned):
    """Even rows T=0.9, odd rows greedy; ragged vocabularies (a partial last
    chunk, a partial 16-byte group), rows that do not start 16-byte aligned,
    and n up to the largest gamma."""
    rng = np.random.default_rng(V * 3 + n)
    B = 6
    _, d = synth.make_logits(rng, B, n, V + 1, 2.0, 0.7, boost_count=min(20, V))
    dt = torch.from_numpy(d)
    if dtype == "bf16":
        dt = dt.to(torch.bfloat16)
    dv = dt.cuda()
    dv = dv[:, :, :V] if aligned else dv[:, :, 1:]          # unaligned rows start one entry in
    df = (dt[:, :, :V] if aligned else dt[:, :, 1:]).float().numpy()
    T = np.where(np.arange(B) % 2 == 0, 0.9, 0.0)
    prm = _prm(B, T)
    with sv.Verifier(B, max(n, 1), V) as v:
        o = _draw(v, dv, prm, 4321 + V)
    _check_draft(o, df, prm, 4321 + V, max_tol=0.2)


def test_draft_rows_without_a_draw(gpu):
    """NaN, +inf and all -inf rows give -1 and NONFINITE_ROW (greedy rows
    too); top-k / top-p rows give -1 and UNSUPPORTED on a handle without
    truncation workspace, and draw on one with it; other rows draw."""
    rng = np.random.default_rng(8)
    B, n, V = 8, 2, 9000
    d = rng.standard_normal((B, n, V)).astype(np.float32)
    d[0, 1, 17] = np.nan
    d[1, 0, 4] = np.inf
    d[2, 1] = -np.inf
    d[3, 0, 5] = np.nan                                     # greedy row
    T = np.array([1, 1, 1, 0, 1, 1, 0.8, 1.2], np.float32)
    k = np.array([0, 0, 0, 0, 5, 0, 0, 0], np.int32)
    p = np.array([1, 1, 1, 1, 1, 0.9, 1, 1], np.float32)
    prm = {"temperature": T, "top_k": k, "top_p": p, "max_new_tokens": np.zeros(B, np.int32)}
    with sv.Verifier(B, n, V) as v:
        o = _draw(v, torch.from_numpy(d).cuda(), prm, 5)
    tok, fl = o["tokens"].cpu().numpy(), o["flags"].cpu().numpy()
    st = o["stats"].cpu().numpy()[..., :3]
    for (b, i) in [(0, 1), (1, 0), (2, 1), (3, 0)]:
        assert tok[b, i] == -1 and fl[b, i] == sv.FLAG_NONFINITE_ROW and np.isnan(st[b, i]).all()
    for b in (4, 5):
        assert (tok[b] == -1).all() and (fl[b] == sv.FLAG_UNSUPPORTED).all() and np.isnan(st[b]).all()
    # every other row against the oracle (same row indices, so same uniforms)
    _check_draft(o, d, prm, 5, max_tol=0.2, skip_rows=(4, 5))
    # with truncation workspace the top-k row draws too, and so does top-p
    # alone on this flat row, whose kept set needs far more than max_top_k
    # candidates per chunk (the exact whole-row truncation)
    with sv.Verifier(B, n, V, max_top_k=16) as v:
        o = _draw(v, torch.from_numpy(d).cuda(), prm, 5)
    _check_draft(o, d, prm, 5, max_tol=0.2)
    assert (o["tokens"][5] >= 0).all() and not (o["flags"][5] & sv.FLAG_CAND_OVERFLOW).any()


@pytest.mark.parametrize("k,p", [(0, 0.9), (0, 0.95), (50, 1.0), (300, 0.9)])
def test_draft_exact_truncation_full_vocab(gpu, k, p):
    """V=152064 bf16 draft rows the candidates cannot settle: flat rows
    (sigma 0.1) with top-p alone, a constant row, a 3000-way tie at the
    top-k threshold, top_k above max_top_k (64); draws and statistics match
    the oracle, and verification from those statistics matches the
    verification that re-reads the draft rows, bit for bit."""
    rng = np.random.default_rng(900 + k + int(100 * p))
    B, n, V = 6, 3, 152064
    d = (rng.standard_normal((B, n, V)) * 0.1).astype(np.float32)
    d[0] = 0.25
    ids = rng.choice(V, size=3030, replace=False)
    d[1, :, ids[:30]] = 3.0
    d[1, :, ids[30:]] = 2.0
    dt = torch.from_numpy(d).to(torch.bfloat16)
    df = dt.float().numpy()
    prm = _prm(B, 1.0, k, p)
    with sv.Verifier(B, n, V, max_top_k=64) as v:
        o = _draw(v, dt.cuda(), prm, 0xE7 + k)
        _check_draft(o, df, prm, 0xE7 + k, max_tol=0.2)
        fl = o["flags"].cpu().numpy()
        assert (o["tokens"].cpu().numpy() >= 0).all()
        assert not (fl & (sv.FLAG_CAND_OVERFLOW | sv.FLAG_UNSUPPORTED)).any()
        t = (df[:, :1] + 0.05 * rng.standard_normal((B, n + 1, V))).astype(np.float32)
        tt = torch.from_numpy(t).to(torch.bfloat16).cuda()
        _verify_both(v, tt, dt.cuda(), o["tokens"], o["stats"], prm, 0xE8 + k)


def test_draft_truncated_full_size(gpu):
    """B=32, 5 positions, V=152064, bf16, T=0.7, top-k 50, top-p 0.9: the
    kept set by the verify kernel's row merge, the draw over it."""
    w = synth.truncated()
    prm = _prm(w.B, w.temperature, w.top_k, w.top_p)
    with sv.Verifier(w.B, w.gamma, w.V, max_top_k=64) as v:
        o = _draw(v, w.draft.cuda(), prm, 0x7A, step=2)
    _check_draft(o, w.draft_f32(), prm, 0x7A, step=2, max_tol=0.05)
    th = o["stats"][..., 2].cpu().numpy()
    assert np.isfinite(th).all()                    # truncated rows carry their threshold


@pytest.mark.parametrize("k,p", [(5, 1.0), (0, 0.8), (12, 0.9)])
def test_draft_truncated_tiny_chi2(gpu, k, p):
    """V=32 rows, 20,000 broadcast copies: the draws follow the truncated q."""
    w = synth.tiny()
    R = 20000
    prm = _prm(R, 1.0, k, p)
    with sv.Verifier(R, 4, 32, max_top_k=16) as v:
        o = _draw(v, w.draft.cuda().expand(R, -1, -1), prm, 0xD1B + k)
    _check_draft(o, w.draft.expand(R, -1, -1).numpy(), prm, 0xD1B + k)
    toks = o["tokens"].cpu().numpy()
    for i in range(4):
        q = oracle.process_row(w.draft_f32()[0, i], 1.0, k, p).probs
        counts = np.bincount(toks[:, i], minlength=32)
        assert counts[q == 0].sum() == 0
        keep = q * R >= 5
        obs, exp = counts[keep], q[keep] * R
        if (~keep & (q > 0)).any():
            obs = np.append(obs, counts[~keep & (q > 0)].sum())
            exp = np.append(exp, q[~keep & (q > 0)].sum() * R)
        assert stats.chisquare(obs, exp * obs.sum() / exp.sum()).pvalue > 1e-3, i


def _verify_both(v, w_t, w_d, tokens, stats_, prm, seed, step=0):
    rp = _rp(prm)
    tok = torch.from_numpy(np.ascontiguousarray(tokens, np.int32)).cuda() if isinstance(tokens, np.ndarray) \
        else tokens
    a = v.verify_sample(w_t, w_d, tok, rp, seed, step, diag=True)
    b = v.verify_sample_qstats(w_t, w_d, stats_, tok, rp, seed, step, diag=True)
    torch.cuda.synchronize()
    for key in ("num_accepted", "out_tokens", "num_emitted", "row_flags"):
        assert torch.equal(a[key], b[key]), key
    for key in ("p_at_draft", "q_at_draft", "residual_sum"):
        x, y = a[key].cpu().numpy(), b[key].cpu().numpy()
        assert np.array_equal(x, y, equal_nan=True), key
    return b


def test_qstats_verify_serving_batch_bitwise(gpu):
    """The drafter's draws and statistics from the sampler, then both verify
    entry points: bit-identical outputs, and parity with the oracle."""
    w = synth.serving_batch()
    prm = _prm(w.B, w.temperature)
    t, d = w.target.cuda(), w.draft.cuda()
    with sv.Verifier(w.B, w.gamma, w.V) as v:
        for step in range(2):
            o = _draw(v, d, prm, w.seed + 1, step)
            out = _verify_both(v, t, d, o["tokens"], o["stats"], prm, w.seed, step)
            toks = o["tokens"].cpu().numpy()
            orc = oracle.verify_sample(w.target_f32(), w.draft_f32(), toks, w.temperature, 0, 1.0, 0,
                                       w.seed, step, keep_weights=True)
            rep = compare(out, orc, toks, w.target_f32(), w.draft_f32(), prm)
            print(rep.summary())
            rep.assert_ok()


def test_qstats_verify_greedy_truncated_mixed(gpu):
    """Rows of every mode in one call (handle with truncation): greedy rows
    ignore the statistics; truncated rows take their kept sets from them."""
    rng = np.random.default_rng(41)
    B, gamma, V = 24, 4, 50000
    t, d = synth.make_logits(rng, B, gamma, V, 3.0, 1.0, boost_count=20)
    tt, dd = torch.from_numpy(t).to(torch.bfloat16), torch.from_numpy(d).to(torch.bfloat16)
    mode = np.arange(B) % 3                                  # 0 sample, 1 greedy, 2 truncated
    T = np.where(mode == 1, 0.0, 0.8).astype(np.float32)
    k = np.where(mode == 2, 40, 0).astype(np.int32)
    p = np.where(mode == 2, 0.9, 1.0).astype(np.float32)
    cap = rng.integers(0, 6, B).astype(np.int32)
    prm = {"temperature": T, "top_k": k, "top_p": p, "max_new_tokens": cap}
    with sv.Verifier(B, gamma, V, max_top_k=64) as v:
        o = _draw(v, dd.cuda(), prm, 77)
        toks = o["tokens"].cpu().numpy()
        df = dd.float().numpy()
        assert (toks >= 0).all()
        out = _verify_both(v, tt.cuda(), dd.cuda(), toks, o["stats"], prm, 79)
    orc = oracle.verify_sample(tt.float().numpy(), df, toks, T, k, p, cap, 79, keep_weights=True)
    rep = compare(out, orc, toks, tt.float().numpy(), df, prm)
    print(rep.summary())
    rep.assert_ok(0.1)


def test_qstats_verify_truncated_full_size_bitwise(gpu):
    """The truncated workload (V=152064, top-k 50, top-p 0.9) through the
    sampler and both verify entry points: bit-identical, and oracle parity."""
    w = synth.truncated()
    prm = _prm(w.B, w.temperature, w.top_k, w.top_p)
    t, d = w.target.cuda(), w.draft.cuda()
    with sv.Verifier(w.B, w.gamma, w.V, max_top_k=64) as v:
        o = _draw(v, d, prm, 0x7B)
        out = _verify_both(v, t, d, o["tokens"], o["stats"], prm, w.seed)
    toks = o["tokens"].cpu().numpy()
    orc = oracle.verify_sample(w.target_f32(), w.draft_f32(), toks, w.temperature, w.top_k,
                               w.top_p, 0, w.seed, keep_weights=True)
    rep = compare(out, orc, toks, w.target_f32(), w.draft_f32(), prm)
    print(rep.summary())
    rep.assert_ok(0.05)


def test_qstats_verify_mixed_full_size_with_eos(gpu):
    """The mixed workload (B=256, gamma=8, V=128256: even rows T=1, odd rows
    greedy, caps 1..9) with an EOS id that some draws hit: the sampler's
    draws and records, both verify entry points bit-identical, oracle parity."""
    w = synth.mixed()
    prm = _prm(w.B, w.temperature, 0, 1.0, w.max_new_tokens)
    t, d = w.target.cuda(), w.draft.cuda()
    with sv.Verifier(w.B, w.gamma, w.V) as v:
        o = _draw(v, d, prm, 0x3C)
        toks = o["tokens"].cpu().numpy()
        eos = int(toks[0, 3])
        out = _verify_both(v, t, d, o["tokens"], o["stats"], prm, w.seed, step=1)
        rp = _rp(prm)
        a = v.verify_sample(t, d, o["tokens"], rp, w.seed, 1, eos)
        b = v.verify_sample_qstats(t, d, o["stats"], o["tokens"], rp, w.seed, 1, eos)
        torch.cuda.synchronize()
    for key in ("num_accepted", "out_tokens", "num_emitted", "row_flags"):
        assert torch.equal(a[key], b[key]), key
    _check_draft(o, w.draft_f32(), prm, 0x3C)
    orc = oracle.verify_sample(w.target_f32(), w.draft_f32(), toks, w.temperature, 0, 1.0,
                               w.max_new_tokens, w.seed, 1, eos, keep_weights=True)
    rep = compare(b, orc, toks, w.target_f32(), w.draft_f32(), prm)
    print(rep.summary())
    rep.assert_ok(0.05)
    em = b["num_emitted"].cpu().numpy()
    assert (em <= w.max_new_tokens).all()


def test_qstats_non_finite_statistics_mark_the_row(gpu):
    """A NaN statistic, a zero sum or a max of -inf makes the row emit
    nothing with NONFINITE_ROW; the other rows are unaffected."""
    w = synth.serving_batch(B=8, V=20000)
    prm = _prm(w.B, w.temperature)
    t, d = w.target.cuda(), w.draft.cuda()
    with sv.Verifier(w.B, w.gamma, w.V) as v:
        o = _draw(v, d, prm, 3)
        st = o["stats"].clone()
        st[1, 0, 1] = float("nan")
        st[2, 0, 1] = 0.0
        st[3, 0, 0] = float("-inf")
        rp = _rp(prm)
        good = v.verify_sample(t, d, o["tokens"], rp, 9)
        bad = v.verify_sample_qstats(t, d, st, o["tokens"], rp, 9)
        torch.cuda.synchronize()
    fl = bad["row_flags"].cpu().numpy()
    em = bad["num_emitted"].cpu().numpy()
    for b in (1, 2, 3):
        assert fl[b] & sv.FLAG_NONFINITE_ROW and em[b] == 0
    keep = [0, 4, 5, 6, 7]
    for key in ("num_accepted", "out_tokens", "num_emitted", "row_flags"):
        assert torch.equal(good[key][keep], bad[key][keep]), key


def test_sampler_argument_errors_and_offsets(gpu):
    """Status codes of specv_sample_draft / specv_verify_sample_qstats for
    bad arguments (through the C ABI directly), no-op calls, and a call
    that fills two middle columns of a wider output."""
    import ctypes
    lib = sv.load_library()
    B, n, V = 4, 2, 300
    d = torch.randn(B, 5, V, device="cuda")
    rp = _rp(_prm(B, 0.9))
    tok = torch.full((B, 5), -7, dtype=torch.int32, device="cuda")
    st = torch.zeros(B, 5, 4, device="cuda")
    with sv.Verifier(B, 5, V) as v:
        h = v._h
        call = lambda **kw: lib.specv_sample_draft(
            h, None, ctypes.c_void_p(kw.get("d", d).data_ptr()), d.stride(0), d.stride(1), 0,
            kw.get("B", B), kw.get("n", n), kw.get("V", V), kw.get("pos0", 0),
            ctypes.c_void_p(rp.data_ptr()), 1, 0, ctypes.c_void_p(tok.data_ptr()),
            ctypes.c_void_p(kw.get("st", st.data_ptr())), kw.get("stride", 5))
        assert call(stride=1) == 2                                   # pos0 + n > out_stride
        assert call(pos0=4) == 2
        assert call(n=6, stride=10) == 5                             # n above max(max_gamma, 1)
        assert call(B=5) == 5                                        # B above max_batch
        assert call(V=301) == 5                                      # V above max_vocab
        assert call(st=st.data_ptr() + 8) == 4                       # records 16-byte aligned
        assert call(n=0) == 0 and call(B=0) == 0                     # no-ops
        torch.cuda.synchronize()
        assert (tok == -7).all()
        # columns 2 and 3 of a width-5 output, positions 2 and 3 of the round
        o = {"tokens": tok, "stats": st}
        v.sample_draft(d[:, 2:4], rp, 1, 0, pos0=2, out=o)
        torch.cuda.synchronize()
        assert (tok[:, [0, 1, 4]] == -7).all() and (tok[:, 2:4] >= 0).all()
        ref = v.sample_draft(d, rp, 1, 0)
        torch.cuda.synchronize()
        assert torch.equal(ref["tokens"][:, 2:4], tok[:, 2:4])
        assert torch.equal(ref["stats"][:, 2:4].view(torch.int32), st[:, 2:4].view(torch.int32))
        # the statistics verify: a short stride and misaligned records are refused
        t = torch.randn(B, 3, V, device="cuda")
        toks = ref["tokens"][:, :2].contiguous()
        outs = [torch.zeros(B * 3, dtype=torch.int32, device="cuda") for _ in range(3)]
        ptr = lambda x: ctypes.c_void_p(x.data_ptr())
        args = lambda sp, ss: (h, None, ptr(t), t.stride(0), t.stride(1), ptr(d), d.stride(0),
                               d.stride(1), ctypes.c_void_p(sp), ss, 0, B, 2, V, ptr(toks), ptr(rp),
                               1, 0, -1, ptr(outs[0]), ptr(outs[1]), ptr(outs[2]), None, None)
        assert lib.specv_verify_sample_qstats(*args(ref["stats"].data_ptr(), 1)) == 2
        assert lib.specv_verify_sample_qstats(*args(ref["stats"].data_ptr() + 4, 5)) == 4
        assert lib.specv_verify_sample_qstats(*args(0, 5)) == 1
