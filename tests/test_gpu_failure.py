"""Failure handling on the GPU: bounded waits that give up.

The kernels' waits for words other workgroups publish are bounded; a wait
that gives up flags its row INTERNAL, and the outputs of such a row are not
valid.  Here the limit is lowered from the host to a single poll
(specv_debug_set_wait_limit), so that waits give up wherever a word is not
out yet at the first look.  Every launch must still end normally; every
row must carry INTERNAL or match the oracle (the rows are classified one by
one, so a row that lost its draw and was not flagged would fail); and once
the limit is restored, calls on the same handle are exact again.  Handles
without truncation workspace only (the verify kernel without the
truncation steps, and the draft sampler's untruncated rows).
"""

import numpy as np
import pytest
import torch

import oracle
import synth
import speculative_decoding_verification_sampling_amd as sv
from parity import compare, compare_draft

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    sv.load_library()
    return torch.device("cuda:0")


@pytest.fixture
def one_poll(gpu):
    """The wait limit at one poll for the test's body, restored after it."""
    sv.debug_set_wait_limit(1)
    try:
        yield
    finally:
        sv.debug_set_wait_limit(0)


def _rows(d, keep, B):
    """Rows ``keep`` of a B-row output or oracle dict (per-row arrays, lists)."""
    out = {}
    for k, v in d.items():
        if isinstance(v, torch.Tensor) and v.dim() >= 1 and v.shape[0] == B:
            out[k] = v.cpu()[keep]
        elif isinstance(v, np.ndarray) and v.ndim >= 1 and v.shape[0] == B:
            out[k] = v[keep]
        elif isinstance(v, list) and len(v) == B:
            out[k] = [v[i] for i in keep]
        else:
            out[k] = v
    return out


def _batch(seed, B=16, gamma=4, V=50001):
    rng = np.random.default_rng(seed)
    t, d = synth.make_logits(rng, B, gamma, V, 3.0, 1.0, boost_count=20)
    T = np.where(np.arange(B) % 4 == 3, 0.0, 0.8).astype(np.float32)      # a greedy row in four
    caps = np.where(np.arange(B) % 5 == 4, 2, 0).astype(np.int32)
    toks = oracle.sample_draft_tokens(d, 1.0, 0, 1.0, seed + 7)
    return t, d, toks, T, caps


def _verify(v, t, d, toks, T, caps, seed, step):
    rp = sv.make_row_params(t.shape[0], T, 0, 1.0, caps)
    out = v.verify_sample(torch.from_numpy(t).to(torch.bfloat16).cuda(),
                          torch.from_numpy(d).to(torch.bfloat16).cuda(),
                          torch.from_numpy(toks).cuda(), rp, seed, step, diag=True)
    torch.cuda.synchronize()
    return out


def test_verify_waits_that_give_up_flag_their_rows(gpu, one_poll):
    B, gamma, V = 16, 4, 50001
    flagged = 0
    with sv.Verifier(B, gamma, V) as v:
        for r in range(3):
            t, d, toks, T, caps = _batch(100 + r)
            tb = torch.from_numpy(t).to(torch.bfloat16).float().numpy()
            db = torch.from_numpy(d).to(torch.bfloat16).float().numpy()
            orc = oracle.verify_sample(tb, db, toks, T, 0, 1.0, caps, 5 + r, 3)
            out = _verify(v, t, d, toks, T, caps, 5 + r, 3)
            flags = out["row_flags"].cpu().numpy()
            internal = (flags & sv.FLAG_INTERNAL) != 0
            flagged += int(internal.sum())
            keep = np.nonzero(~internal)[0]
            prm = {"temperature": T[keep], "top_k": np.zeros(len(keep), np.int32),
                   "top_p": np.ones(len(keep), np.float32)}
            rep = compare(_rows(out, keep, B), _rows(orc, keep, B), toks[keep], tb[keep], db[keep], prm)
            print(f"call {r}: {int(internal.sum())} of {B} rows INTERNAL; others: {rep.summary()}")
            rep.assert_ok(0.5)
    # one poll is far too few for the hand-offs of a 7-chunk row
    assert flagged > 0


def test_calls_after_the_limit_is_restored_are_exact(gpu):
    B, gamma, V = 16, 4, 50001
    t, d, toks, T, caps = _batch(200)
    tb = torch.from_numpy(t).to(torch.bfloat16).float().numpy()
    db = torch.from_numpy(d).to(torch.bfloat16).float().numpy()
    orc = oracle.verify_sample(tb, db, toks, T, 0, 1.0, caps, 11, 4)
    with sv.Verifier(B, gamma, V) as v:
        sv.debug_set_wait_limit(1)
        try:
            _verify(v, t, d, toks, T, caps, 11, 4)
        finally:
            sv.debug_set_wait_limit(0)
        out = _verify(v, t, d, toks, T, caps, 11, 4)
    assert ((out["row_flags"].cpu().numpy() & sv.FLAG_INTERNAL) == 0).all()
    rep = compare(out, orc, toks, tb, db, {"temperature": T, "top_k": np.zeros(B, np.int32),
                                            "top_p": np.ones(B, np.float32)})
    print(rep.summary())
    rep.assert_ok(0.5)


def test_draft_sampler_waits_that_give_up_flag_their_rows(gpu, one_poll):
    B, gamma, V = 16, 3, 50001
    rng = np.random.default_rng(300)
    _, d = synth.make_logits(rng, B, gamma, V, 3.0, 1.0, boost_count=20)
    T = np.where(np.arange(B) % 4 == 3, 0.0, 0.9).astype(np.float32)
    db = torch.from_numpy(d).to(torch.bfloat16)
    with sv.Verifier(B, gamma, V) as v:
        drawn = v.sample_draft(db.cuda(), sv.make_row_params(B, T), seed=17, step=2)
        torch.cuda.synchronize()
    tok = drawn["tokens"].cpu().numpy()
    stats = drawn["stats"].cpu().numpy()
    sflags = stats.view(np.int32)[..., 3]
    internal = (sflags & sv.FLAG_INTERNAL) != 0
    print(f"{int(internal.sum())} of {tok.size} draws INTERNAL")
    assert internal.any()
    # every draw that did not give up is the oracle's
    skip = sorted({int(b) for b in np.nonzero(internal.any(axis=1))[0]})
    rep = compare_draft(tok, stats, db.float().numpy(), T, 17, 2, skip_rows=skip)
    print(rep.summary())
    rep.assert_ok(0.5)
