"""GPU parity at the largest sizes the library accepts: V = 524,288 (64
chunks of 8192, every lane of the chunk-merging waves in use), gamma = 31
(the last accept bit of the row status word) and top_k = 1024, through the
draft sampler and every verify entry point, against the oracle.

Draft logits are a close copy of the target (noise 0.05) so that rounds run
deep and most of the 32 positions are consulted.
"""

import numpy as np
import pytest
import torch

import oracle
import synth
import speculative_decoding_verification_sampling_amd as sv
from parity import compare, compare_draft

pytestmark = pytest.mark.gpu

V_MAX = 524288
GAMMA_MAX = 31
TOPK_MAX = 1024


@pytest.fixture(scope="module")
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    sv.load_library()
    return torch.device("cuda:0")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_largest_vocabulary_and_gamma(gpu, dtype):
    rng = np.random.default_rng(4242 if dtype == "f32" else 4243)
    B = 3
    t, d = synth.make_logits(rng, B, GAMMA_MAX, V_MAX, 3.0, 0.05, boost_count=20)
    tt, dd = torch.from_numpy(t), torch.from_numpy(d)
    if dtype == "bf16":
        tt, dd = tt.to(torch.bfloat16), dd.to(torch.bfloat16)
    tf, df = tt.float().numpy(), dd.float().numpy()
    T = np.array([1.0, 0.0, 0.8], np.float32)
    k = np.array([0, 0, TOPK_MAX], np.int32)
    p = np.array([1.0, 1.0, 0.95], np.float32)
    cap = np.zeros(B, np.int32)
    prm = {"temperature": T, "top_k": k, "top_p": p, "max_new_tokens": cap}
    rp = sv.make_row_params(B, T, k, p, cap)
    td, ddv = tt.cuda(), dd.cuda()
    with sv.Verifier(B, GAMMA_MAX, V_MAX, max_top_k=TOPK_MAX) as v:
        drawn = v.sample_draft(ddv, rp, 7)
        torch.cuda.synchronize()
        rep = compare_draft(drawn["tokens"], drawn["stats"], df, T, 7, 0, 0, k, p)
        print("draw:", rep.summary())
        rep.assert_ok(0.1)
        tok = drawn["tokens"]
        a = v.verify_sample(td, ddv, tok, rp, 11, 0, -1, diag=True)
        b = v.verify_sample_qstats(td, ddv, drawn["stats"], tok, rp, 11, 0, -1, diag=True)
        pm = v.verify_point_mass(td, tok, rp, 11, 0, -1, diag=True)
        g = v.verify_greedy(td, tok)
        torch.cuda.synchronize()
    for key in ("num_accepted", "out_tokens", "num_emitted", "row_flags"):
        assert torch.equal(a[key], b[key]), key
    toks = tok.cpu().numpy()
    orc = oracle.verify_sample(tf, df, toks, T, k, p, cap, 11, keep_weights=True)
    rep = compare(a, orc, toks, tf, df, prm)
    print("verify:", rep.summary())
    rep.assert_ok(0.34)
    assert orc["num_accepted"].max() >= 8                 # the rounds do run deep
    orc_pm = oracle.verify_point_mass(tf, toks, T, k, p, cap, 11, keep_weights=True)
    rep = compare(pm, orc_pm, toks, tf, None, prm)
    print("point mass:", rep.summary())
    rep.assert_ok(0.34)
    orc_g = oracle.verify_greedy(tf, toks)
    rep = compare(g, orc_g, toks, greedy=True)
    print("greedy:", rep.summary())
    rep.assert_ok(0.0)
