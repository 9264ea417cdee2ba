"""Seeded random configurations through every entry point, against the
oracle (GPU).

Each seed draws a shape (B in 1..24, gamma in 0..8, V in 1..70,000 with
ragged tails), a dtype, per-row temperatures (greedy rows included), top-k /
top-p on some rows, caps, an EOS id, and unaligned rows on some seeds; then
runs the drafter's draw, the round with draft logits, the round with the
drafter's statistics (bit-identical to it), the point-mass round and the
greedy round, each compared with the oracle to the bar of ``parity.py``.
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


def _config(seed):
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 25))
    gamma = 0 if seed % 8 == 3 else int(rng.integers(1, 9))
    V = int(rng.choice([1, 2, 31, 1000, 8191, 8200, 16384, 33333, 70000]))
    dtype = "bf16" if rng.random() < 0.6 else "f32"
    aligned = rng.random() < 0.7
    T = np.where(rng.random(B) < 0.25, 0.0, rng.uniform(0.4, 1.6, B)).astype(np.float32)
    trunc = rng.random(B) < 0.4
    k = np.where(trunc & (rng.random(B) < 0.7), rng.integers(1, 40, B), 0).astype(np.int32)
    p = np.where(trunc & (k > 0) & (rng.random(B) < 0.5), rng.uniform(0.5, 0.99, B), 1.0).astype(np.float32)
    cap = np.where(rng.random(B) < 0.3, rng.integers(1, gamma + 3, B), 0).astype(np.int32)
    sd = float(rng.uniform(0.3, 2.5))
    t, d = synth.make_logits(rng, B, max(gamma, 1), V + 1, 2.5, sd, boost_count=min(20, V))
    t, d = t[:, :gamma + 1], d[:, :gamma]
    return dict(B=B, gamma=gamma, V=V, dtype=dtype, aligned=aligned, T=T, k=k, p=p, cap=cap, t=t, d=d)


def _dev(x, dtype, aligned, V):
    tt = torch.from_numpy(np.ascontiguousarray(x))
    if dtype == "bf16":
        tt = tt.to(torch.bfloat16)
    host = tt[..., :V] if aligned else tt[..., 1:]
    dev = tt.cuda()
    dev = dev[..., :V] if aligned else dev[..., 1:]
    return dev, host.float().numpy()


@pytest.mark.parametrize("seed", range(16))
def test_random_configuration(gpu, seed):
    c = _config(1000 + seed)
    B, gamma, V = c["B"], c["gamma"], c["V"]
    print(f"seed {seed}: B={B} gamma={gamma} V={V} {c['dtype']} aligned={c['aligned']}")
    tdev, tf = _dev(c["t"], c["dtype"], c["aligned"], V)
    ddev, df = _dev(c["d"], c["dtype"], c["aligned"], V)
    prm = {"temperature": c["T"], "top_k": c["k"], "top_p": c["p"], "max_new_tokens": c["cap"]}
    rp = sv.make_row_params(B, c["T"], c["k"], c["p"], c["cap"])
    seed_v = 77 + seed
    with sv.Verifier(B, max(gamma, 1), V, max_top_k=64) as v:
        if gamma > 0:
            drawn = v.sample_draft(ddev, rp, seed_v + 1)
            torch.cuda.synchronize()
            rep = compare_draft(drawn["tokens"], drawn["stats"], df, c["T"], seed_v + 1, 0, 0,
                                c["k"], c["p"])
            print("draw:", rep.summary())
            rep.assert_ok(0.2)
            tok = drawn["tokens"]
            stats = drawn["stats"]
        else:
            tok = torch.zeros(B, 0, dtype=torch.int32, device="cuda")
            stats = torch.zeros(B, 0, 4, device="cuda")
        toks = tok.cpu().numpy()
        eos = int(toks[0, gamma // 2]) if gamma > 0 and (toks[0] >= 0).all() else -1
        a = v.verify_sample(tdev, ddev, tok, rp, seed_v, 3, eos, diag=True)
        b = v.verify_sample_qstats(tdev, ddev, stats, tok, rp, seed_v, 3, eos, diag=True) if gamma > 0 \
            else a
        pm = v.verify_point_mass(tdev, tok, rp, seed_v, 3, eos, diag=True)
        torch.cuda.synchronize()
        for key in ("num_accepted", "out_tokens", "num_emitted", "row_flags"):
            assert torch.equal(a[key], b[key]), key
        orc = oracle.verify_sample(tf, df, toks, c["T"], c["k"], c["p"], c["cap"], seed_v, 3, eos,
                                   keep_weights=True)
        rep = compare(a, orc, toks, tf, df, prm)
        print("verify:", rep.summary())
        rep.assert_ok(0.2)
        orc_pm = oracle.verify_point_mass(tf, toks, c["T"], c["k"], c["p"], c["cap"], seed_v, 3, eos,
                                          keep_weights=True)
        rep = compare(pm, orc_pm, toks, tf, None, prm)
        print("point mass:", rep.summary())
        rep.assert_ok(0.2)
        caps = torch.from_numpy(c["cap"]).cuda()
        g = v.verify_greedy(tdev, tok, caps, eos)
        torch.cuda.synchronize()
    orc_g = oracle.verify_greedy(tf, toks, c["cap"], eos)
    rep = compare(g, orc_g, toks, greedy=True)
    print("greedy:", rep.summary())
    rep.assert_ok(0.0)
