"""Verify calls captured into a HIP graph and replayed (through the C ABI, with
torch's graph capture on the current stream).

The call number that tags the records a launch's workgroups exchange, and
selects their set, is taken and advanced on the device, so a replayed launch
(whose arguments are frozen) still gets a new one.  Each replay runs on new
contents of the captured input buffers and is compared, bit for bit, with an
eager call on the same inputs and the same seed and step; eager calls of other
sizes on the same handle run between replays (the records' extent changes),
and some replays follow each other with nothing in between.  The first
replay's outputs are also checked against the oracle.

Covered: specv_verify_sample (sampling, greedy, capped rows), the drafter's
sampler followed by specv_verify_sample_qstats in one graph, and
specv_verify_sample_noalloc.
"""

import numpy as np
import pytest
import torch

import oracle
import synth
import speculative_decoding_verification_sampling_amd as sv
from parity import compare

pytestmark = pytest.mark.gpu

KEYS = ("num_accepted", "out_tokens", "num_emitted", "row_flags")


@pytest.fixture(scope="module")
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    sv.load_library()
    return torch.device("cuda:0")


def _same(a, b, keys=KEYS):
    for k in keys:
        x, y = a[k].cpu(), b[k].cpu()
        if x.dtype == torch.float32:
            assert torch.equal(torch.isnan(x), torch.isnan(y)), k
            x, y = torch.nan_to_num(x, 7.0), torch.nan_to_num(y, 7.0)
        assert torch.equal(x, y), k


def _input_sets(n, B, gamma, V, seed):
    """n seeded (target, draft, tokens) sets of one shape, bfloat16 logits."""
    rng = np.random.default_rng(seed)
    sets = []
    for r in range(n):
        t, d = synth.make_logits(rng, B, gamma, V, 3.0, 0.5 + 0.25 * (r % 3), boost_count=20)
        tt = torch.from_numpy(t).to(torch.bfloat16)
        dd = torch.from_numpy(d).to(torch.bfloat16)
        toks = oracle.sample_draft_tokens(dd.float().numpy(), 1.0, 0, 1.0, 500 + r)
        sets.append((tt.cuda(), dd.cuda(), torch.from_numpy(toks).cuda(), tt.float().numpy(),
                     dd.float().numpy(), toks))
    return sets


def _params(B):
    T = np.where(np.arange(B) % 4 == 3, 0.0, np.where(np.arange(B) % 2 == 0, 1.0, 0.7)).astype(np.float32)
    caps = np.where(np.arange(B) % 5 == 4, 2, 0).astype(np.int32)
    return T, caps


def _clone(o):
    return {k: v.clone() for k, v in o.items()}


def test_verify_sample_replays_match_eager_calls(gpu):
    B, gamma, V = 24, 4, 50001                  # 7 chunks, the last ragged
    T, caps = _params(B)
    rp = sv.make_row_params(B, T, 0, 1.0, caps)
    sets = _input_sets(10, B, gamma, V, 31)
    seed, step = 0x5EED, 11
    # another size for the eager calls between replays
    small = _input_sets(1, 5, 2, 9000, 32)[0]
    rp_small = sv.make_row_params(5, 0.9)
    with sv.Verifier(B, gamma, V) as v:
        t_in = sets[0][0].clone()
        d_in = sets[0][1].clone()
        k_in = sets[0][2].clone()
        v.verify_sample(t_in, d_in, k_in, rp, seed, step)         # loads the kernels
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            out = v.verify_sample(t_in, d_in, k_in, rp, seed, step)
        torch.cuda.synchronize()
        for r, (tt, dd, kk, tf, df, toks) in enumerate(sets):
            t_in.copy_(tt)
            d_in.copy_(dd)
            k_in.copy_(kk)
            g.replay()
            torch.cuda.synchronize()
            got = _clone(out)
            if r < 7:
                # eager work between replays: the same call, and one of another size
                ref = v.verify_sample(tt, dd, kk, rp, seed, step)
                v.verify_sample(small[0], small[1], small[2], rp_small, 3, 1)
                torch.cuda.synchronize()
                _same(got, ref)
            if r == 0:
                orc = oracle.verify_sample(tf, df, toks, T, 0, 1.0, caps, seed, step)
                rep = compare(got, orc, toks, tf, df, {"temperature": T, "top_k": np.zeros(B, np.int32),
                                                      "top_p": np.ones(B, np.float32)})
                rep.assert_ok(0.5)
        # replays 7 .. 9 ran back to back; their eager counterparts now
        for r in range(7, 10):
            t_in.copy_(sets[r][0])
            d_in.copy_(sets[r][1])
            k_in.copy_(sets[r][2])
            g.replay()
            g.replay()                           # twice in a row on the same inputs
            torch.cuda.synchronize()
            got = _clone(out)
            ref = v.verify_sample(sets[r][0], sets[r][1], sets[r][2], rp, seed, step)
            torch.cuda.synchronize()
            _same(got, ref)
            assert (got["row_flags"].cpu().numpy() & sv.FLAG_INTERNAL).sum() == 0


def test_drafter_and_qstats_verify_in_one_graph(gpu):
    B, gamma, V = 16, 3, 40000
    sets = _input_sets(6, B, gamma, V, 41)
    T = np.full(B, 0.8, np.float32)
    rp = sv.make_row_params(B, T)
    with sv.Verifier(B, gamma, V) as v:
        t_in = sets[0][0].clone()
        d_in = sets[0][1].clone()
        drawn = v.sample_draft(d_in, rp, seed=21, step=4)
        v.verify_sample_qstats(t_in, d_in, drawn["stats"], drawn["tokens"], rp, seed=22, step=4)
        torch.cuda.synchronize()
        # the drafter's outputs allocated (and filled) outside the capture, so
        # that the graph holds the two launches only
        gd = {"tokens": torch.full((B, gamma), -1, dtype=torch.int32, device="cuda"),
              "stats": torch.zeros((B, gamma, 4), dtype=torch.float32, device="cuda")}
        gd["flags"] = gd["stats"].view(torch.int32)[..., 3]
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            v.sample_draft(d_in, rp, seed=21, step=4, out=gd)
            out = v.verify_sample_qstats(t_in, d_in, gd["stats"], gd["tokens"], rp, seed=22, step=4)
        torch.cuda.synchronize()
        for r, (tt, dd, _, tf, df, _) in enumerate(sets):
            t_in.copy_(tt)
            d_in.copy_(dd)
            g.replay()
            torch.cuda.synchronize()
            got, got_tok = _clone(out), gd["tokens"].clone()
            e_d = v.sample_draft(dd, rp, seed=21, step=4)
            ref = v.verify_sample_qstats(tt, dd, e_d["stats"], e_d["tokens"], rp, seed=22, step=4)
            torch.cuda.synchronize()
            assert torch.equal(got_tok.cpu(), e_d["tokens"].cpu())
            _same(got, ref)
            if r == 0:
                toks = got_tok.cpu().numpy()
                orc = oracle.verify_sample(tf, df, toks, T, 0, 1.0, 0, 22, 4)
                rep = compare(got, orc, toks, tf, df, {"temperature": T, "top_k": np.zeros(B, np.int32),
                                                      "top_p": np.ones(B, np.float32)})
                rep.assert_ok(0.5)


def test_noalloc_replays_match_eager_calls(gpu):
    B, gamma, V = 12, 3, 30000
    sets = _input_sets(5, B, gamma, V, 51)
    T, caps = _params(B)
    rp = sv.make_row_params(B, T, 0, 1.0, caps)
    t_in = sets[0][0].clone()
    d_in = sets[0][1].clone()
    k_in = sets[0][2].clone()
    sv.verify_sample_noalloc(t_in, d_in, k_in, rp, 9, 2)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = sv.verify_sample_noalloc(t_in, d_in, k_in, rp, 9, 2)
    torch.cuda.synchronize()
    for tt, dd, kk, _, _, _ in sets:
        t_in.copy_(tt)
        d_in.copy_(dd)
        k_in.copy_(kk)
        g.replay()
        torch.cuda.synchronize()
        got = _clone(out)
        ref = sv.verify_sample_noalloc(tt, dd, kk, rp, 9, 2)
        torch.cuda.synchronize()
        _same(got, ref)
