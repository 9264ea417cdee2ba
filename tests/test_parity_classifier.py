"""The parity classifier (tests/parity.py) on hand-made outcomes (CPU).

The oracle runs on small rows; "GPU" outputs are copies of its outputs with
one planted difference each, and the classifier must grade them as the bar
states: identical rows exact; a differing draw inside the 1e-5 CDF window,
an accept decision with the uniform within 1e-5 of the threshold, or a
divergence at a position whose top-p decision was near, tolerated; anything
else (a divergence at another position of a row that had a near top-p
decision elsewhere, a far-off token, a wrong accepted count, bad padding, a
wrong p(d) or residual sum) a failure.
"""

import numpy as np

import oracle
from parity import Report, compare


def _setup(seed=3, B=12, gamma=3, V=50):
    rng = np.random.default_rng(seed)
    t = (rng.standard_normal((B, gamma + 1, V)) * 2).astype(np.float32)
    d = (t[:, :gamma] + rng.standard_normal((B, gamma, V))).astype(np.float32)
    toks = oracle.sample_draft_tokens(d, 1.0, 0, 1.0, 7)
    orc = oracle.verify_sample(t, d, toks, 1.0, 0, 1.0, 0, seed=21, keep_weights=True)
    prm = {"temperature": np.ones(B, np.float32), "top_k": np.zeros(B, np.int32),
           "top_p": np.ones(B, np.float32)}
    return t, d, toks, orc, prm


def _gpu_copy(orc):
    g = {k: np.array(orc[k], copy=True) for k in ("out_tokens", "num_emitted", "num_accepted",
                                                  "row_flags")}
    g["p_at_draft"] = orc["p_at_draft"].astype(np.float32)
    g["q_at_draft"] = orc["q_at_draft"].astype(np.float32)
    g["residual_sum"] = orc["residual_sum"].astype(np.float32)
    return g


def _row_with(orc, kind):
    for b, ev in enumerate(orc["events"]):
        s = ev["sample"]
        if s is not None and s["kind"] == kind:
            return b
    raise AssertionError(f"no row with a {kind} draw")


def test_identical_outputs_are_exact():
    t, d, toks, orc, prm = _setup()
    rep = compare(_gpu_copy(orc), orc, toks, t, d, prm)
    assert not rep.failures and rep.exact == rep.rows


def test_far_token_fails_and_window_token_is_tolerated():
    t, d, toks, orc, prm = _setup()
    b = _row_with(orc, "residual")
    ev = orc["events"][b]["sample"]
    j = ev["pos"]
    w = ev["weights"]
    t0 = int(orc["out_tokens"][b, j])
    far = [v for v in np.nonzero(w > 0)[0] if v != t0]
    lo_u, hi_u = oracle.cdf_interval(w, t0)
    # a token whose interval is far from u fails
    cand = [v for v in far if min(abs(oracle.cdf_interval(w, v)[0] - ev["u"]),
                                  abs(oracle.cdf_interval(w, v)[1] - ev["u"])) > 1e-3]
    g = _gpu_copy(orc)
    g["out_tokens"][b, j] = cand[0]
    rep = compare(g, orc, toks, t, d, prm)
    assert len(rep.failures) == 1
    # move u next to the lower boundary of the oracle token: the previous
    # token with weight is then within the window
    below = [v for v in np.nonzero(w > 0)[0] if v < t0]
    assert below and lo_u > 0
    orc2 = dict(orc)
    orc2["events"] = [dict(e) for e in orc["events"]]
    orc2["events"][b]["sample"] = dict(ev, u=lo_u + 5e-6)
    g = _gpu_copy(orc)
    g["out_tokens"][b, j] = below[-1]
    rep = compare(g, orc2, toks, t, d, prm)
    assert not rep.failures and rep.tolerated["cdf_window"] == 1


def test_accept_window():
    t, d, toks, orc, prm = _setup()
    b = _row_with(orc, "residual")
    j = int(orc["num_accepted"][b])                 # the rejected position
    i, u, pp, qq = orc["events"][b]["accept_tests"][j]
    thr = min(1.0, pp / qq)
    # the GPU accepted d_j instead, and then stopped (a made-up continuation)
    g = _gpu_copy(orc)
    g["num_accepted"][b] = j + 1
    g["out_tokens"][b, j] = toks[b, j]
    g["out_tokens"][b, j + 1:] = -1
    g["num_emitted"][b] = j + 1
    rep = compare(g, orc, toks, t, d, prm)
    assert len(rep.failures) == 1                    # u is not near the threshold
    orc2 = dict(orc)
    orc2["events"] = [dict(e) for e in orc["events"]]
    tests = list(orc["events"][b]["accept_tests"])
    tests[j] = (i, thr + 3e-6, pp, qq)
    orc2["events"][b]["accept_tests"] = tests
    rep = compare(g, orc2, toks, t, d, prm)
    assert not rep.failures and rep.tolerated["accept_window"] == 1


def test_topp_near_only_at_the_diverging_position():
    t, d, toks, orc, prm = _setup()
    b = _row_with(orc, "residual")
    j = int(orc["num_accepted"][b])
    ev = orc["events"][b]["sample"]
    w = ev["weights"]
    t0 = int(orc["out_tokens"][b, j])
    other = [v for v in np.nonzero(w > 0)[0] if v != t0
             and min(abs(oracle.cdf_interval(w, v)[0] - ev["u"]),
                     abs(oracle.cdf_interval(w, v)[1] - ev["u"])) > 1e-3][0]
    g = _gpu_copy(orc)
    g["out_tokens"][b, j] = other
    for near_at, ok in ((j, True), (j + 1, False), ([], False)):
        orc2 = dict(orc)
        orc2["events"] = [dict(e) for e in orc["events"]]
        orc2["events"][b]["topp_near"] = [near_at] if near_at != [] else []
        orc2["row_flags"] = orc["row_flags"].copy()
        if near_at != []:
            orc2["row_flags"][b] |= oracle.FLAG_TOPP_NEAR
        rep = compare(g, orc2, toks, t, d, prm)
        if ok:
            assert not rep.failures and rep.tolerated["topp_near"] == 1
        else:
            assert len(rep.failures) == 1, (near_at, rep.summary())


def test_values_padding_and_counts():
    t, d, toks, orc, prm = _setup()
    b = _row_with(orc, "residual")
    j = int(orc["num_accepted"][b])
    for mutate in ("p", "w", "pad", "acc"):
        g = _gpu_copy(orc)
        if mutate == "p":
            g["p_at_draft"][b, j] *= 1.0 + 5e-5
        elif mutate == "w":
            g["residual_sum"][b] += 5e-5 * max(orc["residual_sum"][b], 1.0)
        elif mutate == "pad":
            g["out_tokens"][b, -1] = 3 if g["num_emitted"][b] < g["out_tokens"].shape[1] else -1
            if g["num_emitted"][b] == g["out_tokens"].shape[1]:
                continue
        else:
            g["num_accepted"][b] += 1
        rep = compare(g, orc, toks, t, d, prm)
        assert len(rep.failures) == 1, mutate


def test_report_counts():
    rep = Report()
    rep.rows, rep.exact = 10, 9
    rep.tolerated["cdf_window"] = 1
    d = rep.as_dict()
    assert d["rows"] == 10 and d["tolerated"]["cdf_window"] == 1 and d["failures"] == 0
