"""Compare a GPU verify result with the oracle's, row by row.

Bar (numbers written here, used by every parity test):

* greedy rows, accepted counts and flags: bit-exact;
* sampled tokens identical, except where floating point legitimately
  decides differently.  Such a row is counted and reported, not failed,
  only when the FIRST event at which the two runs differ is one of:
  - ACCEPT_WINDOW: an accept test whose uniform lies within 1e-5 of the
    acceptance threshold min(1, p/q) (oracle values);
  - CDF_WINDOW: a correction / bonus draw whose GPU token t has the oracle
    interval [C(t-1), C(t)] / W within 1e-5 of the uniform;
  - TOPP_NEAR: the position of that event is one where the oracle found a
    top-p decision within 1e-5 of top_p (its kept set may legitimately
    differ between float32 and float64);
  the positions before the divergence are still checked (values below),
  and the row's later outputs are not compared;
* p_i(d_i), q_i(d_i): relative error <= 1e-5 (absolute floor 1e-30);
* residual sum W: |dW| <= 1e-5 * W + 1e-6.  The floor follows from the
  arithmetic: the GPU forms each p(v) and q(v) in float32 from
  exp2((z - m) * log2(e) / T) / S, whose relative error grows with the
  exponent's size (about |x| * 2^-24 from rounding x, plus a few ulp), so
  the absolute error of the sum of |p - q| over the vocabulary is of order
  1e-7 to 1e-6 whatever W is.  Rows that pass only through the floor are
  counted (``w_floor_only``) and reported with the others.
"""

import os

import numpy as np

import oracle

ACCEPT_WINDOW = 1e-5
CDF_WINDOW = 1e-5
REL_TOL = 1e-5
ABS_FLOOR = 1e-30
W_REL = 1e-5
W_ABS = 1e-6
FLAGS_EXACT = (oracle.FLAG_TOKEN_OOR | oracle.FLAG_NONFINITE_ROW | oracle.FLAG_Q_ZERO
               | oracle.FLAG_RESIDUAL_FALLBACK)


class Report:
    def __init__(self):
        self.rows = 0
        self.exact = 0
        self.tolerated = {"accept_window": 0, "cdf_window": 0, "topp_near": 0}
        self.failures = []
        self.value_checks = 0
        self.w_floor_only = 0

    def fail(self, b, msg):
        self.failures.append(f"row {b}: {msg}")

    def as_dict(self):
        return {"rows": self.rows, "exact": self.exact, "tolerated": dict(self.tolerated),
                "value_checks": self.value_checks, "w_floor_only": self.w_floor_only,
                "failures": len(self.failures)}

    def summary(self):
        return (f"rows={self.rows} exact={self.exact} tolerated={self.tolerated} "
                f"value_checks={self.value_checks} w_floor_only={self.w_floor_only} "
                f"failures={len(self.failures)}")

    def assert_ok(self, max_tolerated_frac=0.02):
        assert not self.failures, self.summary() + "\n" + "\n".join(self.failures[:20])
        tol = sum(self.tolerated.values())
        assert tol <= max(2, max_tolerated_frac * self.rows), self.summary()


def _np(x):
    if hasattr(x, "detach"):
        return x.detach().cpu().numpy()
    return np.asarray(x)


def _weights(o_ev, target_f32, draft_f32, b, T, k, p):
    """Oracle weights of the sampled draw of row b (recomputed on demand)."""
    s = o_ev["sample"]
    if s.get("weights") is not None:
        return s["weights"]
    P = oracle.process_row(target_f32[b, s["pos"]], T, k, p)
    if s["kind"] == "bonus":
        return P.probs
    Q = oracle.process_row(draft_f32[b, s["pos"]], T, k, p)
    w = np.maximum(P.probs - Q.probs, 0.0)
    if not (np.isfinite(w.sum()) and w.sum() > 0):
        w = P.probs
    return w


def _current_name():
    cur = os.environ.get("PYTEST_CURRENT_TEST", "")
    return cur.split(" ")[0] if cur else "outside pytest"


def compare(gpu, orc, tokens, target_f32=None, draft_f32=None, params=None, greedy=False,
            report=None, workload=None):
    """Classify every row; returns the Report (call .assert_ok()).  The
    counts of the rows classified here are added to the session record of
    ``workload`` (default: the running test's id)."""
    rep = report or Report()
    before = rep.as_dict()
    try:
        return _compare(gpu, orc, tokens, target_f32, draft_f32, params, greedy, rep)
    finally:
        record(workload or _current_name(), _delta(rep.as_dict(), before))


def _delta(after, before):
    d = {k: after[k] - before[k] for k in ("rows", "exact", "value_checks", "w_floor_only", "failures")}
    d["tolerated"] = {k: after["tolerated"][k] - before["tolerated"].get(k, 0) for k in after["tolerated"]}
    return d


def _compare(gpu, orc, tokens, target_f32, draft_f32, params, greedy, rep):
    g_tok = _np(gpu["out_tokens"])
    g_emit = _np(gpu["num_emitted"])
    g_acc = _np(gpu["num_accepted"])
    g_flags = _np(gpu["row_flags"])
    tokens = _np(tokens)
    B = g_tok.shape[0]
    for b in range(B):
        rep.rows += 1
        eo = orc["out_tokens"][b, :orc["num_emitted"][b]].tolist()
        eg = g_tok[b, :g_emit[b]].tolist()
        fo = int(orc["row_flags"][b])
        fg = int(g_flags[b])
        n_o, n_g = int(orc["num_accepted"][b]), int(g_acc[b])
        if (g_tok[b, g_emit[b]:] != -1).any():
            rep.fail(b, "padding is not -1")
            continue
        if eo == eg and n_g == n_o and (fo & FLAGS_EXACT) == (fg & FLAGS_EXACT):
            rep.exact += 1
            _check_values(rep, b, gpu, orc, greedy, upto=None, check_w=True)
            continue
        if greedy or (params is not None and params["temperature"][b] == 0):
            rep.fail(b, f"greedy mismatch gpu={eg} oracle={eo} flags {fg}/{fo}")
            continue
        # the first differing event: position j where one run accepted the
        # draft and the other did not, or where both ended the round with
        # different tokens (positions before j agree in outcome and token)
        j = 0
        while (j < min(len(eo), len(eg)) and eo[j] == eg[j] and (j < n_o) == (j < n_g)):
            j += 1
        ev = orc["events"][b]
        tests = {i: (u, pp, qq) for (i, u, pp, qq) in ev["accept_tests"]}
        o_accepted_j = n_o > j
        g_accepted_j = n_g > j
        if j in ev.get("topp_near", ()):
            # the kept set of position j may differ between the precisions:
            # only the positions before it are compared
            rep.tolerated["topp_near"] += 1
            _check_values(rep, b, gpu, orc, greedy, upto=j, check_w=False)
            continue
        if j in tests and o_accepted_j != g_accepted_j:
            u, pp, qq = tests[j]
            thr = min(1.0, pp / qq) if qq > 0 else (1.0 if pp > 0 else 0.0)
            if abs(u - thr) < ACCEPT_WINDOW:
                rep.tolerated["accept_window"] += 1
                _check_values(rep, b, gpu, orc, greedy, upto=j + 1, check_w=False)
            else:
                rep.fail(b, f"accept decision differs at {j}: u={u} thr={thr} gpu={eg} oracle={eo}")
            continue
        s = ev["sample"]
        if s is not None and s["pos"] == j and j < len(eg) and not g_accepted_j:
            T, k, p = (params["temperature"][b], params["top_k"][b], params["top_p"][b])
            w = _weights(ev, target_f32, draft_f32, b, T, k, p)
            t = eg[j]
            if not (0 <= t < len(w)) or w[t] <= 0:
                rep.fail(b, f"GPU sampled token {t} has zero oracle weight at {j}")
                continue
            lo, hi = oracle.cdf_interval(w, t)
            u = s["u"]
            dist = 0.0 if lo <= u <= hi else min(abs(u - lo), abs(u - hi))
            if dist < CDF_WINDOW:
                rep.tolerated["cdf_window"] += 1
                # the same position was sampled from the same weights: the
                # values of every test and the residual sum still agree
                _check_values(rep, b, gpu, orc, greedy, upto=None, check_w=True)
            else:
                rep.fail(b, f"sampled token differs at {j}: gpu {t} [{lo},{hi}] oracle {eo[j]} u={u}")
            continue
        rep.fail(b, f"mismatch gpu={eg} (acc {n_g}, flags {fg}) oracle={eo} "
                    f"(acc {n_o}, flags {fo})")
    return rep


def _check_values(rep, b, gpu, orc, greedy, upto=None, check_w=True):
    """p_i(d_i), q_i(d_i) of the tests at positions < upto (every position
    when None), and the residual sum when check_w."""
    if greedy or "p_at_draft" not in gpu:
        return
    gp = _np(gpu["p_at_draft"])[b]
    gq = _np(gpu["q_at_draft"])[b]
    op = orc["p_at_draft"][b]
    oq = orc["q_at_draft"][b]
    n = len(op) if upto is None else min(upto, len(op))
    for i in range(n):
        if np.isnan(op[i]):
            if not np.isnan(gp[i]):
                rep.fail(b, f"p_at_draft[{i}] written for an untested position")
            continue
        for g, o, name in ((gp[i], op[i], "p"), (gq[i], oq[i], "q")):
            rep.value_checks += 1
            if not abs(g - o) <= REL_TOL * abs(o) + ABS_FLOOR:
                rep.fail(b, f"{name}_at_draft[{i}] gpu={g!r} oracle={o!r} rel={abs(g-o)/max(abs(o),1e-300):.2e}")
    if check_w and "residual_sum" in gpu:
        gw = float(_np(gpu["residual_sum"])[b])
        ow = float(orc["residual_sum"][b])
        rep.value_checks += 1
        err = abs(gw - ow)
        if err > W_REL * ow + W_ABS:
            rep.fail(b, f"residual sum gpu={gw} oracle={ow}")
        elif err > W_REL * ow:
            rep.w_floor_only += 1


# Reports accumulated per workload during a test session; written out as
# JSON at the session's end when SPECV_PARITY_RECORD names a file.
RECORDS = {}


def record(workload, d):
    """Add counts (a Report's ``as_dict()`` or a difference of two) to the
    session record of ``workload``."""
    r = RECORDS.setdefault(workload, {"rows": 0, "exact": 0, "tolerated": {},
                                      "value_checks": 0, "w_floor_only": 0, "failures": 0})
    for key in ("rows", "exact", "value_checks", "w_floor_only", "failures"):
        r[key] += d[key]
    for key, v in d["tolerated"].items():
        r["tolerated"][key] = r["tolerated"].get(key, 0) + v


def compare_draft(gpu_tok, gpu_stats, draft_f32, temperature, seed, step=0, pos0=0,
                  top_k=0, top_p=1.0, report=None, skip_rows=(), workload=None):
    """Compare the draft sampler's outputs for positions pos0 .. pos0+n-1
    (arrays already sliced to those columns; gpu_stats float32 [B, n, 4]
    records (max, sum, threshold, flags bits)) with the oracle's draw and row
    statistics.  Tokens: identical, or (sampled rows) inside the CDF window,
    or (truncated rows) a top-p decision the oracle marked near; greedy
    tokens bit-exact; max and threshold exact; sum within REL_TOL; flags:
    NONFINITE_ROW exactly where the oracle has no draw, TOPP_NEAR allowed.
    Batch rows in ``skip_rows`` are not compared."""
    rep = report or Report()
    before = rep.as_dict()
    try:
        return _compare_draft(gpu_tok, gpu_stats, draft_f32, temperature, seed, step, pos0, top_k,
                              top_p, rep, skip_rows)
    finally:
        record((workload or _current_name()) + " [draft draws]", _delta(rep.as_dict(), before))


def _compare_draft(gpu_tok, gpu_stats, draft_f32, temperature, seed, step, pos0, top_k, top_p, rep,
                   skip_rows):
    d = np.asarray(draft_f32)
    B, n, V = d.shape
    T = np.broadcast_to(np.asarray(temperature, np.float64), (B,))
    K = np.broadcast_to(np.asarray(top_k, np.int64), (B,))
    Pp = np.broadcast_to(np.asarray(top_p, np.float64), (B,))
    o_tok = oracle.sample_draft_tokens(d, T, K, Pp, seed, step, pos0)
    o_st = oracle.draft_row_stats(d, T, K, Pp)
    g_tok, g_st = _np(gpu_tok), _np(gpu_stats)
    g_fl = np.ascontiguousarray(g_st).view(np.int32)[..., 3]
    for b in range(B):
        if b in skip_rows:
            continue
        for i in range(n):
            rep.rows += 1
            t, o = int(g_tok[b, i]), int(o_tok[b, i])
            fl = int(g_fl[b, i]) & ~oracle.FLAG_TOPP_NEAR
            want_flag = oracle.FLAG_NONFINITE_ROW if o < 0 else 0
            if fl != want_flag:
                rep.fail(b, f"pos {pos0 + i}: flags {int(g_fl[b, i])} want {want_flag}")
                continue
            truncated = T[b] > 0 and o >= 0 and ((0 < K[b] < V) or Pp[b] < 1.0)
            Q = oracle.process_row(d[b, i], T[b], K[b], Pp[b]) if truncated else None
            if Q is not None and Q.topp_near:
                # the kept set may legitimately differ between float32 and float64
                rep.tolerated["topp_near"] += 1
                continue
            if T[b] > 0 and o >= 0:
                m, s, th = (float(x) for x in g_st[b, i, :3])
                om, os_, ot = o_st[b, i]
                rep.value_checks += 1
                if m != om or th != ot or not abs(s - os_) <= REL_TOL * os_:
                    rep.fail(b, f"pos {pos0 + i}: stats ({m}, {s}, {th}) oracle ({om}, {os_}, {ot})")
                    continue
            elif not np.isnan(g_st[b, i, :3]).all():
                rep.fail(b, f"pos {pos0 + i}: stats {g_st[b, i, :3]} written for a greedy / undrawn row")
                continue
            if t == o:
                rep.exact += 1
                continue
            if T[b] == 0 or o < 0:
                rep.fail(b, f"pos {pos0 + i}: token {t} oracle {o}")
                continue
            q = (Q if Q is not None else oracle.process_row(d[b, i], T[b], K[b], Pp[b])).probs
            if not (0 <= t < V) or q[t] <= 0:
                rep.fail(b, f"pos {pos0 + i}: token {t} has no draft mass")
                continue
            lo, hi = oracle.cdf_interval(q, t)
            u = float(oracle.philox.uniform(seed, b, pos0 + i, oracle.philox.PURPOSE_DRAFT, step))
            dist = 0.0 if lo <= u <= hi else min(abs(u - lo), abs(u - hi))
            if dist < CDF_WINDOW:
                rep.tolerated["cdf_window"] += 1
            else:
                rep.fail(b, f"pos {pos0 + i}: token {t} [{lo},{hi}] oracle {o} u={u}")
    return rep
