"""One round of speculative verification (oracle side).  TEST INFRASTRUCTURE.

Follows the single-chain pseudo-code 10-1 and section 11.1.2 of
"11.1 核心原理: Draft + Verify 与 Rejection Sampling", and the speculative
sampling description in "Fast Inference from Transformers via Speculative
Decoding":

* target row i (0-based) is the distribution that checks draft token d_i;
  target row gamma is the bonus distribution (11.1.1);
* d_i is accepted with probability min(1, p_i(d_i) / q_i(d_i)): with a
  uniform u in [0, 1) the test is ``u * q < p``, which equals
  ``u < min(1, p / q)`` for q > 0 and accepts a proposal outside q's support
  whenever p > 0 (11.1.2, pseudo-code 10-1);
* the round stops at the first rejection; later drafts are discarded and
  draw no random numbers;
* on a rejection at position i the correction token is drawn from
  norm(max(p_i - q_i, 0)); if that mass is zero or not finite (possible only
  through rounding, or when p_i == q_i with d_i outside both supports) the
  row falls back to p_i and is flagged;
* if all gamma drafts are accepted a bonus token is drawn from p_gamma;
* greedy verification accepts d_i while it equals the target argmax and
  emits the target argmax at the first mismatch (or as the bonus);
* EOS and max_new_tokens end the round early: emission stops after the
  first emitted EOS and after ``max_new_tokens`` tokens, and a bonus or
  correction token that would exceed the cap is not drawn (the remark after
  pseudo-code 10-1).

Sampling by inverse CDF: tokens in ascending index order, t is the smallest
v whose running weight sum exceeds u * W (W the total), clamped to the last
token with positive weight, so a zero-weight token is never returned.

Uniforms: Philox4x32-10 keyed by (seed, row b, position i, purpose, step);
see ``oracle.philox``.

Deterministic proposals (n-gram or prompt-lookup drafts: section 2.1 and
4.2 of the "投机解码 Speculative Decoding" tutorial; the ICML summary's
remark that the approximation model may be an n-gram model or a
context-repeat heuristic) propose d_i with probability one, so their actual
proposal distribution is the point mass on d_i.  ``verify_point_mass`` runs
the same round with q_i = delta(d_i): the test reads u < p_i(d_i), and the
correction distribution norm(max(p_i - delta(d_i), 0)) is p_i with d_i
removed.  No draft logits exist.

The drafter's side: ``sample_draft_tokens`` draws d_i ~ q_i (the processed
draft distribution, inverse CDF with the uniform of purpose DRAFT), and
``draft_row_stats`` gives the statistics a drafter that sampled q_i can hand
to the verifier: over the kept set, m = max z, s = sum exp((z - m) / T) and
the threshold t = min z (-inf without truncation), from which
q_i(v) = [z_v >= t] exp((z_v - m) / T) / s.

Pins (``tests/test_oracle_*.py``): the worked example of 11.1.3, exact
enumeration over all 2^24 uniforms on small rows, the 11.1.3 identities,
E[N] against the closed form of the ICML summary and the tutorial's printed
E(4), E(8) at alpha = 0.7, chi-square tests of the emitted distribution, and
the greedy path against ``torch.argmax``; the drafter's draw by exact
enumeration against ``torch.softmax``, its statistics against
``torch.logsumexp``; ``cdf_interval`` against brute force on exact dyadic
grids (the interval of t is exactly the set of uniforms for which
``inverse_cdf`` returns t), and the reported residual sum against the
reject mass of 11.1.3 (0.2 on the worked example; 1 - sum min(p, q) at the
stopping position, with p and q from ``torch.softmax``)
(``tests/test_oracle_interval_residual.py``).
"""

import numpy as np

from .philox import uniform, PURPOSE_ACCEPT, PURPOSE_RESIDUAL, PURPOSE_BONUS, PURPOSE_DRAFT
from .process import process_row, greedy_argmax

FLAG_TOKEN_OOR = 1 << 0          # a draft token outside [0, V): the row emits nothing
FLAG_NONFINITE_ROW = 1 << 1      # a consulted logits row had NaN / +inf / nothing finite
FLAG_Q_ZERO = 1 << 2             # an accept test met d_i outside q_i's support
FLAG_RESIDUAL_FALLBACK = 1 << 3  # residual mass was zero / not finite: sampled from p_i
FLAG_TOPP_NEAR = 1 << 5          # a top-p decision fell within 1e-5 of top_p

NO_CAP = np.iinfo(np.int64).max


def residual_weights(P, Q):
    """Unnormalised correction distribution max(p - q, 0) (11.1.2)."""
    return np.maximum(P - Q, 0.0)


def inverse_cdf(w, u):
    """Smallest index v with sum(w[:v+1]) > u * sum(w); clamp to last w > 0."""
    w = np.asarray(w, dtype=np.float64)
    W = w.sum()
    c = np.cumsum(w)
    t = int(np.searchsorted(c, u * W, side="right"))
    if t >= len(w):
        t = int(np.nonzero(w > 0)[0][-1])
    return t


def cdf_interval(w, t):
    """[C(t-1), C(t)] / W: the range of u for which ``inverse_cdf`` gives t."""
    w = np.asarray(w, dtype=np.float64)
    W = w.sum()
    c = np.cumsum(w)
    lo = c[t - 1] if t > 0 else 0.0
    return lo / W, c[t] / W


def _broadcast(x, B, dtype):
    a = np.asarray(x, dtype=dtype)
    if a.ndim == 0:
        a = np.full(B, a, dtype=dtype)
    assert a.shape == (B,)
    return a


def _greedy_row(trow, toks, cap, eos_id):
    """Greedy verification of one row. Returns (emitted, n_accepted, flags)."""
    gamma = len(toks)
    emitted = []
    n_acc = 0
    for i in range(gamma + 1):
        if len(emitted) >= cap:
            break
        a = greedy_argmax(trow[i])
        if a is None:
            return [], 0, FLAG_NONFINITE_ROW
        if i < gamma and int(toks[i]) == a:
            emitted.append(a)
            n_acc += 1
            if a == eos_id:
                break
            continue
        emitted.append(a)          # first mismatch: the target's argmax; or the bonus
        break
    return emitted, n_acc, 0


def _sample_row(b, trow, drow, toks, T, k, p, cap, eos_id, seed, step, keep_weights):
    """Stochastic verification of one row, pseudo-code 10-1 order."""
    gamma = len(toks)
    emitted = []
    n_acc = 0
    flags = 0
    p_at = np.full(gamma, np.nan)
    q_at = np.full(gamma, np.nan)
    W_out = 0.0
    ev = {"accept_tests": [], "sample": None, "topp_near": []}
    for i in range(gamma):
        if len(emitted) >= cap:
            return emitted, n_acc, flags, p_at, q_at, W_out, ev
        P = process_row(trow[i], T, k, p)
        Q = process_row(drow[i], T, k, p)
        if P.nonfinite or Q.nonfinite:
            return [], 0, flags | FLAG_NONFINITE_ROW, p_at, q_at, 0.0, ev
        if P.topp_near or Q.topp_near:
            flags |= FLAG_TOPP_NEAR
            ev["topp_near"].append(i)
        d = int(toks[i])
        pd, qd = P.probs[d], Q.probs[d]
        p_at[i], q_at[i] = pd, qd
        if not Q.kept[d]:
            flags |= FLAG_Q_ZERO
        u = float(uniform(seed, b, i, PURPOSE_ACCEPT, step))
        ev["accept_tests"].append((i, u, pd, qd))
        if u * qd < pd:                       # accept with probability min(1, p/q)
            emitted.append(d)
            n_acc += 1
            if d == eos_id:
                return emitted, n_acc, flags, p_at, q_at, W_out, ev
            continue
        # first rejection: correction sample from norm(max(p - q, 0))
        w = residual_weights(P.probs, Q.probs)
        W = w.sum()
        W_out = W
        if not (np.isfinite(W) and W > 0):
            flags |= FLAG_RESIDUAL_FALLBACK
            w = P.probs
        u2 = float(uniform(seed, b, i, PURPOSE_RESIDUAL, step))
        t = inverse_cdf(w, u2)
        ev["sample"] = {"kind": "residual", "pos": i, "u": u2, "W": float(w.sum()),
                        "weights": w if keep_weights else None}
        emitted.append(t)
        return emitted, n_acc, flags, p_at, q_at, W_out, ev
    # every draft accepted: bonus token from p_gamma unless the cap forbids it
    if len(emitted) >= cap:
        return emitted, n_acc, flags, p_at, q_at, W_out, ev
    P = process_row(trow[gamma], T, k, p)
    if P.nonfinite:
        return [], 0, flags | FLAG_NONFINITE_ROW, p_at, q_at, 0.0, ev
    if P.topp_near:
        flags |= FLAG_TOPP_NEAR
        ev["topp_near"].append(gamma)
    u3 = float(uniform(seed, b, gamma, PURPOSE_BONUS, step))
    t = inverse_cdf(P.probs, u3)
    ev["sample"] = {"kind": "bonus", "pos": gamma, "u": u3, "W": float(P.probs.sum()),
                    "weights": P.probs if keep_weights else None}
    emitted.append(t)
    return emitted, n_acc, flags, p_at, q_at, W_out, ev


def _point_mass_row(b, trow, toks, T, k, p, cap, eos_id, seed, step, keep_weights):
    """Stochastic verification of one row against a deterministic proposal:
    pseudo-code 10-1 with q_i the point mass on d_i."""
    gamma = len(toks)
    emitted = []
    n_acc = 0
    flags = 0
    p_at = np.full(gamma, np.nan)
    q_at = np.full(gamma, np.nan)
    W_out = 0.0
    ev = {"accept_tests": [], "sample": None, "topp_near": []}
    for i in range(gamma):
        if len(emitted) >= cap:
            return emitted, n_acc, flags, p_at, q_at, W_out, ev
        P = process_row(trow[i], T, k, p)
        if P.nonfinite:
            return [], 0, flags | FLAG_NONFINITE_ROW, p_at, q_at, 0.0, ev
        if P.topp_near:
            flags |= FLAG_TOPP_NEAR
            ev["topp_near"].append(i)
        d = int(toks[i])
        delta = np.zeros_like(P.probs)
        delta[d] = 1.0                        # q_i: all mass on the proposed token
        pd, qd = P.probs[d], delta[d]
        p_at[i], q_at[i] = pd, qd
        u = float(uniform(seed, b, i, PURPOSE_ACCEPT, step))
        ev["accept_tests"].append((i, u, pd, qd))
        if u * qd < pd:                       # accept with probability min(1, p/q) = p(d)
            emitted.append(d)
            n_acc += 1
            if d == eos_id:
                return emitted, n_acc, flags, p_at, q_at, W_out, ev
            continue
        # first rejection: correction sample from norm(max(p - delta, 0))
        w = residual_weights(P.probs, delta)
        W = w.sum()
        W_out = W
        if not (np.isfinite(W) and W > 0):
            flags |= FLAG_RESIDUAL_FALLBACK
            w = P.probs
        u2 = float(uniform(seed, b, i, PURPOSE_RESIDUAL, step))
        t = inverse_cdf(w, u2)
        ev["sample"] = {"kind": "residual", "pos": i, "u": u2, "W": float(w.sum()),
                        "weights": w if keep_weights else None}
        emitted.append(t)
        return emitted, n_acc, flags, p_at, q_at, W_out, ev
    if len(emitted) >= cap:
        return emitted, n_acc, flags, p_at, q_at, W_out, ev
    P = process_row(trow[gamma], T, k, p)
    if P.nonfinite:
        return [], 0, flags | FLAG_NONFINITE_ROW, p_at, q_at, 0.0, ev
    if P.topp_near:
        flags |= FLAG_TOPP_NEAR
        ev["topp_near"].append(gamma)
    u3 = float(uniform(seed, b, gamma, PURPOSE_BONUS, step))
    t = inverse_cdf(P.probs, u3)
    ev["sample"] = {"kind": "bonus", "pos": gamma, "u": u3, "W": float(P.probs.sum()),
                    "weights": P.probs if keep_weights else None}
    emitted.append(t)
    return emitted, n_acc, flags, p_at, q_at, W_out, ev


def _finish(results, B, gamma):
    out = {
        "num_accepted": np.zeros(B, np.int32),
        "out_tokens": np.full((B, gamma + 1), -1, np.int32),
        "num_emitted": np.zeros(B, np.int32),
        "row_flags": np.zeros(B, np.int32),
        "p_at_draft": np.full((B, gamma), np.nan),
        "q_at_draft": np.full((B, gamma), np.nan),
        "residual_sum": np.zeros(B),
        "events": [],
    }
    for b, r in enumerate(results):
        emitted, n_acc, flags, p_at, q_at, W, ev = r
        out["num_accepted"][b] = n_acc
        out["num_emitted"][b] = len(emitted)
        out["out_tokens"][b, :len(emitted)] = emitted
        out["row_flags"][b] = flags
        out["p_at_draft"][b] = p_at
        out["q_at_draft"][b] = q_at
        out["residual_sum"][b] = W
        out["events"].append(ev)
    return out


def _caps(max_new_tokens, B):
    caps = _broadcast(max_new_tokens, B, np.int64)
    return np.where(caps >= 1, caps, NO_CAP)


def verify_sample(target, draft, tokens, temperature, top_k, top_p, max_new_tokens,
                  seed, step=0, eos_id=-1, keep_weights=False):
    """One verification round for every batch row.

    target: [B, gamma+1, V] logits (float32 or bfloat16 values held in float32),
    draft: [B, gamma, V], tokens: [B, gamma] ints.  Per-row parameters are
    scalars or length-B arrays: temperature (0 = greedy row), top_k (0 = off),
    top_p (1 = off), max_new_tokens (<= 0 = no cap).  Returns a dict of numpy
    arrays (see ``_finish``) plus per-row ``events`` for the parity classifier.
    """
    target = np.asarray(target)
    draft = np.asarray(draft)
    tokens = np.asarray(tokens)
    B, g1, V = target.shape
    gamma = g1 - 1
    assert draft.shape == (B, gamma, V) and tokens.shape == (B, gamma)
    T = _broadcast(temperature, B, np.float64)
    K = _broadcast(top_k, B, np.int64)
    Pp = _broadcast(top_p, B, np.float64)
    caps = _caps(max_new_tokens, B)
    results = []
    for b in range(B):
        toks = tokens[b]
        if ((toks < 0) | (toks >= V)).any():
            results.append(([], 0, FLAG_TOKEN_OOR, np.full(gamma, np.nan),
                            np.full(gamma, np.nan), 0.0, {"accept_tests": [], "sample": None, "topp_near": []}))
            continue
        if T[b] == 0.0:
            em, na, fl = _greedy_row(target[b], toks, caps[b], eos_id)
            results.append((em, na, fl, np.full(gamma, np.nan), np.full(gamma, np.nan), 0.0,
                            {"accept_tests": [], "sample": None, "topp_near": []}))
            continue
        results.append(_sample_row(b, target[b], draft[b], toks, T[b], K[b], Pp[b], caps[b],
                                   eos_id, seed, step, keep_weights))
    return _finish(results, B, gamma)


def verify_point_mass(target, tokens, temperature, top_k, top_p, max_new_tokens, seed, step=0,
                      eos_id=-1, keep_weights=False):
    """One verification round for every batch row against deterministic
    drafts (q_i = the point mass on d_i; no draft logits).  Arguments and
    result as ``verify_sample`` without ``draft``; temperature 0 rows are
    verified greedily."""
    target = np.asarray(target)
    tokens = np.asarray(tokens)
    B, g1, V = target.shape
    gamma = g1 - 1
    assert tokens.shape == (B, gamma)
    T = _broadcast(temperature, B, np.float64)
    K = _broadcast(top_k, B, np.int64)
    Pp = _broadcast(top_p, B, np.float64)
    caps = _caps(max_new_tokens, B)
    results = []
    for b in range(B):
        toks = tokens[b]
        if ((toks < 0) | (toks >= V)).any():
            results.append(([], 0, FLAG_TOKEN_OOR, np.full(gamma, np.nan),
                            np.full(gamma, np.nan), 0.0, {"accept_tests": [], "sample": None, "topp_near": []}))
            continue
        if T[b] == 0.0:
            em, na, fl = _greedy_row(target[b], toks, caps[b], eos_id)
            results.append((em, na, fl, np.full(gamma, np.nan), np.full(gamma, np.nan), 0.0,
                            {"accept_tests": [], "sample": None, "topp_near": []}))
            continue
        results.append(_point_mass_row(b, target[b], toks, T[b], K[b], Pp[b], caps[b], eos_id,
                                       seed, step, keep_weights))
    return _finish(results, B, gamma)


def verify_greedy(target, tokens, max_new_tokens=0, eos_id=-1):
    """Greedy verification of every row (temperature, top-k and top-p ignored)."""
    target = np.asarray(target)
    tokens = np.asarray(tokens)
    B, g1, V = target.shape
    gamma = g1 - 1
    assert tokens.shape == (B, gamma)
    caps = _caps(max_new_tokens, B)
    results = []
    for b in range(B):
        toks = tokens[b]
        if ((toks < 0) | (toks >= V)).any():
            em, na, fl = [], 0, FLAG_TOKEN_OOR
        else:
            em, na, fl = _greedy_row(target[b], toks, caps[b], eos_id)
        results.append((em, na, fl, np.full(gamma, np.nan), np.full(gamma, np.nan), 0.0,
                        {"accept_tests": [], "sample": None, "topp_near": []}))
    return _finish(results, B, gamma)


def draft_row_stats(draft, temperature, top_k=0, top_p=1.0):
    """Statistics of each processed draft row, as a drafter that samples q_i
    can hand them to the verifier: with K the kept set (every finite token
    when no truncation is on; the top-k / top-p set otherwise),
    m = max_{v in K} z_v (the row maximum), s = sum_{v in K} exp((z_v - m)/T)
    and the threshold t = min_{v in K} z_v (-inf when top-k and top-p are
    both off), so that q_i(v) = [z_v >= t] exp((z_v - m)/T) / s (the
    temperature division of the tutorial's section 3.3; q is the truncated
    distribution actually sampled, "11.1 核心原理" 11.1.2).  Rows with
    temperature 0, or with NaN / +inf / no finite logit, get NaN.
    Returns float64 [B, gamma, 3] = (m, s, t)."""
    draft = np.asarray(draft, np.float64)
    B, gamma, V = draft.shape
    T = _broadcast(temperature, B, np.float64)
    K = _broadcast(top_k, B, np.int64)
    Pp = _broadcast(top_p, B, np.float64)
    out = np.full((B, gamma, 3), np.nan)
    for b in range(B):
        if T[b] == 0.0:
            continue
        truncated = (0 < K[b] < V) or Pp[b] < 1.0
        for i in range(gamma):
            Q = process_row(draft[b, i], T[b], K[b], Pp[b])
            if Q.nonfinite:
                continue
            z = draft[b, i][Q.kept]
            m = z.max()
            out[b, i, 0] = m
            out[b, i, 1] = np.exp((z - m) / T[b]).sum()
            out[b, i, 2] = z.min() if truncated else -np.inf
    return out


def sample_draft_tokens(draft, temperature, top_k, top_p, seed, step=0, pos0=0):
    """Harness stand-in for the draft model's sampling: d_i ~ q_i.

    Each d_i is drawn by inverse CDF from the processed draft distribution
    with the uniform of purpose DRAFT.  Rows with temperature 0 take the
    draft argmax (what a greedy drafter emits).  A row with NaN / +inf or
    no finite logit defines no distribution, and gets -1 (no token).
    ``draft[:, i]`` is the round's draft position pos0 + i (the uniform's
    counter), so a drafter that samples one position at a time passes one
    column and its position.
    """
    draft = np.asarray(draft)
    B, gamma, V = draft.shape
    T = _broadcast(temperature, B, np.float64)
    K = _broadcast(top_k, B, np.int64)
    Pp = _broadcast(top_p, B, np.float64)
    toks = np.zeros((B, gamma), np.int32)
    for b in range(B):
        for i in range(gamma):
            if T[b] == 0.0:
                g = greedy_argmax(draft[b, i])
                toks[b, i] = -1 if g is None else g
                continue
            Q = process_row(draft[b, i], T[b], K[b], Pp[b])
            if Q.nonfinite:
                toks[b, i] = -1
                continue
            u = float(uniform(seed, b, pos0 + i, PURPOSE_DRAFT, step))
            toks[b, i] = inverse_cdf(Q.probs, u)
    return toks
