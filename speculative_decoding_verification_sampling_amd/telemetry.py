"""Acceptance telemetry and a dynamic-gamma helper (host side).

What the pages say, restated:

* The expected number of tokens one round yields when every draft is
  accepted independently with probability alpha is
  E(gamma) = (1 - alpha^(gamma+1)) / (1 - alpha) ("Fast Inference from
  Transformers via Speculative Decoding"; the tutorial "投机解码 Speculative
  Decoding", section 2.3, which prints E(4) = 2.77 and E(8) = 3.20 at
  alpha = 0.7).
* The speed-up of a round over plain decoding is about the expected tokens
  divided by the cost of the round, gamma draft steps plus one target
  verification (tutorial, section 2.3; the ICML summary names the draft/target
  step-cost ratio c): E(gamma) / (gamma * c + 1) in target-step units.
* gamma should follow the acceptance: raise it when rounds are fully
  accepted, lower it when the first draft is already rejected (tutorial,
  section 3.2).

``AcceptanceTelemetry`` reads the outputs of verify calls (num_accepted,
num_emitted, row_flags; host or device tensors, or numpy arrays) and keeps,
per draft position, how many accept tests ran and how many passed.  A round
is classified from its outputs alone:

* rejected at n: n drafts accepted and one token more emitted (n < gamma);
* fully accepted: gamma drafts accepted (the bonus may be cut by a cap);
* stopped: as many tokens emitted as accepted, fewer than gamma, so a cap or
  an EOS ended the round before the test at position n ran;
* rows with a data-fault flag (out-of-range token, non-finite row,
  truncation overflow, unsupported truncation, internal) are not counted.

``DynamicGamma`` applies the section 3.2 rule per batch row;
``best_gamma`` picks the gamma that maximises E(gamma) / (gamma * c + 1).
"""

import numpy as np

# row_flags bits that make a round's outcome not a measurement of acceptance
_FAULT_FLAGS = (1 << 0) | (1 << 1) | (1 << 4) | (1 << 6) | (1 << 7)


def expected_tokens(alpha, gamma):
    """E(gamma) = (1 - alpha^(gamma+1)) / (1 - alpha); gamma + 1 at alpha = 1."""
    alpha = float(alpha)
    if alpha >= 1.0:
        return gamma + 1.0
    return (1.0 - alpha ** (gamma + 1)) / (1.0 - alpha)


def speedup(alpha, gamma, c):
    """Expected tokens per round over the round's cost in target steps."""
    return expected_tokens(alpha, gamma) / (gamma * float(c) + 1.0)


def best_gamma(alpha, c, gamma_max=31, gamma_min=1):
    """The gamma in [gamma_min, gamma_max] with the largest ``speedup``
    (the smallest such gamma on ties)."""
    best, best_s = gamma_min, -1.0
    for g in range(gamma_min, gamma_max + 1):
        s = speedup(alpha, g, c)
        if s > best_s * (1 + 1e-12):
            best, best_s = g, s
    return best


def _host(x):
    if x is None:
        return None
    if hasattr(x, "detach"):
        x = x.detach().cpu().numpy()
    return np.asarray(x)


def classify(num_accepted, num_emitted, row_flags, gamma):
    """Per row: (kind, n) with kind 0 = not counted, 1 = rejected at n,
    2 = fully accepted, 3 = stopped by a cap / EOS before the test at n."""
    na = _host(num_accepted).astype(np.int64)
    ne = _host(num_emitted).astype(np.int64)
    fl = _host(row_flags)
    fl = np.zeros_like(na) if fl is None else fl.astype(np.int64)
    kind = np.zeros_like(na)
    ok = (fl & _FAULT_FLAGS) == 0
    full = ok & (na >= gamma)
    rej = ok & (na < gamma) & (ne == na + 1)
    stop = ok & (na < gamma) & (ne == na)
    kind[rej] = 1
    kind[full] = 2
    kind[stop] = 3
    return kind, na


class AcceptanceTelemetry:
    """Running per-position acceptance statistics of verify rounds."""

    def __init__(self, max_gamma=31):
        self.max_gamma = max_gamma
        self.tests = np.zeros(max_gamma, np.int64)      # accept tests run at position i
        self.passed = np.zeros(max_gamma, np.int64)     # ... and passed
        self.rounds = 0
        self.tokens = 0                                  # tokens emitted by counted rounds
        self.full = 0                                    # fully accepted rounds
        self.first_rejected = 0                          # rounds rejected at position 0

    def update(self, out, gamma):
        """Add one call's outputs (a dict with num_accepted, num_emitted and
        optionally row_flags, as the Verifier returns)."""
        if gamma > self.max_gamma:
            raise ValueError("gamma above the telemetry's max_gamma")
        kind, n = classify(out["num_accepted"], out["num_emitted"], out.get("row_flags"), gamma)
        ne = _host(out["num_emitted"]).astype(np.int64)
        counted = kind > 0
        # every counted round passed the tests at positions 0 .. n-1; a
        # rejected round also ran (and failed) the test at n
        acc = np.bincount(np.minimum(n[counted], gamma), minlength=gamma + 1)
        passed = acc[::-1].cumsum()[::-1][1:gamma + 1]       # rounds with n > i
        failed = np.bincount(n[kind == 1], minlength=gamma)[:gamma]
        self.passed[:gamma] += passed
        self.tests[:gamma] += passed + failed
        self.rounds += int(counted.sum())
        self.tokens += int(ne[counted].sum())
        self.full += int((kind == 2).sum())
        self.first_rejected += int(failed[0]) if gamma > 0 else 0

    def position_rates(self):
        """Acceptance rate per draft position (NaN where no test ran)."""
        with np.errstate(invalid="ignore", divide="ignore"):
            return np.where(self.tests > 0, self.passed / np.maximum(self.tests, 1), np.nan)

    def alpha(self):
        """Acceptance rate over all tests (the maximum-likelihood alpha when
        tests pass independently with one probability)."""
        t = self.tests.sum()
        return float(self.passed.sum() / t) if t else float("nan")

    def tokens_per_round(self):
        return self.tokens / self.rounds if self.rounds else float("nan")

    def summary(self, gamma):
        a = self.alpha()
        return {"rounds": self.rounds, "alpha": a,
                "position_rates": self.position_rates()[:gamma].tolist(),
                "tokens_per_round": self.tokens_per_round(),
                "expected_tokens": expected_tokens(a, gamma) if a == a else float("nan"),
                "fully_accepted": self.full, "first_rejected": self.first_rejected}


class DynamicGamma:
    """Per-row draft length following the acceptance (tutorial section 3.2):
    after a fully accepted round the row's gamma grows by one, after a round
    rejected at the first draft it shrinks by one, otherwise it stays;
    always within [gamma_min, gamma_max].  Rounds stopped by a cap / EOS or
    with a data-fault flag leave gamma unchanged.

    A verify call runs one gamma for all its rows, so rows whose gammas
    differ are verified in separate calls (``groups``)."""

    def __init__(self, batch, gamma0=5, gamma_min=1, gamma_max=8):
        if not (1 <= gamma_min <= gamma0 <= gamma_max):
            raise ValueError("need 1 <= gamma_min <= gamma0 <= gamma_max")
        self.gamma_min, self.gamma_max = gamma_min, gamma_max
        self.gammas = np.full(batch, gamma0, np.int64)

    def update(self, out, gamma, rows=None):
        """``out``: the outputs of a call that verified ``rows`` (indices
        into the batch, all of them by default) with draft length ``gamma``."""
        rows = np.arange(len(self.gammas)) if rows is None else np.asarray(rows)
        kind, n = classify(out["num_accepted"], out["num_emitted"], out.get("row_flags"), gamma)
        g = self.gammas[rows]
        g = np.where(kind == 2, g + 1, np.where((kind == 1) & (n == 0), g - 1, g))
        self.gammas[rows] = np.clip(g, self.gamma_min, self.gamma_max)
        return self.gammas

    def groups(self):
        """{gamma: row indices} for the next round."""
        return {int(g): np.nonzero(self.gammas == g)[0] for g in np.unique(self.gammas)}
