"""Per-distribution processing (oracle side).  TEST INFRASTRUCTURE.

"11.1 核心原理", section 11.1.2: p_i and q_i are the distributions each
model actually samples from, after its temperature, top-k / top-p and
constraints; the proposal q must be stored as the truncated distribution
actually sampled, never the untruncated softmax.  The tutorial's section 3.3
divides logits by the temperature before the softmax.

Readings fixed here (the pages do not define these details):

* order: temperature, then top-k, then top-p, then renormalise over the
  kept set; constraints and penalties are out of scope;
* temperature T > 0 divides the logits; T == 0 selects greedy verification
  (handled by the caller, see ``greedy_argmax``);
* top-k keeps every token whose raw logit is >= the k-th largest raw logit
  (counted with multiplicity), so ties at the threshold are all kept and the
  kept set can be larger than k; k <= 0 or k >= V means off.  Dividing by
  T > 0 preserves order, so the set is decided on the raw input values;
* top-p keeps the smallest "value >= t" set (over the top-k survivors) whose
  probability under the top-k-renormalised softmax is >= top_p; tokens tied
  at the boundary value are all kept, the largest logit is always kept;
  top_p >= 1 means off.  When the deciding cumulative mass lies within 1e-5
  of top_p the set may differ between float32 and float64 arithmetic, and
  the row is marked (``topp_near``);
* the greedy argmax is taken over the raw input logits, lowest token index on
  ties (the pages ask only for consistent tie-breaking).

Pins: ``tests/test_oracle_process.py`` checks the softmax against
``torch.softmax`` in float64, and the top-k / top-p sets against a brute
force written from the stated definition with a full sort of every row.
"""

from dataclasses import dataclass

import numpy as np

TOPP_NEAR_WINDOW = 1e-5


@dataclass
class ProcessedRow:
    probs: np.ndarray      # float64 [V], zero outside the kept set
    kept: np.ndarray       # bool [V]
    nonfinite: bool        # NaN / +inf present, or nothing finite in the kept set
    topp_near: bool        # top-p decision within 1e-5 of the threshold


def greedy_argmax(z):
    """Lowest index among the maximal raw logits; None if the row has NaN/+inf
    or no finite value."""
    z = np.asarray(z, dtype=np.float64)
    if np.isnan(z).any() or np.isposinf(z).any() or not np.isfinite(z).any():
        return None
    return int(np.argmax(z))   # numpy returns the first maximal index


def _masked_softmax(x, keep):
    """softmax of x restricted to the tokens in ``keep``; zero elsewhere."""
    out = np.zeros_like(x)
    xs = x[keep]
    m = xs.max()
    e = np.exp(xs - m)
    out[keep] = e / e.sum()
    return out


def process_row(z, temperature, top_k=0, top_p=1.0):
    """Processed distribution of one logits row (temperature > 0)."""
    z = np.asarray(z, dtype=np.float64)     # exact upcast of fp32 / bf16 values
    V = z.shape[0]
    if np.isnan(z).any() or np.isposinf(z).any() or not np.isfinite(z).any():
        return ProcessedRow(np.zeros(V), np.zeros(V, bool), True, False)
    x = z / float(temperature)

    # top-k on raw values, ties at the threshold kept
    if 0 < top_k < V:
        kth = np.sort(z)[::-1][top_k - 1]
        keep = z >= kth
    else:
        keep = np.ones(V, dtype=bool)
    keep &= np.isfinite(z)           # -inf tokens carry no mass
    if not keep.any():
        return ProcessedRow(np.zeros(V), keep, True, False)

    pi = _masked_softmax(x, keep)

    near = False
    if top_p < 1.0:
        # kept tokens by value, descending; the mass of {value >= level} is the
        # running sum at the last token of each run of equal values
        idx = np.nonzero(keep)[0]
        order = np.argsort(-z[idx], kind="stable")
        zs = z[idx][order]
        cum = np.cumsum(pi[idx][order])
        level_end = np.nonzero(np.append(zs[1:] != zs[:-1], True))[0]
        level_mass = cum[level_end]
        j = int(np.searchsorted(level_mass, top_p, side="left"))   # first mass >= top_p
        j = min(j, len(level_end) - 1)
        cut = zs[level_end[j]]
        near = abs(level_mass[j] - top_p) < TOPP_NEAR_WINDOW or (
            j > 0 and abs(level_mass[j - 1] - top_p) < TOPP_NEAR_WINDOW)
        keep = keep & (z >= cut)

    probs = _masked_softmax(x, keep)
    return ProcessedRow(probs, keep, False, near)
