"""Seeded synthetic workloads for the verify step.

This module is the ONLY code that both the CPU oracle's tests and the HIP
path's tests/bench see.  It holds none of the method's arithmetic (no
softmax, no truncation, no acceptance test, no inverse CDF): it draws logits
with numpy's PCG64, casts them to the stored dtype, and stands in for the
draft model when draft tokens are needed.

Logit recipe (shared by the five workloads):

* target logits z ~ N(0, sigma_t^2) i.i.d.; in the "vocabulary-like"
  workloads 20 distinct token ids per (row, position), drawn uniformly without
  replacement, get +8 ("likely" tokens);
* draft logits = target logits + N(0, sigma_d^2) for positions 0..gamma-1;
* stored as float32, or rounded to bfloat16 (round to nearest even, by
  torch on the CPU); every consumer reads the same stored values.

Draft tokens (the draft model's proposals) come from a stand-in sampler:
for untruncated stochastic rows the Gumbel-max trick,
d = argmax_v(z_draft[v] / T + G_v) with G_v standard Gumbel noise from
PCG64, which draws d from softmax(z_draft / T); for greedy rows the draft
argmax.  Workloads whose proposal distribution is truncated (top-k / top-p)
leave ``tokens`` as None: the caller draws them from the truncated proposal.
"""

from dataclasses import dataclass, field

import numpy as np
import torch

BOOST_COUNT = 20
BOOST = 8.0


@dataclass
class Workload:
    name: str
    B: int
    gamma: int
    V: int
    dtype: str                     # "f32" or "bf16"
    target: torch.Tensor           # CPU tensor [B, gamma+1, V] of ``dtype``
    draft: torch.Tensor            # CPU tensor [B, gamma, V]
    tokens: np.ndarray             # int32 [B, gamma] or None
    temperature: np.ndarray        # float32 [B]; 0 = greedy row
    top_k: np.ndarray              # int32 [B]; 0 = off
    top_p: np.ndarray              # float32 [B]; 1 = off
    max_new_tokens: np.ndarray     # int32 [B]; <= 0 = no cap
    seed: int                      # Philox seed of the verify call
    step: int = 0
    eos_id: int = -1
    meta: dict = field(default_factory=dict)

    def target_f32(self):
        """Exact float32 view of the stored target values."""
        return self.target.to(torch.float32).numpy()

    def draft_f32(self):
        return self.draft.to(torch.float32).numpy()

    def bytes_per_element(self):
        return 2 if self.dtype == "bf16" else 4


def _store(x, dtype):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16) if dtype == "bf16" else t


def make_logits(rng, B, gamma, V, sigma_t, sigma_d, boost_count=0, boost=BOOST):
    """target [B, gamma+1, V] and draft [B, gamma, V] float32 logits.

    ``sigma_d`` is a scalar or a per-row array of length B.
    """
    target = rng.standard_normal((B, gamma + 1, V), dtype=np.float32)
    target *= np.float32(sigma_t)
    if boost_count:
        for b in range(B):
            for i in range(gamma + 1):
                ids = rng.choice(V, size=boost_count, replace=False)
                target[b, i, ids] += np.float32(boost)
    sd = np.broadcast_to(np.asarray(sigma_d, np.float32), (B,))
    noise = rng.standard_normal((B, gamma, V), dtype=np.float32)
    noise *= sd[:, None, None]
    draft = target[:, :gamma, :] + noise
    return target, draft


def gumbel_max_tokens(rng, draft_vals, temperature):
    """Stand-in draft sampler: argmax(z / T + Gumbel) per (row, position);
    plain argmax for rows with T == 0.  ``draft_vals`` holds the stored
    (already rounded) draft values as float32."""
    B, gamma, V = draft_vals.shape
    toks = np.zeros((B, gamma), np.int32)
    for b in range(B):
        T = float(temperature[b])
        for i in range(gamma):
            z = draft_vals[b, i].astype(np.float64)
            if T == 0.0:
                toks[b, i] = int(np.argmax(z))
                continue
            g = -np.log(-np.log(rng.random(V) * (1 - 2e-16) + 1e-16))
            toks[b, i] = int(np.argmax(z / T + g))
    return toks


def _params(B, T, k=0, p=1.0, cap=0):
    return (np.broadcast_to(np.asarray(T, np.float32), (B,)).copy(),
            np.broadcast_to(np.asarray(k, np.int32), (B,)).copy(),
            np.broadcast_to(np.asarray(p, np.float32), (B,)).copy(),
            np.broadcast_to(np.asarray(cap, np.int32), (B,)).copy())


def tiny(seed=1001, sample_tokens=False):
    """B=1, gamma=4, V=32, float32; z ~ N(0, 2^2), draft noise N(0, 1); T=1."""
    rng = np.random.default_rng(seed)
    t, d = make_logits(rng, 1, 4, 32, 2.0, 1.0)
    T, k, p, cap = _params(1, 1.0)
    tokens = gumbel_max_tokens(rng, d, T) if sample_tokens else None
    return Workload("tiny-V32-g4-f32", 1, 4, 32, "f32", _store(t, "f32"), _store(d, "f32"),
                    tokens, T, k, p, cap, seed=0x5EED0001)


def llama_vocab(sigma_d, seed=1002):
    """B=1, gamma=4, V=32000, float32; N(0, 3^2) + 20 boosted tokens; T=1."""
    rng = np.random.default_rng(seed)
    t, d = make_logits(rng, 1, 4, 32000, 3.0, sigma_d, BOOST_COUNT)
    T, k, p, cap = _params(1, 1.0)
    tokens = gumbel_max_tokens(rng, d, T)
    return Workload(f"llama-V32000-g4-f32-sd{sigma_d}", 1, 4, 32000, "f32", _store(t, "f32"),
                    _store(d, "f32"), tokens, T, k, p, cap, seed=0x5EED0002 + int(seed))


def llama_vocab_rounds(sigma_d, rounds=1000, seed=1012):
    """The Llama-style workload with fresh logits every round: ``rounds``
    independent rows (B = rounds, gamma=4, V=32000, float32), each drawn as
    ``llama_vocab`` draws its one row (N(0, 3^2) + 20 boosted tokens, draft
    noise sigma_d), with draft tokens from the stand-in sampler; T=1.  The
    data seed depends on sigma_d, so the three noise levels see different
    rows."""
    rng = np.random.default_rng(seed * 1000 + int(round(sigma_d * 10)))
    t, d = make_logits(rng, rounds, 4, 32000, 3.0, sigma_d, BOOST_COUNT)
    T, k, p, cap = _params(rounds, 1.0)
    tokens = gumbel_max_tokens(rng, d, T)
    return Workload(f"llama-rounds{rounds}-V32000-g4-f32-sd{sigma_d}", rounds, 4, 32000, "f32",
                    _store(t, "f32"), _store(d, "f32"), tokens, T, k, p, cap,
                    seed=0x5EED0012 + int(round(sigma_d * 10)))


def serving_batch(seed=1003, B=64, gamma=5, V=128256):
    """B=64, gamma=5, V=128256, bfloat16; N(0, 3^2) + boost, draft noise
    N(0, 1.5^2); T=0.7; no truncation."""
    rng = np.random.default_rng(seed)
    t, d = make_logits(rng, B, gamma, V, 3.0, 1.5, BOOST_COUNT)
    tb, db = _store(t, "bf16"), _store(d, "bf16")
    T, k, p, cap = _params(B, 0.7)
    tokens = gumbel_max_tokens(rng, db.to(torch.float32).numpy(), T)
    return Workload(f"serving-B{B}-V{V}-g{gamma}-bf16", B, gamma, V, "bf16", tb, db, tokens,
                    T, k, p, cap, seed=0x5EED0003)


def truncated(seed=1004, B=32, gamma=5, V=152064):
    """B=32, gamma=5, V=152064, bfloat16 as the serving batch; T=0.7,
    top-k=50, top-p=0.9 on both target and draft.  ``tokens`` is None: the
    proposals must be drawn from the truncated draft distribution."""
    rng = np.random.default_rng(seed)
    t, d = make_logits(rng, B, gamma, V, 3.0, 1.5, BOOST_COUNT)
    T, k, p, cap = _params(B, 0.7, 50, 0.9)
    return Workload(f"truncated-B{B}-V{V}-g{gamma}-bf16-k50-p0.9", B, gamma, V, "bf16",
                    _store(t, "bf16"), _store(d, "bf16"), None, T, k, p, cap, seed=0x5EED0004)


def mixed(seed=1005, B=256, gamma=8, V=128256):
    """B=256, gamma=8, V=128256, bfloat16; per-row draft noise sigma_d ~
    U[0.3, 4.0]; even rows stochastic (T=1), odd rows greedy (T=0, tokens =
    draft argmax); per-row caps max_new_tokens ~ U{1..9}."""
    rng = np.random.default_rng(seed)
    sd = rng.uniform(0.3, 4.0, size=B).astype(np.float32)
    t, d = make_logits(rng, B, gamma, V, 3.0, sd, BOOST_COUNT)
    tb, db = _store(t, "bf16"), _store(d, "bf16")
    T = np.where(np.arange(B) % 2 == 0, 1.0, 0.0).astype(np.float32)
    _, k, p, _ = _params(B, 1.0)
    cap = rng.integers(1, 10, size=B).astype(np.int32)
    tokens = gumbel_max_tokens(rng, db.to(torch.float32).numpy(), T)
    return Workload(f"mixed-B{B}-V{V}-g{gamma}-bf16", B, gamma, V, "bf16", tb, db, tokens,
                    T, k, p, cap, seed=0x5EED0005, meta={"sigma_d": sd})


WORKLOADS = {
    "tiny": tiny,
    "llama_vocab": llama_vocab,
    "llama_vocab_rounds": llama_vocab_rounds,
    "serving_batch": serving_batch,
    "truncated": truncated,
    "mixed": mixed,
}
