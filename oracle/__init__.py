"""CPU oracle for the speculative-sampling verify step.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call,
link or execute anything in this package: only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py``
use it.  It shares no code with the HIP library (no kernels, headers,
helpers, tables or constant generators); the only code both sides see is
the seeded input generator in ``synth/``, which holds none of the method's
arithmetic.

Everything here is plain, slow and meant to be checked against the pages by
eye: numpy in float64, one batch row at a time, one position at a time.

Sources (cited by page title and section):

* "Fast Inference from Transformers via Speculative Decoding" (summary of
  the ICML 2023 paper): speculative sampling, the acceptance rule
  min(1, p/q), the residual distribution norm(max(0, p - q)), the bonus token
  after full acceptance, the acceptance rate alpha and E[N].
* "11.1 核心原理: Draft + Verify 与 Rejection Sampling": position alignment
  (11.1.1), greedy vs stochastic acceptance and the processed proposal q
  (11.1.2), the single-chain pseudo-code 10-1, the proof and worked example
  (11.1.3).
* "投机解码 Speculative Decoding" tutorial: E(gamma) (section 2.3), the
  temperature division (section 3.3).

Parity status of each function is listed in its module header.
"""

from .philox import philox4x32_10, uniform, PURPOSE_DRAFT, PURPOSE_ACCEPT, PURPOSE_RESIDUAL, PURPOSE_BONUS
from .process import process_row, ProcessedRow, greedy_argmax
from .verify import (
    verify_sample,
    verify_point_mass,
    verify_greedy,
    inverse_cdf,
    cdf_interval,
    sample_draft_tokens,
    draft_row_stats,
    FLAG_TOKEN_OOR,
    FLAG_NONFINITE_ROW,
    FLAG_Q_ZERO,
    FLAG_RESIDUAL_FALLBACK,
    FLAG_TOPP_NEAR,
)

__all__ = [
    "philox4x32_10",
    "uniform",
    "PURPOSE_DRAFT",
    "PURPOSE_ACCEPT",
    "PURPOSE_RESIDUAL",
    "PURPOSE_BONUS",
    "process_row",
    "ProcessedRow",
    "greedy_argmax",
    "verify_sample",
    "verify_greedy",
    "inverse_cdf",
    "cdf_interval",
    "sample_draft_tokens",
    "FLAG_TOKEN_OOR",
    "FLAG_NONFINITE_ROW",
    "FLAG_Q_ZERO",
    "FLAG_RESIDUAL_FALLBACK",
    "FLAG_TOPP_NEAR",
]
