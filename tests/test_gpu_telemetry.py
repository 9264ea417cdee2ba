"""Acceptance telemetry read from device outputs of the serving batch,
against the same telemetry over the oracle's outputs for the same inputs."""

import numpy as np
import pytest
import torch

import oracle
import synth
import speculative_decoding_verification_sampling_amd as sv
from speculative_decoding_verification_sampling_amd import telemetry as tm

pytestmark = pytest.mark.gpu


def test_telemetry_on_device_outputs():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    sv.load_library()
    w = synth.serving_batch()
    dev = torch.device("cuda:0")
    prm = sv.make_row_params(w.B, w.temperature, w.top_k, w.top_p, w.max_new_tokens, dev)
    tel_gpu, tel_orc = tm.AcceptanceTelemetry(8), tm.AcceptanceTelemetry(8)
    tf, df = w.target_f32(), w.draft_f32()
    with sv.Verifier(w.B, w.gamma, w.V) as v:
        t, d = w.target.to(dev), w.draft.to(dev)
        tok = torch.from_numpy(w.tokens).to(dev)
        for step in range(3):
            out = v.verify_sample(t, d, tok, prm, w.seed, step)
            tel_gpu.update(out, w.gamma)          # device tensors, read on the host
            orc = oracle.verify_sample(tf, df, w.tokens, w.temperature, w.top_k, w.top_p,
                                       w.max_new_tokens, w.seed, step)
            tel_orc.update(orc, w.gamma)
    assert tel_gpu.rounds == tel_orc.rounds == 3 * w.B
    # parity makes the counts equal up to the rare tolerated boundary cases
    assert np.abs(tel_gpu.tests - tel_orc.tests).sum() <= 2
    assert np.abs(tel_gpu.passed - tel_orc.passed).sum() <= 2
