"""The C-ABI library builds, loads and exports every symbol include/specv.h
declares; host-side argument validation works without a GPU (no compute)."""

import ctypes
import os
import re

import pytest

import speculative_decoding_verification_sampling_amd as sv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_symbols():
    text = open(os.path.join(ROOT, "include", "specv.h")).read()
    return sorted(set(re.findall(r"SPECV_API\s+[\w\s\*]+?\b(specv_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(sv.library_path()):
        from speculative_decoding_verification_sampling_amd import build
        build.build()
    return sv.load_library()


def test_header_declares_the_entry_points():
    assert _declared_symbols() == sorted(sv.EXPORTED_SYMBOLS)


def test_every_declared_symbol_is_exported(lib):
    for name in _declared_symbols():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for code in range(9):
        assert lib.specv_status_string(code)


def test_create_rejects_bad_config_before_touching_a_device(lib):
    bad = [
        sv._Config(0, 0, 5, 1000, 0),        # max_batch < 1
        sv._Config(0, 1, 33, 1000, 0),       # gamma above SPECV_MAX_GAMMA
        sv._Config(0, 1, 5, 0, 0),           # V < 1
        sv._Config(0, 1, 5, 524289, 0),      # V above SPECV_MAX_VOCAB
        sv._Config(0, 1, 5, 1000, 1025),     # top_k above SPECV_MAX_TOP_K
    ]
    for cfg in bad:
        h = ctypes.c_void_p()
        assert lib.specv_create(ctypes.byref(cfg), ctypes.byref(h)) == 6     # SPECV_E_PARAM
        assert not h.value
    assert lib.specv_create(None, None) == 1                                 # SPECV_E_NULL


def test_verify_rejects_null_handle(lib):
    rc = lib.specv_verify_sample(None, None, None, 0, 0, None, 0, 0, 1, 1, 1, 1,
                                 None, None, 0, 0, -1, None, None, None, None, None)
    assert rc == 1
    rc = lib.specv_verify_greedy(None, None, None, 0, 0, 1, 1, 1, 1, None, None, -1,
                                 None, None, None, None)
    assert rc == 1
    rc = lib.specv_verify_point_mass(None, None, None, 0, 0, 1, 1, 1, 1, None, None, 0, 0, -1,
                                     None, None, None, None, None)
    assert rc == 1
    rc = lib.specv_verify_sample_qstats(None, None, None, 0, 0, None, 0, 0, None, 0, 1, 1, 1, 1,
                                        None, None, 0, 0, -1, None, None, None, None, None)
    assert rc == 1
    rc = lib.specv_sample_draft(None, None, None, 0, 0, 1, 1, 1, 1, 0, None, 0, 0,
                                None, None, None, 1)
    assert rc == 1
    assert lib.specv_destroy(None) == 0


def test_row_params_layout():
    import numpy as np
    p = sv.make_row_params(3, temperature=[0.7, 0.0, 1.0], top_k=[0, 50, 5],
                           top_p=[1.0, 0.9, 0.5], max_new_tokens=[0, 3, 9], device="cpu")
    a = p.numpy()
    assert a.shape == (3, 4)
    assert np.allclose(a[:, 0].view(np.float32), [0.7, 0.0, 1.0])
    assert a[:, 1].tolist() == [0, 50, 5]
    assert np.allclose(a[:, 2].view(np.float32), [1.0, 0.9, 0.5])
    assert a[:, 3].tolist() == [0, 3, 9]
