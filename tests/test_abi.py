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
                                None, None, 1)
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


def test_struct_layouts_match_the_binding(tmp_path):
    """The records the binding builds or reads as tensors: specv_row_params
    (4 x 4 bytes: float, int32, float, int32) and specv_draft_stats (float
    max, sum, threshold, int32 flags), compiled from the public header."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    src = tmp_path / "layout.c"
    src.write_text(
        '#include <stddef.h>\n#include <stdio.h>\n#include "specv.h"\n'
        'int main(void) {\n'
        '  printf("%zu %zu %zu %zu %zu\\n", sizeof(specv_row_params), offsetof(specv_row_params, top_k),\n'
        '         offsetof(specv_row_params, top_p), offsetof(specv_row_params, max_new_tokens), 0ul);\n'
        '  printf("%zu %zu %zu %zu\\n", sizeof(specv_draft_stats), offsetof(specv_draft_stats, sum),\n'
        '         offsetof(specv_draft_stats, threshold), offsetof(specv_draft_stats, flags));\n'
        '  return 0;\n}\n')
    exe = tmp_path / "layout"
    inc = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include")
    subprocess.run([gcc, "-std=c99", "-I", inc, str(src), "-o", str(exe)], check=True)
    lines = subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split("\n")
    assert lines[0].split()[:4] == ["16", "4", "8", "12"]
    assert lines[1].split() == ["16", "4", "8", "12"]


def test_binding_exposes_every_entry_point():
    for m in ("verify_sample", "verify_sample_qstats", "verify_point_mass", "verify_greedy",
              "sample_draft", "set_profiling", "profile", "close"):
        assert callable(getattr(sv.Verifier, m, None)), m
