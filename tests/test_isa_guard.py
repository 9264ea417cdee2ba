"""Static guards on the gfx950 code of the verify and draft-sampler kernels (CPU only).

1. A cross-lane read ``v_readlane_b32 sD, vS, sIdx`` returns lane sIdx of vS
   whatever EXEC holds.  When the compiler spills vS and reloads it inside a
   branch that only some lanes take, the reload (``scratch_load``) writes the
   active lanes alone, and a read of another lane returns stale data.  An
   index taken from such a read once sent a load out of bounds.  The kernels
   now read such values with uniform loads; the test fails if any dynamically
   indexed ``v_readlane`` reads a VGPR whose last definition (in program
   order) is a scratch reload.
2. No kernel makes a call, and none uses private memory except the
   six-workgroup verify kernel (k_verify_wide), for a few spilled registers
   (at most 64 bytes per lane).  When the compiler keeps a large step out of
   line, it copies the whole argument block to private memory and reads
   every field from there.  On the truncation kernels that cost a third of
   their time.
"""

import os
import re
import shutil
import subprocess

import pytest

from speculative_decoding_verification_sampling_amd import build as specv_build

_LOADS = ("global_load", "buffer_load", "flat_load", "scratch_load", "ds_read", "ds_load")
_NO_VGPR_DEST = ("v_readlane", "v_readfirstlane", "v_cmp", "v_cmpx")


def _vgprs(operand):
    """VGPR numbers named by an operand such as v7 or v[4:7]."""
    m = re.fullmatch(r"v(\d+)", operand)
    if m:
        return [int(m.group(1))]
    m = re.fullmatch(r"v\[(\d+):(\d+)\]", operand)
    if m:
        return list(range(int(m.group(1)), int(m.group(2)) + 1))
    return []


def _functions(asm):
    funcs, cur = {}, None
    for line in asm.splitlines():
        m = re.match(r"^([A-Za-z_][\w.$]*):", line)
        if m and not line.startswith(".L"):
            cur = m.group(1)
            funcs[cur] = []
            continue
        if cur is None or not line.startswith("\t"):
            continue
        text = line.split(";")[0].strip()
        if not text or text.startswith("."):
            continue
        funcs[cur].append(text)
    return funcs


def stale_lane_reads(asm):
    """(function, instruction) pairs: dynamic readlanes of a spill reload."""
    found = []
    for name, body in _functions(asm).items():
        last_def = {}
        for ins in body:
            op, _, rest = ins.partition(" ")
            ops = [o.strip() for o in rest.split(",")]
            if op == "v_readlane_b32" and len(ops) >= 3:
                src, idx = ops[1], ops[2]
                if idx.startswith("s") and any(last_def.get(v) == "scratch" for v in _vgprs(src)):
                    found.append((name, ins))
                continue
            if not ops or op.startswith(_NO_VGPR_DEST):
                continue
            if op.startswith("v_") or op.startswith(_LOADS):
                kind = "scratch" if op.startswith("scratch_load") else "other"
                for v in _vgprs(ops[0]):
                    last_def[v] = kind
    return found


def test_checker_finds_the_fault_pattern():
    # the shape of the original fault: a lane-masked reload, then a
    # dynamically indexed read of that register
    asm = ("kern:\n"
           "\ts_and_saveexec_b64 s[4:5], vcc\n"
           "\tscratch_load_dword v88, off, s32 offset:12\n"
           "\ts_waitcnt vmcnt(0)\n"
           "\tv_readlane_b32 s20, v88, s3\n"
           "\tv_readlane_b32 s21, v88, 63\n"
           "\tv_mov_b32_e32 v88, 0\n"
           "\tv_readlane_b32 s22, v88, s3\n")
    assert stale_lane_reads(asm) == [("kern", "v_readlane_b32 s20, v88, s3")]


@pytest.fixture(scope="module", params=[("specv_kernels.hip", "k_verify"),
                                        ("specv_draft.hip", "k_sample_draft")])
def compiled(request, tmp_path_factory):
    """(kernel name stem, gfx950 assembly) of one source."""
    if shutil.which(specv_build.hipcc()) is None and not os.path.exists(specv_build.hipcc()):
        pytest.skip("hipcc not available")
    source, kernel = request.param
    src = os.path.join(os.path.dirname(specv_build.__file__), "csrc", source)
    tmp = tmp_path_factory.mktemp("isa")
    out = tmp / "kernels.s"
    flags = [f for f in specv_build.FLAGS if f not in ("-shared", "-fPIC")]
    cmd = [specv_build.hipcc(), *flags, "-I", specv_build.INCLUDE, "-I", os.path.dirname(src),
           "--offload-device-only", "-S", src, "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True, cwd=str(tmp))
    assert r.returncode == 0, r.stderr[-2000:]
    asm = out.read_text()
    assert kernel in asm
    return kernel, asm


def test_no_dynamic_lane_read_of_a_spill_reload(compiled):
    _, asm = compiled
    assert stale_lane_reads(asm) == []


def private_use(asm):
    """(kernel, private bytes per lane) of kernels with private memory, and
    the number of call instructions."""
    sizes = re.findall(r"\.name:\s+(\S+)\s*\n\s+\.private_segment_fixed_size:\s+(\d+)", asm)
    return [(n, int(v)) for n, v in sizes if int(v) > 0], len(re.findall(r"\bs_swappc_b64\b", asm))


def test_private_use_checker():
    asm = ("    .name:           kern_a\n    .private_segment_fixed_size: 0\n"
           "    .name:           kern_b\n    .private_segment_fixed_size: 368\n"
           "\ts_swappc_b64 s[30:31], s[0:1]\n")
    assert private_use(asm) == ([("kern_b", 368)], 1)


# private bytes per lane allowed for spills in the six-workgroup verify kernel
WIDE_SPILL_BYTES = 64


def test_kernels_use_no_private_memory_and_make_no_calls(compiled):
    kernel, asm = compiled
    pairs = re.findall(r"\.name:\s+\S+\s*\n\s+\.private_segment_fixed_size:", asm)
    assert len(pairs) >= 4, "kernel metadata not found"
    used, calls = private_use(asm)
    assert calls == 0
    assert [(n, v) for n, v in used if not ("k_verify_wide" in n and v <= WIDE_SPILL_BYTES)] == []
