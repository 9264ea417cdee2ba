"""Python binding of libspecv, the speculative-sampling verify step for MI355X.

Argument marshalling only: every step of the verify path runs in the HIP
kernels of ``libspecv.so``.  PyTorch supplies device memory (tensors) and
the stream (``torch.cuda.current_stream()``); no torch computation happens
on the path.  Build the library first with
``python -m speculative_decoding_verification_sampling_amd.build``; if it is
missing, importing works but every call raises.

    v = Verifier(max_batch=64, max_gamma=5, max_vocab=128256)
    params = make_row_params(64, temperature=0.7, device="cuda")
    out = v.verify_sample(target, draft, tokens, params, seed=1234)
    out["out_tokens"], out["num_emitted"], out["num_accepted"], out["row_flags"]
"""

import ctypes
import os

import numpy as np
import torch

__all__ = [
    "Verifier",
    "make_row_params",
    "load_library",
    "library_path",
    "SpecvError",
    "FLAG_TOKEN_OOR",
    "FLAG_NONFINITE_ROW",
    "FLAG_Q_ZERO",
    "FLAG_RESIDUAL_FALLBACK",
    "FLAG_CAND_OVERFLOW",
    "FLAG_TOPP_NEAR",
    "FLAG_UNSUPPORTED",
    "FLAG_INTERNAL",
    "EXPORTED_SYMBOLS",
    "read_ceiling",
    "verify_sample_noalloc",
    "debug_set_wait_limit",
]

_HERE = os.path.dirname(os.path.abspath(__file__))

FLAG_TOKEN_OOR = 1 << 0
FLAG_NONFINITE_ROW = 1 << 1
FLAG_Q_ZERO = 1 << 2
FLAG_RESIDUAL_FALLBACK = 1 << 3
FLAG_CAND_OVERFLOW = 1 << 4
FLAG_TOPP_NEAR = 1 << 5
FLAG_UNSUPPORTED = 1 << 6
FLAG_INTERNAL = 1 << 7

SPECV_F32 = 0
SPECV_BF16 = 1

EXPORTED_SYMBOLS = ("specv_create", "specv_verify_sample", "specv_verify_point_mass",
                    "specv_verify_sample_qstats", "specv_sample_draft", "specv_verify_greedy",
                    "specv_destroy", "specv_status_string", "specv_set_profiling",
                    "specv_get_profile", "specv_get_profile_samples", "specv_read_ceiling",
                    "specv_verify_sample_noalloc", "specv_debug_set_wait_limit")


class SpecvError(RuntimeError):
    pass


class _Config(ctypes.Structure):
    _fields_ = [("device", ctypes.c_int), ("max_batch", ctypes.c_int),
                ("max_gamma", ctypes.c_int), ("max_vocab", ctypes.c_int),
                ("max_top_k", ctypes.c_int)]


class _Diag(ctypes.Structure):
    _fields_ = [("p_at_draft", ctypes.c_void_p), ("q_at_draft", ctypes.c_void_p),
                ("residual_sum", ctypes.c_void_p)]


_lib = None


def library_path():
    return os.environ.get("SPECV_LIBRARY", os.path.join(_HERE, "libspecv.so"))


def load_library():
    """Load libspecv.so (once).  Raises SpecvError if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise SpecvError(f"libspecv.so not found at {path}; build it with "
                         "`python -m speculative_decoding_verification_sampling_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i32, i64, u32, u64 = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                              ctypes.c_uint32, ctypes.c_uint64)
    lib.specv_create.argtypes = [ctypes.POINTER(_Config), ctypes.POINTER(vp)]
    lib.specv_create.restype = ctypes.c_int
    lib.specv_destroy.argtypes = [vp]
    lib.specv_destroy.restype = ctypes.c_int
    lib.specv_status_string.argtypes = [ctypes.c_int]
    lib.specv_status_string.restype = ctypes.c_char_p
    lib.specv_verify_sample.argtypes = [
        vp, vp,
        vp, i64, i64,
        vp, i64, i64,
        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
        vp, vp,
        u64, u32, i32,
        vp, vp, vp, vp,
        ctypes.POINTER(_Diag)]
    lib.specv_verify_sample.restype = ctypes.c_int
    lib.specv_verify_point_mass.argtypes = [
        vp, vp,
        vp, i64, i64,
        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
        vp, vp,
        u64, u32, i32,
        vp, vp, vp, vp,
        ctypes.POINTER(_Diag)]
    lib.specv_verify_point_mass.restype = ctypes.c_int
    lib.specv_verify_sample_qstats.argtypes = [
        vp, vp,
        vp, i64, i64,
        vp, i64, i64,
        vp, i64,
        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
        vp, vp,
        u64, u32, i32,
        vp, vp, vp, vp,
        ctypes.POINTER(_Diag)]
    lib.specv_verify_sample_qstats.restype = ctypes.c_int
    lib.specv_sample_draft.argtypes = [
        vp, vp,
        vp, i64, i64,
        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
        vp, u64, u32,
        vp, vp, i64]
    lib.specv_sample_draft.restype = ctypes.c_int
    lib.specv_verify_greedy.argtypes = [
        vp, vp,
        vp, i64, i64,
        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
        vp, vp, i32,
        vp, vp, vp, vp]
    lib.specv_verify_greedy.restype = ctypes.c_int
    lib.specv_set_profiling.argtypes = [vp, ctypes.c_int]
    lib.specv_set_profiling.restype = ctypes.c_int
    lib.specv_get_profile.argtypes = [vp, ctypes.c_int, ctypes.POINTER(ctypes.c_int),
                                      ctypes.POINTER(ctypes.c_double)]
    lib.specv_get_profile.restype = ctypes.c_int
    lib.specv_get_profile_samples.argtypes = [vp, ctypes.c_int, ctypes.POINTER(ctypes.c_float),
                                              ctypes.POINTER(ctypes.c_int)]
    lib.specv_get_profile_samples.restype = ctypes.c_int
    lib.specv_read_ceiling.argtypes = [vp, vp, i64, ctypes.c_int, vp]
    lib.specv_read_ceiling.restype = ctypes.c_int
    lib.specv_verify_sample_noalloc.argtypes = [ctypes.c_int] + lib.specv_verify_sample.argtypes[1:]
    lib.specv_verify_sample_noalloc.restype = ctypes.c_int
    _lib = lib
    return lib


def _check(status, what):
    if status != 0:
        msg = load_library().specv_status_string(status).decode()
        raise SpecvError(f"{what} failed: status {status} ({msg})")


def make_row_params(B, temperature=1.0, top_k=0, top_p=1.0, max_new_tokens=0, device="cuda"):
    """specv_row_params[B] as an int32 tensor [B, 4] on ``device``.

    Columns: temperature (float32 bits), top_k, top_p (float32 bits),
    max_new_tokens.  Each argument is a scalar or a length-B sequence.
    """
    rec = np.zeros(B, dtype=[("t", "<f4"), ("k", "<i4"), ("p", "<f4"), ("cap", "<i4")])
    rec["t"] = temperature
    rec["k"] = top_k
    rec["p"] = top_p
    rec["cap"] = max_new_tokens
    host = torch.from_numpy(rec.view(np.int32).reshape(B, 4).copy())
    return host.to(device)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return SPECV_BF16
    if t.dtype == torch.float32:
        return SPECV_F32
    raise SpecvError(f"unsupported logits dtype {t.dtype} (float32 or bfloat16)")


def _rows(t, name, lead):
    if not t.is_cuda:
        raise SpecvError(f"{name} must be a device tensor")
    if t.dim() != 3 or (lead is not None and t.shape[0] != lead):
        raise SpecvError(f"{name} must be [B, positions, V], got {tuple(t.shape)}")
    if t.shape[2] > 1 and t.stride(2) != 1:
        raise SpecvError(f"{name} must be contiguous along the vocabulary")
    return t.stride(0), t.stride(1)


def verify_sample_noalloc(target, draft, tokens, row_params, seed, step=0, eos_id=-1, out=None,
                          diag=False):
    """specv_verify_sample_noalloc: Verifier.verify_sample without a handle,
    for callers that cannot allocate device memory (the library's static
    per-device scratch array; B <= 256, gamma <= 15, V <= 262144, no
    truncated rows).  Runs on the current torch device and stream.  The
    output tensors are allocated here unless ``out`` (and, with ``diag``,
    its diagnostics) are given."""
    B, g1, V = target.shape
    gamma = g1 - 1
    tsb, tsp = _rows(target, "target", None)
    dsb = dsp = 0
    if gamma > 0:
        dsb, dsp = _rows(draft, "draft", B)
        if draft.shape[1] != gamma or draft.shape[2] != V or draft.dtype != target.dtype:
            raise SpecvError("draft must be [B, gamma, V] with the target's dtype")
    for t, n in ((tokens, "tokens"), (row_params, "row_params")):
        if t.dtype != torch.int32 or not t.is_contiguous() or not t.is_cuda:
            raise SpecvError(f"{n} must be a contiguous int32 device tensor")
    if tokens.shape != (B, gamma) or row_params.shape != (B, 4):
        raise SpecvError("tokens must be [B, gamma] and row_params [B, 4]")
    dev = target.device
    if out is None:
        z = dict(dtype=torch.int32, device=dev)
        out = {"num_accepted": torch.empty(B, **z), "out_tokens": torch.empty(B, gamma + 1, **z),
               "num_emitted": torch.empty(B, **z), "row_flags": torch.empty(B, **z)}
    d = None
    if diag:
        for key, shape in (("p_at_draft", (B, gamma)), ("q_at_draft", (B, gamma)), ("residual_sum", (B,))):
            if key not in out:
                out[key] = torch.empty(*shape, dtype=torch.float32, device=dev)
        d = _Diag(out["p_at_draft"].data_ptr(), out["q_at_draft"].data_ptr(),
                  out["residual_sum"].data_ptr())
    st = load_library().specv_verify_sample_noalloc(
        dev.index if dev.index is not None else torch.cuda.current_device(),
        ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream),
        _ptr(target), tsb, tsp, _ptr(draft if gamma > 0 else None), dsb, dsp,
        _dtype_code(target), B, gamma, V, _ptr(tokens), _ptr(row_params),
        int(seed) & 0xFFFFFFFFFFFFFFFF, int(step) & 0xFFFFFFFF, int(eos_id),
        _ptr(out["num_accepted"]), _ptr(out["out_tokens"]), _ptr(out["num_emitted"]),
        _ptr(out.get("row_flags")), ctypes.byref(d) if d is not None else None)
    _check(st, "specv_verify_sample_noalloc")
    return out


def read_ceiling(buf, grid, sink):
    """One streaming read of the device tensor ``buf`` (its bytes, a multiple
    of 16) by ``grid`` workgroups on the current stream (measurement aid);
    ``sink`` is an int32 device tensor of at least ``grid`` entries."""
    nbytes = buf.numel() * buf.element_size()
    if not buf.is_cuda or not buf.is_contiguous() or sink.numel() < grid or sink.dtype != torch.int32:
        raise SpecvError("read_ceiling needs a contiguous device buffer and an int32 sink of grid entries")
    st = load_library().specv_read_ceiling(ctypes.c_void_p(torch.cuda.current_stream().cuda_stream),
                                           _ptr(buf), nbytes, int(grid), _ptr(sink))
    _check(st, "specv_read_ceiling")


def debug_set_wait_limit(polls, device=None):
    """Failure-path tests only: the polls every bounded wait of the kernels
    makes before it gives up and flags its row INTERNAL (0 restores the
    default).  Process-wide for the device."""
    dev = torch.cuda.current_device() if device is None else int(device)
    fn = load_library().specv_debug_set_wait_limit
    fn.argtypes = [ctypes.c_int, ctypes.c_int32]
    fn.restype = ctypes.c_int
    _check(fn(dev, int(polls)), "specv_debug_set_wait_limit")


class Verifier:
    """A libspecv handle: owns the device workspace for calls up to the given
    maxima.  Calls run on the current torch stream of the handle's device."""

    def __init__(self, max_batch, max_gamma, max_vocab, max_top_k=0, device=0):
        lib = load_library()
        self.device = int(device)
        cfg = _Config(self.device, int(max_batch), int(max_gamma), int(max_vocab), int(max_top_k))
        h = ctypes.c_void_p()
        _check(lib.specv_create(ctypes.byref(cfg), ctypes.byref(h)), "specv_create")
        self._h = h
        self.max_batch, self.max_gamma, self.max_vocab = max_batch, max_gamma, max_vocab
        self.max_top_k = max_top_k

    def close(self):
        if getattr(self, "_h", None) is not None and self._h.value:
            load_library().specv_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def set_profiling(self, enable=True):
        """Record HIP events around each kernel of later calls."""
        _check(load_library().specv_set_profiling(self._h, int(bool(enable))), "specv_set_profiling")

    def profile(self, reset=True):
        """(calls, summed kernel milliseconds) over profiled calls; waits for
        the recorded events."""
        n = ctypes.c_int()
        ms = ctypes.c_double()
        _check(load_library().specv_get_profile(self._h, int(bool(reset)), ctypes.byref(n),
                                                ctypes.byref(ms)),
               "specv_get_profile")
        return n.value, ms.value

    def profile_samples(self, max_samples=1 << 16):
        """Per-call kernel milliseconds recorded since the last reset (numpy
        float32); waits for the recorded events, does not reset."""
        buf = (ctypes.c_float * max_samples)()
        n = ctypes.c_int()
        _check(load_library().specv_get_profile_samples(self._h, max_samples, buf, ctypes.byref(n)),
               "specv_get_profile_samples")
        return np.frombuffer(buf, dtype=np.float32, count=n.value).copy()

    def _stream(self):
        return ctypes.c_void_p(torch.cuda.current_stream(self.device).cuda_stream)

    def _outputs(self, B, gamma, device, out):
        if out is not None:
            return out
        z = dict(dtype=torch.int32, device=device)
        return {"num_accepted": torch.empty(B, **z), "out_tokens": torch.empty(B, gamma + 1, **z),
                "num_emitted": torch.empty(B, **z), "row_flags": torch.empty(B, **z)}

    def verify_sample(self, target, draft, tokens, row_params, seed, step=0, eos_id=-1,
                      out=None, diag=False):
        """Stochastic verification.  target [B, gamma+1, V], draft [B, gamma, V]
        (same dtype), tokens int32 [B, gamma], row_params from make_row_params.
        Returns a dict of device tensors (plus p_at_draft, q_at_draft,
        residual_sum when ``diag``).  Asynchronous on the current stream."""
        return self._verify_two_model(target, draft, None, tokens, row_params, seed, step, eos_id,
                                      out, diag)

    def verify_sample_qstats(self, target, draft, draft_stats, tokens, row_params, seed, step=0,
                             eos_id=-1, out=None, diag=False):
        """Stochastic verification reusing the drafter's row statistics:
        draft_stats float32 [B, >= gamma, 4] records (max, sum, threshold,
        flags as int32 bits) per draft row, as ``sample_draft`` returns them.
        Otherwise as verify_sample."""
        return self._verify_two_model(target, draft, draft_stats, tokens, row_params, seed, step,
                                      eos_id, out, diag)

    def _verify_two_model(self, target, draft, draft_stats, tokens, row_params, seed, step, eos_id,
                          out, diag):
        B, g1, V = target.shape
        gamma = g1 - 1
        tsb, tsp = _rows(target, "target", None)
        dsb = dsp = 0
        if gamma > 0:
            dsb, dsp = _rows(draft, "draft", B)
            if draft.shape[1] != gamma or draft.shape[2] != V or draft.dtype != target.dtype:
                raise SpecvError("draft must be [B, gamma, V] with the target's dtype")
        for t, n in ((tokens, "tokens"), (row_params, "row_params")):
            if t.dtype != torch.int32 or not t.is_contiguous() or not t.is_cuda:
                raise SpecvError(f"{n} must be a contiguous int32 device tensor")
        if tokens.shape != (B, gamma) or row_params.shape != (B, 4):
            raise SpecvError("tokens must be [B, gamma] and row_params [B, 4]")
        o = self._outputs(B, gamma, target.device, out)
        d = None
        if diag:
            o["p_at_draft"] = torch.empty(B, gamma, dtype=torch.float32, device=target.device)
            o["q_at_draft"] = torch.empty(B, gamma, dtype=torch.float32, device=target.device)
            o["residual_sum"] = torch.empty(B, dtype=torch.float32, device=target.device)
            d = _Diag(o["p_at_draft"].data_ptr(), o["q_at_draft"].data_ptr(),
                      o["residual_sum"].data_ptr())
        common = (_dtype_code(target), B, gamma, V,
                  _ptr(tokens), _ptr(row_params),
                  int(seed) & 0xFFFFFFFFFFFFFFFF, int(step) & 0xFFFFFFFF, int(eos_id),
                  _ptr(o["num_accepted"]), _ptr(o["out_tokens"]), _ptr(o["num_emitted"]),
                  _ptr(o.get("row_flags")),
                  ctypes.byref(d) if d is not None else None)
        drows = (_ptr(target), tsb, tsp, _ptr(draft if gamma > 0 else None), dsb, dsp)
        if draft_stats is None:
            st = load_library().specv_verify_sample(self._h, self._stream(), *drows, *common)
            _check(st, "specv_verify_sample")
            return o
        if (draft_stats.dtype != torch.float32 or not draft_stats.is_cuda or draft_stats.dim() != 3
                or draft_stats.shape[0] != B or draft_stats.shape[1] < gamma
                or draft_stats.shape[2] != 4 or not draft_stats.is_contiguous()):
            raise SpecvError("draft_stats must be a contiguous float32 [B, >= gamma, 4] device tensor")
        st = load_library().specv_verify_sample_qstats(
            self._h, self._stream(), *drows, _ptr(draft_stats), draft_stats.shape[1], *common)
        _check(st, "specv_verify_sample_qstats")
        return o

    def sample_draft(self, draft, row_params, seed, step=0, pos0=0, width=None, out=None):
        """Draft-side sampler: d_i ~ q_i for positions pos0 .. pos0 + n - 1
        of the round, from draft logits [B, n, V] (float32 or bfloat16), with
        each row's statistics for verify_sample_qstats.  Returns
        {"tokens": int32 [B, width], "stats": float32 [B, width, 4],
        "flags": int32 [B, width]}: stats holds (max, sum, threshold, flags
        bits) records and "flags" is a view of their last field.  ``width``
        defaults to pos0 + n; pass ``out`` (such a dict) to fill columns of
        existing tensors, e.g. one position per call.  Asynchronous on the
        current stream."""
        B, n, V = draft.shape
        dsb, dsp = _rows(draft, "draft", None)
        if row_params.dtype != torch.int32 or not row_params.is_contiguous() or row_params.shape != (B, 4):
            raise SpecvError("row_params must be a contiguous int32 [B, 4] device tensor")
        if out is None:
            w = pos0 + n if width is None else int(width)
            st = torch.full((B, w, 4), float("nan"), dtype=torch.float32, device=draft.device)
            st.view(torch.int32)[..., 3] = 0
            out = {"tokens": torch.full((B, w), -1, dtype=torch.int32, device=draft.device),
                   "stats": st, "flags": st.view(torch.int32)[..., 3]}
        tok, sts = out["tokens"], out.get("stats")
        w = tok.shape[1]
        if tok.dtype != torch.int32 or not tok.is_contiguous() or tok.shape[0] != B:
            raise SpecvError("tokens output must be a contiguous int32 [B, width] tensor")
        if sts is not None and (sts.dtype != torch.float32 or not sts.is_contiguous()
                                or tuple(sts.shape) != (B, w, 4)):
            raise SpecvError("stats output must be a contiguous float32 [B, width, 4] tensor")
        st = load_library().specv_sample_draft(
            self._h, self._stream(), _ptr(draft), dsb, dsp, _dtype_code(draft), B, n, V, int(pos0),
            _ptr(row_params), int(seed) & 0xFFFFFFFFFFFFFFFF, int(step) & 0xFFFFFFFF,
            _ptr(tok), _ptr(sts), w)
        _check(st, "specv_sample_draft")
        return out

    def verify_point_mass(self, target, tokens, row_params, seed, step=0, eos_id=-1, out=None,
                          diag=False):
        """Stochastic verification against deterministic drafts (q_i is the
        point mass on d_i; no draft logits).  target [B, gamma+1, V], tokens
        int32 [B, gamma], row_params from make_row_params.  Returns a dict of
        device tensors as verify_sample."""
        B, g1, V = target.shape
        gamma = g1 - 1
        tsb, tsp = _rows(target, "target", None)
        for t, n in ((tokens, "tokens"), (row_params, "row_params")):
            if t.dtype != torch.int32 or not t.is_contiguous() or not t.is_cuda:
                raise SpecvError(f"{n} must be a contiguous int32 device tensor")
        if tokens.shape != (B, gamma) or row_params.shape != (B, 4):
            raise SpecvError("tokens must be [B, gamma] and row_params [B, 4]")
        o = self._outputs(B, gamma, target.device, out)
        d = None
        if diag:
            o["p_at_draft"] = torch.empty(B, gamma, dtype=torch.float32, device=target.device)
            o["q_at_draft"] = torch.empty(B, gamma, dtype=torch.float32, device=target.device)
            o["residual_sum"] = torch.empty(B, dtype=torch.float32, device=target.device)
            d = _Diag(o["p_at_draft"].data_ptr(), o["q_at_draft"].data_ptr(),
                      o["residual_sum"].data_ptr())
        st = load_library().specv_verify_point_mass(
            self._h, self._stream(),
            _ptr(target), tsb, tsp,
            _dtype_code(target), B, gamma, V,
            _ptr(tokens), _ptr(row_params),
            int(seed) & 0xFFFFFFFFFFFFFFFF, int(step) & 0xFFFFFFFF, int(eos_id),
            _ptr(o["num_accepted"]), _ptr(o["out_tokens"]), _ptr(o["num_emitted"]),
            _ptr(o.get("row_flags")),
            ctypes.byref(d) if d is not None else None)
        _check(st, "specv_verify_point_mass")
        return o

    def verify_greedy(self, target, tokens, max_new_tokens=None, eos_id=-1, out=None):
        """Greedy verification.  target [B, gamma+1, V], tokens int32 [B, gamma],
        max_new_tokens int32 [B] device tensor or None."""
        B, g1, V = target.shape
        gamma = g1 - 1
        tsb, tsp = _rows(target, "target", None)
        if tokens.dtype != torch.int32 or not tokens.is_contiguous() or tokens.shape != (B, gamma):
            raise SpecvError("tokens must be a contiguous int32 [B, gamma] device tensor")
        if max_new_tokens is not None and (max_new_tokens.dtype != torch.int32 or
                                           max_new_tokens.shape != (B,)):
            raise SpecvError("max_new_tokens must be an int32 [B] device tensor")
        o = self._outputs(B, gamma, target.device, out)
        st = load_library().specv_verify_greedy(
            self._h, self._stream(),
            _ptr(target), tsb, tsp,
            _dtype_code(target), B, gamma, V,
            _ptr(tokens), _ptr(max_new_tokens), int(eos_id),
            _ptr(o["num_accepted"]), _ptr(o["out_tokens"]), _ptr(o["num_emitted"]),
            _ptr(o.get("row_flags")))
        _check(st, "specv_verify_greedy")
        return o
