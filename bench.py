"""Throughput of the speculative-sampling verify step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--sets S] [--no-cpu-baseline]
                    [--workload serving|point-mass|drafted|truncated|mixed|tiny|llama]

Workload (default): the serving batch, B=64 rows, gamma=5 drafts, V=128256
bfloat16 logits (target [64, 6, 128256], draft [64, 5, 128256]), T=0.7,
synthetic logits (N(0, 3^2) with 20 boosted tokens per position, draft =
target + N(0, 1.5^2)), draft tokens drawn from the draft distribution.  A
step is one call of the whole verify path over one batch.  Inputs are
resident in HBM; ``--sets`` distinct copies of them are rotated so that the
256 MB memory-side cache cannot serve a call from the previous one.

``--workload point-mass`` runs the same target logits against deterministic
drafts (the argmax of the draft logits, standing in for n-gram /
prompt-lookup proposals) through ``specv_verify_point_mass``, which reads no
draft logits.

``--workload truncated`` (B=32, gamma=5, V=152064, bf16, T=0.7, top-k 50 and
top-p 0.9 on both distributions, draft tokens drawn by ``specv_sample_draft``
from the truncated draft distribution) and ``--workload mixed`` (B=256,
gamma=8, V=128256, bf16, even rows T=1, odd rows greedy, per-row caps 1..9)
run the other synthetic configurations through ``specv_verify_sample``.
``--workload tiny`` (B=1, gamma=4, V=32, fp32) and ``--workload llama``
(B=1, gamma=4, V=32000, fp32, draft noise 1.5) are the latency-bound
single-row configurations: their line reports microseconds per call.

``--workload drafted`` runs the drafter's side too: a step is gamma calls of
``specv_sample_draft`` (one per position, as an autoregressive drafter
samples d_i before computing the next position's logits), each drawing
d_i ~ q_i for the 64 rows and returning the rows' statistics, then one
``specv_verify_sample_qstats``, which reads no draft row for its accept
tests.

Prints one JSON line: verified rows/s (``value``), per-call kernel time
(mean, median, p10, p90), the achieved HBM bandwidth of the dominant kernel
on its algorithmic bytes against MI355X's 8 TB/s, the bytes the kernel
actually moved by rocprofv3 counters (when a counter file taken on the
current kernel sources exists) and their rate, the device's one-pass read
rate measured in the same run, a check of every timed call's flags, and the
CPU oracle timed on this host (one process, then a pool over the host's
cores), whose first batch is the first timed call's inputs and is compared
with the GPU's outputs of that call.
"""

import argparse
import hashlib
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
METRIC = "verified rows/sec + achieved HBM GB/s (% peak), V=128256 γ=5 B=64 bf16"
METRICS = {
    "point-mass": ("verified rows/sec + achieved HBM GB/s (% peak), point-mass drafts, "
                   "V=128256 γ=5 B=64 bf16"),
    "truncated": ("verified rows/sec + achieved HBM GB/s (% peak), top-k 50 top-p 0.9, "
                  "V=152064 γ=5 B=32 bf16"),
    "mixed": ("verified rows/sec + achieved HBM GB/s (% peak), half greedy rows, caps 1..9, "
              "V=128256 γ=8 B=256 bf16"),
    "drafted": ("verified rows/sec + achieved HBM GB/s (% peak), drafter-sampled proposals "
                "with row statistics, V=128256 γ=5 B=64 bf16"),
    "tiny": "verified rows/sec (latency-bound: µs per call), V=32 γ=4 B=1 f32",
    "llama": "verified rows/sec (latency-bound: µs per call), V=32000 γ=4 B=1 f32",
}
PEAK_HBM_GBPS = 8000.0
KERNEL_SRC = os.path.join(ROOT, "speculative_decoding_verification_sampling_amd", "csrc",
                          "specv_kernels.hip")
TRAFFIC_FILES = {
    ("serving", "k_verify"): os.path.join(ROOT, "profiles", "traffic_k_verify_serving_batch.json"),
    ("point-mass", "k_verify"): os.path.join(ROOT, "profiles", "traffic_k_verify_point_mass.json"),
    ("drafted", "k_verify"): os.path.join(ROOT, "profiles", "traffic_k_verify_drafted.json"),
    ("drafted", "k_sample_draft"): os.path.join(ROOT, "profiles", "traffic_k_sample_draft_drafted.json"),
    ("truncated", "k_verify"): os.path.join(ROOT, "profiles", "traffic_k_verify_truncated.json"),
    ("mixed", "k_verify"): os.path.join(ROOT, "profiles", "traffic_k_verify_mixed.json"),
}
HOST_POOL_CAP = 16          # worker processes: the host share of one GPU


def algorithmic_bytes(B, gamma, V, es, caps, eos_cut, greedy, point_mass=False, qstats=False):
    """Logits bytes the round may consult: per row, target rows
    min(cap, gamma+1) and, for stochastic rows, draft rows: min(cap, gamma)
    of them with draft logits alone, at most one (the row where the round
    stops) with the drafter's statistics, none for point-mass drafts."""
    total = 0
    for b in range(B):
        cap = caps[b] if caps[b] >= 1 else 1 << 30
        cap = min(cap, eos_cut[b])
        nt = min(cap, gamma + 1)
        nd = 0 if greedy[b] or point_mass else min(cap, gamma)
        if qstats:
            nd = min(nd, 1)
        total += (nt + nd) * V * es
    return int(total)


def sampler_bytes(B, V, es):
    """One specv_sample_draft launch at one position: every draft row read
    once, and per row a token, two statistics and a flag word written."""
    return B * V * es + B * (4 + 8 + 4)


def kernel_source_hash():
    """Hash of the device-code sources (every file under csrc/ except the
    host-side C ABI and the measurement aid), so that counter figures are
    dropped once a kernel changes."""
    h = hashlib.sha256()
    d = os.path.dirname(KERNEL_SRC)
    for name in sorted(os.listdir(d)):
        if name in ("specv_api.hip", "specv_measure.hip") or not name.endswith((".hip", ".hpp")):
            continue
        with open(os.path.join(d, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def stored_traffic(workload, kernel="k_verify"):
    """HBM bytes per launch of ``kernel`` on ``workload`` from committed
    rocprofv3 counter runs, or None when absent or taken on different kernel
    sources."""
    try:
        with open(TRAFFIC_FILES[(workload, kernel)]) as f:
            t = json.load(f)
    except (KeyError, OSError, ValueError):
        return None
    if t.get("kernel_source_hash") != kernel_source_hash():
        return None
    return t.get("bytes_per_launch")


def make_workload(name):
    """The synthetic workload (CPU tensors) and its draft tokens; ``None``
    tokens mean the GPU draws them (truncated) or the drafter does (drafted)."""
    import synth
    import torch
    if name == "tiny":
        w = synth.tiny(sample_tokens=True)
    elif name == "llama":
        w = synth.llama_vocab(1.5)
    elif name == "truncated":
        w = synth.truncated()
    elif name == "mixed":
        w = synth.mixed()
    else:
        w = synth.serving_batch()
    if name == "point-mass":
        # deterministic drafts stand in for n-gram / prompt-lookup proposals
        tokens = w.draft.to(torch.float32).numpy().argmax(-1).astype(np.int32)
    elif name == "truncated":
        tokens = None
    else:
        tokens = w.tokens
    return w, tokens


# ---------------------------------------------------------------- CPU oracle leg
_POOL_STATE = {}


def _oracle_batch(step):
    """One whole batch of the workload through the oracle at ``step`` (runs
    in a pool worker forked with the inputs in _POOL_STATE)."""
    import oracle
    s = _POOL_STATE
    w = s["w"]
    if s["kind"] == "drafted":
        toks = oracle.sample_draft_tokens(s["df"], w.temperature, w.top_k, w.top_p, w.seed + 1, step)
        return oracle.verify_sample(s["tf"], s["df"], toks, w.temperature, w.top_k, w.top_p,
                                    w.max_new_tokens, w.seed, step)
    if s["kind"] == "point-mass":
        return oracle.verify_point_mass(s["tf"], s["tokens"], w.temperature, w.top_k, w.top_p,
                                        w.max_new_tokens, w.seed, step)
    return oracle.verify_sample(s["tf"], s["df"], s["tokens"], w.temperature, w.top_k, w.top_p,
                                w.max_new_tokens, w.seed, step)


def _pool_task(step):
    _oracle_batch(step)
    return step


def cpu_oracle_leg(kind, w, tokens, first_step, budget_s):
    """The oracle as it stands, timed on this host over whole batches of the
    workload at successive steps (first_step, first_step + 1, ...): first
    one process, then a pool of worker processes over the host's cores (one
    batch per task).  Returns the baseline record and the oracle's output of
    the first batch, whose inputs are those of the first timed GPU call.
    Runs before anything initialises the GPU, so that the pool's fork is
    safe."""
    import multiprocessing as mp
    import oracle
    tf = w.target_f32()
    df = w.draft_f32()
    if tokens is None:
        # truncated: the GPU draws the proposals with the Philox drafter; the
        # oracle's drafter gives the same draws for its own run
        tokens = oracle.sample_draft_tokens(df, w.temperature, w.top_k, w.top_p, w.seed + 1)
    _POOL_STATE.update(w=w, tf=tf, df=df, tokens=tokens, kind=kind)
    t0 = time.perf_counter()
    first = _oracle_batch(first_step)
    steps = 1
    while time.perf_counter() - t0 < budget_s / 2:
        _oracle_batch(first_step + steps)
        steps += 1
    single_s = time.perf_counter() - t0
    single = w.B * steps / single_s
    n = max(1, min(HOST_POOL_CAP, len(os.sched_getaffinity(0))))
    per_worker = max(1, int(np.ceil(steps / single_s * budget_s / 2)))
    tasks = [first_step + i for i in range(n * per_worker)]
    ctx = mp.get_context("fork")
    t0 = time.perf_counter()
    with ctx.Pool(n) as pool:
        done = sum(1 for _ in pool.imap_unordered(_pool_task, tasks))
    pool_s = time.perf_counter() - t0
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    rec = {
        "value": w.B * done / pool_s,
        "unit": "verified rows/s",
        "cores": n,
        "kind": "oracle",
        "sample": (f"{done} whole batches (B={w.B}) of the same workload at steps {first_step}.., "
                   f"{pool_s:.1f} s, numpy float64, a pool of {n} worker processes (one batch per task)"),
        "single_process": {"value": single, "unit": "verified rows/s", "cores": 1,
                           "sample": f"{steps} whole batches, {single_s:.1f} s, one process"},
        "cpu_model": model or platform.processor(),
        "numpy": np.__version__,
        "host_cpus_visible": len(os.sched_getaffinity(0)),
    }
    return rec, first, tokens


def check_first_call(kind, w, gpu_out, orc, gpu_tokens, oracle_tokens, step):
    """Classify the GPU's first timed call against the oracle's output of the
    same inputs (the bar of tests/parity.py).  When the GPU's proposals
    (drawn on the device for the truncated workload) differ from the
    oracle's draw, the oracle's batch is run again on the GPU's proposals."""
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import oracle
    from parity import compare
    if kind in ("serving", "truncated", "mixed", "tiny", "llama") and not np.array_equal(gpu_tokens,
                                                                                          oracle_tokens):
        orc = oracle.verify_sample(w.target_f32(), w.draft_f32(), gpu_tokens, w.temperature, w.top_k,
                                   w.top_p, w.max_new_tokens, w.seed, step)
    prm = {"temperature": w.temperature, "top_k": w.top_k, "top_p": w.top_p}
    rep = compare(gpu_out, orc, gpu_tokens, w.target_f32(),
                  None if kind == "point-mass" else w.draft_f32(), prm, workload=f"bench {kind}")
    d = rep.as_dict()
    d["first_failures"] = rep.failures[:3]
    return d


# ---------------------------------------------------------------- GPU leg
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--sets", type=int, default=4)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=16.0, help="seconds of oracle time")
    ap.add_argument("--no-read-ceiling", action="store_true")
    ap.add_argument("--workload", choices=("serving", "point-mass", "drafted", "truncated", "mixed",
                                           "tiny", "llama"),
                    default="serving")
    ap.add_argument("--copy-reference", type=int, default=0, metavar="MIB",
                    help="only run --steps device copies of MIB MiB (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the verify step shards by batch row with no exchange; see the design notes)",
              file=sys.stderr)
        sys.exit(2)

    sys.path.insert(0, ROOT)
    kind = args.workload
    point_mass = kind == "point-mass"
    drafted = kind == "drafted"
    truncated = kind == "truncated"
    first_step = 1000
    if not args.copy_reference:
        w, tok_np = make_workload(kind)
        cpu = orc_first = cpu_tokens = None
        if not args.no_cpu_baseline:
            cpu, orc_first, cpu_tokens = cpu_oracle_leg(kind, w, tok_np, first_step, args.cpu_budget)

    import torch
    import speculative_decoding_verification_sampling_amd as sv

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    if args.copy_reference:
        # a plain copy of known size: rocprofv3 FETCH_SIZE / WRITE_SIZE of these
        # launches calibrate the counters against bytes actually moved
        n = args.copy_reference * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_reference_bytes_each_way": n * 4, "launches": args.steps}))
        return
    sv.load_library()

    B, gamma, V = w.B, w.gamma, w.V
    max_top_k = 64 if truncated else 0
    if truncated:
        # proposals from the truncated draft distribution, drawn on the device
        with sv.Verifier(B, gamma, V, max_top_k=max_top_k) as vd:
            rp = sv.make_row_params(B, w.temperature, w.top_k, w.top_p, w.max_new_tokens, dev)
            tok_np = vd.sample_draft(w.draft.to(dev), rp, w.seed + 1)["tokens"].cpu().numpy()
    sets = []
    for _ in range(max(1, args.sets)):
        t = w.target.to(dev)
        d = None if point_mass else w.draft.to(dev)
        # one [B, 1, V] view per position, for the drafter's per-position calls
        cols = [d[:, i:i + 1] for i in range(gamma)] if drafted else None
        sets.append((t, d, cols))
    tokens = torch.from_numpy(np.ascontiguousarray(tok_np, np.int32)).to(dev)
    params = sv.make_row_params(B, w.temperature, w.top_k, w.top_p, w.max_new_tokens, dev)
    v = sv.Verifier(B, gamma, V, max_top_k=max_top_k)
    vs = sv.Verifier(B, gamma, V) if drafted else None      # the drafter's handle, timed apart
    drawn = None
    if drafted:
        drawn = {"tokens": torch.full((B, gamma), -1, dtype=torch.int32, device=dev),
                 "stats": torch.zeros(B, gamma, 4, dtype=torch.float32, device=dev)}

    def outputs(n):
        z = dict(dtype=torch.int32, device=dev)
        return {"num_accepted": torch.zeros(n, B, **z), "out_tokens": torch.zeros(n, B, gamma + 1, **z),
                "num_emitted": torch.zeros(n, B, **z), "row_flags": torch.zeros(n, B, **z)}

    def view(o, i):
        return {k: x[i] for k, x in o.items()}

    def call(k, step, out):
        t, d, cols = sets[k % len(sets)]
        if point_mass:
            return v.verify_point_mass(t, tokens, params, w.seed, step, -1, out=out)
        if drafted:
            for i in range(gamma):
                vs.sample_draft(cols[i], params, w.seed + 1, step, i, out=drawn)
            return v.verify_sample_qstats(t, d, drawn["stats"], drawn["tokens"], params, w.seed, step,
                                          -1, out=out)
        return v.verify_sample(t, d, tokens, params, w.seed, step, -1, out=out)

    es = w.bytes_per_element()
    eos_cut = [1 << 30] * B
    greedy = [bool(t == 0) for t in w.temperature]
    per_launch = {"k_verify": algorithmic_bytes(B, gamma, V, es, w.max_new_tokens, eos_cut, greedy,
                                                point_mass, qstats=drafted)}
    if drafted:
        per_launch["k_sample_draft"] = sampler_bytes(B, V, es)

    # The read ceiling is measured first: after the oracle leg the device has
    # idled for seconds, and its clocks take milliseconds of load to come back
    # up (the first 20 calls after 5 s idle ran at 46-53 us against 35.5 us
    # warm); this pass keeps it busy for tens of milliseconds before the
    # warm-up steps.
    read = None
    if not args.no_read_ceiling and kind not in ("tiny", "llama"):
        read = read_ceiling(sv, torch, dev, per_launch["k_verify"], len(sets))

    scratch = outputs(1)
    call(0, 0, view(scratch, 0))
    torch.cuda.synchronize()
    for i in range(args.warmup):
        call(i, i, view(scratch, 0))
    torch.cuda.synchronize()

    # the timed region: every call writes outputs of its own, checked afterwards
    timed = outputs(args.steps)
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    # a ~0.1 ms spin on the stream ahead of the start event, so that the host
    # has submitted the first calls by the time the device reaches it: the
    # window then holds the K calls back to back, not the latency of the
    # first submission to an idle device
    torch.cuda._sleep(250_000)
    e0.record(stream)
    for i in range(args.steps):
        call(i, first_step + i, view(timed, i))
    e1.record(stream)
    torch.cuda.synchronize()
    ms_total = e0.elapsed_time(e1)
    ms_step = ms_total / args.steps

    flags = timed["row_flags"].cpu().numpy()
    bad_internal = int(((flags & sv.FLAG_INTERNAL) != 0).sum())
    bad_nonfinite = int(((flags & sv.FLAG_NONFINITE_ROW) != 0).sum())
    bad_other = int(((flags & (sv.FLAG_TOKEN_OOR | sv.FLAG_CAND_OVERFLOW | sv.FLAG_UNSUPPORTED)) != 0).sum())
    emitted = timed["num_emitted"].cpu().numpy()
    tokens_per_call = float(emitted.sum(axis=1).mean())
    first_out = {k: x[0].cpu() for k, x in timed.items()}

    # per-kernel durations from HIP events recorded by the library on the
    # stream the kernels run on (attached to the dispatches themselves)
    handles = [("k_verify", v, 1)] + ([("k_sample_draft", vs, gamma)] if drafted else [])
    for _, h, _ in handles:
        h.set_profiling(True)
        h.profile(reset=True)
    for i in range(args.steps):
        call(i, first_step + i, view(scratch, 0))
    torch.cuda.synchronize()
    avg_us, dist_us = {}, {}
    for name, h, per_step in handles:
        samples = h.profile_samples() * 1e3
        n, ms_kernel = h.profile(reset=True)
        h.set_profiling(False)
        assert n == args.steps * per_step, (name, n)
        avg_us[name] = ms_kernel / n * 1e3
        dist_us[name] = {"mean": avg_us[name], "median": float(np.median(samples)),
                         "p10": float(np.percentile(samples, 10)),
                         "p90": float(np.percentile(samples, 90)), "calls": int(n)}

    roof = {}
    for name, _, per_step in handles:
        achieved = per_launch[name] / (avg_us[name] * 1e-6) / 1e9
        traffic = stored_traffic(kind, name)
        roof[name] = {
            "bound": "hbm",
            "kernel": name,
            "achieved": achieved,
            "peak": PEAK_HBM_GBPS,
            "unit": "GB/s",
            "frac": achieved / PEAK_HBM_GBPS,
            "traffic": traffic,
            "algorithmic_bytes_per_launch": per_launch[name],
            "launches_per_step": per_step,
        }
        if traffic is not None:
            # what the kernel actually moved (counter bytes), at its mean duration
            tg = traffic / (avg_us[name] * 1e-6) / 1e9
            roof[name]["traffic_gbps"] = tg
            roof[name]["traffic_frac"] = tg / PEAK_HBM_GBPS
    # the dominant kernel: the one with the most device time per step
    dominant = max(roof, key=lambda n: avg_us[n] * roof[n]["launches_per_step"])
    step_bytes = sum(per_launch[n] * roof[n]["launches_per_step"] for n in roof)

    rows_per_s = B / (ms_step * 1e-3)
    desc = {
        "point-mass": "serving batch, deterministic drafts (argmax of target + noise 1.5), no draft logits",
        "drafted": ("serving batch, draft noise 1.5, drafts drawn on the device one position per call "
                    "with the rows' statistics, verified with those statistics"),
        "truncated": ("truncated batch, T=0.7, top-k 50, top-p 0.9 on target and draft, draft noise 1.5, "
                      "drafts drawn on the device from the truncated draft distribution"),
        "mixed": ("mixed batch, even rows T=1 and odd rows greedy, per-row draft noise U[0.3, 4], "
                  "caps U{1..9}"),
        "tiny": "tiny exactness workload, z ~ N(0, 2^2), draft noise 1, T=1",
        "llama": "Llama-style vocabulary, N(0, 3^2) + 20 boosted tokens, draft noise 1.5, T=1",
    }.get(kind, "serving batch, T=0.7, draft noise 1.5")
    boosted = "" if kind == "tiny" else ", 20 boosted tokens"
    dt = "bf16" if w.dtype == "bf16" else "f32"
    line = {
        "metric": METRICS.get(kind, METRIC),
        "value": rows_per_s,
        "unit": "verified rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dt,
        "data": "synthetic",
        "config": {"workload": f"B={B} gamma={gamma} V={V} {dt}{boosted}, {desc}",
                   "B": B, "gamma": gamma, "V": V, "rotated_input_sets": len(sets)},
        "us_per_call": ms_step * 1e3,
        "emitted_tokens_per_s": tokens_per_call / (ms_step * 1e-3),
        "step_hbm_gbps_algorithmic": step_bytes / (ms_step * 1e-3) / 1e9,
        "kernel_us": avg_us,
        "kernel_us_dist": dist_us,
        "timed_outputs_checked": {"calls": args.steps, "rows": int(flags.size),
                                  "internal": bad_internal, "nonfinite": bad_nonfinite,
                                  "overflow_oor_unsupported": bad_other},
        "roofline": roof[dominant],
    }
    if read is not None:
        line["read_ceiling"] = read
    if drafted:
        line["roofline_other"] = [roof[n] for n in roof if n != dominant]
    if cpu is not None:
        if drafted:
            # the proposals of the timed calls are drawn inside the step and not kept
            cpu["first_timed_call_vs_oracle"] = None
        else:
            cpu["first_timed_call_vs_oracle"] = check_first_call(
                kind, w, first_out, orc_first, np.asarray(tok_np), np.asarray(cpu_tokens), first_step)
        line["cpu_baseline"] = cpu
    v.close()
    if vs is not None:
        vs.close()
    print(json.dumps(line), flush=True)
    if bad_internal or bad_nonfinite or bad_other:
        print(f"timed outputs carry error flags: {line['timed_outputs_checked']}", file=sys.stderr)
        sys.exit(3)
    if cpu is not None and cpu["first_timed_call_vs_oracle"] and cpu["first_timed_call_vs_oracle"]["failures"]:
        print("the first timed call differs from the oracle", file=sys.stderr)
        sys.exit(4)


def read_ceiling(sv, torch, dev, nbytes, nsets, reps=120):
    """The device's one-pass read rate for buffers of ``nbytes`` (rounded up
    to 16): ``nsets`` distinct buffers read in rotation by the library's
    plain streaming kernel, at a few grid sizes; the best grid's mean."""
    n16 = (nbytes + 15) // 16
    bufs = [torch.empty(n16 * 4, dtype=torch.int32, device=dev).fill_(i + 1) for i in range(nsets)]
    best = None
    for grid in (1024, 2048, 4096, 8192):
        sink = torch.zeros(grid, dtype=torch.int32, device=dev)
        for i in range(4):
            sv.read_ceiling(bufs[i % nsets], grid, sink)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(reps):
            sv.read_ceiling(bufs[i % nsets], grid, sink)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) / reps * 1e3
        gbps = n16 * 16 / (us * 1e-6) / 1e9
        if best is None or gbps > best["gbps"]:
            best = {"gbps": gbps, "us_per_read": us, "grid": grid}
    best.update({"bytes": n16 * 16, "frac_of_peak": best["gbps"] / PEAK_HBM_GBPS,
                 "kernel": "specv_read_ceiling (16-byte loads, 32 KB in flight per workgroup)",
                 "rotated_buffers": nsets})
    del bufs
    return best


if __name__ == "__main__":
    main()
