"""Throughput of the speculative-sampling verify step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--sets S] [--no-cpu-baseline]
                    [--workload serving|point-mass|drafted|truncated|mixed]

Workload: the serving batch, B=64 rows, gamma=5 drafts, V=128256 bfloat16
logits (target [64, 6, 128256], draft [64, 5, 128256]), T=0.7, synthetic
logits (N(0, 3^2) with 20 boosted tokens per position, draft = target +
N(0, 1.5^2)), draft tokens drawn from the draft distribution.  A step is one
call of the whole verify path over one batch.  Inputs are resident in HBM;
``--sets`` distinct copies of them are rotated so that the 256 MB
memory-side cache cannot serve a call from the previous one.

``--workload point-mass`` runs the same target logits against deterministic
drafts (the argmax of the draft logits, standing in for n-gram /
prompt-lookup proposals) through ``specv_verify_point_mass``, which reads no
draft logits.

``--workload truncated`` (B=32, gamma=5, V=152064, bf16, T=0.7, top-k 50 and
top-p 0.9 on both distributions, draft tokens drawn by ``specv_sample_draft``
from the truncated draft distribution) and ``--workload mixed`` (B=256,
gamma=8, V=128256, bf16, even rows T=1, odd rows greedy, per-row caps 1..9)
run the other synthetic configurations through ``specv_verify_sample``.

``--workload drafted`` runs the drafter's side too: a step is gamma calls of
``specv_sample_draft`` (one per position, as an autoregressive drafter
samples d_i before computing the next position's logits), each drawing
d_i ~ q_i for the 64 rows and returning the rows' statistics, then one
``specv_verify_sample_qstats``, which reads no draft row for its accept
tests.

Prints one JSON line: verified rows/s (``value``), the achieved HBM bandwidth
of the dominant kernel (the streaming statistics kernel) on its algorithmic
bytes against MI355X's 8 TB/s, and the CPU oracle timed on this host.
"""

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
METRIC = "verified rows/sec + achieved HBM GB/s (% peak), V=128256 γ=5 B=64 bf16"
METRIC_POINT_MASS = ("verified rows/sec + achieved HBM GB/s (% peak), point-mass drafts, "
                     "V=128256 γ=5 B=64 bf16")
METRIC_TRUNCATED = ("verified rows/sec + achieved HBM GB/s (% peak), top-k 50 top-p 0.9, "
                    "V=152064 γ=5 B=32 bf16")
METRIC_MIXED = ("verified rows/sec + achieved HBM GB/s (% peak), half greedy rows, caps 1..9, "
                "V=128256 γ=8 B=256 bf16")
METRIC_DRAFTED = ("verified rows/sec + achieved HBM GB/s (% peak), drafter-sampled proposals "
                  "with row statistics, V=128256 γ=5 B=64 bf16")
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
    host-side C ABI), so that counter figures are dropped once a kernel
    changes."""
    h = hashlib.sha256()
    d = os.path.dirname(KERNEL_SRC)
    for name in sorted(os.listdir(d)):
        if name == "specv_api.hip" or not name.endswith((".hip", ".hpp")):
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
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_hash") != kernel_source_hash():
        return None
    return t.get("bytes_per_launch")


def cpu_baseline(w, tokens, point_mass, budget_s=15.0, drafted=False):
    """The oracle as it stands, on this host, over whole batches of the same
    workload at successive steps until about ``budget_s`` seconds (with
    ``drafted``, the oracle's draft draw of every position comes first)."""
    import oracle
    tf, df = w.target_f32(), w.draft_f32()
    rows = 0
    steps = 0
    t0 = time.perf_counter()
    while True:
        if drafted:
            toks = oracle.sample_draft_tokens(df, w.temperature, w.top_k, w.top_p, w.seed + 1, steps)
            oracle.verify_sample(tf, df, toks, w.temperature, w.top_k, w.top_p,
                                 w.max_new_tokens, w.seed, steps)
        elif point_mass:
            oracle.verify_point_mass(tf, tokens, w.temperature, w.top_k, w.top_p,
                                     w.max_new_tokens, w.seed, steps)
        else:
            oracle.verify_sample(tf, df, tokens, w.temperature, w.top_k, w.top_p,
                                 w.max_new_tokens, w.seed, steps)
        rows += w.B
        steps += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    return {"value": rows / el, "unit": "verified rows/s", "cores": 1, "kind": "oracle",
            "sample": f"{steps} full batches (B={w.B}, steps 0..{steps - 1}) of the same workload, "
                      f"{el:.1f} s, numpy float64, one process, one thread"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--sets", type=int, default=4)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--workload", choices=("serving", "point-mass", "drafted", "truncated", "mixed"),
                    default="serving")
    ap.add_argument("--copy-reference", type=int, default=0, metavar="MIB",
                    help="only run --steps device copies of MIB MiB (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the verify step shards by batch row with no exchange; see the design notes)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    sys.path.insert(0, ROOT)
    import synth
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

    point_mass = args.workload == "point-mass"
    drafted = args.workload == "drafted"
    truncated = args.workload == "truncated"
    w = {"truncated": synth.truncated, "mixed": synth.mixed}.get(args.workload, synth.serving_batch)()
    B, gamma, V = w.B, w.gamma, w.V
    max_top_k = 64 if truncated else 0
    # deterministic drafts stand in for n-gram / prompt-lookup proposals
    tok_np = (w.draft.to(torch.float32).numpy().argmax(-1).astype(np.int32) if point_mass
              else w.tokens)
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
    tokens = torch.from_numpy(tok_np).to(dev)
    params = sv.make_row_params(B, w.temperature, w.top_k, w.top_p, w.max_new_tokens, dev)
    out = None
    v = sv.Verifier(B, gamma, V, max_top_k=max_top_k)
    vs = sv.Verifier(B, gamma, V) if drafted else None      # the drafter's handle, timed apart
    drawn = None
    if drafted:
        drawn = {"tokens": torch.full((B, gamma), -1, dtype=torch.int32, device=dev),
                 "stats": torch.zeros(B, gamma, 4, dtype=torch.float32, device=dev)}

    def call(k, step):
        t, d, cols = sets[k % len(sets)]
        if point_mass:
            return v.verify_point_mass(t, tokens, params, w.seed, step, -1, out=out)
        if drafted:
            for i in range(gamma):
                vs.sample_draft(cols[i], params, w.seed + 1, step, i, out=drawn)
            return v.verify_sample_qstats(t, d, drawn["stats"], drawn["tokens"], params, w.seed, step,
                                          -1, out=out)
        return v.verify_sample(t, d, tokens, params, w.seed, step, -1, out=out)

    out = call(0, 0)
    torch.cuda.synchronize()
    for i in range(args.warmup):
        call(i, i)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(args.steps):
        call(i, 1000 + i)
    e1.record(stream)
    torch.cuda.synchronize()
    ms_total = e0.elapsed_time(e1)
    ms_step = ms_total / args.steps

    # emitted tokens per call, averaged over a few steps (outside the timed region)
    em = []
    for i in range(8):
        o = call(i, 1000 + i)
        torch.cuda.synchronize()
        em.append(int(o["num_emitted"].sum()))
    tokens_per_call = float(np.mean(em))

    # per-kernel durations from HIP events recorded by the library on the
    # stream the kernels run on (attached to the dispatches themselves)
    handles = [("k_verify", v, 1)] + ([("k_sample_draft", vs, gamma)] if drafted else [])
    for _, h, _ in handles:
        h.set_profiling(True)
        h.profile(reset=True)
    for i in range(args.steps):
        call(i, 1000 + i)
    torch.cuda.synchronize()
    avg_us = {}
    for name, h, per_step in handles:
        n, ms_kernel = h.profile(reset=True)
        h.set_profiling(False)
        assert n == args.steps * per_step, (name, n)
        avg_us[name] = ms_kernel / n * 1e3

    es = w.bytes_per_element()
    eos_cut = [1 << 30] * B
    greedy = [bool(t == 0) for t in w.temperature]
    per_launch = {"k_verify": algorithmic_bytes(B, gamma, V, es, w.max_new_tokens, eos_cut, greedy,
                                                point_mass, qstats=drafted)}
    if drafted:
        per_launch["k_sample_draft"] = sampler_bytes(B, V, es)
    roof = {}
    for name, _, per_step in handles:
        achieved = per_launch[name] / (avg_us[name] * 1e-6) / 1e9
        roof[name] = {
            "bound": "hbm",
            "kernel": name,
            "achieved": achieved,
            "peak": PEAK_HBM_GBPS,
            "unit": "GB/s",
            "frac": achieved / PEAK_HBM_GBPS,
            "traffic": stored_traffic(args.workload, name),
            "algorithmic_bytes_per_launch": per_launch[name],
            "launches_per_step": per_step,
        }
    # the dominant kernel: the one with the most device time per step
    dominant = max(roof, key=lambda n: avg_us[n] * roof[n]["launches_per_step"])
    step_bytes = sum(per_launch[n] * roof[n]["launches_per_step"] for n in roof)

    rows_per_s = B / (ms_step * 1e-3)
    if point_mass:
        desc = "serving batch, deterministic drafts (argmax of target + noise 1.5), no draft logits"
    elif drafted:
        desc = ("serving batch, draft noise 1.5, drafts drawn on the device one position per call "
                "with the rows' statistics, verified with those statistics")
    elif truncated:
        desc = ("truncated batch, T=0.7, top-k 50, top-p 0.9 on target and draft, draft noise 1.5, "
                "drafts drawn on the device from the truncated draft distribution")
    elif args.workload == "mixed":
        desc = ("mixed batch, even rows T=1 and odd rows greedy, per-row draft noise U[0.3, 4], "
                "caps U{1..9}")
    else:
        desc = "serving batch, T=0.7, draft noise 1.5"
    metric = {"point-mass": METRIC_POINT_MASS, "drafted": METRIC_DRAFTED, "truncated": METRIC_TRUNCATED,
              "mixed": METRIC_MIXED}.get(args.workload, METRIC)
    line = {
        "metric": metric,
        "value": rows_per_s,
        "unit": "verified rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"B={B} gamma={gamma} V={V} bf16, 20 boosted tokens, {desc}",
                   "B": B, "gamma": gamma, "V": V, "rotated_input_sets": len(sets)},
        "emitted_tokens_per_s": tokens_per_call / (ms_step * 1e-3),
        "step_hbm_gbps_algorithmic": step_bytes / (ms_step * 1e-3) / 1e9,
        "kernel_us": avg_us,
        "roofline": roof[dominant],
    }
    if drafted:
        line["roofline_other"] = [roof[n] for n in roof if n != dominant]
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, tok_np, point_mass, drafted=drafted)
    v.close()
    if vs is not None:
        vs.close()
    print(json.dumps(line), flush=True)

if __name__ == "__main__":
    main()
