#!/usr/bin/env python3
"""Throughput of the KDA RecoverSSM verify + commit on one MI355X.

One step = the fused conv update + speculative verify of one KDA layer
followed by the commit of the accepted tokens, on the seeded decode batch of
the headline workload: 256 requests, 32 heads, head dim 128, 4 draft tokens
each, a 512-slot fp32 state pool in per-slot pages, dim-first conv state,
lower-bound gate (-5), commit lengths uniform in 1..4.  Inputs are resident in
HBM before timing starts; consecutive steps reuse the same buffers (every
step verifies from, and commits into, the same 256 checkpoints; the 512 MiB
of live state per step exceeds the 256 MB last-level cache, and verify and
commit walk the requests in the same order, so each state tile returns from
HBM).

Prints one JSON line.  `value` is verified tokens per second (draft tokens
verified per step / step time over K back-to-back steps); `roofline`
describes the kernel that takes the most time per step, from HIP events
around its launches; `kernels` gives each kernel's median, p10 and p90 over
the timed steps, the median of single synchronized launches, and the
median of single launches that each follow an untimed 1 GiB write (which
evicts the caches), so that any help from the last-level cache between
kernels shows up as a difference; `cpu_baseline`
times the fp64 CPU oracle on a bounded sample of the same workload.

  python bench.py [--steps K] [--warmup W] [--workload NAME]
  python bench.py --copy-calibration   # plain copy for HBM counter scaling
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor figure
PROFILE_DIR = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = {
    "kda_verify_grid_kernel": "kda_verify.hip",
    "kda_commit_grid_kernel": "kda_commit.hip",
}


def kernel_sha(kernel: str) -> str:
    """Hash of the sources a kernel is built from (for matching counters
    recorded under profiles/ with the kernel that runs now)."""
    csrc = os.path.join(ROOT, "linear_attention_speculative_amd", "csrc")
    h = hashlib.sha256()
    for name in (KERNEL_SOURCES[kernel], "kda_device.hpp", "kda_internal.hpp"):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def algorithmic_bytes(wl) -> dict:
    """Bytes the method must move per launch (each state tile read once by
    the verify, read and written once by the commit; every activation,
    record and conv byte once), from the workload's seeded metadata."""
    import numpy as np
    H, D, Q, W = wl.H, wl.D, wl.Q, wl.W
    e_act = 2 if wl.act == "bf16" else 4
    e_w = 2 if wl.weight == "bf16" else 4
    e_out = 2 if wl.out_dtype == "bf16" else 4
    e_kg = 2 if wl.kg_dtype == "bf16" else 4
    C = 3 * H * D
    qsl = wl.query_start_loc.cpu().numpy().astype(np.int64)
    slots = wl.state_indices.cpu().numpy()
    lens = wl.commit_lens.cpu().numpy()
    per_launch = C * W * e_w + 4 * H + 4 * H * D + 4 * (3 * wl.B + 1)
    verify = per_launch
    commit = 4 * H + 4 * H * D + 8 * wl.B   # gate params, slots + lens
    tokens = 0
    for b in range(wl.B):
        q = int(min(max(qsl[b + 1] - qsl[b], 0), Q))
        tokens += q
        if q == 0:
            continue
        if not 0 < slots[b] < wl.N:
            verify += q * H * D * e_out
            continue
        verify += 4 * H * D * D                          # state tile read
        verify += (W - 1) * C * e_act                    # conv history
        verify += (W - 2 + q) * C * e_act                # conv roll write
        verify += q * (C * e_act + H * D * e_act + H * e_act   # x, gate, beta
                       + H * D * e_out                   # out
                       + 4 * H * D + 2 * H * D * e_kg)   # records
        n = int(min(max(lens[b], 0), Q))
        if n > 0:
            commit += 8 * H * D * D + n * (4 * H * D + 2 * H * D * e_kg)
    return dict(verify=verify, commit=commit, tokens=tokens)


def traffic_from_profiles(kernel: str, workload: str):
    """HBM bytes per launch measured with rocprofv3 counters, if a summary
    for this kernel, workload and source hash is committed."""
    path = os.path.join(PROFILE_DIR, f"{kernel}_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_sha") != kernel_sha(kernel):
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(wl, seconds: float, max_passes: int = 8) -> dict:
    """The fp64 oracle, as it stands, single-threaded, on the requests of
    the same workload taken in order, 16 at a time (verify + commit), until
    `seconds` of CPU time have passed; passes over the whole batch repeat
    (at most `max_passes`) when one pass takes less than that."""
    import contextlib
    try:
        from threadpoolctl import threadpool_limits
        limit = threadpool_limits(limits=1)
    except ImportError:  # pragma: no cover
        limit = contextlib.nullcontext()
    import oracle
    from workloads.sample import snapshot
    L = wl.layers[0]
    lens = wl.commit_lens.cpu().numpy()
    tokens, spent, done = 0, 0.0, 0
    with limit:
        while spent < seconds and done < wl.B * max_passes:
            start = done % wl.B
            reqs = list(range(start, min(start + 16, wl.B)))
            sample = snapshot(wl, 0, reqs)
            t0 = time.perf_counter()
            ref = oracle.conv_update_verify(**sample.inputs)
            oracle.commit(layers=[dict(
                state=sample.inputs["state"], correction=ref["correction"],
                key_gate=ref["key_gate"], A_log=sample.inputs["A_log"],
                dt_bias=sample.inputs["dt_bias"],
                use_lower_bound=L.use_lower_bound,
                lower_bound=L.lower_bound)],
                state_indices=sample.new_slot, commit_lens=lens[reqs],
                spec_query_len=wl.Q,
                record_rows=None if wl.record_rows is None
                else sample.new_row)
            spent += time.perf_counter() - t0
            tokens += sum(min(len(t), wl.Q) for t in sample.tok)
            done += len(reqs)
    return {"value": tokens / spent, "unit": "verified tokens/s", "cores": 1,
            "kind": "oracle",
            "sample": f"{done} request verifies + commits "
                      f"({done / wl.B:.2f} passes over the {wl.B}-request "
                      f"batch), {tokens} tokens in {spent:.1f} s, numpy "
                      "fp64, 1 thread"}


def copy_calibration(gib: float = 1.0, reps: int = 5) -> None:
    """A plain device copy of known size, for scaling HBM byte counters."""
    import torch
    n = int(gib * (1 << 30)) // 4
    src = torch.ones(n, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n * 4, "copy_bytes_written": n * 4,
                      "reps": reps}), flush=True)


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="headline")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="time budget of the CPU-oracle sample (0: skip)")
    ap.add_argument("--cold", type=int, default=10,
                    help="launches timed after a cache-evicting write")
    ap.add_argument("--copy-calibration", action="store_true")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: this path runs on a single MI355X "
              "and has no multi-GPU mode (requests and heads shard with no "
              "exchange between GPUs).", file=sys.stderr)
        return 2
    if args.copy_calibration:
        copy_calibration()
        return 0

    import torch
    from workloads import make_workload
    from workloads import drive

    wl = make_workload(args.workload, "cuda", out_dtype="act")
    nbytes = algorithmic_bytes(wl)
    counter = torch.zeros(1, dtype=torch.int32, device="cuda")
    ctx = drive.commit_context(wl)

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        drive.verify(wl, 0, counter)
        if ev is not None:
            ev[1].record()
        ctx.commit(wl.state_indices, wl.commit_lens,
                   record_rows=wl.record_rows)
        if ev is not None:
            ev[2].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print(f"# warmup done ({args.warmup} steps)", file=sys.stderr, flush=True)

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)]
              for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(events[k])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps
    v_all = sorted(e[0].elapsed_time(e[1]) * 1e3 for e in events)
    c_all = sorted(e[1].elapsed_time(e[2]) * 1e3 for e in events)
    v_ms = sum(v_all) / args.steps / 1e3
    c_ms = sum(c_all) / args.steps / 1e3
    print(f"# timed {args.steps} steps: {ms_step:.4f} ms/step (verify "
          f"{v_ms * 1e3:.1f} us, commit {c_ms * 1e3:.1f} us)",
          file=sys.stderr, flush=True)

    def quant(xs, q):
        return xs[min(len(xs) - 1, int(q * len(xs)))]

    # Cold launches: each after an untimed 1 GiB write.
    scratch = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
    cold_v, cold_c = [], []
    for k in range(args.cold):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        scratch.fill_(float(k))
        ev[0].record()
        drive.verify(wl, 0, counter)
        ev[1].record()
        scratch.fill_(float(k) + 0.5)
        ev[2].record()
        ctx.commit(wl.state_indices, wl.commit_lens,
                   record_rows=wl.record_rows)
        ev[3].record()
        torch.cuda.synchronize()
        cold_v.append(ev[0].elapsed_time(ev[1]) * 1e3)
        cold_c.append(ev[2].elapsed_time(ev[3]) * 1e3)
    del scratch
    cold_v.sort()
    cold_c.sort()
    # The same single launches without the evicting write: the difference
    # to the back-to-back steps is launch ramp-up and drain, the difference
    # to the cold launches is what the caches kept between kernels.
    iso_v, iso_c = [], []
    for k in range(args.cold):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        torch.cuda.synchronize()
        ev[0].record()
        drive.verify(wl, 0, counter)
        ev[1].record()
        torch.cuda.synchronize()
        ev[2].record()
        ctx.commit(wl.state_indices, wl.commit_lens,
                   record_rows=wl.record_rows)
        ev[3].record()
        torch.cuda.synchronize()
        iso_v.append(ev[0].elapsed_time(ev[1]) * 1e3)
        iso_c.append(ev[2].elapsed_time(ev[3]) * 1e3)
    iso_v.sort()
    iso_c.sort()

    tokens = nbytes["tokens"]
    kernels = {
        "kda_verify_grid_kernel": (nbytes["verify"], v_ms),
        "kda_commit_grid_kernel": (nbytes["commit"], c_ms),
    }
    dom = max(kernels, key=lambda k: kernels[k][1])
    by, ms = kernels[dom]
    achieved = by / (ms * 1e-3) / 1e9
    traffic = traffic_from_profiles(dom, args.workload)
    result = {
        "metric": "verified tokens/s (KDA verify+commit, H=32 K=V=128, Q=4)",
        "value": tokens / (ms_step * 1e-3),
        "unit": "verified tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded decode batch, bf16 activations, fp32 "
                "state)",
        "config": {"workload": f"{args.workload}: B={wl.B} H={wl.H} "
                               f"K=V={wl.D} Q={wl.Q} layers=1 "
                               f"pool={wl.N} slots "
                               f"conv={'dim-first' if wl.conv_dim_first else 'token-first'}",
                   "batch": wl.B, "heads": wl.H, "head_dim": wl.D,
                   "window": wl.Q, "tokens_per_step": tokens},
        "roofline": {"bound": "hbm", "achieved": achieved,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": dom, "bytes_per_launch": by,
                     "us_per_launch": ms * 1e3},
        "step_hbm": {"bytes": nbytes["verify"] + nbytes["commit"],
                     "GB/s": (nbytes["verify"] + nbytes["commit"])
                     / (ms_step * 1e-3) / 1e9,
                     "frac": (nbytes["verify"] + nbytes["commit"])
                     / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS,
                     "verify_us": v_ms * 1e3, "commit_us": c_ms * 1e3,
                     "verify_GB/s": nbytes["verify"] / (v_ms * 1e-3) / 1e9,
                     "commit_GB/s": nbytes["commit"] / (c_ms * 1e-3) / 1e9},
        "kernels": {
            name: {"median_us": quant(xs, 0.5), "p10_us": quant(xs, 0.1),
                   "p90_us": quant(xs, 0.9),
                   "single_launch_median_us": quant(si, 0.5) if si else None,
                   "cold_median_us": quant(cs, 0.5) if cs else None}
            for name, xs, si, cs in (
                ("kda_verify_grid_kernel", v_all, iso_v, cold_v),
                ("kda_commit_grid_kernel", c_all, iso_c, cold_c))},
    }
    if args.cpu_seconds > 0:
        print("# cpu baseline ...", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
