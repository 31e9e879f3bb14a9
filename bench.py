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
verified per step / step time over K back-to-back steps, timed as one
replay of a HIP graph that holds the K steps; `ms_per_step_eager` is the
same K steps launched one by one with nothing between the launches,
`--eager` reports that instead); `roofline` describes the kernel that takes
the most time per step, from HIP events that the library records from the
kernels' own dispatch (kda_set_launch_events: an event recorded on the
stream between two launches adds its marker's gap, 6-11 us here, to the
kernel it brackets), over K more eager steps; `kernels` gives each kernel's
median, p10 and p90 over those steps, the median of single synchronized
launches, and the
median of single launches that each follow an untimed write and read of a
1 GiB buffer (which evicts the caches and leaves no dirty lines for the
timed kernel to write back), so that any help from the last-level cache
between kernels shows up as a difference; `cold_step` is the whole step
after the same eviction (median of `--cold` steps, one event pair from the
first kernel's dispatch to the last kernel's end); `cpu_baseline`
times the fp64 CPU oracle on a bounded sample of the same workload;
`step_hbm.frac_of_copy` relates the step's bandwidth to a plain 1 GiB
device copy timed in the same run; `deferred_form` (headline only) times
the same batch in the deferred form
(see `--workload fused`) as context for the headline figure.

Other workloads (`--workload`), each one JSON line of the same form:
  large     24 layers: 24 verifies, then one commit launch over all layers
            (B=256, Q=8);
  deferred  the deferred sequence at scale (B=1024, two layers): per layer
            one fused launch that folds the previous step's pending records
            into the checkpoint and then verifies;
  align     the headline batch under prefix caching (16-token state
            blocks): verify of the running block, then the commit plan,
            conv compaction and align-mode commit in one fused launch;
  align3    the align workload with the commit step as three launches
            (plan, conv compaction, commit);
  unfused   the headline batch through the unfused verify
            (kda_recoverssm_verify_qkv: q | k | v arrive convolved, no conv
            state) and the commit;
  fused     the headline batch in the deferred form: each step is one
            launch that folds the previous step's accepted positions into
            the checkpoints and then verifies (the same verify and commit
            work per step, one state pass fewer);
  tiny      2 requests, 2 heads, head dim 16, Q=3, fp32: `value` is the CPU
            seconds of one oracle pass (verify + commit of the whole
            workload); the GPU step time is reported beside it;
  single    one request at the full head shape (B=1, token-first conv):
            launch-latency bound, so the absolute microseconds per
            verify + commit are the figure (graph-replayed and eager);
  ragged    64 requests with ragged windows (q uniform in 1..4) and 10%
            null slots, verify only; its state (about 116 MiB) fits the
            256 MB last-level cache, so every timed launch follows an
            untimed 1 GiB write and read that evicts it.
The default run (headline) is the one the throughput figure is quoted on.
`--cold-steps` times any workload that way (an evicting write and read
before every timed step, the step timed from its first kernel's start to
its last kernel's end by one pair of dispatch-recorded events; a pair per
phase would add its own gap between the kernels).

  python bench.py [--steps K] [--warmup W] [--workload NAME] [--cold-steps]
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
METRIC = ("verified tokens/s + % HBM peak (KDA verify+commit, H=32 K=V=128, "
          "Q=4)")
EVICT_BYTES = 1 << 30          # the cache-evicting buffer before cold steps


def evict_caches(buf, k: float) -> None:
    """Untimed: write the 1 GiB buffer, then read it back.  The write alone
    would evict the caches but leave up to 256 MB of dirty last-level-cache
    lines, which the next (timed) kernel would then write back to HBM
    (measured: 148 us for a 127 us verify); the read leaves clean lines."""
    buf.fill_(k)
    buf.sum()
# workloads whose every timed launch is cold (the state fits the caches)
COLD_WORKLOADS = ("ragged",)
PROFILE_DIR = os.path.join(ROOT, "profiles")
ALIGN_BLOCK_SIZE = 16          # tokens per state block, align workload
KERNEL_SOURCES = {
    "kda_verify_grid_kernel": "kda_verify_kernels.hpp",
    "kda_verify_vtile_kernel": "kda_verify_kernels.hpp",
    "kda_verify_kernel": "kda_verify_kernels.hpp",
    "kda_commit_grid_kernel": "kda_commit.hip",
    "kda_commit_plan_kernel": "kda_plan.hip",
    "kda_compact_conv_kernel": "kda_plan.hip",
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


def algorithmic_bytes(wl, pending=None, boundary=None, conv=True) -> dict:
    """Bytes the method must move per launch (each state tile read once by
    the verify, read and written once by the commit; every activation,
    record and conv byte once), from the workload's seeded metadata.
    `pending` (per request): the fused deferred flush also reads that many
    records and writes the state tile back.  `boundary` (per request, the
    boundary length or 0): align mode also writes the boundary state, and
    the compaction moves three conv entries per channel to each of the
    final and boundary slots.  `conv` False: the unfused verify (the input
    row is already convolved: no taps, history or roll)."""
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
    per_launch = (C * W * e_w if conv else 0) + 4 * H + 4 * H * D \
        + 4 * (3 * wl.B + 1)
    verify = per_launch
    commit = 4 * H + 4 * H * D + 8 * wl.B   # gate params, slots + lens
    flush = 0
    compact = 0
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
        if conv:
            verify += (W - 1) * C * e_act                # conv history
            verify += (W - 2 + q) * C * e_act            # conv roll write
        verify += q * (C * e_act + H * D * e_act + H * e_act   # x, gate, beta
                       + H * D * e_out                   # out
                       + 4 * H * D + 2 * H * D * e_kg)   # records
        n = int(min(max(lens[b], 0), Q))
        if n > 0:
            commit += 8 * H * D * D + n * (4 * H * D + 2 * H * D * e_kg)
            if boundary is not None:
                compact += 2 * (W - 1) * C * e_act
                if boundary[b] > 0:
                    commit += 4 * H * D * D
                    compact += 2 * (W - 1) * C * e_act
        if pending is not None:
            m = int(min(max(pending[b], 0), Q))
            if m > 0:
                flush += 4 * H * D * D + m * (4 * H * D + 2 * H * D * e_kg)
    return dict(verify=verify, commit=commit, tokens=tokens, flush=flush,
                compact=compact)


SCHEDULES = {"default": 0, "per-item": 1, "tickets": 2, "v-tiles": 3}


def verify_kernel(wl, schedule: int, v_tiles: int) -> str:
    """Name of the kernel the plain verify of `wl` launches (the default
    schedule runs one workgroup per item up to 65535 requests)."""
    if schedule == SCHEDULES["v-tiles"]:
        return "kda_verify_vtile_kernel"
    if schedule == SCHEDULES["tickets"] or wl.B > 65535:
        return "kda_verify_kernel"
    return "kda_verify_grid_kernel"


def build_phases(name, wl, drive, torch, schedule=0, v_tiles=0):
    """The launches of one step of workload `name`, as phases timed with
    events on both sides: (kernel, algorithmic bytes per step, launches per
    step, function).  Returns (phases, verified tokens per step, config
    note)."""
    import numpy as np
    # ticket counter + one arrival counter per (request, head)
    counter = drive.counter(wl)
    L = len(wl.layers)
    if name in ("deferred", "fused"):
        nb = algorithmic_bytes(wl, pending=wl.commit_lens.cpu().numpy())

        def fused():
            for layer in range(L):
                drive.verify(wl, layer, counter, pending_lens=wl.commit_lens)
        return ([("kda_verify_grid_kernel", (nb["verify"] + nb["flush"]) * L,
                  L, fused)], nb["tokens"] * L,
                f"layers={L} fused flush+verify, pending "
                f"{int(wl.commit_lens.min())}..{int(wl.commit_lens.max())}")
    ctx = drive.commit_context(wl, conv=name in ("align", "align3"))
    if name in ("align", "align3"):
        from workloads.gen import running_block_tables
        bs = ALIGN_BLOCK_SIZE
        table, computed = running_block_tables(
            wl.state_indices.cpu().numpy(), wl.N, bs, seed=5)
        lens = wl.commit_lens.cpu().numpy()
        boundary = np.where(computed + lens >= bs, bs - computed, 0)
        nb = algorithmic_bytes(wl, boundary=boundary)
        table_t = torch.as_tensor(table, device="cuda")
        computed_t = torch.as_tensor(computed, device="cuda")
        ones = torch.ones(wl.B, dtype=torch.int32, device="cuda")
        kw = drive.verify_kwargs(wl, 0, counter)
        kw["num_accepted_tokens"] = ones
        from linear_attention_speculative_amd import conv_update_verify

        def verify():
            conv_update_verify(**kw)

        if name == "align3":
            # the same commit step as three launches: plan, compaction,
            # commit (the plan's four arrays carry between them)
            plan_out = tuple(torch.empty(wl.B, dtype=torch.int32,
                                         device="cuda") for _ in range(4))
            lens_o, final_o, bnd_o, blens_o = plan_out

            def plan():
                ctx.plan(wl.commit_lens, wl.state_indices,
                         wl.query_start_loc, block_table=table_t,
                         num_computed_tokens=computed_t,
                         mamba_block_size=bs, out=plan_out)

            def compact():
                ctx.compact(wl.state_indices, lens_o, final_o, bnd_o,
                            blens_o)

            def commit3():
                ctx.commit(wl.state_indices, lens_o, final_o,
                           boundary_state_indices=bnd_o,
                           boundary_recovery_lens=blens_o)
            # plan: metadata in (lens, slots, computed counts, one table
            # entry, query starts), four int32 arrays out
            plan_bytes = 4 * (wl.B + 1) + 4 * 4 * wl.B + 4 * 4 * wl.B
            return ([("kda_verify_grid_kernel", nb["verify"], 1, verify),
                     ("kda_commit_plan_kernel", plan_bytes, 1, plan),
                     ("kda_compact_conv_kernel", nb["compact"], 1, compact),
                     ("kda_commit_grid_kernel", nb["commit"], 1, commit3)],
                    nb["tokens"],
                    f"layers=1 align bs={bs}, {int((boundary > 0).sum())} "
                    "boundaries per step, commit step as three launches")

        def commit():
            ctx.commit_step(wl.commit_lens, wl.state_indices,
                            wl.query_start_loc, block_table=table_t,
                            num_computed_tokens=computed_t,
                            mamba_block_size=bs)
        # one launch: the commit kernel plans and compacts inline
        return ([("kda_verify_grid_kernel", nb["verify"], 1, verify),
                 ("kda_commit_grid_kernel", nb["commit"] + nb["compact"], 1,
                  commit)], nb["tokens"],
                f"layers=1 align bs={bs}, {int((boundary > 0).sum())} "
                "boundaries per step, fused commit step")
    if name == "unfused":
        nb = algorithmic_bytes(wl, conv=False)

        def verify_qkv():
            drive.verify_qkv(wl, 0, counter)

        def commit_u():
            ctx.commit(wl.state_indices, wl.commit_lens,
                       record_rows=wl.record_rows)
        return ([("kda_verify_grid_kernel", nb["verify"], 1, verify_qkv),
                 ("kda_commit_grid_kernel", nb["commit"], 1, commit_u)],
                nb["tokens"], "layers=1 unfused verify (convolved q|k|v)")
    nb = algorithmic_bytes(wl)
    vname = verify_kernel(wl, schedule, v_tiles)

    def verify_all():
        for layer in range(L):
            drive.verify(wl, layer, counter, schedule=schedule,
                         v_tiles=v_tiles)

    if name == "ragged":
        # verify only; the commit of this batch is exercised by the tests
        return ([(vname, nb["verify"] * L, L,
                  verify_all)], nb["tokens"] * L,
                f"layers={L} verify only, {int((wl.state_indices == 0).sum())} "
                "null slots")

    def commit():
        ctx.commit(wl.state_indices, wl.commit_lens,
                   record_rows=wl.record_rows)
    return ([(vname, nb["verify"] * L, L, verify_all),
             ("kda_commit_grid_kernel", nb["commit"] * L, 1, commit)],
            nb["tokens"] * L, f"layers={L}")


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


def host_threads() -> dict:
    """CPU threads this process may use, and the BLAS thread setting numpy
    would use by default (before the one-thread limit below)."""
    info = {"host_cores": len(os.sched_getaffinity(0))}
    try:
        from threadpoolctl import threadpool_info
        info["blas"] = [{"api": p.get("internal_api"),
                         "num_threads": p.get("num_threads")}
                        for p in threadpool_info()]
    except ImportError:  # pragma: no cover
        info["blas"] = None
    return info


def _one_thread():
    import contextlib
    try:
        from threadpoolctl import threadpool_limits
        return threadpool_limits(limits=1)
    except ImportError:  # pragma: no cover
        return contextlib.nullcontext()


def _oracle_pass(wl, reqs, oracle, snapshot):
    """Oracle verify + commit of layer 0 for `reqs`; returns (seconds spent
    in the oracle, verified tokens)."""
    L = wl.layers[0]
    lens = wl.commit_lens.cpu().numpy()
    sample = snapshot(wl, 0, reqs)
    t0 = time.perf_counter()
    ref = oracle.conv_update_verify(**sample.inputs)
    oracle.commit(layers=[dict(
        state=sample.inputs["state"], correction=ref["correction"],
        key_gate=ref["key_gate"], A_log=sample.inputs["A_log"],
        dt_bias=sample.inputs["dt_bias"],
        use_lower_bound=L.use_lower_bound, lower_bound=L.lower_bound)],
        state_indices=sample.new_slot, commit_lens=lens[reqs],
        spec_query_len=wl.Q,
        record_rows=None if wl.record_rows is None else sample.new_row)
    spent = time.perf_counter() - t0
    return spent, sum(min(len(t), wl.Q) for t in sample.tok)


def cpu_baseline(wl, seconds: float, max_passes: int = 8) -> dict:
    """The fp64 oracle, as it stands, single-threaded, on the requests of
    the same workload taken in order, 16 at a time (verify + commit), until
    `seconds` of CPU time have passed; passes over the whole batch repeat
    (at most `max_passes`) when one pass takes less than that."""
    import oracle
    from workloads.sample import snapshot
    tokens, spent, done = 0, 0.0, 0
    with _one_thread():
        while spent < seconds and done < wl.B * max_passes:
            start = done % wl.B
            reqs = list(range(start, min(start + 16, wl.B)))
            dt, tok = _oracle_pass(wl, reqs, oracle, snapshot)
            spent += dt
            tokens += tok
            done += len(reqs)
    return dict({"value": tokens / spent, "unit": "verified tokens/s",
                 "cores": 1, "kind": "oracle",
                 "sample": f"{done} request verifies + commits "
                           f"({done / wl.B:.2f} passes over the {wl.B}-request "
                           f"batch), {tokens} tokens in {spent:.1f} s, numpy "
                           "fp64, 1 thread (BLAS limited to 1)"},
                **host_threads())


def oracle_seconds(wl, seconds: float = 3.0) -> dict:
    """CPU seconds of one oracle pass over the whole workload (verify +
    commit of every request), single-threaded: median over repeated passes
    until `seconds` have passed (at least 5)."""
    import oracle
    from workloads.sample import snapshot
    times, tok = [], 0
    with _one_thread():
        while sum(times) < seconds or len(times) < 5:
            dt, tok = _oracle_pass(wl, list(range(wl.B)), oracle, snapshot)
            times.append(dt)
    times.sort()
    return dict({"value": times[len(times) // 2], "unit": "s", "cores": 1,
                 "kind": "oracle", "passes": len(times),
                 "min_s": times[0], "max_s": times[-1],
                 "sample": f"the whole workload ({wl.B} requests, {tok} "
                           "tokens) per pass, numpy fp64, 1 thread"},
                **host_threads())


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
                    help="launches timed after a cache-evicting write and "
                         "read")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--eager", action="store_true",
                    help="time the K steps as eager launches, not as one "
                         "replay of a HIP graph holding them")
    ap.add_argument("--schedule", default="default", choices=list(SCHEDULES),
                    help="verify schedule of the headline-form workloads")
    ap.add_argument("--v-tiles", type=int, default=0,
                    help="workgroups per (request, head) for --schedule "
                         "v-tiles (0: the library's choice)")
    ap.add_argument("--cold-steps", action="store_true",
                    help="precede every timed step with an untimed 1 GiB "
                         "write and read that evict the caches; the step "
                         "time is then taken from events around its "
                         "launches")
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

    cfg_name = "headline" if args.workload in ("align", "align3", "fused",
                                               "unfused") \
        else args.workload
    wl = make_workload(cfg_name, "cuda", out_dtype="act")
    phases, tokens, note = build_phases(args.workload, wl, drive, torch,
                                        SCHEDULES[args.schedule],
                                        args.v_tiles)
    if args.schedule != "default" or args.v_tiles:
        note += f" verify schedule={args.schedule} v_tiles={args.v_tiles}"
    P = len(phases)
    cold_steps = args.cold_steps or args.workload in COLD_WORKLOADS
    evict = torch.empty(EVICT_BYTES // 4, dtype=torch.float32,
                        device="cuda") if cold_steps else None

    from linear_attention_speculative_amd import set_launch_events

    def step(ev=None):
        # ev: per phase a (start, stop) pair of events that the library
        # records from the kernels' own dispatch (the first launch's start,
        # the last launch's end); an event recorded on the stream between
        # launches would add its marker's gap to the kernel it brackets
        for i, (_, _, n, fn) in enumerate(phases):
            if ev is not None:
                set_launch_events(ev[i][0], ev[i][1], n)
            fn()
            if ev is not None and set_launch_events(None, None, 0) != 0:
                raise RuntimeError(f"phase {phases[i][0]} launched fewer "
                                   f"than {n} kernels")

    def step_whole(pair):
        # one (start, stop) pair around the whole step: the first launch's
        # dispatch to the last launch's end, with no event between phases
        total = sum(n for (_, _, n, _) in phases)
        set_launch_events(pair[0], pair[1], total)
        for (_, _, _, fn) in phases:
            fn()
        if set_launch_events(None, None, 0) != 0:
            raise RuntimeError("a step launched fewer kernels than armed")

    def new_events():
        out = []
        for _ in range(P):
            pair = (torch.cuda.Event(enable_timing=True),
                    torch.cuda.Event(enable_timing=True))
            for e in pair:
                e.record()                 # creates the event
            out.append(pair)
        return out

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print(f"# warmup done ({args.warmup} steps)", file=sys.stderr, flush=True)

    # The step time: K eager steps with nothing between the launches (cold
    # steps: each after an untimed cache-evicting write and read, timed from
    # its first kernel's start to its last kernel's end by one event pair
    # that the library records from the kernels' own dispatch).
    events = [new_events() for _ in range(args.steps)]
    whole = [new_events()[0] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        if evict is not None:
            evict_caches(evict, float(k))  # untimed: before the first kernel
            step_whole(whole[k])
        else:
            step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps
    if evict is not None:
        ms_step = sum(e[0].elapsed_time(e[1]) for e in whole) / args.steps
    # per-kernel durations: K more steps (cold ones after the same eviction)
    # with every phase's launches timed from their own dispatch
    for k in range(args.steps):
        if evict is not None:
            evict_caches(evict, float(k) + 0.25)
        step(events[k])
    torch.cuda.synchronize()
    if evict is not None:
        ms_phased = sum(e[0][0].elapsed_time(e[P - 1][1])
                        for e in events) / args.steps
        print(f"# cold steps: {ms_step:.4f} ms/step with one event pair; "
              f"{ms_phased:.4f} ms with an event pair per phase",
              file=sys.stderr, flush=True)
    # per phase: microseconds per launch (a phase of n launches / n)
    per = [sorted(e[i][0].elapsed_time(e[i][1]) * 1e3 / phases[i][2]
                  for e in events) for i in range(P)]
    mean_ms = [sum(x) / args.steps / 1e3 for x in per]
    print(f"# timed {args.steps} steps: {ms_step:.4f} ms/step ("
          + ", ".join(f"{ph[0]} {m * 1e3:.1f} us/launch"
                      for ph, m in zip(phases, mean_ms)) + ")",
          file=sys.stderr, flush=True)

    # The figure reported: the same K steps captured in one HIP graph and
    # replayed once (after an untimed replay), so that host launch overhead
    # stays out of the step time.  Falls back to the eager time if the
    # capture fails.
    timing, ms_eager = ("cold" if evict is not None else "eager"), ms_step
    if not args.eager and evict is None:
        try:
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                step()
            torch.cuda.current_stream().wait_stream(side)
            torch.cuda.synchronize()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                for _ in range(args.steps):
                    step()
            graph.replay()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            graph.replay()
            torch.cuda.synchronize()
            ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
            timing = "graph"
            del graph
            print(f"# graph replay of {args.steps} steps: {ms_step:.4f} "
                  "ms/step", file=sys.stderr, flush=True)
        except RuntimeError as exc:
            print(f"# graph capture failed ({exc}); eager timing",
                  file=sys.stderr, flush=True)

    def quant(xs, q):
        return xs[min(len(xs) - 1, int(q * len(xs)))]

    # Cold phases: each after an untimed 1 GiB write and read; then the same
    # single phases without it.  The difference to the back-to-back steps
    # is launch ramp-up and drain, the difference between the two is what
    # the caches kept between kernels.
    scratch = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
    cold = [[] for _ in range(P)]
    iso = [[] for _ in range(P)]
    def timed(fn, n):
        """One phase, its launches timed from their own dispatch."""
        ev = new_events()[0]
        set_launch_events(ev[0], ev[1], n)
        fn()
        if set_launch_events(None, None, 0) != 0:
            raise RuntimeError("a phase launched fewer kernels than armed")
        torch.cuda.synchronize()
        return ev[0].elapsed_time(ev[1]) * 1e3 / n

    for k in range(args.cold):
        for i, (_, _, n, fn) in enumerate(phases):
            evict_caches(scratch, float(k) + 0.5 * i)
            cold[i].append(timed(fn, n))
    # Whole cold steps (warm runs only; a --cold-steps run times its steps
    # this way already): each after the eviction, one event pair from the
    # first kernel's dispatch to the last kernel's end.
    cold_step = []
    if evict is None:
        for k in range(args.cold):
            evict_caches(scratch, float(k) + 0.75)
            pair = new_events()[0]
            step_whole(pair)
            torch.cuda.synchronize()
            cold_step.append(pair[0].elapsed_time(pair[1]))
        cold_step.sort()
    del scratch
    for k in range(args.cold):
        for i, (_, _, n, fn) in enumerate(phases):
            torch.cuda.synchronize()
            iso[i].append(timed(fn, n))
    for xs in cold + iso:
        xs.sort()

    # A plain 1 GiB device copy on the same GPU, for the fraction of what
    # this HBM sustains for streaming read + write traffic.
    csrc = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    cdst = torch.empty_like(csrc)
    for _ in range(2):
        cdst.copy_(csrc)
    cev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    torch.cuda.synchronize()
    cev[0].record()
    for _ in range(5):
        cdst.copy_(csrc)
    cev[1].record()
    torch.cuda.synchronize()
    copy_gbs = 2 * csrc.numel() * 4 * 5 / (cev[0].elapsed_time(cev[1]) *
                                           1e-3) / 1e9
    del csrc, cdst

    dom = max(range(P), key=lambda i: mean_ms[i] * phases[i][2])
    kname, by_step, n_launch, _ = phases[dom]
    ms = mean_ms[dom]
    by = by_step / n_launch
    achieved = by / (ms * 1e-3) / 1e9
    traffic = traffic_from_profiles(kname, args.workload)
    step_bytes = sum(ph[1] for ph in phases)
    result = {
        "metric": METRIC if args.workload == "headline" else
        f"verified tokens/s ({args.workload} workload)",
        "value": tokens / (ms_step * 1e-3),
        "unit": "verified tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "timing": timing,
        "ms_per_step_eager": ms_eager,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded decode batch, bf16 activations, fp32 "
                "state)",
        "us_per_step": ms_step * 1e3,
        "config": {"workload": f"{args.workload}: B={wl.B} H={wl.H} "
                               f"K=V={wl.D} Q={wl.Q} {note} "
                               f"pool={wl.N} slots "
                               f"conv={'dim-first' if wl.conv_dim_first else 'token-first'}",
                   "batch": wl.B, "heads": wl.H, "head_dim": wl.D,
                   "window": wl.Q, "tokens_per_step": tokens},
        "roofline": {"bound": "hbm", "achieved": achieved,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": kname, "bytes_per_launch": by,
                     "us_per_launch": ms * 1e3,
                     # the same kernel launched after an untimed 1 GiB
                     # write and read that evict the caches (median of --cold)
                     "cold": None if not cold[dom] else {
                         "us_per_launch": quant(cold[dom], 0.5),
                         "achieved": by / (quant(cold[dom], 0.5) * 1e-6)
                         / 1e9,
                         "frac": by / (quant(cold[dom], 0.5) * 1e-6) / 1e9
                         / HBM_PEAK_GBS}},
        "step_hbm": dict(
            {"bytes": step_bytes,
             "GB/s": step_bytes / (ms_step * 1e-3) / 1e9,
             "frac": step_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS,
             "copy_GB/s": copy_gbs,
             "frac_of_copy": step_bytes / (ms_step * 1e-3) / 1e9 / copy_gbs},
            **{f"{ph[0]}_us_per_launch": m * 1e3
               for ph, m in zip(phases, mean_ms)},
            **{f"{ph[0]}_GB/s": ph[1] / ph[2] / (m * 1e-3) / 1e9
               for ph, m in zip(phases, mean_ms)}),
        # the whole step after an untimed 1 GiB write and read (median of
        # --cold steps)
        "cold_step": None if not cold_step else {
            "ms_per_step": quant(cold_step, 0.5),
            "value": tokens / (quant(cold_step, 0.5) * 1e-3),
            "frac": step_bytes / (quant(cold_step, 0.5) * 1e-3) / 1e9
            / HBM_PEAK_GBS},
        "kernels": {
            ph[0]: {"median_us": quant(per[i], 0.5),
                    "p10_us": quant(per[i], 0.1),
                    "p90_us": quant(per[i], 0.9),
                    "single_launch_median_us":
                        quant(iso[i], 0.5) if iso[i] else None,
                    "cold_median_us": quant(cold[i], 0.5) if cold[i] else None,
                    "launches_per_step": ph[2]}
            for i, ph in enumerate(phases)},
    }
    if args.workload == "headline":
        # Context, not the headline figure: the same batch in the deferred
        # form of the state page (commit of the previous step folded into
        # this step's verify launch).
        fphases, ftokens, fnote = build_phases("fused", wl, drive, torch)
        ffn = fphases[0][3]
        for _ in range(args.warmup):
            ffn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            ffn()
        torch.cuda.synchronize()
        fms = (time.perf_counter() - t0) * 1e3 / args.steps
        fby = fphases[0][1]
        result["deferred_form"] = {
            "value": ftokens / (fms * 1e-3), "unit": "verified tokens/s",
            "ms_per_step": fms, "step": fnote,
            "GB/s": fby / (fms * 1e-3) / 1e9,
            "frac": fby / (fms * 1e-3) / 1e9 / HBM_PEAK_GBS}
        print(f"# deferred form: {fms:.4f} ms/step", file=sys.stderr,
              flush=True)
    if args.workload == "tiny":
        # the small workload's figure is the oracle's CPU time; the GPU
        # step time stays beside it
        cpu = oracle_seconds(wl)
        result.update(metric="CPU seconds of one oracle pass (tiny workload: "
                             "verify + commit)",
                      value=cpu["value"], unit="s", higher_is_better=False,
                      dtype="f64", gpu_verified_tokens_per_s=result["value"])
        result["cpu_baseline"] = cpu
    elif args.cpu_seconds > 0:
        print("# cpu baseline ...", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
