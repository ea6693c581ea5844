"""Throughput of one draft-tree step (build + tree attention + verify + compact) on one GPU.

Default workload: the TALON tree on the Llama-3-8B attention-layer shape (1 sequence,
32 query / 8 KV heads, head dim 128, bf16, KV prefix 2048, budget B = 60, root Top-K 10,
gate alpha 0.1, vocab 128256, greedy verification). Inputs are seeded synthetic arrays
resident in HBM before timing starts. Prints one JSON line.

The ``cpu_baseline`` leg times the float64 CPU oracle on the same workload (a bounded
number of steps) and is the only part of this file that touches the oracle.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
MFMA_F32_PEAK_TFLOPS = 157.3    # MI355X fp32 vector
METRIC = "draft-tree verify steps/sec + tree tokens/sec, % roofline, Llama-3-8B shape"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="c2_talon_llama3_8b")
    ap.add_argument("--seed", type=int, default=None)
    ap.add_argument("--launch", choices=["graph", "eager"], default="eager",
                    help="replay the step as a captured HIP graph, or launch its kernels one by one")
    ap.add_argument("--separate-compact", action="store_true",
                    help="compact the KV cache in its own launch instead of inside the verification")
    ap.add_argument("--event-every", type=int, default=16,
                    help="record per-stage events on every n-th timed step")
    ap.add_argument("--cpu-steps", type=int, default=4, help="oracle steps for cpu_baseline (0: skip)")
    ap.add_argument("--decode-steps", type=int, default=0,
                    help="also run a decoding loop of this many steps on one growing KV cache and add "
                         "its rates and bookkeeping to the line as `decode` (0: skip)")
    ap.add_argument("--gamma", type=float, default=0.1,
                    help="draft-to-target cost ratio for the decoding loop's Speedup = E[A]/(1 + gamma eta)")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="before timing, run one device-to-device copy of this many MiB (a reference "
                         "kernel of known traffic for HBM byte counters); not part of any timing")
    return ap.parse_args()


def algorithmic_work(step, wl):
    """Bytes (and flops) each stage must move/compute for this step, from the built tree.

    Build: every draft row the builder expands, read once. Attention: prefix K/V once per
    KV head, tree K/V, Q in and O out; flops 4*Hq*D per visible (query, key) pair. Verify:
    greedy reads each node's target row once; rejection sampling reads, at each node the
    walk visits (the accepted path), its target row and, when it has children, its draft
    row (residual passes re-read those rows). Compaction: K and V rows of the path, read
    and written once.
    """
    import numpy as np
    cfg = wl.cfg
    esz = 2 if cfg.dtype == "bf16" else 4
    n_nodes = step.tree.n_nodes.cpu().numpy()
    depth = step.tree.depth.cpu().numpy()
    layers = step.tree.layers.cpu().numpy()
    anc = step.tree.anc.cpu().numpy().view(np.uint64)
    plen = step.verify_out[1].cpu().numpy()
    paths = step.verify_out[0].cpu().numpy()
    parents = step.tree.parent.cpu().numpy()
    out = {"build": {"bytes": 0.0}, "attention": {"bytes": 0.0, "flops": 0.0},
           "verify": {"bytes": 0.0}, "compact": {"bytes": 0.0}}
    row = cfg.V * esz
    for s in range(cfg.S):
        N = int(n_nodes[s])
        P = int(wl.P[s])
        if cfg.build == "talon":
            out["build"]["bytes"] += int(np.sum(depth[s, :N] < int(layers[s]))) * row
        elif cfg.build == "spine":
            out["build"]["bytes"] += int(np.sum(np.asarray(wl.widths) > 0)) * row
        elif cfg.build == "opt":
            W, rows = 1, 0
            for _ in range(int(layers[s])):
                rows += W
                W = min(cfg.n, W * min(cfg.n, cfg.V))
            out["build"]["bytes"] += rows * row
        else:  # given shape: parents and masks only
            out["build"]["bytes"] += N * (3 * 4 + 8 + 8 * step.tree.words)
        vis = sum(bin(int(w)).count("1") for w in anc[s, :N].ravel())
        out["attention"]["bytes"] += (2 * P * cfg.Hkv * cfg.D + 2 * N * cfg.Hkv * cfg.D
                                      + 2 * N * cfg.Hq * cfg.D) * esz
        out["attention"]["flops"] += 4.0 * cfg.Hq * cfg.D * (N * P + vis)
        if cfg.verify == "greedy":   # every node's argmax decides which paths match
            out["verify"]["bytes"] += N * row
        else:   # p and q are needed only where the walk goes: the nodes of the accepted path
            internal = set(int(x) for x in parents[s, 1:N])
            for v in paths[s, :int(plen[s])]:
                out["verify"]["bytes"] += row * (2 if int(v) in internal else 1)
        out["compact"]["bytes"] += 4 * int(plen[s]) * cfg.Hkv * cfg.D * esz
    out["verify_compact"] = {"bytes": out["verify"]["bytes"] + out["compact"]["bytes"]}
    return out


def talon_rows_name(cfg) -> str:
    """TALON's row kernel: bf16 rows in 32768-value parts, fp32 rows in chunks."""
    return "talon_rows_bf16_kernel" if cfg.dtype == "bf16" else "talon_rows_kernel"


def kernel_work(step, wl, work):
    """Algorithmic bytes (and flops) of one launch of each kernel of the step, from the
    stage figures: the kernel that streams a stage's rows or keys carries its work, the
    stage's small follow-up kernels (selections, merges of partials) carry none."""
    cfg = wl.cfg
    out = {}
    if cfg.build == "talon":
        out[talon_rows_name(cfg)] = dict(work["build"])
    elif cfg.build == "spine":
        out["spine_bf16_kernel+spine_kernel"] = dict(work["build"])
    elif cfg.build == "opt":
        out["opt_rows_bf16_kernel+opt_rows_kernel+opt_root_bf16_kernel+opt_root_kernel"] = dict(work["build"])
    else:
        out["given_tree_kernel"] = dict(work["build"])
    att = "attn_bf16_kernel" if cfg.dtype == "bf16" else "attn_f32_kernel"
    out[att] = dict(work["attention"])
    if cfg.verify == "greedy":
        # bf16 rows go through the part kernel, fp32 rows through the chunk kernel
        out["verify_greedy_bf16_kernel+verify_greedy_kernel"] = dict(work["verify_compact"] if step.fuse_compact
                                                                     else work["verify"])
    else:
        out["sample_walk_kernel"] = dict(work["verify_compact"] if step.fuse_compact else work["verify"])
    if not step.fuse_compact:
        out["compact_kernel"] = dict(work["compact"])
    return out


# The kernels each stage launches (a stage's time is the HIP-event time of all of them;
# rocprofv3 --kernel-trace lists them separately, and their averages add up to it).
STAGE_KERNELS = {
    "build": lambda c: {"talon": [talon_rows_name(c), "talon_select_kernel"],
                        "spine": ["spine_bf16_kernel", "spine_kernel"],
                        "opt": ["opt_init_kernel", "opt_root_bf16_kernel", "opt_root_kernel", "opt_rows_bf16_kernel",
                                "opt_rows_kernel",
                                "opt_bound_kernel",
                                "opt_collect_kernel", "opt_select_kernel", "opt_finalize_kernel"],
                        "given": ["given_tree_kernel"]}[c.build],
    "attention": lambda c: (["attn_bf16_kernel", "attn_combine_rows_kernel"] if c.dtype == "bf16"
                            else ["attn_f32_kernel"]),
    "verify": lambda c: (["verify_greedy_bf16_kernel", "verify_greedy_kernel"] if c.verify == "greedy"
                         else ["sample_walk_kernel"]),
    "compact": lambda c: ["compact_kernel"],
    "verify_compact": lambda c: (["verify_greedy_bf16_kernel or verify_greedy_kernel (compacts the cache)"]
                                 if c.verify == "greedy"
                                 else ["sample_walk_kernel (compacts the cache)"]),
}


def kernel_stage(kernel: str, fused: bool) -> str:
    """The stage (launch group of DraftTreeStep) a kernel belongs to."""
    if kernel.startswith(("talon_", "spine_", "opt_", "given_")):
        return "build"
    if kernel.startswith("attn_"):
        return "attention"
    if kernel.startswith(("verify_", "sample_")):
        return "verify_compact" if fused else "verify"
    return "compact"


def csrc_sha256() -> str:
    """Hash of the kernel sources; recorded traffic counts are used only while it matches."""
    import hashlib
    csrc = os.path.join(ROOT, "draft_tree_verification_build_amd", "csrc")
    h = hashlib.sha256()
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".h")):
            h.update(f.encode())
            with open(os.path.join(csrc, f), "rb") as fh:
                h.update(fh.read())
    return h.hexdigest()


def recorded_traffic(workload: str, stage: str):
    """HBM bytes per launch measured with rocprofv3 counters for this workload and stage, or None."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f).get(workload)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("csrc_sha256") != csrc_sha256():
        return None
    return rec.get(stage)


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(wl, steps: int):
    """The oracle on the host: `steps` whole steps with one thread, then with every core this
    process may run on (numpy's BLAS threads; the oracle's loops stay in one thread)."""
    from threadpoolctl import threadpool_limits
    from oracle import step as ostep
    ncores = len(os.sched_getaffinity(0))
    legs = {}
    for label, limit in (("one_thread", 1), ("all_cores", ncores)):
        with threadpool_limits(limits=limit):
            t0 = time.perf_counter()
            for _ in range(steps):
                ostep.run_step(wl)
            legs[label] = steps / (time.perf_counter() - t0)
    return {"value": legs["all_cores"], "unit": "steps/s", "cores": ncores, "kind": "oracle",
            "sample": f"{steps} whole oracle steps (build, attention, verify, compact) of the same "
                      f"workload, float64 numpy, per leg",
            "one_thread": {"value": legs["one_thread"], "cores": 1}, "cpu_model": cpu_model()}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the draft-tree step has no multi-GPU path)", file=sys.stderr)
        return 2
    import numpy as np
    import torch
    from draft_tree_verification_build_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        from draft_tree_verification_build_amd import build_lib
        build_lib.build()
    from draft_tree_verification_build_amd.step import DraftTreeStep
    from workloads import make_workload
    from workloads.configs import CONFIG_ORDER

    seed = args.seed if args.seed is not None else CONFIG_ORDER.index(args.config) + 1
    if args.copy_mib > 0:
        n = args.copy_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    wl = make_workload(args.config, seed)
    cfg = wl.cfg
    step = DraftTreeStep(wl, "cuda", fuse_compact=not args.separate_compact)
    stream = torch.cuda.current_stream()
    stages = [name for name, _ in step.stages()]
    fns = [fn for _, fn in step.stages()]

    for _ in range(args.warmup):
        step.run()
    torch.cuda.synchronize()
    st = step.ws_status()
    if any(v != 0 for v in st.values()):
        print(f"device status after warmup: {st}", file=sys.stderr)
        return 1

    # Optionally one step captured as a HIP graph (the step makes no host round trip and no
    # allocation once warm), replayed on the launch stream. Measured on MI355X, replay only
    # pays off where the host's launch work is the bound (c1: 35 -> 27.5 us per step); for
    # the larger steps it adds about 0.7 us per kernel (c2: 68.4 -> 72.9 us), so eager
    # launches are the default.
    graph = None
    if args.launch == "graph":
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step.run()
        for _ in range(3):
            graph.replay()
        torch.cuda.synchronize()
        st = step.ws_status()
        if any(v != 0 for v in st.values()):
            print(f"device status after graph replays: {st}", file=sys.stderr)
            return 1
    run_step = graph.replay if graph is not None else step.run

    # Whole-step timing. Every `event_every`-th step of the same timed loop runs its stages as
    # separate launches with HIP events on the launch stream around each stage; a record
    # between two kernels adds a gap of a few microseconds, so sampling keeps that cost inside
    # the timed region at about 1%.
    # Every `every`-th step also carries HIP events: steps k = 0, every, ... around each
    # stage (torch events on the launch stream); steps k = every/2, every + every/2, ...
    # around each kernel (the library's own events, recorded on the stream it launches on).
    from draft_tree_verification_build_amd import api
    every = max(2, args.event_every)
    sampled = list(range(0, args.steps, every))
    ktimed = set(range(every // 2, args.steps, every)) or {args.steps - 1}
    ev = {k: [torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)] for k in sampled}
    api.kernel_timing(False, reset=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        e = ev.get(k)
        if e is None:
            if k in ktimed:
                api.kernel_timing(True)
                step.run()
                api.kernel_timing(False)
            else:
                run_step()
            continue
        e[0].record(stream)
        for j, fn in enumerate(fns):
            fn()
            e[j + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ktimes = api.kernel_times()
    st = step.ws_status()
    if any(v != 0 for v in st.values()):
        print(f"device status after the timed steps: {st}", file=sys.stderr)
        return 1
    stage_ms = {name: float(np.mean([ev[k][j].elapsed_time(ev[k][j + 1]) for k in sampled]))
                for j, name in enumerate(stages)}

    work = algorithmic_work(step, wl)
    ms = wall * 1e3 / args.steps
    steps_s = args.steps / wall
    tree_tokens = float(step.tree.n_nodes.sum().item() - cfg.S)  # draft nodes, root excluded
    stage_report = {}
    for name in stages:
        t = stage_ms[name] * 1e-3
        w = work[name]
        gbs = w["bytes"] / t / 1e9 if t > 0 else 0.0
        rep = {"ms": stage_ms[name], "bytes": w["bytes"], "GB/s": gbs, "hbm_frac": gbs / HBM_PEAK_GBS}
        if "flops" in w:
            tf = w["flops"] / t / 1e12 if t > 0 else 0.0
            peak = MFMA_BF16_PEAK_TFLOPS if cfg.dtype == "bf16" else MFMA_F32_PEAK_TFLOPS
            rep.update({"flops": w["flops"], "TFLOP/s": tf, "mfma_frac": tf / peak})
        stage_report[name] = rep
    # Per kernel: mean event time per launch and per step; the dominant kernel (most time per
    # step) gives `roofline`: its algorithmic bytes (or flops) per launch over its mean launch
    # time, against 8 TB/s HBM or 2.5 PFLOP/s dense bf16 MFMA.
    nk = max(1, len(ktimed))
    kwork = kernel_work(step, wl, work)
    kernels = {}
    for name, (tot, cnt) in ktimes.items():
        kernels[name] = {"launches_per_step": cnt / nk, "ms_per_launch": tot / cnt, "ms_per_step": tot / nk}
    for key, w in kwork.items():   # a work entry may cover several kernels ("a+b")
        parts = [kernels[n] for n in key.split("+") if n in kernels]
        if not parts:
            continue
        launches = sum(p["launches_per_step"] for p in parts)
        ms_launch = sum(p["ms_per_step"] for p in parts) / launches
        for n in key.split("+"):
            if n in kernels:
                kernels[n]["work_of"] = key
        per = {"bytes": w["bytes"] / launches}
        if "flops" in w:
            per["flops"] = w["flops"] / launches
        kernels[key] = {**kernels.get(key, {}), "launches_per_step": launches, "ms_per_launch": ms_launch,
                        "ms_per_step": ms_launch * launches, **{f"{k}_per_launch": v for k, v in per.items()}}
    scored = {n: k for n, k in kernels.items() if "bytes_per_launch" in k}
    dom = max(kernels, key=lambda n: kernels[n]["ms_per_step"]) if kernels else None
    if dom is not None and "bytes_per_launch" not in kernels[dom]:
        # the most expensive kernel moves no algorithmic data (a selection or a merge of
        # partials): the roofline goes to the most expensive kernel that streams data, and
        # the line names both
        slowest = dom
        dom = max(scored, key=lambda n: scored[n]["ms_per_step"])
    else:
        slowest = dom
    kd = kernels[dom]
    t = kd["ms_per_launch"] * 1e-3
    gbs = kd["bytes_per_launch"] / t / 1e9
    flops = kd.get("flops_per_launch")
    ridge = (MFMA_BF16_PEAK_TFLOPS * 1e12) / (HBM_PEAK_GBS * 1e9)
    if flops is not None and flops / max(kd["bytes_per_launch"], 1) > ridge and cfg.dtype == "bf16":
        tf = flops / t / 1e12
        roof = {"bound": "mfma", "achieved": tf, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": tf / MFMA_BF16_PEAK_TFLOPS}
    else:
        roof = {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS}
    roof["traffic"] = recorded_traffic(cfg.name, dom)
    roof["kernel"] = dom
    roof["ms_per_launch"] = kd["ms_per_launch"]
    roof["bytes_per_launch"] = kd["bytes_per_launch"]
    if flops is not None:
        roof["flops_per_launch"] = flops
    if slowest != dom:
        roof["slowest_kernel"] = slowest
    stage = kernel_stage(dom.split("+")[0], step.fuse_compact)
    roof["stage"] = {"name": stage, **stage_report[stage]}

    out = {
        "metric": METRIC, "value": steps_s, "unit": "steps/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": cfg.dtype, "data": "synthetic",
        "config": {"workload": cfg.name, "seed": seed, "S": cfg.S, "Hq": cfg.Hq, "Hkv": cfg.Hkv,
                   "D": cfg.D, "P": cfg.P, "V": cfg.V, "N": cfg.N, "build": cfg.build,
                   "verify": cfg.verify, "launch": args.launch,
                   "compaction": "separate" if args.separate_compact else "in verification"},
        "tree_tokens_per_s": tree_tokens * steps_s,
        "roofline": roof,
        "stages": stage_report,
        "stage_samples": len(sampled),
        "kernels": kernels,
        "kernel_samples": nk,
    }
    if args.decode_steps > 0:
        out["decode"] = decode_loop(args.config, seed, args.decode_steps, args.gamma)
    if args.cpu_steps > 0:
        out["cpu_baseline"] = cpu_baseline(wl, args.cpu_steps)
    print(json.dumps(out), flush=True)
    return 0


def decode_loop(config: str, seed: int, steps: int, gamma: float) -> dict:
    """A decoding loop of ``steps`` draft-tree steps on one KV cache that grows by each
    step's accepted path. Every step's inputs are generated and uploaded before timing, and
    step 0 (which allocates the workspaces) runs untimed; the timed region holds steps
    1 .. steps-1, the writes of each step's tree keys and values after the current prefix,
    and the host's read of the accepted lengths after every step. E[A], eta and Speedup
    cover all steps."""
    import numpy as np
    import torch
    from draft_tree_verification_build_amd.decode import DraftTreeDecoder
    from draft_tree_verification_build_amd import goose
    from workloads import config_by_name, make_step_inputs
    cfg = config_by_name(config)
    adaptive = cfg.build == "spine"   # GOOSE: each step's topology from the spine acceptance so far
    policy = goose.SpineTopology(cfg.N - 1) if adaptive else None
    topo = {0: policy.plan()} if adaptive else {}

    def inputs(t):
        if not adaptive:
            return make_step_inputs(config, seed, t)
        L, w = topo[t]
        return make_step_inputs(config, seed, t, n_spine=L, n_forks=len(w), spine_widths=tuple(w))

    dec = DraftTreeDecoder(inputs, steps, "cuda")

    def observe(t, rec):
        L = topo[t][0]
        policy.observe([goose.spine_accepted(rec["path"][s][:int(rec["A"][s]) + 1], L) for s in range(dec.S)], L)
        topo[t + 1] = policy.plan()

    if adaptive:   # topologies depend on results: inputs are made and uploaded step by step, untimed
        wall = 0.0
        for t in range(steps):
            up = dec.upload(t)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            rec = dec.step(t, up)
            if t > 0:
                wall += time.perf_counter() - t0
            observe(t, rec)
    else:
        ups = [dec.upload(t) for t in range(steps)]
        dec.step(0, ups[0])   # untimed: the first step allocates the workspaces
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for t in range(1, steps):
            dec.step(t, ups[t])
        wall = time.perf_counter() - t0
    books = dec.bookkeeping(gamma)
    timed = steps - 1
    emitted = float(sum(int(r["A"].sum()) + len(r["A"]) for r in dec.log[1:]))
    return {"steps": steps, "timed_steps": timed, "ms_per_step": wall * 1e3 / timed, "steps_per_s": timed / wall,
            "emitted_tokens_per_s": emitted / wall, "sequences": len(books),
            "E_A": float(np.mean([b["E_A"] for b in books])), "eta": float(np.mean([b["eta"] for b in books])),
            "gamma": gamma, "speedup": float(np.mean([b["speedup"] for b in books])),
            "P_final": [int(p) for p in dec.P_host],
            **({"topology": "GOOSE adaptive", "spine_lengths": [int(topo[t][0]) for t in range(steps)]}
               if adaptive else {}),
            **({"E_A_predicted": float(np.mean([r["E_A_predicted"].mean() for r in dec.log])),
                "A_realised": float(np.mean([r["A"].mean() for r in dec.log]))}
               if cfg.build == "opt" else {})}


if __name__ == "__main__":
    rc = main()
    if rc:
        sys.exit(rc)
    # a clean run ends by falling off the script: some profilers only flush their output on
    # this path, not on the SystemExit one
