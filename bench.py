"""Benchmark of the fused bidirectional selective scan (and SS2D cross-scan) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config N | --all] [--no-cpu] [--v2] [--bwd]
                    [--d-state 32] [--front]

A step is one call of the hot path over one batch of seeded synthetic input already resident in
HBM.  The default workload is the Vim-Ti layer scan (batch 128, d_inner 384, L 197, d_state 16,
bf16 activations, fp32 state), the configuration the metric is quoted on.  R input/output sets
are rotated so that at least 1 GiB is touched between reuses and the 256 MB Infinity Cache cannot
serve the inputs.  Rank 0 prints one JSON line per workload.  ``--v2`` runs the Vim workloads
through the entry point whose backward branch has its own u_b, Δ_raw_b and bias_b; ``--bwd``
times the backward pass (all gradients) of the Vim workloads instead of the forward; ``--d-state
32`` runs the workloads (forward or backward) with 32 states instead of 16; ``--front`` times the front
convolution that produces the scan input followed by the scan.
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
# ALU roofline of the recurrence.  One state update (token, channel, direction, state) needs one
# exp2 and four fp32 VALU ops (Δ·A', h·a, h + Δu·B, y + C·h).  MI355X: 256 CUs at 2.4 GHz; fp32
# vector peak 157.3 TFLOP/s = 128 FMA lanes per CU per clock; transcendentals issue at a quarter of
# that, 32 lanes per CU per clock.  So one update costs at least 4/128 + 1/32 = 1/16 CU-clock and
# the peak is 256 * 2.4e9 * 16 = 9.83e12 updates/s.
CUS, CLOCK_HZ = 256, 2.4e9
ALU_PEAK_UPD_S = CUS * CLOCK_HZ / (4.0 / 128 + 1.0 / 32)
# Backward: per state update the forward state must be rebuilt (one exp2 and three VALU ops: Δ·A',
# h·a, h + Δu·B) and the adjoint walked (nine VALU ops with the decay reused: g·C, λ, a·h_{t-1},
# λ·(a h_{t-1}), the dΔ and dA accumulations, Σ λ B, and the dB and dC terms), so at least
# 12/128 + 1/32 = 1/8 CU-clock per update: 4.92e12 updates/s.
ALU_PEAK_BWD_UPD_S = CUS * CLOCK_HZ / (12.0 / 128 + 1.0 / 32)
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SRC = os.path.join(ROOT, "selective_state_space_41_amd", "csrc", "vmscan.hip")

METRIC = "scan tokens·channels/s (fwd, bidir) and achieved HBM GB/s vs peak, 1 GPU"


def algorithmic_bytes(cfg, v2=False):
    """Bytes the call must move at minimum: every input read once, the output written once."""
    c = cfg
    esz = 4 if c["dtype"] == "f32" else 2
    N = c["d_state"]
    if c["kind"] == "vim":
        nb, nd, L = c["batch"], c["dim"], c["seqlen"]
        act = (6 if v2 else 4) * nb * nd * L * esz   # u, delta_raw, z, out (+ u_b, delta_raw_b)
        bc = 4 * nb * N * L * esz                 # B, C, B_b, C_b
        par = 2 * nd * N * 4 + (4 if v2 else 3) * nd * 4   # A_log, A_b_log; D, D_b, bias (+ bias_b)
        return act + bc + par, nb * nd * L
    nb, nd, L = c["batch"], c["dim"], c["H"] * c["W"]
    act = 2 * nb * nd * L * esz                   # x, out
    dr = 4 * nb * nd * L * esz                    # delta_raw, four directions
    bc = 2 * 4 * nb * N * L * esz                 # B, C, four directions
    par = 4 * nd * N * 4 + 2 * 4 * nd * 4
    return act + dr + bc + par, nb * nd * L


def state_updates(cfg):
    """Recurrence state updates per call: tokens * channels * directions * d_state."""
    dirs = 2 if cfg["kind"] == "vim" else 4
    seq = cfg["seqlen"] if cfg["kind"] == "vim" else cfg["H"] * cfg["W"]
    return cfg["batch"] * cfg["dim"] * seq * dirs * cfg["d_state"]


def source_digest():
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def traffic_record(workload):
    """HBM traffic per launch from the committed rocprofv3 counter summary, if it was taken on
    the current kernel source; else None."""
    path = os.path.join(PROFILES, f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_sha256_16") != source_digest():
        return None
    return rec.get("traffic_bytes_per_launch")


def _db_rows(path, sql):
    import glob
    import sqlite3
    rows = []
    for f in sorted(glob.glob(os.path.join(path, "**", "*.db"), recursive=True)):
        con = sqlite3.connect(f)
        rows += con.execute(sql).fetchall()
        con.close()
    if not rows:
        raise SystemExit(f"no rocprofv3 results under {path}")
    return rows


def _counter_kib(path, counter, like):
    """Mean of a counter per dispatch (KiB for FETCH_SIZE/WRITE_SIZE) over the dispatches of the
    kernels whose name contains ``like``, from a rocprofv3 --pmc result database."""
    rows = _db_rows(path, "select kernel_name, counter_name, value from counters_collection")
    vals = [v for k, c, v in rows if c == counter and like in k]
    if not vals:
        raise SystemExit(f"{counter}: no dispatch of a kernel matching {like!r} under {path}")
    return sum(vals) / len(vals), len(vals)


def summarize_kernels(path, command, out_txt):
    """Per-kernel duration table (rocprofv3 --kernel-trace result database) written as text."""
    rows = _db_rows(path, "select name, count(*), avg(duration), min(duration), max(duration), sum(duration) "
                          "from kernels group by name")
    rows.sort(key=lambda r: -r[5])
    lines = [f"command: {command}", "", f"{'calls':>6} {'avg us':>10} {'min us':>10} {'max us':>10}  kernel"]
    for name, n, avg, mn, mx, _ in rows:
        lines.append(f"{n:6d} {avg / 1e3:10.2f} {mn / 1e3:10.2f} {mx / 1e3:10.2f}  {name[:140]}")
    with open(out_txt, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize_counters(out_txt, like, runs):
    """Mean per dispatch of every counter in rocprofv3 --pmc runs, for the kernel matching
    ``like``; ``runs`` is a list of (result_dir, command)."""
    lines = [f"kernel: dispatches whose name contains {like!r}; values are means per dispatch", ""]
    for path, command in runs:
        rows = _db_rows(path, "select kernel_name, counter_name, value from counters_collection")
        acc = {}
        for k, c, v in rows:
            if like in k:
                acc.setdefault(c, []).append(v)
        lines.append(f"command: {command}")
        for c in sorted(acc):
            lines.append(f"  {c:28s} {sum(acc[c]) / len(acc[c]):16.6g}   (n={len(acc[c])})")
        lines.append("")
    with open(out_txt, "w") as f:
        f.write("\n".join(lines))
    print("\n".join(lines))


def summarize_traffic(workload, like, dirs, commands):
    """HBM bytes per launch of the kernel matching ``like``: FETCH_SIZE and WRITE_SIZE (KiB per
    dispatch), each scaled by what the same counter reads for a plain 1 GiB device copy."""
    f_kib, nf = _counter_kib(dirs["fetch"], "FETCH_SIZE", like)
    w_kib, nw = _counter_kib(dirs["write"], "WRITE_SIZE", like)
    cf_kib, _ = _counter_kib(dirs["copy_fetch"], "FETCH_SIZE", "copy")
    cw_kib, _ = _counter_kib(dirs["copy_write"], "WRITE_SIZE", "copy")
    gib = float(1 << 30)
    rs, ws = gib / (cf_kib * 1024), gib / (cw_kib * 1024)
    rd, wr = f_kib * 1024 * rs, w_kib * 1024 * ws
    rec = {"workload": workload, "kernel_match": like, "source_sha256_16": source_digest(),
           "fetch_kib_per_dispatch": f_kib, "write_kib_per_dispatch": w_kib, "dispatches": [nf, nw],
           "copy_fetch_kib_per_GiB": cf_kib, "copy_write_kib_per_GiB": cw_kib,
           "read_scale": rs, "write_scale": ws, "read_bytes": rd, "write_bytes": wr,
           "traffic_bytes_per_launch": int(round(rd + wr)), "commands": commands}
    os.makedirs(PROFILES, exist_ok=True)
    with open(os.path.join(PROFILES, f"traffic_{workload}.json"), "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(rec, indent=1))


def _cpu_worker(args):
    cfg_id, bsel, min_s = args
    import oracle as O
    import synth
    p = synth.make_vim_inputs(cfg_id)
    sl = slice(bsel[0], bsel[1])
    reps, t0 = 0, time.perf_counter()
    while True:   # repeat the slice until this worker has computed for at least min_s seconds
        O.vim_bidir(p["u"][sl], p["delta_raw"][sl], p["z"][sl], p["A_log"], p["A_b_log"], p["B"][sl], p["C"][sl],
                    p["B_b"][sl], p["C_b"][sl], p["D"], p["D_b"], p["delta_bias"])
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= min_s:
            return reps, dt


def cpu_baseline(cfg_id, cfg, min_s=1.0):
    """The fp64 oracle on the same workload: the batches of the Vim-Ti scan are split into
    slices over a process pool (one process per host core, at most 16: the host share of a
    one-GPU machine, whatever os.cpu_count() reports; both counts are recorded) and each process repeats
    its slice for at least ``min_s`` seconds.  Throughput = tokens·channels computed / slowest
    worker's compute time (input generation excluded)."""
    import multiprocessing as mp
    host = os.cpu_count() or 1
    workers = max(1, min(16, host))  # a one-GPU machine's share of the host is 16 cores
    nb = cfg["batch"]
    per = math.ceil(nb / workers)
    slices = [(cfg_id, (i, min(nb, i + per)), min_s) for i in range(0, nb, per)]
    ctx = mp.get_context("spawn")
    with ctx.Pool(len(slices)) as pool:
        res = pool.map(_cpu_worker, slices)
    tpb = cfg["dim"] * cfg["seqlen"]
    work = sum(r * (b[1][1] - b[1][0]) * tpb for (r, _), b in zip(res, slices))
    wall = max(t for _, t in res)
    return {"value": work / wall, "unit": "tokens·channels/s", "cores": len(slices), "host_cores": host,
            "kind": "oracle",
            "sample": f"{cfg['name']}: batch slices of {per} (all {nb} batches), each repeated for >= {min_s:.0f} s "
                      f"in its own process (fp64 numpy oracle); {sum(t for _, t in res):.1f} CPU-s in total, "
                      f"slowest worker {wall:.2f} s"}


def cpu_sample(kind, cfg_id, cfg, min_s=3.0):
    """The fp64 oracle of one bench leg on a bounded sample of its workload: one batch, in this
    process (one core; the oracle is plain elementwise numpy), repeated for at least ``min_s``
    seconds.  ``kind``: "v2", "n32", "bwd", "front"."""
    import numpy as np
    import oracle as O
    import synth
    N = cfg["d_state"]
    if cfg["kind"] == "vim":
        p = synth.make_vim_v2_inputs(cfg_id, batch=1, d_state=N)
        toks = cfg["dim"] * cfg["seqlen"]
        v2args = lambda q: (q["u"], q["delta_raw"], q["delta_bias"], q["u_b"], q["delta_raw_b"], q["delta_bias_b"],
                            q["z"], q["A_log"], q["A_b_log"], q["B"], q["C"], q["B_b"], q["C_b"], q["D"], q["D_b"])
        if kind == "bwd":
            dout = np.random.default_rng(1).standard_normal(p["u"].shape)
            fn = lambda: O.vim_bidir_v2_bwd(*v2args(p), dout)
            what = "vim_bidir_v2_bwd (all 15 gradients)"
        elif kind == "front":
            c = synth.make_conv1d_inputs(cfg_id, batch=1)

            def fn():
                q = dict(p)
                q["u"] = O.conv1d_silu(c["x"], c["conv_w"], c["conv_b"])
                q["u_b"] = O.conv1d_silu(c["x"], c["conv_w_b"], c["conv_b_b"], reverse=True)
                return O.vim_bidir_v2(*v2args(q))
            what = "conv1d_silu (both branches) + vim_bidir_v2"
        elif kind == "v2":
            fn = lambda: O.vim_bidir_v2(*v2args(p))
            what = "vim_bidir_v2"
        else:
            fn = lambda: O.vim_bidir(p["u"], p["delta_raw"], p["z"], p["A_log"], p["A_b_log"], p["B"], p["C"],
                                     p["B_b"], p["C_b"], p["D"], p["D_b"], p["delta_bias"])
            what = f"vim_bidir (d_state {N})"
    else:
        p = synth.make_ss2d_inputs(cfg_id, batch=1, d_state=N)
        toks = cfg["dim"] * cfg["H"] * cfg["W"]
        args = (p["delta_raw"], p["A_log"], p["B"], p["C"], p["D"], p["delta_bias"])
        if kind == "bwd":
            dout = np.random.default_rng(1).standard_normal(p["x"].shape)
            fn = lambda: O.ss2d_cross_scan_bwd(p["x"], *args, None, dout)
            what = "ss2d_cross_scan_bwd (all gradients)"
        elif kind == "front":
            c = synth.make_conv2d_inputs(cfg_id, batch=1)
            fn = lambda: O.ss2d_cross_scan(O.conv2d_silu(c["x"], c["conv_w"], c["conv_b"]), *args)
            what = "conv2d_silu + ss2d_cross_scan"
        else:
            fn = lambda: O.ss2d_cross_scan(p["x"], *args)
            what = f"ss2d_cross_scan (d_state {N})"
    reps, t0 = 0, time.perf_counter()
    while True:
        fn()
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= min_s:
            break
    return {"value": reps * toks / dt, "unit": "tokens·channels/s", "cores": 1, "kind": "oracle",
            "sample": f"{cfg['name']}: batch 1 of {cfg['batch']}, {what}, repeated {reps}x in {dt:.1f} s on one "
                      f"core (fp64 numpy oracle)"}


VIM_ACT = ("u", "delta_raw", "z", "B", "C", "B_b", "C_b")
VIM_PAR = ("A_log", "A_b_log", "D", "D_b", "delta_bias")
V2_ACT = ("u_b", "delta_raw_b")
V2_PAR = ("delta_bias_b",)


def make_sets(cfg_id, cfg, nsets, torch, v2=False):
    """Set 0 comes from the seeded generator (the parity inputs); further rotation sets are drawn on
    the device from a seeded torch generator with the same distributions."""
    import numpy as np
    import synth
    dt = torch.bfloat16 if cfg["dtype"] == "bf16" else torch.float32
    dev = torch.device("cuda", 0)
    g = torch.Generator(device=dev)
    g.manual_seed(41_000 + cfg_id)
    sets = []
    if cfg["kind"] == "vim":
        mk = synth.make_vim_v2_inputs if v2 else synth.make_vim_inputs
        p = mk(cfg_id, d_state=cfg["d_state"])
        act_names = VIM_ACT + (V2_ACT if v2 else ())
        par = {k: torch.from_numpy(np.ascontiguousarray(p[k])).to(dev) for k in VIM_PAR + (V2_PAR if v2 else ())}
        base = {k: torch.from_numpy(np.ascontiguousarray(p[k])).to(dev).to(dt) for k in act_names}
        for s in range(nsets):
            if s == 0:
                act = base
            else:
                act = {k: torch.randn(v.shape, generator=g, device=dev, dtype=torch.float32).to(dt) for k, v in base.items()}
            act["out"] = torch.empty_like(act["u"])
            sets.append((act, par))
    else:
        p = synth.make_ss2d_inputs(cfg_id, d_state=cfg["d_state"])
        act_names = ("x", "delta_raw", "B", "C")
        par = {k: torch.from_numpy(np.ascontiguousarray(p[k])).to(dev) for k in ("A_log", "D", "delta_bias")}
        base = {k: torch.from_numpy(np.ascontiguousarray(p[k])).to(dev).to(dt) for k in act_names}
        for s in range(nsets):
            act = base if s == 0 else {k: torch.randn(v.shape, generator=g, device=dev, dtype=torch.float32).to(dt)
                                       for k, v in base.items()}
            act["out"] = torch.empty_like(act["x"])
            sets.append((act, par))
    return sets


def bench_config(cfg_id, steps, warmup, with_cpu, torch, V, v2=False, d_state=None, lane_scan=False):
    import synth
    cfg = with_d_state(cfg_id, d_state)
    v2 = v2 and cfg["kind"] == "vim"
    nbytes, toks = algorithmic_bytes(cfg, v2)
    layers = cfg.get("layers", 1)
    per_set = nbytes
    nsets = max(1, math.ceil((1 << 30) / per_set)) if layers == 1 else layers
    sets = []
    if cfg["kind"] == "vim" and layers > 1:
        # one set per layer, each with its own seed (all 24 layers run back to back on distinct buffers)
        import numpy as np
        dt = torch.bfloat16
        dev = torch.device("cuda", 0)
        for layer in range(layers):
            mk = synth.make_vim_v2_inputs if v2 else synth.make_vim_inputs
            p = mk(cfg_id, layer=layer, d_state=cfg["d_state"])
            act = {k: torch.from_numpy(np.ascontiguousarray(p[k])).to(dev).to(dt) for k in VIM_ACT + (V2_ACT if v2 else ())}
            act["out"] = torch.empty_like(act["u"])
            par = {k: torch.from_numpy(np.ascontiguousarray(p[k])).to(dev) for k in VIM_PAR + (V2_PAR if v2 else ())}
            sets.append((act, par))
    else:
        sets = make_sets(cfg_id, cfg, nsets, torch, v2)
    dev = torch.device("cuda", 0)
    ws = None
    lane_scan = lane_scan and cfg["kind"] == "vim"
    chunk_len = V.CHUNK_LANE_SCAN if lane_scan else 0
    if cfg["kind"] == "vim":
        wsb = V.lib.vmscan_fwd_bidir_workspace_bytes_ex(cfg["batch"], cfg["dim"], cfg["seqlen"], cfg["d_state"],
                                                        1 if cfg["dtype"] == "bf16" else 0, chunk_len)
    else:
        wsb = V.lib.ss2d_cross_scan_workspace_bytes(cfg["batch"], cfg["dim"], cfg["H"], cfg["W"], cfg["d_state"],
                                                    1 if cfg["dtype"] == "bf16" else 0)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev)

    def prepare(i, stage=3):
        """The call on rotation set i, validated and marshalled once (the timed loops then make only
        the C calls)."""
        act, par = sets[i]
        if v2:
            return V.vmscan_fwd_bidir_v2(act["u"], act["delta_raw"], par["delta_bias"], act["u_b"], act["delta_raw_b"],
                                         par["delta_bias_b"], act["z"], par["A_log"], par["A_b_log"], act["B"],
                                         act["C"], act["B_b"], act["C_b"], par["D"], par["D_b"], out=act["out"],
                                         workspace=ws, stage=stage, prepare=True, chunk_len=chunk_len)
        if cfg["kind"] == "vim":
            return V.vmscan_fwd_bidir(act["u"], act["delta_raw"], act["z"], par["A_log"], par["A_b_log"], act["B"],
                                      act["C"], act["B_b"], act["C_b"], par["D"], par["D_b"], par["delta_bias"],
                                      out=act["out"], workspace=ws, stage=stage, prepare=True, chunk_len=chunk_len)
        return V.ss2d_cross_scan_fwd(act["x"], act["delta_raw"], par["A_log"], act["B"], act["C"], par["D"],
                                     par["delta_bias"], out=act["out"], workspace=ws, prepare=True)

    full = [prepare(i) for i in range(len(sets))]
    for i in range(warmup):
        full[i % len(sets)]()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)   # the binding launches on this stream
    # The step: one whole call (all kernels of the path), back to back.
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    for i in range(steps):
        ev[i].record(stream)
        full[(warmup + i) % len(sets)]()
    ev[steps].record(stream)
    torch.cuda.synchronize()
    total_ms = ev[0].elapsed_time(ev[steps])
    step_ms = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(steps))
    # The dominant kernel on its own (Vim: the scan stage, timed between events after its
    # preparation stage); SS2D: the whole call.
    split = cfg["kind"] == "vim"
    if split:
        prep = [prepare(i, stage=1) for i in range(len(sets))]
        scan = [prepare(i, stage=2) for i in range(len(sets))]
        ek = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        torch.cuda.synchronize()
        for i in range(steps):
            j = (warmup + i) % len(sets)
            prep[j]()
            ek[i][0].record(stream)
            scan[j]()
            ek[i][1].record(stream)
        torch.cuda.synchronize()
        kern_ms = sum(a.elapsed_time(b) for a, b in ek) / steps
    else:
        kern_ms = total_ms / steps
    ms = total_ms / steps
    value = toks / (ms * 1e-3)
    gbs = nbytes / (ms * 1e-3) / 1e9
    upd = state_updates(cfg)
    alu = upd / (kern_ms * 1e-3)
    dtype = "f32"  # arithmetic and state are fp32; activations are stored as cfg["dtype"]
    is_default = cfg_id == 1 and cfg["d_state"] == synth.CONFIGS[cfg_id]["d_state"]
    roof = {"bound": "alu", "achieved": round(alu / 1e9, 1), "peak": round(ALU_PEAK_UPD_S / 1e9, 1), "unit": "Gupd/s",
            "frac": round(alu / ALU_PEAK_UPD_S, 4), "traffic": traffic_record(cfg["name"]),
            "kernel": ((("lane_scan_kernel<bf16> (vmscan_fwd_bidir" if lane_scan else "scan_pair_kernel<bf16, vim> (scan stage of vmscan_fwd_bidir") +
                        ("_v2)" if v2 else ")")) if split else
                       "all kernels of the call (transpose, chunk states, both SS2D pairs)"),
            "kernel_avg_us": round(kern_ms * 1000, 2),
            "updates_per_launch": upd,
            "call_frac": round(upd / (ms * 1e-3) / ALU_PEAK_UPD_S, 4),
            "hbm": {"achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                    "algorithmic_bytes_per_step": nbytes}}
    rec = {
        "metric": METRIC,
        "value": value,
        "unit": "tokens·channels/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic",
        "config": {"workload": cfg["name"] + ("_sepbwd" if v2 else "") + ("_lanescan" if lane_scan else ""),
                   "batch": cfg["batch"], "dim": cfg["dim"],
                   "seqlen": cfg.get("seqlen", cfg.get("H", 0) * cfg.get("W", 0)), "d_state": cfg["d_state"],
                   "io_dtype": cfg["dtype"], "rotation_sets": len(sets),
                   "step_ms_p10_p50_p90": [step_ms[len(step_ms) // 10], step_ms[len(step_ms) // 2],
                                           step_ms[(9 * len(step_ms)) // 10]]},
        "roofline": roof,
    }
    if v2:
        rec["config"]["backward_branch"] = "separate u_b, delta_raw_b, delta_bias_b"
    if cfg["kind"] == "ss2d":
        rec["config"]["H"] = cfg["H"]
        rec["config"]["W"] = cfg["W"]
    if with_cpu and is_default and not v2:
        rec["cpu_baseline"] = cpu_baseline(cfg_id, cfg)
    elif with_cpu and (v2 or cfg["d_state"] != synth.CONFIGS[cfg_id]["d_state"]):
        rec["cpu_baseline"] = cpu_sample("v2" if v2 else "n32", cfg_id, cfg)
    return rec


def with_d_state(cfg_id, d_state):
    """The workload's configuration, at another state size if ``d_state`` differs from its own."""
    import synth
    cfg = dict(synth.CONFIGS[cfg_id])
    if d_state and d_state != cfg["d_state"]:
        cfg["d_state"] = d_state
        cfg["name"] = cfg["name"] + f"_n{d_state}"
    return cfg


def bench_bwd(cfg_id, steps, warmup, torch, V, v2=False, with_cpu=False, d_state=None):
    """Backward pass (vmscan_bwd_bidir_v2, every gradient) of a Vim workload; with shared inputs
    (the forward of vmscan_fwd_bidir) unless ``v2``.  The timed region is the whole call."""
    import numpy as np
    import synth
    cfg = with_d_state(cfg_id, d_state)
    if cfg["kind"] != "vim":
        return bench_ss2d_bwd(cfg_id, steps, warmup, torch, V, with_cpu, d_state)
    dev = torch.device("cuda", 0)
    dt = torch.bfloat16 if cfg["dtype"] == "bf16" else torch.float32
    N = cfg["d_state"]
    p = synth.make_vim_v2_inputs(cfg_id, d_state=N)
    act = {k: torch.from_numpy(np.ascontiguousarray(p[k])).to(dev).to(dt) for k in VIM_ACT + V2_ACT}
    par = {k: torch.from_numpy(np.ascontiguousarray(p[k])).to(dev) for k in VIM_PAR + V2_PAR}
    if not v2:
        act["u_b"], act["delta_raw_b"], par["delta_bias_b"] = act["u"], act["delta_raw"], par["delta_bias"]
    g = torch.Generator(device=dev)
    g.manual_seed(42_000 + cfg_id)
    dout = torch.randn(act["u"].shape, generator=g, device=dev, dtype=torch.float32).to(dt)
    nb, nd, L = act["u"].shape
    wsb = V.lib.vmscan_bwd_bidir_v2_workspace_bytes(nb, nd, L, N, 1 if cfg["dtype"] == "bf16" else 0)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev)

    # validated once; each call rewrites the same gradient tensors
    call, outs = V.vmscan_bwd_bidir_v2(act["u"], act["delta_raw"], par["delta_bias"], act["u_b"], act["delta_raw_b"],
                                       par["delta_bias_b"], act["z"], par["A_log"], par["A_b_log"], act["B"], act["C"],
                                       act["B_b"], act["C_b"], par["D"], par["D_b"], dout, shared=not v2, workspace=ws,
                                       prepare=True)
    for _ in range(warmup):
        call()
    stream = torch.cuda.current_stream(dev)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    upd = state_updates(cfg)
    alu = upd / (ms * 1e-3)
    toks = nb * nd * L
    del outs
    rec = {
        "metric": "scan tokens·channels/s (bwd: all gradients of the bidirectional scan), 1 GPU",
        "value": toks / (ms * 1e-3), "unit": "tokens·channels/s", "n_gpus": 1, "steps": steps, "warmup": warmup,
        "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": cfg["name"] + ("_sepbwd" if v2 else "") + "_backward", "batch": nb, "dim": nd,
                   "seqlen": L, "d_state": N, "io_dtype": cfg["dtype"], "branches": "separate" if v2 else "shared"},
        "roofline": {"bound": "alu", "achieved": round(alu / 1e9, 1), "peak": round(ALU_PEAK_BWD_UPD_S / 1e9, 1),
                     "unit": "Gupd/s", "frac": round(alu / ALU_PEAK_BWD_UPD_S, 4), "traffic": None,
                     "kernel": "all kernels of vmscan_bwd_bidir_v2 (forward with saved sum, gate, adjoint scan, "
                               "reductions)", "kernel_avg_us": round(ms * 1000, 2), "updates_per_launch": upd},
    }
    if with_cpu:
        rec["cpu_baseline"] = cpu_sample("bwd", cfg_id, cfg)
    return rec


def front_bytes(cfg):
    """Algorithmic bytes of the front convolution: x read once, its outputs written once (u and
    u_b for Vim; the row-major and transposed copies for SS2D); weights are negligible."""
    esz = 4 if cfg["dtype"] == "f32" else 2
    n = cfg["batch"] * cfg["dim"] * (cfg["seqlen"] if cfg["kind"] == "vim" else cfg["H"] * cfg["W"])
    return 3 * n * esz


def bench_front(cfg_id, steps, warmup, torch, V, with_cpu=False):
    """Front convolution + scan as one step: Vim: conv1d + SiLU for both branches
    (vmscan_conv1d_silu_fwd) then the scan with a separate backward branch; SS2D: the 3 x 3
    conv2d + SiLU writing both layouts (ss2d_conv2d_silu_fwd) then the cross-scan reading the
    transposed copy (ss2d_cross_scan_fwd_xt).  Input sets are drawn on the device and rotated
    so that at least 1 GiB is touched between reuses."""
    import numpy as np
    import synth
    cfg = synth.CONFIGS[cfg_id]
    dev = torch.device("cuda", 0)
    dt = torch.bfloat16 if cfg["dtype"] == "bf16" else torch.float32
    g = torch.Generator(device=dev)
    g.manual_seed(44_000 + cfg_id)
    rnd = lambda shape: torch.randn(shape, generator=g, device=dev, dtype=torch.float32).to(dt)
    vim = cfg["kind"] == "vim"
    if vim:
        c = synth.make_conv1d_inputs(cfg_id)
        p = synth.make_vim_v2_inputs(cfg_id, batch=1)  # parameters only
        nb, nd, L = cfg["batch"], cfg["dim"], cfg["seqlen"]
        N = cfg["d_state"]
        act_shapes = {k: (nb, nd, L) for k in ("x", "delta_raw", "delta_raw_b", "z")}
        act_shapes.update({k: (nb, N, L) for k in ("B", "C", "B_b", "C_b")})
        par = {k: torch.from_numpy(np.ascontiguousarray(p[k])).to(dev) for k in VIM_PAR + V2_PAR}
        wsb = V.lib.vmscan_fwd_bidir_workspace_bytes(nb, nd, L, N, 1 if dt == torch.bfloat16 else 0)
        toks = nb * nd * L
    else:
        c = synth.make_conv2d_inputs(cfg_id)
        p = synth.make_ss2d_inputs(cfg_id, batch=1)
        nb, nd, H, W = cfg["batch"], cfg["dim"], cfg["H"], cfg["W"]
        L, N = H * W, cfg["d_state"]
        act_shapes = {"x": (nb, nd, H, W), "delta_raw": (nb, 4, nd, L), "B": (nb, 4, N, L), "C": (nb, 4, N, L)}
        par = {k: torch.from_numpy(np.ascontiguousarray(p[k])).to(dev) for k in ("A_log", "D", "delta_bias")}
        wsb = V.lib.ss2d_cross_scan_workspace_bytes(nb, nd, H, W, N, 1 if dt == torch.bfloat16 else 0)
        toks = nb * nd * L
    wts = {k: torch.from_numpy(np.ascontiguousarray(v)).to(dev) for k, v in c.items() if k.startswith("conv_")}
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev)
    esz = 2 if dt == torch.bfloat16 else 4
    per_set = sum(int(np.prod(s)) for s in act_shapes.values()) * esz + 3 * toks * esz
    nsets = max(1, math.ceil((1 << 30) / per_set))
    sets = []
    for _ in range(nsets):
        a = {k: rnd(s) for k, s in act_shapes.items()}
        a["u"], a["u_b"] = torch.empty_like(a["x"]), torch.empty_like(a["x"])
        if not vim:
            a["xT"] = torch.empty((nb, nd, W, H), dtype=dt, device=dev)
        a["out"] = torch.empty_like(a["x"])
        sets.append(a)

    def front(a):
        if vim:
            V.conv1d_silu_fwd(a["x"], wts["conv_w"], wts["conv_b"], wts["conv_w_b"], wts["conv_b_b"], u=a["u"],
                              u_b=a["u_b"])
        else:
            V.ss2d_conv2d_silu_fwd(a["x"], wts["conv_w"], wts["conv_b"], x_out=a["u"], xT_out=a["xT"])

    scans = []
    for a in sets:
        if vim:
            scans.append(V.vmscan_fwd_bidir_v2(a["u"], a["delta_raw"], par["delta_bias"], a["u_b"], a["delta_raw_b"],
                                               par["delta_bias_b"], a["z"], par["A_log"], par["A_b_log"], a["B"],
                                               a["C"], a["B_b"], a["C_b"], par["D"], par["D_b"], out=a["out"],
                                               workspace=ws, prepare=True))
        else:
            scans.append(V.ss2d_cross_scan_fwd(a["u"], a["delta_raw"], par["A_log"], a["B"], a["C"], par["D"],
                                               par["delta_bias"], out=a["out"], workspace=ws, xT=a["xT"],
                                               prepare=True))

    for i in range(warmup):
        front(sets[i % nsets])
        scans[i % nsets]()
    stream = torch.cuda.current_stream(dev)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        k = (warmup + i) % nsets
        ev[i][0].record(stream)
        front(sets[k])
        ev[i][1].record(stream)
        scans[k]()
        ev[i][2].record(stream)
    torch.cuda.synchronize()
    ms = ev[0][0].elapsed_time(ev[-1][2]) / steps
    front_ms = sum(e[0].elapsed_time(e[1]) for e in ev) / steps
    scan_ms = sum(e[1].elapsed_time(e[2]) for e in ev) / steps
    fb = front_bytes(cfg)
    gbs = fb / (front_ms * 1e-3) / 1e9
    upd = state_updates(cfg)
    alu = upd / (scan_ms * 1e-3)
    rec = {
        "metric": METRIC + " (front convolution + scan)",
        "value": toks / (ms * 1e-3), "unit": "tokens·channels/s", "n_gpus": 1, "steps": steps, "warmup": warmup,
        "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": cfg["name"] + "_front", "batch": nb, "dim": nd, "seqlen": L, "d_state": N,
                   "io_dtype": cfg["dtype"], "rotation_sets": nsets,
                   "front": "conv1d d_conv 4 + SiLU, both branches" if vim else "conv2d 3x3 + SiLU, row-major and transposed"},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "conv1d_flat_kernel" if vim else "conv2d_front_kernel",
                     "kernel_avg_us": round(front_ms * 1000, 2), "algorithmic_bytes_per_launch": fb,
                     "scan": {"bound": "alu", "achieved": round(alu / 1e9, 1), "peak": round(ALU_PEAK_UPD_S / 1e9, 1),
                              "unit": "Gupd/s", "frac": round(alu / ALU_PEAK_UPD_S, 4),
                              "avg_us": round(scan_ms * 1000, 2)}},
    }
    if with_cpu:
        rec["cpu_baseline"] = cpu_sample("front", cfg_id, cfg)
    return rec


def bench_ss2d_bwd(cfg_id, steps, warmup, torch, V, with_cpu=False, d_state=None):
    """Backward pass of the SS2D cross-scan (ss2d_cross_scan_bwd, every gradient, no gate as in
    the 56x56 workload); the timed region is the whole call."""
    import numpy as np
    import synth
    cfg = with_d_state(cfg_id, d_state)
    dev = torch.device("cuda", 0)
    dt = torch.bfloat16 if cfg["dtype"] == "bf16" else torch.float32
    N = cfg["d_state"]
    p = synth.make_ss2d_inputs(cfg_id, d_state=N)
    act = {k: torch.from_numpy(np.ascontiguousarray(p[k])).to(dev).to(dt) for k in ("x", "delta_raw", "B", "C")}
    par = {k: torch.from_numpy(np.ascontiguousarray(p[k])).to(dev) for k in ("A_log", "D", "delta_bias")}
    g = torch.Generator(device=dev)
    g.manual_seed(43_000 + cfg_id)
    dout = torch.randn(act["x"].shape, generator=g, device=dev, dtype=torch.float32).to(dt)
    nb, nd, H, W = act["x"].shape
    wsb = V.lib.ss2d_cross_scan_bwd_workspace_bytes(nb, nd, H, W, N, 1 if cfg["dtype"] == "bf16" else 0)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev)

    call, outs = V.ss2d_cross_scan_bwd(act["x"], act["delta_raw"], par["A_log"], act["B"], act["C"], par["D"],
                                       par["delta_bias"], None, dout, workspace=ws, prepare=True)
    for _ in range(max(1, warmup)):
        call()
    stream = torch.cuda.current_stream(dev)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    upd = state_updates(cfg)
    alu = upd / (ms * 1e-3)
    toks = nb * nd * H * W
    rec = {
        "metric": "scan tokens·channels/s (bwd: all gradients of the SS2D cross-scan), 1 GPU",
        "value": toks / (ms * 1e-3), "unit": "tokens·channels/s", "n_gpus": 1, "steps": steps, "warmup": warmup,
        "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": cfg["name"] + "_backward", "batch": nb, "dim": nd, "H": H, "W": W, "d_state": N,
                   "io_dtype": cfg["dtype"]},
        "roofline": {"bound": "alu", "achieved": round(alu / 1e9, 1), "peak": round(ALU_PEAK_BWD_UPD_S / 1e9, 1),
                     "unit": "Gupd/s", "frac": round(alu / ALU_PEAK_BWD_UPD_S, 4), "traffic": None,
                     "kernel": "all kernels of ss2d_cross_scan_bwd (transposes, two pairs of adjoint scans, reductions)",
                     "kernel_avg_us": round(ms * 1000, 2), "updates_per_launch": upd},
    }
    if with_cpu:
        rec["cpu_baseline"] = cpu_sample("bwd", cfg_id, cfg)
    return rec


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=1)
    ap.add_argument("--all", action="store_true", help="one line per workload (configs 0-4)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--v2", action="store_true", help="Vim workloads with a separate backward branch (u_b, delta_raw_b, bias_b)")
    ap.add_argument("--bwd", action="store_true", help="time the backward pass (every gradient) of the workloads")
    ap.add_argument("--front", action="store_true",
                    help="time the front convolution (conv1d / conv2d + SiLU) followed by the scan")
    ap.add_argument("--lane-scan", action="store_true",
                    help="Vim workloads through the lane-scan path (associative scan over positions, no chunk pass)")
    ap.add_argument("--d-state", type=int, default=None, choices=(16, 32),
                    help="state size of the workloads, forward or backward (default: the workload's own, 16)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run only a plain 1 GiB device-to-device copy (counter calibration for FETCH_SIZE/WRITE_SIZE)")
    ap.add_argument("--summarize-kernels", nargs=3, metavar=("RESULT_DIR", "COMMAND", "OUT_TXT"),
                    help="write the per-kernel table of a rocprofv3 --kernel-trace run (no GPU needed)")
    ap.add_argument("--summarize-traffic", nargs=7,
                    metavar=("WORKLOAD", "KERNEL_MATCH", "FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR", "COPY_WRITE_DIR",
                             "COMMANDS_JSON"),
                    help="write profiles/traffic_<workload>.json from four rocprofv3 --pmc runs (no GPU needed)")
    ap.add_argument("--summarize-counters", nargs="+", metavar="ARG",
                    help="OUT_TXT KERNEL_MATCH then pairs RESULT_DIR COMMAND of rocprofv3 --pmc runs (no GPU needed)")
    args = ap.parse_args()
    if args.summarize_counters:
        a = args.summarize_counters
        summarize_counters(a[0], a[1], list(zip(a[2::2], a[3::2])))
        return
    if args.summarize_kernels:
        summarize_kernels(*args.summarize_kernels)
        return
    if args.summarize_traffic:
        w, like, fd, wd, cfd, cwd, cmds = args.summarize_traffic
        summarize_traffic(w, like, {"fetch": fd, "write": wd, "copy_fetch": cfd, "copy_write": cwd}, json.loads(cmds))
        return
    if args.gpus != 1:
        print(f"bench.py: runs on one GPU only (got --gpus {args.gpus}); multi-GPU sharding over batch and "
              "channels is not implemented.", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    if args.calibrate_copy:
        # A plain copy of a known size: its FETCH_SIZE/WRITE_SIZE per dispatch give the scale that
        # turns the same counters of the scan kernels into bytes.
        n = (1 << 30) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(max(1, args.steps)):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "copy", "bytes_read_per_dispatch": n * 4, "bytes_written_per_dispatch": n * 4,
                          "dispatches": max(1, args.steps)}), flush=True)
        return
    import selective_state_space_41_amd as V
    cfgs = [0, 1, 2, 3, 4] if args.all else [args.config]
    for c in cfgs:
        if args.front:
            rec = bench_front(c, args.steps, args.warmup, torch, V, not args.no_cpu)
        elif args.bwd:
            rec = bench_bwd(c, args.steps, args.warmup, torch, V, args.v2, not args.no_cpu, args.d_state)
            if rec is None:
                continue
        else:
            rec = bench_config(c, args.steps, args.warmup, not args.no_cpu, torch, V, args.v2, args.d_state,
                               args.lane_scan)
        print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
