"""Benchmark of the local MoE FFN forward on one MI355X.

One step = one moe_forward call through the C ABI (route -> dispatch maps
-> gate/up GEMM with fused SiLU*up -> down GEMM -> combine) on the current
stream over one batch of synthetic input, inputs resident in HBM. Default
workload: the Mixtral-shaped bf16 batch (T=4096, H=4096, I=14336, E=8,
top_k=2, renormalize). Prints one JSON line.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
                    [--router grouped | --special | --train | --quant 8|4] [--no-graph]

moe_forward (or, for the epilogue, grouped-router and special-experts lines,
the same steps as separate calls) records HIP events on its stream at the
stage boundaries of every timed step; the gate/up stage (the dominant
kernel, plus its tile plan) gives the roofline figure. The CPU baseline
times the oracle on the first tokens of the same workload. The forward lines
also time the step replayed from a HIP graph (`graph_replay`).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE fwd tokens/s; expert GEMM TFLOP/s (% MFMA peak); combine GB/s (% HBM)"
# Grouped-limited sigmoid router of --router grouped (the DeepSeek-V3 family's settings).
GROUPED = {"groups": 8, "selected_groups": 4, "group_top_two": True, "scale": 2.5}
PEAK_TFLOPS = {"bf16": 2500.0, "f16": 2500.0, "f32": 157.3}
PEAK_HBM_GBS = 8000.0
# Which roof bounds the gate/up GEMM of each workload (flops per weight byte:
# ~2*rows-per-expert; the MI355X ridge is ~310 bf16 FLOP per HBM byte).
# Tokens of each workload the CPU oracle runs on (its cost is dominated by
# decoding the touched experts' weights to fp64 and the fp64 GEMMs).
CPU_TOKENS = {"tiny_fp32": 64, "mixtral_8x_bf16": 4096, "many_expert_zipf_bf16": 1024,
              "dsv3_share_rmsnorm_bf16": 8, "decode_nan_rows_bf16": 16}
BOUND = {"tiny_fp32": "alu", "mixtral_8x_bf16": "mfma", "many_expert_zipf_bf16": "mfma",
         "dsv3_share_rmsnorm_bf16": "hbm", "decode_nan_rows_bf16": "hbm"}


FORWARD_SOURCES = ("combine.hip", "common.h", "gemm.hip", "schedule.h")


def kernel_source_hash(sources=FORWARD_SOURCES) -> str:
    """sha256/16 over the sources the profiled kernels are compiled from (for
    the forward lines the GEMM and combine kernels and their device helpers):
    counters taken on other sources no longer describe the kernels."""
    import hashlib
    d = os.path.join(ROOT, "mixture_experts_ffn_top_amd", "csrc")
    h = hashlib.sha256()
    for n in sources:
        h.update(n.encode())
        h.update(open(os.path.join(d, n), "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, kernel: str):
    """HBM bytes per launch of `kernel` (for the quantised and training lines:
    per step of the launches their roofline covers) from the committed
    rocprofv3 FETCH_SIZE / WRITE_SIZE runs (profiles/counters.json, scaled by
    the copy-kernel calibration), or None when the kernel sources changed
    after they were taken."""
    try:
        data = json.load(open(os.path.join(ROOT, "profiles", "counters.json")))[workload]
    except (OSError, KeyError, ValueError):
        return None
    if kernel_source_hash(tuple(data.get("sources", FORWARD_SOURCES))) != data.get("kernel_source_sha16"):
        return None
    return data["traffic_bytes_per_launch"].get(kernel)


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="mixtral_8x_bf16")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=0,
                    help="tokens of the workload the CPU oracle runs on (default: a per-workload "
                         "sample of roughly 5-30 s)")
    ap.add_argument("--train", action="store_true",
                    help="time one first-order training step (forward with the experts' cache, "
                         "then combine, expert, dispatch and router backward) instead of the forward")
    ap.add_argument("--quant", type=int, default=0, choices=(0, 4, 8),
                    help="time the forward with weight-only INT8 or INT4 experts (decode-sized workloads)")
    ap.add_argument("--groups", type=int, default=0,
                    help="scale groups along K for --quant (default 1 for INT8, 4 for INT4)")
    ap.add_argument("--router", choices=("softmax", "grouped"), default="softmax",
                    help="grouped: the grouped-limited sigmoid router (8 groups, 4 kept, top-two "
                         "group scores, a correction bias, scale 2.5) in place of the softmax top-k")
    ap.add_argument("--special", action="store_true",
                    help="E/32 zero, E/32 copy and E/32 constant experts after the E experts and a "
                         "per-token activity mask (7/8 of the tokens active) in the combine")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the extra timing of the same step replayed from a HIP graph")
    ap.add_argument("--no-targets", action="store_true",
                    help="default line only: skip the two HBM measurements reported beside it (the "
                         "decode weight stream and the DeepSeek-V3-shaped combine + Add + RMSNorm)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES",
                    help="only run a plain device-to-device copy of BYTES bytes 5 times (the "
                         "reference kernel for scaling HBM byte counters), then exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the path has no "
              "multi-GPU mode", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.calibrate_copy:
        a = torch.ones(args.calibrate_copy, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "copy", "bytes_read": args.calibrate_copy,
                          "bytes_written": args.calibrate_copy, "launches": 5}), flush=True)
        return

    from mixture_experts_ffn_top_amd import inputs as I
    from mixture_experts_ffn_top_amd import moe

    w = I.workload(args.workload)
    T, H, I_, E, k = w.T, w.H, w.I, w.E, w.top_k
    R = T * k
    td = {"bf16": torch.bfloat16, "f32": torch.float32}[w.dtype]
    if args.workload not in BOUND:
        raise SystemExit(f"unknown workload {args.workload}")
    dev = "cuda"
    torch.cuda.set_device(0)
    moe.lib()

    def to_dev(a, dtype=w.dtype):
        if dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)

    # ---- inputs (host generation, then resident in HBM) --------------------
    t0 = time.time()
    grouped = args.router == "grouped"
    if (grouped or args.special) and (args.quant or args.train):
        raise SystemExit("--router grouped and --special time the forward; not with --quant / --train")
    if grouped and args.special:
        raise SystemExit("--router grouped and --special are separate lines")
    if grouped and (E % GROUPED["groups"] or E // GROUPED["groups"] < 2
                    or k > GROUPED["selected_groups"] * (E // GROUPED["groups"])):
        raise SystemExit("--router grouped needs E divisible by 8 with at least two experts a group "
                         "(top-two group scores) and top_k within the kept groups")
    x = I.tokens_for(w)
    bias = I.router_bias(w) if grouped else None
    n_sp = max(1, E // 32)
    if args.special:
        z, sp_a1, sp_a2, sp_v, sp_active = I.special_expert_inputs(w, n_sp, n_sp, n_sp)
    else:
        z = I.logits_for(w)
    if args.quant:
        return run_quant(args, w, x, z, to_dev)
    n_cpu = min(args.cpu_tokens or CPU_TOKENS[args.workload], T)
    keep = set()
    if not args.no_cpu_baseline:
        from oracle import moe_oracle as O
        if grouped:
            idx_s, _ = O.route_sigmoid_grouped(z[:n_cpu], "f32", bias, k, GROUPED["groups"],
                                               GROUPED["selected_groups"], True, w.renormalize,
                                               GROUPED["scale"])
        else:
            idx_s, _ = O.route(z[:n_cpu], "f32", k, w.renormalize)
        keep = set(int(e) for e in idx_s.ravel() if int(e) < E)
    wt = {}
    kept = {e: {} for e in keep}
    for name in ("w_gate", "w_up", "w_down"):
        shape = (E, I_, H) if name != "w_down" else (E, H, I_)
        t = torch.empty(shape, dtype=td, device=dev)
        for e0 in range(0, E, 16):
            ex = list(range(e0, min(E, e0 + 16)))
            a = I.expert_weights(w, name, ex)
            t[ex[0]:ex[-1] + 1].copy_(torch.from_numpy(a.view(np.int16) if w.dtype == "bf16" else a).view(td))
            for i, e in enumerate(ex):
                if e in kept:
                    kept[e][name] = a[i].copy()
            del a
        wt[name] = t
    xd, zd = to_dev(x), to_dev(z, "f32")
    torch.cuda.synchronize()
    log(f"inputs ready in {time.time() - t0:.1f}s: {args.workload} T={T} H={H} I={I_} E={E} k={k}")

    if args.train:
        return run_train(args, w, x, z, xd, zd, wt, kept, n_cpu)

    # ---- buffers ----------------------------------------------------------
    idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    wts = torch.empty((T, k), dtype=torch.float32, device=dev)
    out = torch.empty((T, H), dtype=td, device=dev)
    ws = torch.empty(moe.moe_forward_workspace_size(T, H, I_, E, k, td, torch.float32),
                     dtype=torch.uint8, device=dev)

    stages = ["route", "dispatch", "gate_up", "down", "combine"]
    if w.epilogue or grouped or args.special:
        # the split calls, with events recorded between them on this stream:
        # the combine fused with the shared-expert term, residual Add and
        # RMSNorm (epilogue workloads), the grouped router, special experts
        offsets_d = torch.empty(E + 1, dtype=torch.int32, device=dev)
        sor = torch.empty(R, dtype=torch.int32, device=dev)
        ros = torch.empty(R, dtype=torch.int32, device=dev)
        h = torch.empty((R, I_), dtype=td, device=dev)
        y = torch.empty((R, H), dtype=td, device=dev)
        ws_d = torch.empty(moe.moe_dispatch_workspace_size(T, k, E), dtype=torch.uint8, device=dev)
        ws_g = torch.empty(moe.moe_experts_gemm_workspace_size(R, E, H, I_, td), dtype=torch.uint8,
                           device=dev)
        if w.epilogue:
            sh, res, gam = I.epilogue_inputs(w)
            shd, resd, gamd = to_dev(sh), to_dev(res), to_dev(gam, "f32")
            yo = torch.empty((T, H), dtype=td, device=dev)
            rstd = torch.empty(T, dtype=torch.float32, device=dev)
            stages[-1] = "combine_add_rmsnorm"
        if args.special:
            a1d, a2d, vd = to_dev(sp_a1), to_dev(sp_a2), to_dev(sp_v)
            actd = torch.from_numpy(sp_active).to(dev)
            stages[-1] = "combine_special" + ("_add_rmsnorm" if w.epilogue else "")
        bd = to_dev(bias, "f32") if grouped else None

        def step(ev=None):
            def mark(i):
                if ev is not None:
                    ev[i].record()
            mark(0)
            if grouped:
                moe.moe_route_sigmoid_grouped(zd, k, GROUPED["groups"], GROUPED["selected_groups"],
                                              GROUPED["group_top_two"], w.renormalize,
                                              GROUPED["scale"], bias=bd, indices=idx, weights=wts)
            else:
                moe.moe_route(zd, k, w.renormalize, indices=idx, weights=wts)
            mark(1)
            if args.special:
                moe.moe_dispatch_masked(idx, E, active=actd, ws=ws_d, offsets=offsets_d,
                                        slot_of_row=sor, row_of_slot=ros)
            else:
                moe.moe_dispatch(idx, E, ws=ws_d, offsets=offsets_d, slot_of_row=sor, row_of_slot=ros)
            mark(2)
            moe.moe_experts_gate_up(xd, offsets_d, wt["w_gate"], wt["w_up"], row_map=sor, map_div=k,
                                    rows=R, h=h, ws=ws_g)
            mark(3)
            moe.moe_experts_down(h, offsets_d, wt["w_down"], expert_out=y, ws=ws_g)
            mark(4)
            if args.special:
                moe.moe_combine_special(y, ros, idx, wts, E, n_sp, n_sp, n_sp, ori_x=xd,
                                        const_alpha1=a1d, const_alpha2=a2d, const_v=vd, active=actd,
                                        shared=shd if w.epilogue else None,
                                        out=yo if w.epilogue else out,
                                        residual=resd if w.epilogue else None,
                                        gamma=gamd if w.epilogue else None, eps=w.eps,
                                        x_out=out if w.epilogue else None,
                                        rstd=rstd if w.epilogue else None)
            elif w.epilogue:
                moe.moe_combine_add_rmsnorm(y, ros, wts, resd, gamd, w.eps, shared=shd, y=yo,
                                            x_out=out, rstd=rstd)
            else:
                moe.moe_combine(y, ros, wts, out=out)
            mark(5)
    else:
        def step(ev=None):
            moe.moe_forward(xd, zd, k, w.renormalize, wt["w_gate"], wt["w_up"], wt["w_down"],
                            out=out, indices_out=idx, weights_out=wts, ws=ws, stage_events=ev)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"warmup done ({args.warmup} steps)")

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(args.steps)]
    for ev in evs:  # create the events before the timed region
        for e_ in ev:
            e_.record()
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for s in range(args.steps):
        step(evs[s])
    torch.cuda.synchronize()
    t_end = time.perf_counter()
    elapsed = t_end - t_start
    log(f"timed {args.steps} steps in {elapsed:.3f}s")
    if w.epilogue or grouped or args.special:
        offsets = offsets_d.cpu()
    else:
        offsets = torch.from_numpy(np.concatenate([[0], np.cumsum(np.bincount(idx.cpu().numpy().ravel(),
                                                                                minlength=E))])).int()
    R_disp = int(offsets[E])  # dispatched rows (fewer than T*k with special experts or the mask)

    stage_ms = {name: float(np.mean([evs[s][i].elapsed_time(evs[s][i + 1]) for s in range(args.steps)]))
                for i, name in enumerate(stages)}
    ms_step = elapsed / args.steps * 1e3
    tokens_per_s = T * args.steps / elapsed

    # ---- roofline of the dominant kernel (gate/up grouped GEMM) -----------
    es = 2 if w.dtype == "bf16" else 4
    counts = np.diff(offsets.cpu().numpy())
    touched = int((counts > 0).sum())
    flops_gate_up = 4.0 * R_disp * H * I_  # two [R,H]x[H,I] products per launch
    flops_down = 2.0 * R_disp * H * I_
    # bytes a launch must move at least: touched experts' weights, its input
    # rows and its output rows
    bytes_gate_up = touched * 2 * I_ * H * es + T * H * es + R_disp * I_ * es
    bytes_down = touched * H * I_ * es + R_disp * I_ * es + R_disp * H * es
    gu_s = stage_ms["gate_up"] / 1e3
    bound = BOUND[args.workload]
    if bound == "hbm":
        achieved, peak, unit = bytes_gate_up / gu_s / 1e9, PEAK_HBM_GBS, "GB/s"
    else:
        achieved, peak, unit = flops_gate_up / gu_s / 1e12, PEAK_TFLOPS[w.dtype], "TFLOP/s"
    if w.dtype == "f32":
        kname = "simt_gemm_kernel<gate_up>"
    elif R <= 4 * E:  # the library's weight-streaming path for decode-sized batches
        kname = "skinny_gate_up_kernel<bf16>"
    else:
        kname = "mfma_gemm_kernel<bf16,gate_up>"
    roofline = {"bound": bound, "achieved": round(achieved, 1), "peak": peak, "unit": unit,
                "frac": round(achieved / peak, 4),
                "traffic": measured_traffic(args.workload, kname),
                "kernel": kname, "covers": "the gate/up launch (both GEMMs: expert_gemm_frac_peak)",
                "algorithmic_per_launch": flops_gate_up if bound != "hbm" else bytes_gate_up}
    gemm_s = (stage_ms["gate_up"] + stage_ms["down"]) / 1e3
    expert_tflops = (flops_gate_up + flops_down) / gemm_s / 1e12
    if args.special:
        # dispatched expert rows; the token row once for each token with a
        # copy or constant slot; the constant experts' rows; ids, weights,
        # maps and the mask; then as below
        ids = idx.cpu().numpy().astype(np.int64)
        on = sp_active.astype(bool)[:, None]
        cc = ((ids >= E + n_sp) & (ids < E + 3 * n_sp) & on).any(axis=1).sum()
        comb_bytes = R_disp * H * es + int(cc) * H * es + n_sp * H * es + R * 12 + T
        comb_bytes += (4 * T * H * es + 4 * H + 4 * T) if w.epilogue else T * H * es
    elif w.epilogue:  # expert rows, weights, maps, shared, residual, gamma in; y, x_out, rstd out
        comb_bytes = R * H * es + R * 4 + R * 4 + 4 * T * H * es + 4 * H + 4 * T
    else:
        comb_bytes = R * H * es + R * 4 + R * 4 + T * H * es
    comb_gbs = comb_bytes / (stage_ms[stages[-1]] / 1e3) / 1e9
    extra = {
        "stages_ms": {k_: round(v, 4) for k_, v in stage_ms.items()},
        "expert_gemm_tflops": round(expert_tflops, 1),
        "expert_gemm_frac_peak": round(expert_tflops / PEAK_TFLOPS[w.dtype], 4),
        "expert_gemm_weight_gbs": round((bytes_gate_up + bytes_down) / gemm_s / 1e9, 1),
        "combine_gbs": round(comb_gbs, 1),
        "combine_frac_hbm": round(comb_gbs / PEAK_HBM_GBS, 4),
        "experts_touched": touched,
    }
    if grouped:  # the grouped router's own kernel: logits, bias in; ids, weights out
        route_bytes = 4 * T * E + 4 * E + 8 * T * k
        extra["route_gbs"] = round(route_bytes / (stage_ms["route"] / 1e3) / 1e9, 1)
    if args.special:
        extra["rows_dispatched"] = R_disp

    if args.workload == "mixtral_8x_bf16" and not (grouped or args.special or args.no_targets):
        extra.update(measure_targets(args, torch, moe, I))

    # ---- CPU baseline: the oracle on the first tokens of the workload -----
    cpu = None
    if not args.no_cpu_baseline:
        from oracle import moe_oracle as O
        cores = len(os.sched_getaffinity(0))
        wo = lambda e: (kept[e]["w_gate"], kept[e]["w_up"], kept[e]["w_down"])  # noqa: E731
        log(f"cpu baseline: oracle on {n_cpu} tokens")
        c0 = time.perf_counter()
        xs, zs = x[:n_cpu], z[:n_cpu]
        if grouped:
            O.forward_sigmoid_grouped(xs, zs, "f32", bias, k, GROUPED["groups"],
                                      GROUPED["selected_groups"], GROUPED["group_top_two"],
                                      w.renormalize, GROUPED["scale"], wo, E, w.dtype)
            what = "grouped sigmoid route, dispatch, fp64 SwiGLU experts, combine"
        elif args.special:
            ids_s, wts_s = O.route(zs, "f32", k, w.renormalize)
            act_s = sp_active[:n_cpu]
            d_s = O.dispatch(ids_s, E, xs, active=act_s)
            y_s = O.experts_forward_dispatched(d_s["x_disp"], d_s["offsets"], wo, w.dtype)
            if y_s is None:
                y_s = O.round_to(np.zeros((0, H)), w.dtype)
            sp_args = (y_s, d_s["row_of_slot"], ids_s, wts_s, "f32", n_cpu, k, w.dtype, E, n_sp, n_sp,
                       n_sp, xs, sp_a1, sp_a2, sp_v, act_s)
            if w.epilogue:
                sh_s, res_s, gam_s = I.epilogue_inputs(w)
                O.combine_add_rmsnorm_special(res_s[:n_cpu], gam_s, w.eps, *sp_args, shared=sh_s[:n_cpu])
            else:
                O.combine_special(*sp_args)
            what = "route over experts and special experts, masked dispatch, fp64 SwiGLU experts, special combine"
        else:
            O.forward(xs, zs, "f32", k, w.renormalize, wo, E, w.dtype)
            what = "route, dispatch, fp64 SwiGLU experts, combine"
        c_el = time.perf_counter() - c0
        cpu = {"value": round(n_cpu / c_el, 2), "unit": "tokens/s", "cores": cores, "kind": "oracle",
               "sample": f"first {n_cpu} of {T} tokens of {args.workload}; {what}; {c_el:.1f}s wall"}

    # ---- the same step replayed from a HIP graph (launch gaps removed) -----
    # Reported beside the eager figures (which stay `value`): one step
    # captured once, then replayed K times.
    graph = None
    if not args.no_graph:
        try:
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                step()
            torch.cuda.current_stream().wait_stream(side)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step()
            for _ in range(3):
                g.replay()
            torch.cuda.synchronize()
            g0 = time.perf_counter()
            for _ in range(args.steps):
                g.replay()
            torch.cuda.synchronize()
            g_el = time.perf_counter() - g0
            graph = {"ms_per_step": round(g_el / args.steps * 1e3, 4),
                     "tokens_per_s": round(T * args.steps / g_el, 1)}
        except RuntimeError as ex:  # capture not available: report the eager figures only
            log(f"graph replay skipped: {ex}")

    res = {
        "metric": METRIC, "value": round(tokens_per_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": args.workload, "T": T, "H": H, "I": I_, "E": E, "top_k": k,
                   "renormalize": w.renormalize, "logits_dtype": "f32"},
        "roofline": roofline, "cpu_baseline": cpu, "device": device_info(torch),
    }
    res["graph_replay"] = graph
    if grouped:
        res["config"]["router"] = dict(GROUPED, kind="sigmoid_grouped", bias="N(0, 0.05^2)")
        res["metric"] = METRIC + "; grouped-limited sigmoid router"
    if args.special:
        res["config"]["special_experts"] = {"zero": n_sp, "copy": n_sp, "const": n_sp,
                                            "active_tokens": int(sp_active.sum())}
        res["metric"] = METRIC + "; special experts and activity mask in the combine"
    res.update(extra)
    print(json.dumps(res), flush=True)


def device_info(torch):
    """The device the line was measured on: name, compute units, memory, the
    highest shader clock level the amdgpu kernel driver lists (sysfs; null
    where it cannot be read), the peaks the fractions use and a measured
    1 GiB device copy (read + written bytes over its median time of 5)."""
    p = torch.cuda.get_device_properties(0)
    info = {"name": p.name, "arch": p.gcnArchName.split(":")[0], "compute_units": p.multi_processor_count,
            "memory_gib": round(p.total_memory / 2**30, 1), "peak_bf16_tflops": PEAK_TFLOPS["bf16"],
            "peak_hbm_gbs": PEAK_HBM_GBS, "max_sclk_mhz": None}
    bus = f"{p.pci_domain_id:04x}:{p.pci_bus_id:02x}:{p.pci_device_id:02x}.0"
    try:
        with open(f"/sys/bus/pci/devices/{bus}/pp_dpm_sclk") as f:
            mhz = [int(tok.lower().replace("mhz", "")) for line in f for tok in line.split()[1:2]
                   if tok.lower().endswith("mhz")]
        info["max_sclk_mhz"] = max(mhz) if mhz else None
    except (OSError, ValueError):
        pass
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    b.copy_(a)
    times = []
    for _ in range(5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        b.copy_(a)
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    del a, b
    torch.cuda.empty_cache()
    info["copy_1gib_gbs"] = round(2 * n / (float(np.median(times)) / 1e3) / 1e9, 1)
    return info


def _device_weights(w, torch, td, I):
    """The workload's expert weights, generated expert by expert on the host
    and copied to the device."""
    out = {}
    for name in ("w_gate", "w_up", "w_down"):
        shape = (w.E, w.I, w.H) if name != "w_down" else (w.E, w.H, w.I)
        t = torch.empty(shape, dtype=td, device="cuda")
        for e0 in range(0, w.E, 16):
            ex = list(range(e0, min(w.E, e0 + 16)))
            a = I.expert_weights(w, name, ex)
            t[ex[0]:ex[-1] + 1].copy_(torch.from_numpy(a.view(np.int16)).view(td))
        out[name] = t
    return out


def measure_targets(args, torch, moe, I):
    """The two HBM-bound steps measured beside the default line, each on its
    workload's full shape with inputs resident in HBM, timed with HIP events
    on the stream the kernels run on:
      - the decode weight stream: moe_forward on the decode workload (T 16,
        H 4096, I 1536, E 128, top-8); both expert GEMMs' algorithmic bytes
        (the touched experts' gate, up and down weights, plus their input and
        output rows) over the median duration of the two GEMM stages;
      - the epilogue: moe_combine_add_rmsnorm on the DeepSeek-V3-shaped batch
        (T 2048, H 7168, top-8) from seeded expert rows and the routing maps
        of that workload's logits, with the shared-expert term, residual and
        gamma; its algorithmic bytes (expert rows, maps, weights, shared,
        residual and gamma in; y, x_out and rstd out) over its duration. Its
        352.5 MB would partly stay in the 256 MB MALL between back-to-back
        calls on the same buffers, so three input sets (1.06 GB) rotate: each
        call reads buffers last touched two calls earlier. The K calls run
        back to back between two events (the launch gaps amortised)."""
    td = torch.bfloat16
    res = {}
    # decode weight stream
    w = I.workload("decode_nan_rows_bf16")
    T, H, I_, E, k = w.T, w.H, w.I, w.E, w.top_k
    wt = _device_weights(w, torch, td, I)
    xd = torch.from_numpy(I.tokens_for(w).view(np.int16)).view(td).cuda()
    zd = torch.from_numpy(I.logits_for(w)).cuda()
    out = torch.empty((T, H), dtype=td, device="cuda")
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    offs = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    ws = torch.empty(moe.moe_forward_workspace_size(T, H, I_, E, k, td, torch.float32), dtype=torch.uint8,
                     device="cuda")
    for _ in range(args.warmup):
        moe.moe_forward(xd, zd, k, w.renormalize, wt["w_gate"], wt["w_up"], wt["w_down"], out=out, ws=ws,
                        indices_out=idx, offsets_out=offs)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for ev in evs:
        moe.moe_forward(xd, zd, k, w.renormalize, wt["w_gate"], wt["w_up"], wt["w_down"], out=out, ws=ws,
                        indices_out=idx, offsets_out=offs, stage_events=ev)
    torch.cuda.synchronize()
    # the median over the timed calls (one late call does not move it); the
    # mean is reported beside it
    gemm_all = [ev[2].elapsed_time(ev[4]) for ev in evs]
    gemm_ms, gemm_mean = float(np.median(gemm_all)), float(np.mean(gemm_all))
    counts = np.diff(offs.cpu().numpy())
    touched, rows = int((counts > 0).sum()), int(counts.sum())
    stream_bytes = touched * 3 * I_ * H * 2 + (T * H + 2 * rows * I_ + rows * H) * 2
    gbs = stream_bytes / (gemm_ms / 1e3) / 1e9
    res["hbm_decode_weight_stream_frac"] = round(gbs / PEAK_HBM_GBS, 4)
    res["hbm_decode_weight_stream"] = {"workload": w.name, "experts_touched": touched,
                                       "bytes": stream_bytes, "ms": round(gemm_ms, 4), "ms_mean": round(gemm_mean, 4),
                                       "gbs": round(gbs, 1), "stat": f"median of {len(gemm_all)} calls"}
    del wt
    torch.cuda.empty_cache()
    # combine + shared + residual Add + RMSNorm at the DeepSeek-V3-shaped batch
    w = I.workload("dsv3_share_rmsnorm_bf16")
    T, H, E, k = w.T, w.H, w.E, w.top_k
    R = T * k
    zd = torch.from_numpy(I.logits_for(w)).cuda()
    idx, wts = moe.moe_route(zd, k, w.renormalize)
    d = moe.moe_dispatch(idx, E)
    y = torch.from_numpy(I.store(I.normal(w.seed, "expert_out", (R, H)), "bf16").view(np.int16)).view(td).cuda()
    sh, rs, gam = I.epilogue_inputs(w)
    shd, rsd = (torch.from_numpy(a.view(np.int16)).view(td).cuda() for a in (sh, rs))
    gamd = torch.from_numpy(gam).cuda()
    sets = []
    for i in range(3):  # the same values in three places
        sets.append(dict(y=y if i == 0 else y.clone(), sh=shd if i == 0 else shd.clone(),
                         rs=rsd if i == 0 else rsd.clone(), ros=d["row_of_slot"].clone(), w=wts.clone(),
                         yo=torch.empty((T, H), dtype=td, device="cuda"),
                         xo=torch.empty((T, H), dtype=td, device="cuda"),
                         rstd=torch.empty(T, dtype=torch.float32, device="cuda")))

    def epilogue(i):
        b = sets[i % 3]
        moe.moe_combine_add_rmsnorm(b["y"], b["ros"], b["w"], b["rs"], gamd, w.eps, shared=b["sh"], y=b["yo"],
                                    x_out=b["xo"], rstd=b["rstd"])

    for i in range(max(args.warmup, 3)):
        epilogue(i)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for i in range(args.steps):
        epilogue(i)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / args.steps
    ep_bytes = R * H * 2 + R * 4 + R * 4 + 4 * T * H * 2 + 4 * H + 4 * T
    gbs = ep_bytes / (ms / 1e3) / 1e9
    res["hbm_epilogue_frac"] = round(gbs / PEAK_HBM_GBS, 4)
    res["hbm_epilogue"] = {"workload": w.name, "kernel": "combine_norm_kernel", "bytes": ep_bytes,
                           "ms": round(ms, 4), "gbs": round(gbs, 1),
                           "inputs": "three rotating sets, each last touched two calls earlier"}
    log(f"targets: decode weight stream {res['hbm_decode_weight_stream_frac']:.3f} of HBM, "
        f"epilogue {res['hbm_epilogue_frac']:.3f}")
    return res


def run_quant(args, w, x, z, to_dev):
    """The forward with weight-only quantised experts (moe_forward_quant) on
    the current stream; stage events as moe_forward. Roofline: the gate/up
    stage's weight-streaming bytes (codes + scales of the touched experts,
    tokens, h) against HBM."""
    import torch
    from mixture_experts_ffn_top_amd import inputs as I
    from mixture_experts_ffn_top_amd import moe

    T, H, I_, E, k = w.T, w.H, w.I, w.E, w.top_k
    R = T * k
    bits = args.quant
    groups = args.groups or (1 if bits == 8 else 4)
    if R > 4 * E or w.dtype != "bf16":
        raise SystemExit("the quantised path serves decode-sized bf16 batches (T * top_k <= 4 E)")
    t0 = time.time()
    q, sc = {}, {}
    for name in ("w_gate", "w_up", "w_down"):
        qh, sh = I.quant_expert_weights(w, name, bits, groups)
        q[name], sc[name] = torch.from_numpy(qh).cuda(), to_dev(sh)
        if not args.no_cpu_baseline:
            q[name + "_host"], sc[name + "_host"] = qh, sh
    xd, zd = to_dev(x), to_dev(z, "f32")
    torch.cuda.synchronize()
    log(f"quantised inputs ready in {time.time() - t0:.1f}s: INT{bits}, {groups} group(s)")
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    wts = torch.empty((T, k), dtype=torch.float32, device="cuda")
    out = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(moe.moe_forward_workspace_size(T, H, I_, E, k, torch.bfloat16, torch.float32),
                     dtype=torch.uint8, device="cuda")
    scales = (sc["w_gate"], sc["w_up"], sc["w_down"])

    def step(ev=None):
        moe.moe_forward_quant(xd, zd, k, w.renormalize, q["w_gate"], q["w_up"], q["w_down"], bits, scales,
                              groups=groups, out=out, indices_out=idx, weights_out=wts, ws=ws, stage_events=ev)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(args.steps)]
    for ev in evs:
        for e_ in ev:
            e_.record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for s_ in range(args.steps):
        step(evs[s_])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t1
    stages = ["route", "dispatch", "gate_up", "down", "combine"]
    stage_ms = {n: float(np.mean([evs[s_][i].elapsed_time(evs[s_][i + 1]) for s_ in range(args.steps)]))
                for i, n in enumerate(stages)}
    touched = len(np.unique(idx.cpu().numpy()))
    wbytes_gu = touched * 2 * I_ * H * bits // 8 + touched * 2 * I_ * groups * 2
    wbytes_dn = touched * H * I_ * bits // 8 + touched * H * groups * 2
    # moe_forward_quant runs both expert GEMMs between the gate_up and down
    # events: the roofline covers the two launches of skinny_quant_kernel
    # (codes + scales of the touched experts, tokens in, h out and back in,
    # expert rows out) over that stage
    bytes_experts = wbytes_gu + wbytes_dn + T * H * 2 + 2 * R * I_ * 2 + R * H * 2
    exp_s = (stage_ms["gate_up"] + stage_ms["down"]) / 1e3
    gbs = bytes_experts / exp_s / 1e9
    qkernel = f"skinny_quant_kernel<bf16,gate_up|down,INT{bits}> (both launches)"
    roofline = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(gbs / PEAK_HBM_GBS, 4),
                "traffic": measured_traffic(f"{args.workload}+int{bits}", qkernel),
                "kernel": qkernel, "algorithmic_per_launch": bytes_experts}
    cpu = None
    if not args.no_cpu_baseline:
        from oracle import moe_oracle as O
        n = min(args.cpu_tokens or 4, T)
        cores = len(os.sched_getaffinity(0))
        idx_s, w_s = O.route(z[:n], "f32", k, w.renormalize)
        d = O.dispatch(idx_s, E, x[:n])
        quant_of = lambda e: tuple((q[nm + "_host"][e], sc[nm + "_host"][e], None)  # noqa: E731
                                   for nm in ("w_gate", "w_up", "w_down"))
        c0 = time.perf_counter()
        y = O.experts_forward_quant(d["x_disp"], d["offsets"], quant_of, bits, groups, w.dtype)
        O.combine(y, d["row_of_slot"], w_s, "f32", n, k, w.dtype)
        c_el = time.perf_counter() - c0
        cpu = {"value": round(n / c_el, 3), "unit": "tokens/s", "cores": cores, "kind": "oracle",
               "sample": f"first {n} of {T} tokens of {args.workload} with INT{bits} experts; dequantised "
                         f"fp64 SwiGLU experts and combine; {c_el:.1f}s wall"}
    res = {
        "metric": f"MoE fwd tokens/s with weight-only INT{bits} experts", "value": round(T * args.steps / elapsed, 1),
        "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(elapsed / args.steps * 1e3, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{args.workload}+int{bits}", "T": T, "H": H, "I": I_, "E": E, "top_k": k,
                   "bits": bits, "groups": groups},
        "roofline": roofline, "cpu_baseline": cpu, "device": device_info(torch),
        "stages_ms": {k_: round(v, 4) for k_, v in stage_ms.items()},
        "weight_stream_gbs": round((wbytes_gu + wbytes_dn) / exp_s / 1e9, 1),
        "experts_touched": touched,
    }
    print(json.dumps(res), flush=True)


TRAIN_STAGES = ["route", "router_weights", "dispatch", "experts_fwd", "combine",
                "combine_bwd", "experts_bwd", "dispatch_bwd", "router_bwd"]
TRAIN_CPU_TOKENS = {"tiny_fp32": 64, "mixtral_8x_bf16": 16, "many_expert_zipf_bf16": 64,
                    "dsv3_share_rmsnorm_bf16": 4, "decode_nan_rows_bf16": 16}


def run_train(args, w, x, z, xd, zd, wt, kept, n_cpu):
    """One training step through the C ABI: the routing plan's selection, its
    fp32 weights (selected_router_weights), dispatch with x_disp, the experts'
    training forward (cache of g, u, h), combine; then combine_backward,
    the experts' backward, dispatch_backward and the router backward, with a
    fixed synthetic gradient of the output. Stage events on this stream."""
    import torch
    from mixture_experts_ffn_top_amd import moe

    T, H, I_, E, k = w.T, w.H, w.I, w.E, w.top_k
    R = T * k
    if w.dtype != "bf16":
        raise SystemExit("the training path runs on the bf16/f16 matrix cores; pick a bf16 workload")
    td, dev = torch.bfloat16, "cuda"
    from mixture_experts_ffn_top_amd import inputs as I
    go_host = I.grad_output_for(w)
    grad_out = torch.from_numpy(go_host.view(np.int16)).view(td).to(dev)
    idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    wts_plan = torch.empty((T, k), dtype=torch.float32, device=dev)
    wts = torch.empty((T, k), dtype=torch.float32, device=dev)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    sor = torch.empty(R, dtype=torch.int32, device=dev)
    ros = torch.empty(R, dtype=torch.int32, device=dev)
    x_disp = torch.empty((R, H), dtype=td, device=dev)
    y = torch.empty((R, H), dtype=td, device=dev)
    out = torch.empty((T, H), dtype=td, device=dev)
    cache = torch.empty(R * 3 * I_, dtype=td, device=dev)
    dexp = torch.empty((R, H), dtype=td, device=dev)
    dw = torch.empty((T, k), dtype=torch.float32, device=dev)
    dinput = torch.empty((R, H), dtype=td, device=dev)
    dgate = torch.empty((E, I_, H), dtype=torch.float32, device=dev)
    dup = torch.empty_like(dgate)
    ddown = torch.empty((E, H, I_), dtype=torch.float32, device=dev)
    dx = torch.empty((T, H), dtype=td, device=dev)
    dz = torch.empty((T, E), dtype=torch.float32, device=dev)
    ws_d = torch.empty(moe.moe_dispatch_workspace_size(T, k, E), dtype=torch.uint8, device=dev)
    ws_f = torch.empty(moe.lib().moe_experts_forward_training_workspace_size(R, E, H, I_, moe.BF16),
                       dtype=torch.uint8, device=dev)
    ws_b = torch.empty(moe.lib().moe_experts_backward_workspace_size(R, E, H, I_, moe.BF16),
                       dtype=torch.uint8, device=dev)
    scoring = moe.SOFTMAX

    def step(ev=None):
        def mark(i):
            if ev is not None:
                ev[i].record()
        mark(0)
        moe.moe_route(zd, k, w.renormalize, indices=idx, weights=wts_plan)
        mark(1)
        moe.moe_router_weights(zd, idx, scoring, w.renormalize, 1.0, weights=wts)
        mark(2)
        moe.moe_dispatch(idx, E, xd, ws=ws_d, offsets=offsets, slot_of_row=sor, row_of_slot=ros,
                         x_disp=x_disp)
        mark(3)
        moe.moe_experts_forward_training(x_disp, offsets, wt["w_gate"], wt["w_up"], wt["w_down"], rows=R,
                                         expert_out=y, cache=cache, ws=ws_f)
        mark(4)
        moe.moe_combine(y, ros, wts, out=out)
        mark(5)
        moe.moe_combine_backward(y, ros, wts, grad_out, k, dexpert=dexp, dweights=dw)
        mark(6)
        moe.moe_experts_backward(x_disp, offsets, wt["w_gate"], wt["w_up"], wt["w_down"], cache, dexp, rows=R,
                                 dinput=dinput, dgate=dgate, dup=dup, ddown=ddown, ws=ws_b)
        mark(7)
        moe.moe_dispatch_backward(dinput, ros, T, k, dx=dx)
        mark(8)
        moe.moe_router_backward(zd, idx, dw, scoring, w.renormalize, 1.0, grad_logits=dz)
        mark(9)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"train warmup done ({args.warmup} steps)")
    n_ev = len(TRAIN_STAGES) + 1
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(n_ev)] for _ in range(args.steps)]
    for ev in evs:
        for e_ in ev:
            e_.record()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s_ in range(args.steps):
        step(evs[s_])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    log(f"timed {args.steps} training steps in {elapsed:.3f}s")
    stage_ms = {name: float(np.mean([evs[s_][i].elapsed_time(evs[s_][i + 1]) for s_ in range(args.steps)]))
                for i, name in enumerate(TRAIN_STAGES)}
    # the experts' backward: dh (2RHI), dinput (4RHI), ddown (2RHI), dgate|dup (4RHI)
    flops_bwd = 12.0 * R * H * I_
    flops_fwd = 6.0 * R * H * I_
    bwd_tf = flops_bwd / (stage_ms["experts_bwd"] / 1e3) / 1e12
    fwd_tf = flops_fwd / (stage_ms["experts_fwd"] / 1e3) / 1e12
    tkernel = "moe_experts_backward (4 train_gemm_kernel launches + tile prefix)"
    roofline = {"bound": "mfma", "achieved": round(bwd_tf, 1), "peak": PEAK_TFLOPS["bf16"], "unit": "TFLOP/s",
                "frac": round(bwd_tf / PEAK_TFLOPS["bf16"], 4),
                "traffic": measured_traffic(f"{args.workload}+train", tkernel),
                "kernel": tkernel, "algorithmic_per_launch": flops_bwd}
    cpu = None
    if not args.no_cpu_baseline:
        from oracle import moe_oracle as O
        n = min(args.cpu_tokens or TRAIN_CPU_TOKENS.get(args.workload, 16), T)
        cores = len(os.sched_getaffinity(0))
        idx_s, _ = O.route(z[:n], "f32", k, w.renormalize)
        need = sorted(set(int(e) for e in idx_s.ravel()))
        if all(e in kept for e in need):
            wo = lambda e: (kept[e]["w_gate"], kept[e]["w_up"], kept[e]["w_down"])  # noqa: E731
            sub = {e: i for i, e in enumerate(need)}
            go = go_host[:n]
            log(f"cpu baseline: oracle training step on {n} tokens")
            c0 = time.perf_counter()
            wr = O.router_selected_weights(z[:n], "f32", idx_s, O.SOFTMAX, w.renormalize, 1.0)
            idx_l = np.vectorize(sub.get)(idx_s).astype(np.uint32)
            d = O.dispatch(idx_l, len(need), x[:n])
            wl = lambda i: wo(need[i])  # noqa: E731
            y_r, g_r, u_r, h_r = O.experts_forward_training(d["x_disp"], d["offsets"], wl, w.dtype)
            O.combine(y_r, d["row_of_slot"], wr, "f32", n, k, w.dtype)
            de, dwr = O.combine_backward(y_r, d["row_of_slot"], wr, "f32", go, n, k, w.dtype)
            di, _, _, _ = O.experts_backward(d["x_disp"], d["offsets"], wl, g_r, u_r, h_r, de, w.dtype)
            O.dispatch_backward(di, d["row_of_slot"], n, k, H, w.dtype)
            O.router_selected_backward(z[:n], "f32", idx_s, dwr, O.SOFTMAX, w.renormalize, 1.0)
            c_el = time.perf_counter() - c0
            cpu = {"value": round(n / c_el, 3), "unit": "tokens/s", "cores": cores, "kind": "oracle",
                   "sample": f"training step on the first {n} of {T} tokens of {args.workload} "
                             f"({len(need)} experts); {c_el:.1f}s wall"}
    res = {
        "metric": "MoE training step tokens/s (forward with cache + backward)",
        "value": round(T * args.steps / elapsed, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(elapsed / args.steps * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": args.workload + "+train", "T": T, "H": H, "I": I_, "E": E, "top_k": k,
                   "scoring": "softmax", "normalize": w.renormalize},
        "roofline": roofline, "cpu_baseline": cpu, "device": device_info(torch),
        "stages_ms": {k_: round(v, 4) for k_, v in stage_ms.items()},
        "experts_fwd_tflops": round(fwd_tf, 1), "experts_bwd_tflops": round(bwd_tf, 1),
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
