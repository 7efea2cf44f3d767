"""Benchmark of the vertical-slash sparse attention hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input that is
already resident in HBM: sparse-index build (scores + top-p) -> active region
-> sparse attention forward -> backward (delta, dQ, dK, dV).

Default workload: the Qwen2.5-3B-shaped layer at 131072 tokens (16 q heads,
2 kv heads, head dim 128, bf16, top-p 0.95), forward + backward.

Prints one JSON line with the effective sparse-attention TFLOP/s of the whole
step (effective FLOPs = 4*d*A forward + 10*d*A backward, A = active entries
summed over q heads), tokens/s, per-stage times, the roofline of the sparse
forward kernel and the fp64 oracle timed on the host as a CPU baseline.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                       [--no-cpu-baseline]

Ring simulation (a workload with P > 1, e.g. --workload qwen512k_cp32): every
rank's steps of the ring run one after another on the one GPU, each timed
alone; prints a separate report line (per-step times and load imbalance,
striped vs zigzag, fused vs separate merge), not the headline line.
"""
import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "effective sparse-attn TFLOP/s fwd+bwd + tokens/s at 128K, 1 MI355X"
MFMA_BF16_PEAK_TFLOPS = 2500.0
MFMA_F32_PEAK_TFLOPS = 157.3
HBM_PEAK_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="qwen128k")
    ap.add_argument("--top-p", type=float, default=None)
    ap.add_argument("--operands", choices=("f16", "bf16"), default="f16",
                    help="attention operand format for bf16 workloads: exact fp16 copies (converted inside the "
                         "timed step, single fp16 P/dS) or the bf16 inputs (hi + lo bf16 P/dS)")
    ap.add_argument("--bwd-streams", type=int, choices=(1, 2), default=1,
                    help="2: run the dQ part on a second stream, concurrently with the dK/dV parts")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-budgets", action="store_true", help="skip the budget-rule report (after the timed steps)")
    ap.add_argument("--no-bf16-operands", action="store_true",
                    help="skip the second timing of the step with bf16 operands (kernel traces of the fp16 path)")
    ap.add_argument("--no-packed", action="store_true",
                    help="skip the per-kv-head index / head-pair forward report (after the timed steps)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target oracle sample time")
    ap.add_argument("--copy-probe", action="store_true", help="run only a 1 GiB device copy (counter scaling)")
    ap.add_argument("--layouts", default="striped,zigzag", help="ring simulation: layouts to compare")
    ap.add_argument("--ring-reps", type=int, default=3, help="ring simulation: timed repetitions (median)")
    ap.add_argument("--report-md", default=None, help="ring simulation: also write a markdown summary here")
    return ap.parse_args()


def main():
    args = parse()
    if args.copy_probe:
        copy_probe()
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: it times one rank's share of the sparse path on a "
              "single MI355X and has no multi-GPU mode (use --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import torch
    import dynamic_sparse_attention_index_amd as vs
    from synth import config_by_name, generate

    cfg = config_by_name(args.workload)
    if args.top_p is not None:
        cfg = config_by_name(args.workload, top_p=args.top_p)
    if cfg.P != 1:
        ring_report(args, cfg)
        return
    dev = torch.device("cuda:0")
    N, Hq, Hkv, D = cfg.N, cfg.Hq, cfg.Hkv, cfg.D
    T = N // 64
    tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32

    t0 = time.time()
    host = generate(cfg)
    q = torch.tensor(host["q"]).to(dev, tdt)
    k = torch.tensor(host["k"]).to(dev, tdt)
    v = torch.tensor(host["v"]).to(dev, tdt)
    do = torch.tensor(host["do"]).to(dev, tdt)
    gen_s = time.time() - t0

    lay = vs.layout("contig", 1, N)
    vert_s = torch.empty(Hq, N, device=dev)
    slash_s = torch.empty(Hq, T, device=dev)
    vidx = torch.empty(Hq, N, dtype=torch.int32, device=dev)
    vcnt = torch.empty(Hq, dtype=torch.int32, device=dev)
    sidx = torch.empty(Hq, T, dtype=torch.int32, device=dev)
    scnt = torch.empty(Hq, dtype=torch.int32, device=dev)
    ws = torch.empty(vs.index_workspace_size(Hq, Hkv, N, D), dtype=torch.uint8, device=dev)
    q_last = q[:, N - cfg.last_q:]
    vs.vs_index_build(q_last, k, lay, cfg.scale, cfg.top_p, vert_s, slash_s, vidx, vcnt, sidx, scnt, ws)
    torch.cuda.synchronize()
    max_s = int(scnt.max().item())
    mask = vs.Mask(Hq, Hkv, lay, tile_cap=Hq * T * (max_s + 1))
    o = torch.empty(Hq, N, D, device=dev)
    lse = torch.empty(Hq, N, device=dev)
    delta = torch.empty(Hq, N, device=dev)
    dq = torch.empty(Hq, N, D, device=dev)     # written whole by the backward step
    dk = torch.empty(Hkv, N, D, device=dev)
    dv = torch.empty(Hkv, N, D, device=dev)
    stream = torch.cuda.current_stream()

    # fp16 operands: exact copies of the bf16 inputs, made inside every timed
    # step (q, k, v before the forward; dO before the backward)
    f16_main = args.operands == "f16" and cfg.dtype == "bf16" and D == 128
    conv_status = torch.zeros(1, dtype=torch.int32, device=dev)
    if f16_main:
        q16, k16, v16, do16 = (torch.empty(x.shape, dtype=torch.float16, device=dev) for x in (q, k, v, do))

    stages = ("index", "mask", "convert_qkv", "fwd", "bwd_prep", "dq", "dkdv", "dkdv_vert")
    ev = {name: [] for name in stages}
    two = args.bwd_streams == 2 and cfg.backward
    side = torch.cuda.Stream(device=dev) if two else None    # default priority, like every stream here

    def step(record, f16=f16_main, ev=ev):
        aq, ak, av, ado = (q16, k16, v16, do16) if f16 else (q, k, v, do)
        marks = [torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)] if record else None
        dq_ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) if record else None

        def mark(i):
            if record:
                marks[i].record(stream)
        mark(0)
        vs.vs_index_build(q_last, k, lay, cfg.scale, cfg.top_p, vert_s, slash_s, vidx, vcnt, sidx, scnt, ws, stream)
        mark(1)
        vs.vs_block_mask(vidx, vcnt, sidx, scnt, 0, 0, mask, stream)
        mark(2)
        if f16:
            for src, dst in ((q, q16), (k, k16), (v, v16)):
                vs.vs_convert_f16(src, dst, conv_status, stream)
        mark(3)
        vs.vs_attn_fwd(aq, ak, av, mask, cfg.scale, o, lse, 0, stream)
        mark(4)
        if cfg.backward:
            if f16:     # delta and the fp16 copy of dO in one pass over dO
                vs.vs_attn_bwd_prep_f16(o, do, do16, delta, conv_status, stream)
            else:
                vs.vs_attn_bwd_prep(o, ado, delta, stream)
            mark(5)
            # dq and the slash dk/dv write their outputs whole; the vertical part adds after them
            if two:
                # dq (writes dq only) on the side stream, dk/dv parts on the launch stream
                fork, join = torch.cuda.Event(), torch.cuda.Event()
                fork.record(stream)
                side.wait_event(fork)
                if record:
                    dq_ev[0].record(side)
                vs.vs_attn_bwd_parts(aq, ak, av, ado, lse, delta, mask, cfg.scale, dq, dk, dv,
                                     vs.VS_BWD_DQ | vs.VS_BWD_OVERWRITE, side)
                if record:
                    dq_ev[1].record(side)
                join.record(side)
            else:
                vs.vs_attn_bwd_parts(aq, ak, av, ado, lse, delta, mask, cfg.scale, dq, dk, dv,
                                     vs.VS_BWD_DQ | vs.VS_BWD_OVERWRITE, stream)
            mark(6)
            vs.vs_attn_bwd_parts(aq, ak, av, ado, lse, delta, mask, cfg.scale, dq, dk, dv,
                                 vs.VS_BWD_DKDV | vs.VS_BWD_OVERWRITE, stream)
            mark(7)
            vs.vs_attn_bwd_parts(aq, ak, av, ado, lse, delta, mask, cfg.scale, dq, dk, dv, vs.VS_BWD_DKDV_VERT,
                                 stream)
        else:
            for i in (5, 6, 7):
                mark(i)
        mark(8)
        if two:
            stream.wait_event(join)
        if record:
            for i, name in enumerate(stages):
                ev[name].append(dq_ev if (two and name == "dq") else (marks[i], marks[i + 1]))

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    status = int(mask.arrays()["status"].item())
    if status != 0:
        raise RuntimeError(f"mask status {status}")
    if int(conv_status.item()) != 0:
        raise RuntimeError("an input is outside the fp16 range: run with --operands bf16")
    t_start = time.perf_counter()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    if int(conv_status.item()) != 0:
        raise RuntimeError("fp16 conversion range error in the timed steps")
    ms_per_step = wall * 1e3 / args.steps
    stage_ms = {kname: float(np.mean([a.elapsed_time(b) for a, b in pairs])) for kname, pairs in ev.items()}
    f16 = f16_main

    # The same step with the bf16 inputs as operands (hi + lo bf16 P and dS,
    # no copies), timed right after on the same inputs and index: the format
    # the pages train in, beside the fp16 headline.
    bf16_operands = None
    if f16_main and cfg.backward and not args.no_bf16_operands:
        ev_b = {name: [] for name in stages}
        for _ in range(args.warmup):
            step(False, f16=False, ev=ev_b)
        torch.cuda.synchronize()
        tb = time.perf_counter()
        for _ in range(args.steps):
            step(True, f16=False, ev=ev_b)
        torch.cuda.synchronize()
        ms_b = (time.perf_counter() - tb) * 1e3 / args.steps
        bf16_operands = {"ms_per_step": round(ms_b, 4),
                         "stage_ms": {kname: round(float(np.mean([a.elapsed_time(b) for a, b in pairs])), 4)
                                      for kname, pairs in ev_b.items()}}

    arrs = mask.arrays()
    n_active = arrs["n_active"]
    A = int(n_active.sum().item())
    tp = arrs["tile_ptr"].cpu().numpy()
    tcol = arrs["tile_col"][: int(tp[-1])].cpu().numpy()
    n_diag = int(((tcol & vs.TILE_DIAG) != 0).sum())
    A_slash = 4096 * (len(tcol) - n_diag) + 2080 * n_diag     # entries inside listed slash tiles
    A_vert = A - A_slash                                       # vertical entries outside them
    # entries the kernels compute: every listed tile whole (the diagonal
    # tile's upper half is masked), and the vertical columns of a query block
    # gathered 64 at a time into whole 64 x 64 tiles
    vend = arrs["vert_end"].cpu().numpy().astype(np.int64)
    computed_slash = 4096 * len(tcol)
    computed_vert = 4096 * int(((vend + 63) // 64).sum())
    tile_fill = {"slash_tiles": round(A_slash / max(computed_slash, 1), 4),
                 "vertical_chunks": round(A_vert / max(computed_vert, 1), 4),
                 "all": round(A / max(computed_slash + computed_vert, 1), 4),
                 "computed_entries": computed_slash + computed_vert,
                 "note": "active entries / entries the forward and dQ kernels compute (whole 64x64 tiles: "
                         "listed slash tiles, and vertical columns gathered 64 per tile)"}
    total_causal = Hq * N * (N + 1) // 2
    sparsity = 1.0 - A / total_causal
    eff_flops = (4 + (10 if cfg.backward else 0)) * D * A
    tflops = eff_flops / (ms_per_step * 1e-3) / 1e12
    attn_ms = sum(stage_ms[x] for x in ("convert_qkv", "fwd", "bwd_prep"))
    if two:   # dq overlaps the dk/dv parts
        attn_ms += max(stage_ms["dq"], stage_ms["dkdv"] + stage_ms["dkdv_vert"])
    else:
        attn_ms += stage_ms["dq"] + stage_ms["dkdv"] + stage_ms["dkdv_vert"]
    attn_tflops = eff_flops / (attn_ms * 1e-3) / 1e12

    # Roofline of the dominant kernel. Each timed kernel stage below is exactly
    # one kernel launch (convert_qkv is three). Algorithmic FLOPs per active entry (FlashAttention-2
    # convention, 14 d in total): forward 4 d; dK/dV kernels 8 d (recompute S,
    # dP, dV, dK) over their entries; dQ kernel 2 d.
    peak = MFMA_BF16_PEAK_TFLOPS if cfg.dtype == "bf16" else MFMA_F32_PEAK_TFLOPS
    if cfg.dtype == "bf16" and D == 128:
        op = "f16" if f16 else "bf16"
        kn = {"fwd": f"attn_fwd_{op}_d128_kernel", "dq": f"dq_{op}_d128_kernel",
              "dkdv": f"dkdv_{op}_d128_kernel", "dkdv_vert": f"dkdv_vert_{op}_d128_kernel"}
    else:
        tn = "bf16" if cfg.dtype == "bf16" else "float"
        kn = {"fwd": f"attn_fwd_kernel<{tn}, {D}>", "dq": f"dq_kernel<{tn}, {D}>",
              "dkdv": f"dkdv_kernel<{tn}, {D}>", "dkdv_vert": f"dkdv_vert_kernel<{tn}, {D}>"}
    kernels = {"fwd": (kn["fwd"], 4 * D * A)}
    if cfg.backward:
        kernels.update({"dq": (kn["dq"], 2 * D * A),
                        "dkdv": (kn["dkdv"], 8 * D * A_slash),
                        "dkdv_vert": (kn["dkdv_vert"], 8 * D * A_vert)})
    per_kernel = {}
    for st, (kname, flops) in kernels.items():
        tf = flops / (stage_ms[st] * 1e-3) / 1e12
        per_kernel[st] = {"kernel": kname, "ms": round(stage_ms[st], 4), "tflops": round(tf, 2),
                          "frac_mfma_peak": round(tf / peak, 4)}
    dom = max(per_kernel, key=lambda x: per_kernel[x]["ms"])
    dk_name, dk_flops = kernels[dom]
    # strict count (no recomputation credited): forward 4 d, dK/dV 6 d (dP, dV,
    # dK), dQ 2 d, vertical dK/dV 6 d
    strict_per = {"fwd": 4, "dq": 2, "dkdv": 6, "dkdv_vert": 6}
    strict_flops = strict_per[dom] * D * (A_slash if dom == "dkdv" else A_vert if dom == "dkdv_vert" else A)
    roofline = {"kernel": dk_name, "bound": "mfma", "achieved": per_kernel[dom]["tflops"], "peak": peak,
                "unit": "TFLOP/s", "frac": per_kernel[dom]["frac_mfma_peak"],
                "traffic": stored_traffic(dk_name),
                "traffic_kind": "bytes per launch between L2 and the data fabric (FETCH_SIZE + WRITE_SIZE, "
                                "scaled by a copy of known size): HBM plus Infinity Cache hits",
                "algorithmic_flops_per_launch": dk_flops,
                "frac_strict": round(strict_flops / (stage_ms[dom] * 1e-3) / 1e12 / peak, 4),
                "mean_launch_ms": round(stage_ms[dom], 4)}

    # Index pass (scores + top-p): algorithmic bytes = K read once + the last
    # query rows + vertical and slash scores written; FLOPs = two passes of
    # 2 * last_q * N * d per q head (row statistics, then the masses).
    esz = 2 if cfg.dtype == "bf16" else 4
    idx_bytes = Hkv * N * D * esz + Hq * cfg.last_q * D * esz + 4 * Hq * N + 4 * Hq * T
    idx_flops = 2 * 2 * cfg.last_q * N * D * Hq
    index_pass = {"ms": round(stage_ms["index"], 4), "algorithmic_bytes": idx_bytes,
                  "gbs": round(idx_bytes / (stage_ms["index"] * 1e-3) / 1e9, 1),
                  "frac_hbm_peak": round(idx_bytes / (stage_ms["index"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                  "tflops": round(idx_flops / (stage_ms["index"] * 1e-3) / 1e12, 2),
                  "frac_mfma_peak": round(idx_flops / (stage_ms["index"] * 1e-3) / 1e12 / peak, 4)}
    strict_tflops = (4 + (8 if cfg.backward else 0)) * D * A / (ms_per_step * 1e-3) / 1e12

    budgets = None if args.no_budgets else budget_report(vs, torch, Hq, Hkv, N, lay, vert_s, slash_s, cfg.top_p,
                                                         stream)

    packed = None
    if not args.no_packed and D == 128 and (Hq // Hkv) % 2 == 0 and cfg.dtype == "bf16":
        aq, ak, av = (q16, k16, v16) if f16 else (q, k, v)   # the headline's operands
        packed = packed_report(vs, torch, cfg, lay, vert_s, slash_s, aq, ak, av, o, lse, stream)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(cfg, host, vidx, vcnt, sidx, scnt, args.cpu_seconds, tflops_unit=True)

    line = {
        "metric": METRIC, "value": round(tflops, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f16" if f16 else cfg.dtype, "data": "synthetic",
        "inputs": cfg.dtype,
        "operands": ("fp16 copies of the bf16 inputs (exact for 2^-17 <= |x| < 65536, smaller magnitudes "
                     "rounded to 2^-24 spacing; converted inside the step), single fp16 P/dS, "
                     "fp32 accumulation") if f16 else f"{cfg.dtype} inputs as given",
        "bwd_streams": args.bwd_streams,
        "config": {"workload": cfg.name, "Hq": Hq, "Hkv": Hkv, "seq_len": N, "head_dim": D,
                   "top_p": cfg.top_p, "last_q": cfg.last_q, "backward": cfg.backward, "mean_c": cfg.c,
                   "seed": cfg.seed},
        "tokens_per_s": round(N / (ms_per_step * 1e-3), 1),
        "attn_only_tflops": round(attn_tflops, 3),
        "stage_ms": {kk: round(vv, 4) for kk, vv in stage_ms.items()},
        "kernels": per_kernel,
        "active_entries": A, "active_slash_tiles": A_slash, "active_vertical": A_vert, "tile_fill": tile_fill,
        "sparsity": round(sparsity, 5), "effective_flops": eff_flops,
        "strict_algorithmic_tflops": round(strict_tflops, 3), "index_pass": index_pass,
        "roofline": roofline, "cpu_baseline": cpu, "budgets": budgets, "gqa_packed": packed,
        "bf16_operands": (None if bf16_operands is None else dict(
            bf16_operands, value=round(eff_flops / (bf16_operands["ms_per_step"] * 1e-3) / 1e12, 3),
            unit="TFLOP/s", note="the same step on the bf16 inputs as attention operands (hi + lo bf16 P and "
                                 "dS, no fp16 copies), timed in this run after the headline steps")),
        "gen_s": round(gen_s, 1),
    }
    print(json.dumps(line), flush=True)


def packed_report(vs, torch, cfg, lay, vert_s, slash_s, q, k, v, o, lse, stream, reps=10):
    """The per-kv-head index (one top-p per kv head on its q heads' mean
    scores) on the workload's own scores, and the sparse forward on it run
    two ways: one q head per workgroup (vs_attn_fwd) and two q heads of a kv
    group per workgroup sharing the K/V tile copies (vs_attn_fwd_packed).
    Mean kernel time over `reps` launches each."""
    dev = vert_s.device
    N, Hq, Hkv = cfg.N, cfg.Hq, cfg.Hkv
    T = N // 64
    vidx = torch.empty(Hq, N, dtype=torch.int32, device=dev)
    sidx = torch.empty(Hq, T, dtype=torch.int32, device=dev)
    vcnt, scnt = (torch.empty(Hq, dtype=torch.int32, device=dev) for _ in range(2))
    gws = torch.empty(vs.index_select_group_workspace_size(Hq, Hkv, N), dtype=torch.uint8, device=dev)
    vs.vs_index_select_group(vert_s, slash_s, Hq, Hkv, N, cfg.top_p, vidx, vcnt, sidx, scnt, gws, stream)
    torch.cuda.synchronize()
    m = vs.Mask(Hq, Hkv, lay, tile_cap=Hq * T * (int(scnt.max().item()) + 1))
    vs.vs_block_mask(vidx, vcnt, sidx, scnt, 0, 0, m, stream)
    status = torch.zeros(1, dtype=torch.int32, device=dev)

    def timed(fn):
        fn()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps
    t_sel = timed(lambda: vs.vs_index_select_group(vert_s, slash_s, Hq, Hkv, N, cfg.top_p, vidx, vcnt, sidx, scnt,
                                                   gws, stream))
    t1 = timed(lambda: vs.vs_attn_fwd(q, k, v, m, cfg.scale, o, lse, 0, stream))
    o1 = o.clone()
    t2 = timed(lambda: vs.vs_attn_fwd_packed(q, k, v, m, cfg.scale, o, lse, status, 0, stream))
    arr = m.arrays()
    if int(arr["status"].item()) != 0 or int(status.item()) != 0:
        raise RuntimeError("packed report: mask or pair status")
    same = bool(torch.equal(o1, o))
    A = int(arr["n_active"].sum().item())
    f = 4 * cfg.D * A
    return {"select_ms": round(t_sel, 4), "mean_verticals": round(float(vcnt.float().mean()), 1),
            "mean_slashes": round(float(scnt.float().mean()), 1),
            "sparsity": round(1.0 - A / (Hq * N * (N + 1) // 2), 5),
            "fwd_ms": round(t1, 4), "fwd_packed_ms": round(t2, 4),
            "fwd_tflops": round(f / (t1 * 1e-3) / 1e12, 2), "fwd_packed_tflops": round(f / (t2 * 1e-3) / 1e12, 2),
            "packed_equals_unpacked": same}


def budget_report(vs, torch, Hq, Hkv, N, lay, vert_s, slash_s, top_p, stream, target=0.95, reps=20):
    """The three budget rules on the workload's own scores: selection time
    (one launch sequence, mean over `reps`), mean kept counts and the
    sparsity of the mask they give. The fixed-count budget is sized for
    `target` sparsity (the pages' hand-fixed 95%): counts proportional to the
    top-p means, scaled by bisection until the mask just reaches it."""
    dev = vert_s.device
    T = N // 64
    vidx = torch.empty(Hq, N, dtype=torch.int32, device=dev)
    vcnt = torch.empty(Hq, dtype=torch.int32, device=dev)
    sidx = torch.empty(Hq, T, dtype=torch.int32, device=dev)
    scnt = torch.empty(Hq, dtype=torch.int32, device=dev)
    sws = torch.empty(vs.index_select_workspace_size(Hq, N), dtype=torch.uint8, device=dev)
    total_causal = Hq * N * (N + 1) // 2

    def run(budget, p, kv, ks):
        vs.vs_index_select_budget(vert_s, slash_s, Hq, N, budget, p, kv, ks, vidx, vcnt, sidx, scnt, sws, stream)

    def sparsity():
        torch.cuda.synchronize()
        m = vs.Mask(Hq, Hkv, lay, tile_cap=Hq * T * (int(scnt.max().item()) + 1))
        vs.vs_block_mask(vidx, vcnt, sidx, scnt, 0, 0, m, stream)
        torch.cuda.synchronize()
        arr = m.arrays()
        if int(arr["status"].item()) != 0:
            raise RuntimeError("mask status in budget report")
        return 1.0 - int(arr["n_active"].sum().item()) / total_causal

    def entry(budget, p, kv, ks):
        run(budget, p, kv, ks)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            run(budget, p, kv, ks)
        e1.record(stream)
        sp = sparsity()
        return {"select_ms": round(e0.elapsed_time(e1) / reps, 4), "mean_verticals": round(float(vcnt.float().mean()), 1),
                "mean_slashes": round(float(scnt.float().mean()), 1), "sparsity": round(sp, 5)}

    out = {"top_p": dict(entry(vs.VS_BUDGET_TOP_P, top_p, 0, 0), p=top_p)}
    mv, ms = out["top_p"]["mean_verticals"], out["top_p"]["mean_slashes"]
    lo, hi = 0.0, 4.0                               # scale of the counts; sparsity falls as it grows
    for _ in range(16):
        mid = 0.5 * (lo + hi)
        run(vs.VS_BUDGET_TOP_K, 0.0, max(1, round(mid * mv)), max(1, round(mid * ms)))
        if sparsity() >= target:
            lo = mid
        else:
            hi = mid
    kv, ks = max(1, round(lo * mv)), max(1, round(lo * ms))
    out["top_k"] = dict(entry(vs.VS_BUDGET_TOP_K, 0.0, kv, ks), k_vert=kv, k_slash=ks, target_sparsity=target)
    out["joint_top_p"] = dict(entry(vs.VS_BUDGET_JOINT_TOP_P, top_p, 0, 0), p=top_p)
    return out


def ring_report(args, cfg):
    """Ring simulation of one sequence at P ranks on one GPU.

    All shards stay resident in storage order (rank r's rows are rows
    r*N/P .. of the storage-order tensors). For each layout: the global index
    over the storage-order keys, then for every rank r and ring step s
    (source shard (r - s) mod P) the step's active region, the forward with
    the merge fused into its epilogue, and after the forward of all steps the
    backward of every step. Each (r, s) kernel group is timed alone with HIP
    events on the launch stream; reported times are medians over repetitions.
    Communication between ranks is not part of it (one GPU). With fp16
    operands every rank's q, k, v, dO shard is converted once before its ring
    (the shard a rank sends round the ring is then already fp16); that
    one-time conversion is timed over all shards at once and reported per
    rank (total / P) beside the steps.
    """
    import torch
    import dynamic_sparse_attention_index_amd as vs
    from synth import generate
    from synth.inputs import layout_permutation

    dev = torch.device("cuda:0")
    N, Hq, Hkv, D, P = cfg.N, cfg.Hq, cfg.Hkv, cfg.D, cfg.P
    T, QB = N // 64, N // 64 // P
    tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    t0 = time.time()
    host = generate(cfg)
    gen_s = time.time() - t0
    stream = torch.cuda.current_stream()

    def timed(fn):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        fn()
        b.record(stream)
        return a, b

    out = {"metric": f"ring simulation: one rank's sparse fwd+bwd ring steps, {N} tokens at P={P}, 1 MI355X",
           "unit": "ms", "workload": cfg.name, "Hq": Hq, "Hkv": Hkv, "seq_len": N, "P": P, "head_dim": D,
           "dtype": cfg.dtype, "data": "synthetic", "reps": args.ring_reps, "gen_s": round(gen_s, 1),
           "operands": args.operands if cfg.dtype == "bf16" and D == 128 else cfg.dtype,
           "bwd_streams": args.bwd_streams,
           "communication": "excluded (one GPU; every rank's steps run in turn)", "layouts": {}}
    def progress(msg):
        print(f"[ring {time.time() - t0:6.1f}s] {msg}", file=sys.stderr, flush=True)

    for kind in args.layouts.split(","):
        progress(f"{kind}: inputs")
        perm = np.concatenate([layout_permutation(kind, N, P, r) for r in range(P)])
        q = torch.tensor(host["q"][:, perm]).to(dev, tdt)
        k = torch.tensor(host["k"][:, perm]).to(dev, tdt)
        v = torch.tensor(host["v"][:, perm]).to(dev, tdt)
        do = torch.tensor(host["do"][:, perm]).to(dev, tdt)
        lay = vs.layout(kind, P, N)
        f16 = args.operands == "f16" and cfg.dtype == "bf16" and D == 128
        t_conv = None
        if f16:
            conv_status = torch.zeros(1, dtype=torch.int32, device=dev)
            aq, ak, av, ado = (torch.empty(x.shape, dtype=torch.float16, device=dev) for x in (q, k, v, do))
            # all P shards at once (bandwidth-bound, linear in size): per rank = total / P
            qc, kc, vc, doc = (x.contiguous() for x in (q, k, v, do))
            t_conv = []
            for rep in range(-1, args.ring_reps):
                e = timed(lambda: [vs.vs_convert_f16(x, y, conv_status, stream)
                                   for x, y in ((qc, aq), (kc, ak), (vc, av), (doc, ado))])
                torch.cuda.synchronize()
                if rep >= 0:
                    t_conv.append(e[0].elapsed_time(e[1]) / P)
            if int(conv_status.item()) != 0:
                raise RuntimeError("an input is outside the fp16 range: run with --operands bf16")
            del qc, kc, vc, doc
        else:
            aq, ak, av, ado = q, k, v, do
        # global index over the storage-order keys; the last rows are global
        # rows N - last_q .. N - 1, wherever they are stored. One-position
        # stripes: the index takes the keys in global order (the lists are
        # global either way), and the per-rank passes are not offered.
        last_rows = np.nonzero(np.isin(perm, np.arange(N - cfg.last_q, N)))[0]
        order = np.argsort(perm[last_rows])
        q_last = q[:, torch.tensor(last_rows[order], device=dev)].contiguous()
        s1 = kind == "striped1"
        idx_lay, k_idx = lay, k
        if s1:
            idx_lay = vs.layout("contig", 1, N)
            k_idx = torch.tensor(host["k"]).to(dev, tdt)
        vert_s = torch.empty(Hq, N, device=dev)
        slash_s = torch.empty(Hq, T, device=dev)
        vidx = torch.empty(Hq, N, dtype=torch.int32, device=dev)
        vcnt = torch.empty(Hq, dtype=torch.int32, device=dev)
        sidx = torch.empty(Hq, T, dtype=torch.int32, device=dev)
        scnt = torch.empty(Hq, dtype=torch.int32, device=dev)
        ws = torch.empty(vs.index_workspace_size(Hq, Hkv, N, D), dtype=torch.uint8, device=dev)

        def index():
            vs.vs_index_build(q_last, k_idx, idx_lay, cfg.scale, cfg.top_p, vert_s, slash_s, vidx, vcnt, sidx, scnt,
                              ws, stream)
        index()
        torch.cuda.synchronize()
        t_index = []
        for _ in range(args.ring_reps):
            ev = timed(index)
            torch.cuda.synchronize()
            t_index.append(ev[0].elapsed_time(ev[1]))
        # the same index built the distributed way: every rank's two passes on
        # its own shard (a slice of the storage order), the gathered (max, sum)
        # slots between them, then the selection (exchanges excluded)
        all_stats = torch.empty(P, Hq, 64, 2, device=dev)
        vert_d, slash_d = torch.empty_like(vert_s), torch.empty_like(slash_s)
        vidx_d, vcnt_d = torch.empty_like(vidx), torch.empty_like(vcnt)
        sidx_d, scnt_d = torch.empty_like(sidx), torch.empty_like(scnt)
        nl = N // P
        sws = torch.empty(vs.index_select_workspace_size(Hq, N), dtype=torch.uint8, device=dev)
        t_d1, t_d2, t_d3 = [], [], []
        for rep in range(-1, 0 if s1 else args.ring_reps):
            if s1:
                break
            e1 = [timed(lambda: vs.vs_index_rank_stats(q_last, k[:, r * nl:(r + 1) * nl], lay, r, cfg.scale,
                                                       all_stats[r], ws, stream)) for r in range(P)]
            e2 = [timed(lambda: vs.vs_index_rank_mass(q_last, k[:, r * nl:(r + 1) * nl], lay, r, cfg.scale,
                                                      all_stats, vert_d, slash_d, ws, stream)) for r in range(P)]
            e3 = timed(lambda: vs.vs_index_select(vert_d, slash_d, Hq, N, cfg.top_p, vidx_d, vcnt_d, sidx_d,
                                                  scnt_d, sws, stream))
            torch.cuda.synchronize()
            if rep >= 0:
                t_d1.append(max(a.elapsed_time(b) for a, b in e1))
                t_d2.append(max(a.elapsed_time(b) for a, b in e2))
                t_d3.append(e3[0].elapsed_time(e3[1]))
        same_sel = bool(torch.equal(vcnt_d, vcnt) and torch.equal(scnt_d, scnt)) if not s1 else None
        if same_sel:
            for h in range(Hq):
                same_sel = same_sel and torch.equal(vidx_d[h, :int(vcnt[h])], vidx[h, :int(vcnt[h])]) and \
                    torch.equal(sidx_d[h, :int(scnt[h])], sidx[h, :int(scnt[h])])
        score_rel = None if s1 else float(((vert_d - vert_s).abs() / vert_s.abs().clamp_min(1e-30)).max().item())
        # tiles per query block: one per selected diagonal, two under one-position stripes
        cap = Hq * QB * ((2 if s1 else 1) * int(scnt.max().item()) + 1)
        t_mask = np.zeros((args.ring_reps, P, P))
        t_fwd = np.zeros((args.ring_reps, P, P))
        t_bwd = np.zeros((args.ring_reps, P, P))
        t_prep = np.zeros((args.ring_reps, P))
        act = np.zeros((P, P), dtype=np.int64)
        computed = np.zeros((P, P), dtype=np.int64)   # entries the forward computes (whole 64x64 tiles)
        o = torch.empty(Hq, QB * 64, D, device=dev)
        lse = torch.empty(Hq, QB * 64, device=dev)
        delta = torch.empty(Hq, QB * 64, device=dev)
        dq = torch.empty(Hq, QB * 64, D, device=dev)
        dk = torch.zeros(P, Hkv, QB * 64, D, device=dev)   # per source shard
        dv = torch.zeros(P, Hkv, QB * 64, D, device=dev)
        side = torch.cuda.Stream(device=dev) if args.bwd_streams == 2 else None   # default priority

        def bwd_step(qr, kc, vc, dor, m, dks, dvs):
            """One step's backward: one launch sequence, or with two streams dQ on
            the side stream concurrently with the dK/dV parts (the step's end
            event on the launch stream waits for both)."""
            if side is None:
                vs.vs_attn_bwd(qr, kc, vc, dor, lse, delta, m, cfg.scale, dq, dks, dvs, stream)
                return
            fork, join = torch.cuda.Event(), torch.cuda.Event()
            fork.record(stream)
            side.wait_event(fork)
            vs.vs_attn_bwd_parts(qr, kc, vc, dor, lse, delta, m, cfg.scale, dq, dks, dvs, vs.VS_BWD_DQ, side)
            join.record(side)
            vs.vs_attn_bwd_parts(qr, kc, vc, dor, lse, delta, m, cfg.scale, dq, dks, dvs,
                                 vs.VS_BWD_DKDV | vs.VS_BWD_DKDV_VERT, stream)
            stream.wait_event(join)

        for rep in range(-1, args.ring_reps):       # rep -1: warm-up
            progress(f"{kind}: per-step mode, repetition {rep + 1} of {args.ring_reps} (first: warm-up)")
            dk.zero_()
            dv.zero_()
            for r in range(P):
                rows = slice(r * QB * 64, (r + 1) * QB * 64)
                qr, dor = aq[:, rows], ado[:, rows]
                o.zero_()
                lse.fill_(-math.inf)
                dq.zero_()
                masks, evs = [], []
                for st in range(P):
                    src = (r - st) % P
                    cols = slice(src * QB * 64, (src + 1) * QB * 64)
                    m = vs.Mask(Hq, Hkv, lay, cap)
                    e_m = timed(lambda: vs.vs_block_mask(vidx, vcnt, sidx, scnt, r, st, m, stream))
                    e_f = timed(lambda: vs.vs_attn_fwd(qr, ak[:, cols], av[:, cols], m, cfg.scale, o, lse, 1, stream))
                    masks.append(m)
                    evs.append((e_m, e_f))
                e_p = timed(lambda: vs.vs_attn_bwd_prep(o, dor, delta, stream))
                ebs = []
                for st in range(P):
                    src = (r - st) % P
                    cols = slice(src * QB * 64, (src + 1) * QB * 64)
                    ebs.append(timed(lambda: bwd_step(qr, ak[:, cols], av[:, cols], dor, masks[st], dk[src],
                                                      dv[src])))
                torch.cuda.synchronize()
                if rep >= 0:
                    t_prep[rep, r] = e_p[0].elapsed_time(e_p[1])
                    for st in range(P):
                        (a, b), (c, d) = evs[st]
                        t_mask[rep, r, st] = a.elapsed_time(b)
                        t_fwd[rep, r, st] = c.elapsed_time(d)
                        t_bwd[rep, r, st] = ebs[st][0].elapsed_time(ebs[st][1])
                else:
                    for st, m in enumerate(masks):
                        arr = m.arrays()
                        if int(arr["status"].item()) != 0:
                            raise RuntimeError(f"mask status {int(arr['status'].item())} at rank {r} step {st}")
                        act[r, st] = int(arr["n_active"].sum().item())
                        chunks = int(((arr["vert_end"].long() + 63) // 64).sum().item())
                        computed[r, st] = 4096 * (int(arr["tile_ptr"][-1].item()) + chunks)
                del masks
        tm, tf, tb = (np.median(x, axis=0) for x in (t_mask, t_fwd, t_bwd))
        tp = np.median(t_prep, axis=0)                 # per rank, once per ring
        t = tf + tb                                    # attention time of step s on rank r
        mean_r = t.mean(axis=0)
        max_r = t.max(axis=0)
        cmean, cmax = act.mean(axis=0), act.max(axis=0)
        ring_ms = float(max_r.sum())                   # the ring waits for the slowest rank each step
        # the whole ring of a rank: every step's active region, forward and
        # backward (slowest rank per step) plus the rank's one delta pass
        tall = tm + tf + tb
        ring_all_ms = float(tall.max(axis=0).sum() + tp.max())
        A_total = int(act.sum())
        # resident mode: a rank's masks of every step built up front (one
        # launch sequence for all steps, vs_block_mask_ring), then the
        # forward of all its steps in one launch (the online softmax carried
        # across the steps in the kernel: no per-step merge) and the backward
        # of all its steps in one call; k/v hold every shard in storage order
        # (not offered under one-position stripes)
        res_masks = [vs.Mask(Hq, Hkv, lay, cap) for _ in range(P)]
        dk_res = torch.empty(Hkv, N, D, device=dev)
        dv_res = torch.empty(Hkv, N, D, device=dev)
        t_res = np.zeros((args.ring_reps, P, 4))      # mask, fwd, prep, bwd per rank
        for rep in range(-1, -1 if s1 else args.ring_reps):
            progress(f"{kind}: resident mode, repetition {rep + 1} of {args.ring_reps} (first: warm-up)")
            for r in range(P):
                rows = slice(r * QB * 64, (r + 1) * QB * 64)
                qr, dor = aq[:, rows], ado[:, rows]
                e_m = timed(lambda: vs.vs_block_mask_ring(vidx, vcnt, sidx, scnt, r, res_masks, stream))
                e_f = timed(lambda: vs.vs_attn_fwd_ring(qr, ak, av, res_masks, cfg.scale, o, lse, 0, stream))
                e_p = timed(lambda: vs.vs_attn_bwd_prep(o, dor, delta, stream))
                e_b = timed(lambda: vs.vs_attn_bwd_ring(qr, ak, av, dor, lse, delta, res_masks, cfg.scale, dq, dk_res,
                                                        dv_res, vs.VS_BWD_ALL | vs.VS_BWD_OVERWRITE, stream))
                torch.cuda.synchronize()
                if rep >= 0:
                    for i, (a_, b_) in enumerate((e_m, e_f, e_p, e_b)):
                        t_res[rep, r, i] = a_.elapsed_time(b_)
        tr = np.median(t_res, axis=0)                 # [rank, part]
        rank_ms = np.maximum(tr.sum(axis=1), 1e-9)
        res_ms = float(rank_ms.max())
        A_rank = act.sum(axis=1)
        r3 = (lambda x: None) if s1 else (lambda x: round(x, 3))
        r2 = (lambda x: None) if s1 else (lambda x: round(x, 2))
        del res_masks, dk_res, dv_res
        # merge: separate kernel vs fused into the forward, rank 0's steps
        o_step = torch.empty_like(o)
        l_step = torch.empty_like(lse)
        fused, split = [], []
        r = 0
        qr = aq[:, 0:QB * 64]
        for st in range(P):
            src = (r - st) % P
            cols = slice(src * QB * 64, (src + 1) * QB * 64)
            m = vs.Mask(Hq, Hkv, lay, cap)
            vs.vs_block_mask(vidx, vcnt, sidx, scnt, r, st, m, stream)
            ef = timed(lambda: vs.vs_attn_fwd(qr, ak[:, cols], av[:, cols], m, cfg.scale, o, lse, 1, stream))
            es1 = timed(lambda: vs.vs_attn_fwd(qr, ak[:, cols], av[:, cols], m, cfg.scale, o_step, l_step, 0, stream))
            es2 = timed(lambda: vs.vs_merge_lse(o, lse, o_step, l_step, stream))
            torch.cuda.synchronize()
            fused.append(ef[0].elapsed_time(ef[1]))
            split.append(es1[0].elapsed_time(es1[1]) + es2[0].elapsed_time(es2[1]))
            del m
        out["layouts"][kind] = {
            "index_ms": round(float(np.median(t_index)), 4),
            "convert_f16_ms_per_rank": round(float(np.median(t_conv)), 4) if t_conv else None,
            "index_distributed_pass1_ms_max_rank": round(float(np.median(t_d1)), 4) if t_d1 else None,
            "index_distributed_pass2_ms_max_rank": round(float(np.median(t_d2)), 4) if t_d2 else None,
            "index_distributed_select_ms": round(float(np.median(t_d3)), 4) if t_d3 else None,
            "index_distributed_exchange_bytes": None if s1 else P * Hq * 64 * 2 * 4 + Hq * (N + T) * 4,
            "index_distributed_same_selection": same_sel,
            "index_distributed_max_rel_score_diff": None if s1 else float(f"{score_rel:.3e}"),
            "mask_ms_per_step_mean": round(float(tm.mean()), 4),
            "fwd_ms_per_step_mean": round(float(tf.mean()), 4),
            "bwd_ms_per_step_mean": round(float(tb.mean()), 4),
            "step_time_imbalance_mean": round(float((max_r / mean_r).mean()), 4),
            "step_time_imbalance_max": round(float((max_r / mean_r).max()), 4),
            "step_count_imbalance_mean": round(float((cmax / np.maximum(cmean, 1)).mean()), 4),
            "step_count_imbalance_max": round(float((cmax / np.maximum(cmean, 1)).max()), 4),
            "ring_time_imbalance": round(float(max_r.sum() / mean_r.sum()), 4),
            "worker_total_imbalance": round(float(t.sum(axis=1).max() / t.sum(axis=1).mean()), 4),
            "ring_ms_fwd_bwd": round(ring_ms, 3),
            "ring_ms_with_mask_and_prep": round(ring_all_ms, 3),
            "bwd_prep_ms_per_rank": round(float(tp.mean()), 4),
            "per_gpu_tokens_per_s": round((N / P) / (ring_all_ms * 1e-3), 1),
            "per_gpu_effective_tflops": round(14 * D * A_total / P / (ring_all_ms * 1e-3) / 1e12, 2),
            "per_gpu_effective_tflops_attention_only": round(14 * D * A_total / P / (ring_ms * 1e-3) / 1e12, 2),
            "active_entries": A_total,
            "tile_fill_fwd": round(A_total / max(int(computed.sum()), 1), 4),
            "merge_fused_ms_per_step": round(float(np.mean(fused)), 4),
            "merge_separate_ms_per_step": round(float(np.mean(split)), 4),
            "resident_ring_ms_max_rank": r3(res_ms),
            "resident_parts_ms_max_rank": None if s1 else
            {k_: round(float(tr[int(np.argmax(rank_ms)), i]), 3)
             for i, k_ in enumerate(("masks", "fwd", "bwd_prep", "bwd"))},
            "resident_rank_imbalance": None if s1 else round(float(rank_ms.max() / rank_ms.mean()), 4),
            "resident_per_gpu_tokens_per_s": None if s1 else round((N / P) / (res_ms * 1e-3), 1),
            "resident_per_gpu_effective_tflops": r2(14 * D * float(A_rank[int(np.argmax(rank_ms))]) /
                                                    (res_ms * 1e-3) / 1e12),
            "resident_effective_tflops_mean_rank": r2(float(np.mean(14 * D * A_rank / (rank_ms * 1e-3) / 1e12))),
        }
        del q, k, v, do, dk, dv, aq, ak, av, ado, k_idx
        torch.cuda.empty_cache()
    print(json.dumps(out), flush=True)
    if args.report_md:
        with open(args.report_md, "w") as f:
            f.write(f"# Ring simulation report: {cfg.name} ({N} tokens, P = {P}, {Hq}/{Hkv} heads, d {D}, "
                    f"{cfg.dtype})\n\n")
            f.write("Command (repository root, one MI355X): `python bench.py --workload " + cfg.name +
                    f" --layouts {args.layouts} --ring-reps {args.ring_reps}"
                    f" --report-md <path>`\n\n")
            f.write("Every rank's ring steps run one after another on the one GPU (communication excluded); "
                    "times are medians over repetitions of each (rank, step) kernel group timed alone. "
                    "Per-step mode: one active-region build, one forward (merge fused) and one backward call per "
                    "step. Resident mode (`resident_*`): a rank's masks of all steps built up front by one launch "
                    "sequence (vs_block_mask_ring), then one "
                    "forward launch over all its steps (vs_attn_fwd_ring: the online softmax carried across the "
                    "steps, O written once) and one backward call (vs_attn_bwd_ring: dQ accumulated across the "
                    "steps, the key-major parts over every step's shard in one grid); its time per rank is "
                    "masks + forward + delta + backward. Under one-position stripes (`striped1`: rank r holds "
                    "the positions n with n mod P = r) the index is built on the keys in global order, the "
                    "per-rank index passes and the resident mode are not offered (empty cells), and "
                    "`tile_fill_fwd` (active entries / entries of the listed tiles and vertical chunks the "
                    "forward computes) shows how thin a selected diagonal becomes inside a local tile.\n\n")
            keys = list(next(iter(out["layouts"].values())).keys())
            f.write("| quantity | " + " | ".join(out["layouts"]) + " |\n|---|" + "---|" * len(out["layouts"]) + "\n")
            for kk in keys:
                f.write(f"| {kk} | " + " | ".join("—" if out["layouts"][L][kk] is None else str(out["layouts"][L][kk])
                                                  for L in out["layouts"]) + " |\n")


def stored_traffic(kernel):
    """L2-to-fabric bytes per launch of `kernel` (HBM traffic plus Infinity
    Cache hits) from the committed counter summary (profiles/counters.json:
    FETCH_SIZE and WRITE_SIZE runs scaled by the same counters' reading for a
    copy of known size), or None when absent or
    when the kernel's source file or the shared kernel headers have changed
    since the counters were taken (one SHA-256 over all of them)."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "counters.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path)).get(kernel)
    if not rec:
        return None
    h = hashlib.sha256()
    for rel in [rec["source"]] + rec.get("headers", []):
        path = os.path.join(ROOT, rel)
        if not os.path.exists(path):
            return None
        h.update(open(path, "rb").read())
    if h.hexdigest() != rec["source_sha256"]:
        return None
    return int(rec["l2_miss_bytes_per_launch"])


def copy_probe():
    """A plain device copy of known size, for scaling the HBM byte counters."""
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_read": n, "copy_probe_bytes_written": n, "launches": 3}))


def cpu_baseline(cfg, host, vidx, vcnt, sidx, scnt, seconds, tflops_unit=True):
    """Time the fp64 oracle on the host cores on the same workload.

    Index: the oracle's index step over every q head, in full. Active region:
    the oracle's per-block description (tile list, vertical prefix, active
    count) of a seeded sample of (head, query block) items, extrapolated by
    item count. Attention: forward (+ backward) of random (head, 64-row block)
    items for about `seconds`, extrapolated linearly in active entries. The
    attention sample runs again with BLAS limited to one thread (a third of
    the time budget) for a single-thread figure.
    """
    import torch  # noqa: F401  (for .cpu())
    from threadpoolctl import threadpool_info, threadpool_limits
    from oracle import index as oi
    from oracle import attention as oa
    from oracle import mask as om

    N, Hq, Hkv, D = cfg.N, cfg.Hq, cfg.Hkv, cfg.D
    cores = len(os.sched_getaffinity(0))
    blas = [x for x in threadpool_info() if x.get("user_api") == "blas"]
    blas_threads = max((int(x["num_threads"]) for x in blas), default=None)
    vc, sc = vcnt.cpu().numpy(), scnt.cpu().numpy()
    vert = [vidx[h, :vc[h]].cpu().numpy().astype(np.int64) for h in range(Hq)]
    slash = [sidx[h, :sc[h]].cpu().numpy().astype(np.int64) for h in range(Hq)]
    QB = N // 64
    # index, every head
    t0 = time.perf_counter()
    oi.build_index(host["q"][:, N - cfg.last_q:], host["k"], cfg.scale, N, cfg.top_p)
    t_index = time.perf_counter() - t0
    # active region, sampled blocks
    rng = np.random.default_rng(1)
    n_mask = 0
    t_mask = 0.0
    while t_mask < seconds / 6 and n_mask < 256:
        h, I = int(rng.integers(Hq)), int(rng.integers(QB))
        t0 = time.perf_counter()
        om.step_description("contig", N, 1, 0, 0, vert, slash, heads=[h], blocks=[I])
        t_mask += time.perf_counter() - t0
        n_mask += 1
    t_mask_full = t_mask * Hq * QB / max(n_mask, 1)
    pos = np.arange(N)

    def attn_sample(budget, seed):
        rng = np.random.default_rng(seed)
        done_active, t_attn, items = 0, 0.0, 0
        while t_attn < budget and items < 4096:
            h = int(rng.integers(Hq))
            I = int(rng.integers(QB))
            g = h * Hkv // Hq
            rows = pos[64 * I:64 * I + 64]
            t0 = time.perf_counter()
            M, _, _ = om.active(rows, pos, vert[h], slash[h])
            used = M.any(axis=0)
            kk, vv = host["k"][g, used], host["v"][g, used]
            oa.forward_rows(host["q"][h, rows], kk, vv, M[:, used], cfg.scale)
            if cfg.backward:
                oa.backward_rows(host["q"][h, rows], kk, vv, M[:, used], cfg.scale, host["do"][h, rows])
            t_attn += time.perf_counter() - t0
            done_active += int(M.sum())
            items += 1
        return t_attn, done_active, items

    A_total = sum(om.active_count(N, vert[h], slash[h]) for h in range(Hq))
    t_attn, done_active, items = attn_sample(seconds, 0)
    t_attn_full = t_attn * A_total / max(done_active, 1)
    with threadpool_limits(1):
        t1, done1, items1 = attn_sample(seconds / 3, 2)
        t0 = time.perf_counter()
        oi.build_index(host["q"][:1, N - cfg.last_q:], host["k"][:1], cfg.scale, N, cfg.top_p)
        t_index1 = (time.perf_counter() - t0) * Hq
    t_attn1_full = t1 * A_total / max(done1, 1)
    t_total = t_index + t_mask_full + t_attn_full
    t_total1 = t_index1 + t_mask_full + t_attn1_full
    eff = (4 + (10 if cfg.backward else 0)) * D * A_total
    return {"value": round(eff / t_total / 1e12, 6), "unit": "TFLOP/s", "cores": cores,
            "blas_threads": blas_threads, "kind": "oracle",
            "tokens_per_s": round(N / t_total, 3),
            "stage_s": {"index": round(t_index, 2), "mask_extrapolated": round(t_mask_full, 1),
                        "attention_extrapolated": round(t_attn_full, 1)},
            "seconds_measured": round(t_index + t_mask + t_attn + t1 + t_index1 / Hq, 1),
            "single_thread": {"value": round(eff / t_total1 / 1e12, 6), "unit": "TFLOP/s", "blas_threads": 1,
                              "stage_s": {"index_extrapolated": round(t_index1, 2),
                                          "attention_extrapolated": round(t_attn1_full, 1)},
                              "sample": f"index step of 1 of {Hq} q heads (x{Hq}); fwd+bwd of {items1} random "
                                        f"items = {done1} active entries, extrapolated; the active-region "
                                        f"time of the threaded run"},
            "sample": f"index step of all {Hq} q heads in full; active-region description of {n_mask} random "
                      f"(head, 64-row block) items of {Hq * QB}, extrapolated by item count; fwd+bwd of {items} "
                      f"random (head, block) items = {done_active} of {A_total} active entries, extrapolated "
                      f"linearly in active entries; numpy fp64, BLAS threads {blas_threads}"}


if __name__ == "__main__":
    main()
