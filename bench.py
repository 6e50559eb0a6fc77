"""Benchmark of the MoE layer of a prefill step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c3_dsv3_bf16]

One step is one moe_layer call -- router GEMM + group-limited top-k, dispatch,
grouped SwiGLU FFN (bf16 MFMA, shared expert included), combine -- over one
batch of synthetic inputs already resident in HBM.  The default workload is the
DeepSeek-V3-shaped prefill layer: T=8192 tokens, H=7168, 256 routed experts
(top-8, sigmoid, 8 groups keep 4, renormalised x2.5) + 1 shared expert, SwiGLU
intermediate 2048, bf16 weights and activations, fp32 accumulation, bf16
output.  Inputs follow the workload's distributions (activations N(0,1),
weights N(0, 1/fan_in)) from the seeded counter-based generator.

Prints one JSON line: value = layer TFLOP/s (algorithmic: 6*H*I per routed
(token, expert) pair and per token for the shared expert, plus 2*T*H*E for the
router), tokens/s, the fraction of the bf16 dense MFMA peak, a per-stage
breakdown timed with HIP events on the launch stream, the roofline of the
dominant stage (the grouped FFN: bound by whichever of flop / MFMA peak and
algorithmic bytes / HBM peak takes longer, both fractions reported), and the
oracle's CPU throughput on a bounded sample of the same arithmetic.

--workload c5_dsv3_ep_fp8 times the fp8 grouped FFN alone on one GPU's
expert-parallel share (65536 dispatched rows over 8 local experts, e4m3 with
block scales): a step is one moe_grouped_ffn call, against the fp8 peak.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_FP8_TFLOPS = 5000.0   # MI355X dense fp8 (e4m3) MFMA
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E
METRIC = "MoE-layer TFLOP/s + tokens/s (1 GPU, DSV3 prefill shape); % of MFMA peak"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_grouped_ffn_c3_dsv3_bf16.json")
FFN_SOURCES = [os.path.join(ROOT, "expert_layer_amd", "csrc", f) for f in ("gemm_bf16.hip", "common.hpp")]


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default="c3_dsv3_bf16")
    p.add_argument("--fp8-experts", action="store_true",
                   help="a bf16 layer workload with e4m3 experts (128x128 block scales): moe_layer quantises the "
                        "activations per token inside the router's pass over x and runs the experts in fp8")
    p.add_argument("--tokens", type=int, default=0,
                   help="override the workload's token count T (the small-T, weight-streaming regime)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-extra", action="store_true",
                   help="the default run also times the c4 (skewed routing) layer and the c5 fp8 grouped FFN as "
                        "extra keys of its line; this leaves them out")
    p.add_argument("--rowmajor-weights", action="store_true",
                   help="time the row-major weight layout instead of the tiled one")
    p.add_argument("--fp4-weights", action="store_true",
                   help="with the fp8 FFN workload or --fp8-experts: MXFP4 expert weights (E2M1, E8M0 per 32) "
                        "instead of e4m3 ones")
    p.add_argument("--weight-table", type=int, default=0, metavar="N",
                   help="read the expert weights through a device pointer table of N layers (the N layers' "
                        "tables point at the one weight set, each in its own expert order) and run the steps "
                        "over the layers in turn")
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU time of the oracle sample")
    p.add_argument("--traffic-run", action="store_true",
                   help="the program to run under rocprofv3 --pmc: CAL_RUNS plain streaming kernels (torch.neg "
                        "over CAL_BYTES of fp32, as many bytes written) to scale the counters, then warmup + steps "
                        "passes of the stage calls on the workload's routing, with the expert weights drawn by "
                        "torch.randn (their values do not change which bytes the kernels move; a few hundred "
                        "dispatches in all); with --fp8-experts, warmup + steps moe_route_quantize calls (the route "
                        "with the per-token quantisation of x) on the workload's router inputs instead; prints no "
                        "JSON line")
    p.add_argument("--no-clock", action="store_true", help="accepted for older command lines; does nothing")
    p.add_argument("--pmc-summary", nargs="+", metavar="DB",
                   help="no GPU: print, per kernel, the per-dispatch average of every counter in these rocprofv3 "
                        "--pmc result databases (a markdown table), and exit")
    p.add_argument("--clock-from", nargs=2, metavar=("SQ_DB", "KT_STATS_CSV"),
                   help="no GPU: from a --pmc run with GRBM_GUI_ACTIVE and SQ_VALU_MFMA_BUSY_CYCLES of a --traffic-run "
                        "and the kernel_stats.csv of a --kernel-trace --stats run, write the grouped FFN kernels' "
                        "clock under load and MFMA utilisation to the clock file, exit")
    p.add_argument("--traffic-from", nargs=2, metavar=("FETCH_DB", "WRITE_DB"),
                   help="no GPU: read two rocprofv3 --pmc result databases of a --traffic-run (FETCH_SIZE, then "
                        "WRITE_SIZE), write the grouped FFN's HBM bytes per launch to the traffic file, exit")
    return p.parse_args()


CAL_BYTES = 1 << 30
CAL_RUNS = 3
# the grouped FFN's kernels, as name prefixes (GEMM1 has a streamed-weights instance)
FFN_KERNELS = ("ffn_build_tiles", "ffn_gemm_bf16<0", "ffn_gemm_bf16<1")


def calibrate_copy(dev):
    import torch
    a = torch.ones(CAL_BYTES // 4, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(CAL_RUNS):
        torch.neg(a, out=b)
    torch.cuda.synchronize()
    del a, b
    torch.cuda.empty_cache()


def _pmc_per_dispatch(db, counter):
    """{dispatch_id: (kernel_name, value)} of one counter in a rocprofv3 results database."""
    import sqlite3
    con = sqlite3.connect(db)
    out = {}
    for name, cname, val, disp in con.execute(
            "select kernel_name, counter_name, value, dispatch_id from counters_collection"):
        if cname != counter:
            continue
        n, v = out.get(disp, (name, 0.0))
        out[disp] = (n, v + float(val))
    con.close()
    return out


def traffic_from(fetch_db, write_db, workload):
    """HBM bytes per moe_grouped_ffn launch: FETCH_SIZE and WRITE_SIZE (KiB per
    dispatch) summed over the launch's three kernels, each scaled so that the
    calibration kernel reads and writes exactly CAL_BYTES."""
    res = {"workload": workload, "source_hash": ffn_source_hash()}
    total = 0.0
    for key, db, counter in (("fetch", fetch_db, "FETCH_SIZE"), ("write", write_db, "WRITE_SIZE")):
        d = _pmc_per_dispatch(db, counter)
        cal = [v for n, v in d.values() if "neg_kernel" in n]
        if len(cal) < 1:
            raise SystemExit(f"{db}: no calibration dispatch (profile bench.py --traffic-run)")
        cal_kib = sum(cal) / len(cal)
        scale = CAL_BYTES / (cal_kib * 1024.0)
        per = {k: [v for n, v in d.values() if k in n] for k in FFN_KERNELS}
        launches = len(per["ffn_build_tiles"])
        if launches == 0 or any(len(v) != launches for v in per.values()):
            raise SystemExit(f"{db}: FFN dispatch counts differ: { {k: len(v) for k, v in per.items()} }")
        b = {k: sum(v) / launches * 1024.0 * scale for k, v in per.items()}
        res[f"{key}_calibration_kib"] = cal_kib
        res[f"{key}_scale"] = scale
        res[f"{key}_bytes_per_launch"] = sum(b.values())
        res[f"{key}_bytes_per_kernel"] = b
        res[f"{key}_launches"] = launches
        total += sum(b.values())
    res["hbm_bytes_per_launch"] = total
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(res, f, indent=1)
    print(json.dumps(res))


def _short(name):
    """A kernel's name without its return type, namespaces and arguments."""
    n = name.replace("void ", "").replace("(anonymous namespace)::", "").replace("moe::", "")
    return n.split("(")[0].strip()


def _pmc_dispatches(db):
    """{dispatch_id: (kernel name, {counter: [value per instance]})} of a
    rocprofv3 --pmc results database."""
    import sqlite3
    con = sqlite3.connect(db)
    out = {}
    for name, cname, val, disp in con.execute(
            "select kernel_name, counter_name, value, dispatch_id from counters_collection"):
        out.setdefault(disp, (name, {}))[1].setdefault(cname, []).append(float(val))
    con.close()
    return out


def pmc_summary(dbs):
    """Per kernel and counter: the value of a dispatch (summed over the
    counter's instances), averaged over the kernel's dispatches, from
    rocprofv3 --pmc databases."""
    rows = {}
    for db in dbs:
        for name, cs in _pmc_dispatches(db).values():
            for c, v in cs.items():
                rows.setdefault((_short(name), c), []).append(sum(v))
    counters = sorted({c for _, c in rows})
    kernels = sorted({k for k, _ in rows})
    print("| kernel | dispatches | " + " | ".join(counters) + " |")
    print("|---|---:|" + "---:|" * len(counters))
    for k in kernels:
        n = max(len(rows.get((k, c), [])) for c in counters)
        vals = []
        for c in counters:
            v = rows.get((k, c))
            vals.append(f"{sum(v) / len(v):.6g}" if v else "")
        print(f"| {k} | {n} | " + " | ".join(vals) + " |")


SIMDS = 1024  # MI355X: 256 CUs x 4 SIMDs
XCDS = 8      # GRBM_GUI_ACTIVE has one instance per XCD; the database holds their sum
CLOCK_FILE = os.path.join(ROOT, "profiles", "clock_grouped_ffn_c3_dsv3_bf16.json")


def clock_from(sq_db, kt_stats_csv, workload):
    """The GPU clock under the grouped FFN's load and its MFMA utilisation:
    per kernel, GRBM_GUI_ACTIVE (busy cycles, summed over the 8 XCDs, so / 8
    per XCD) over the kernel's average duration from a --kernel-trace --stats run of
    the same build on the same box, and SQ_VALU_MFMA_BUSY_CYCLES over those
    cycles times the SIMD count.  Written to the clock file with the FFN
    sources' hash."""
    import csv
    disp = _pmc_dispatches(sq_db)
    dur = {}
    for r in csv.DictReader(open(kt_stats_csv)):
        dur[_short(r["Name"])] = float(r["AverageNs"]) * 1e-9
    res = {"workload": workload, "source_hash": ffn_source_hash(), "kernels": {}}
    names = sorted({_short(n) for n, _ in disp.values() if _short(n).startswith(FFN_KERNELS[1:])})
    for k in names:
        grbm = [sum(cs["GRBM_GUI_ACTIVE"]) / XCDS for n, cs in disp.values()
                if _short(n) == k and "GRBM_GUI_ACTIVE" in cs]
        busy = [sum(cs["SQ_VALU_MFMA_BUSY_CYCLES"]) for n, cs in disp.values()
                if _short(n) == k and "SQ_VALU_MFMA_BUSY_CYCLES" in cs]
        if not grbm or k not in dur:
            raise SystemExit(f"no GRBM_GUI_ACTIVE or duration for {k}")
        cyc = sum(grbm) / len(grbm)
        e = {"grbm_cycles": cyc, "avg_s": dur[k], "clock_ghz": round(cyc / dur[k] / 1e9, 3)}
        if busy:
            e["mfma_busy_frac"] = round(sum(busy) / len(busy) / (cyc * SIMDS), 4)
        res["kernels"][k] = e
    os.makedirs(os.path.dirname(CLOCK_FILE), exist_ok=True)
    with open(CLOCK_FILE, "w") as f:
        json.dump(res, f, indent=1)
    print(json.dumps(res))


def ffn_source_hash() -> str:
    h = hashlib.sha256()
    for f in FFN_SOURCES:
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def main():
    a = parse()
    if a.traffic_from:
        traffic_from(*a.traffic_from, a.workload)
        return
    if a.pmc_summary:
        pmc_summary(a.pmc_summary)
        return
    if a.clock_from:
        clock_from(*a.clock_from, a.workload)
        return
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import expert_layer_amd as moe
    import synth

    dev = torch.device("cuda:0")
    if a.traffic_run:
        calibrate_copy(dev)
    s = synth.config(a.workload, **({"T": a.tokens} if a.tokens else {}))
    if s.dtype == "fp8":
        res = bench_fp8_ffn(a, s, dev)
    elif a.fp8_experts:
        res = bench_fp8_layer(a, s, dev)
    elif s.dtype != "bf16":
        raise SystemExit("bench.py times the bf16 layers (c2/c3/c4) and the fp8 grouped FFN (c5)")
    else:
        res = bench_bf16_layer(a, s, dev)
    if res is None:  # a traffic run prints no line
        return
    default_run = (a.workload == "c3_dsv3_bf16" and not a.tokens and not a.fp8_experts and not a.weight_table
                   and not a.rowmajor_weights and not a.no_extra)
    if default_run:
        # the skewed-routing layer and the fp8 expert-parallel share, timed the
        # same way in the same run (their own keys; `value` stays the c3 layer)
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        extra = {}
        for name in ("c4_qwen3_skew_bf16", "c5_dsv3_ep_fp8"):
            se = synth.config(name)
            r = bench_fp8_ffn(a, se, dev) if se.dtype == "fp8" else bench_bf16_layer(a, se, dev, extra=True)
            extra[name] = summary(r)
            torch.cuda.synchronize()
            torch.cuda.empty_cache()
        res["extra_workloads"] = extra
    print(json.dumps(res), flush=True)


def summary(r):
    """The figures of another workload's line that ride along the main one."""
    keep = ("metric", "value", "unit", "ms_per_step", "dtype", "config", "tokens_per_s", "stages")
    out = {k: r[k] for k in keep if k in r}
    rf = r["roofline"]
    out["roofline"] = {k: rf[k] for k in ("bound", "achieved", "peak", "unit", "frac", "mfma_frac", "hbm_frac",
                                           "roofline_ms") if k in rf}
    return out


def bench_bf16_layer(a, s, dev, extra=False):
    """A bf16 layer workload (c2/c3/c4): a step is one moe_layer call.  With
    `extra`, a line that rides along the main one: no CPU baseline, no clock
    sampling, no host-dispatch figures."""
    import numpy as np
    import torch

    import expert_layer_amd as moe
    import synth

    T, H, E, k, I = s.T, s.H, s.E, s.k, s.I
    c = moe.make_cfg(T=T, H=H, E=E, k=k, I=I, n_groups=s.n_groups, topk_groups=s.topk_groups,
                     score_fn=moe.MOE_SCORE_SIGMOID if s.score == "sigmoid" else moe.MOE_SCORE_SOFTMAX,
                     renormalize=s.renormalize, routed_scale=s.routed_scale, has_shared=s.shared,
                     I_shared=s.I_shared, act_dtype=moe.MOE_BF16, y_dtype=moe.MOE_BF16, out_dtype=moe.MOE_BF16)

    # ---- inputs, resident in HBM before timing
    t_gen = time.time()
    x, w_r, bias = synth.router_inputs(s, dev)
    if a.traffic_run:
        def rnd(*shape):
            return (torch.randn(*shape, device=dev) / math.sqrt(shape[-1])).to(torch.bfloat16)
        wg, wu, wd = rnd(E, I, H), rnd(E, I, H), rnd(E, H, I)
        sh = (rnd(s.I_shared, H), rnd(s.I_shared, H), rnd(H, s.I_shared)) if s.shared else (None, None, None)
    else:
        wg = torch.empty((E, I, H), dtype=torch.bfloat16, device=dev)
        wu = torch.empty_like(wg)
        wd = torch.empty((E, H, I), dtype=torch.bfloat16, device=dev)
        for e in range(E):
            wg[e], wu[e], wd[e] = synth.expert_weights(s, e, dev)
        sh = synth.shared_weights(s, dev) if s.shared else (None, None, None)
    w = moe.weights(wg, wu, wd, sh_gate=sh[0], sh_up=sh[1], sh_down=sh[2])
    tiled_buf = None
    if not a.rowmajor_weights or extra:
        # weights are static: tiled once at load time, outside the timed region
        w, tiled_buf = moe.tile_weights(c, w, dev)
        del wg, wu, wd, sh
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    ws = moe.workspace(c, moe.MOE_STAGE_LAYER, dev)
    ws_layers = [w]
    table = layer_ids = None
    if a.weight_table > 0 and not extra:
        # layer l's expert e is the weight set's expert (e + 37 l) mod E: each
        # layer reads all E experts' bytes, as distinct weights would
        n_l = a.weight_table
        base = moe.moe_weight_table(c, [w])
        G = E + (1 if s.shared else 0)
        entries = []
        for li in range(n_l):
            for e in range(G):
                src = (e + 37 * li) % E if e < E else E
                entries += base[src * 6:(src + 1) * 6]
        table = torch.tensor(entries, dtype=torch.int64, device=dev)
        layer_ids = torch.arange(n_l, dtype=torch.int32, device=dev)
        ws_layers = [moe.weights(None, None, None, layout=w.layout, table=table,
                                 layer=layer_ids.data_ptr() + 4 * li, n_layers=n_l) for li in range(n_l)]
    torch.cuda.synchronize()
    print(f"[bench] inputs ready in {time.time() - t_gen:.1f}s; workspace {ws.numel() / 2**30:.2f} GiB",
          file=sys.stderr, flush=True)

    stream = torch.cuda.current_stream()

    def step(i):
        moe.moe_layer(c, w_r, bias, ws_layers[i % len(ws_layers)], x, out, ws, stream)

    ms_step = wall = None
    if not a.traffic_run:
        for i in range(a.warmup):
            step(i)
        torch.cuda.synchronize()

        # ---- timed region: K whole-layer steps
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        ev0.record(stream)
        for i in range(a.steps):
            step(i)
        ev1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        ms_step = ev0.elapsed_time(ev1) / a.steps

    dispatch = None
    if table is not None and not a.traffic_run:
        # Host cost of issuing one layer: an eager moe_layer call (argument
        # checks and 9 kernel launches) against the replay of a graph captured
        # once with the layer id read on the device, the id of the next layer
        # written by a fill kernel ahead of each replay (the ids are already on
        # the device, so the host need not wait for them).
        torch.cuda.synchronize()
        h0 = time.perf_counter()
        for i in range(a.steps):
            step(i)
        h_eager = (time.perf_counter() - h0) / a.steps
        torch.cuda.synchronize()
        lay = torch.zeros(1, dtype=torch.int32, device=dev)
        wg_ = moe.weights(None, None, None, layout=w.layout, table=table, layer=lay, n_layers=a.weight_table)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            moe.moe_layer(c, w_r, bias, wg_, x, out, ws)
        torch.cuda.synchronize()
        ev2, ev3 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        h0 = time.perf_counter()
        ev2.record(stream)
        for i in range(a.steps):
            lay.fill_(i % a.weight_table)
            g.replay()
        ev3.record(stream)
        h_graph = (time.perf_counter() - h0) / a.steps
        torch.cuda.synchronize()
        dispatch = {"eager_host_us_per_layer": round(h_eager * 1e6, 1),
                    "graph_host_us_per_layer": round(h_graph * 1e6, 1),
                    "graph_ms_per_step": round(ev2.elapsed_time(ev3) / a.steps, 4)}
        del g

    # ---- per-stage breakdown: moe_layer is these four stage calls with m_tile 16
    # and the indexed x_perm (the permute writes the maps, GEMM1 reads x through
    # row_src; bit-identical results); events between the stages on the launch
    # stream
    R = T * k
    c = moe.make_cfg(T=T, H=H, E=E, k=k, I=I, n_groups=s.n_groups, topk_groups=s.topk_groups,
                     score_fn=c.score_fn, renormalize=s.renormalize, routed_scale=s.routed_scale,
                     has_shared=s.shared, I_shared=s.I_shared, act_dtype=moe.MOE_BF16, y_dtype=moe.MOE_BF16,
                     out_dtype=moe.MOE_BF16, m_tile=16, x_layout=moe.MOE_LAYOUT_INDEXED)
    rows = moe.moe_max_rows(c)
    ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    tw = torch.empty((T, k), dtype=torch.float32, device=dev)
    counts = torch.empty(E, dtype=torch.int32, device=dev)
    offs = torch.empty(E + 1, dtype=torch.int32, device=dev)
    row_src = torch.empty(rows, dtype=torch.int32, device=dev)
    tok_row = torch.empty((T, k), dtype=torch.int32, device=dev)
    x_perm = moe.x_perm_buffer(c, dev)
    y_rows = torch.empty((rows, H), dtype=torch.bfloat16, device=dev)
    y_sh = torch.empty((T, H), dtype=torch.bfloat16, device=dev) if s.shared else None
    ws_r = moe.workspace(c, moe.MOE_STAGE_ROUTE, dev)
    ws_p = moe.workspace(c, moe.MOE_STAGE_PERMUTE, dev)
    ws_f = moe.workspace(c, moe.MOE_STAGE_FFN, dev)
    names = ["route", "permute", "grouped_ffn", "combine"]

    def stage_step(evs, i):
        w = ws_layers[i % len(ws_layers)]
        evs[0].record(stream)
        moe.moe_route(c, x, w_r, bias, None, None, ids, tw, ws_r, stream)
        evs[1].record(stream)
        moe.moe_permute(c, x, None, ids, counts, offs, row_src, tok_row, x_perm, None, ws_p, stream)
        evs[2].record(stream)
        moe.moe_grouped_ffn(c, rows, x, None, offs, w, None, y_rows, y_sh, ws_f, stream, row_src=row_src)
        evs[3].record(stream)
        moe.moe_combine(c, y_rows, tok_row, tw, y_sh, out, stream)
        evs[4].record(stream)

    for i in range(a.warmup if a.traffic_run else 2):
        stage_step([torch.cuda.Event(enable_timing=True) for _ in range(5)], i)
    torch.cuda.synchronize()
    stage_ms = np.zeros(4)
    all_evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(a.steps)]
    for i, evs in enumerate(all_evs):
        stage_step(evs, i)
    torch.cuda.synchronize()
    for evs in all_evs:
        stage_ms += np.array([evs[i].elapsed_time(evs[i + 1]) for i in range(4)])
    stage_ms /= a.steps
    if a.traffic_run:
        print(f"[bench] traffic run done: {a.warmup + a.steps} stage passes, grouped FFN "
              f"{stage_ms[2]:.3f} ms", flush=True)
        return None

    # ---- algorithmic work
    I_sh = s.I_shared if s.shared else 0
    ffn_flop = 6.0 * H * I * R + 6.0 * H * I_sh * T
    router_flop = 2.0 * T * H * E
    layer_flop = ffn_flop + router_flop
    w_bytes = 3.0 * E * H * I * 2 + 3.0 * H * I_sh * 2
    bytes_ = {
        "route": T * H * 2 + E * H * 2 + T * k * 8,
        # the maps only: ids read, counts/offsets/row_src/tok_row written (the
        # payload gather is GEMM1's A load)
        "permute": T * k * 4 + E * 8 + rows * 4 + T * k * 4,
        "grouped_ffn": w_bytes + R * H * 2 + T * H * 2 * bool(s.shared) + (R + T * bool(s.shared)) * H * 2,
        "combine": R * H * 2 + T * H * 2 * bool(s.shared) + T * H * 2 + T * k * 8,
    }
    tflops = layer_flop / (ms_step * 1e-3) / 1e12
    stages = {}
    for i, n in enumerate(names):
        ms = float(stage_ms[i])
        st = {"ms": round(ms, 4), "GB/s": round(bytes_[n] / (ms * 1e-3) / 1e9, 1),
              "hbm_frac": round(bytes_[n] / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
        if n == "grouped_ffn":
            st["TFLOP/s"] = round(ffn_flop / (ms * 1e-3) / 1e12, 1)
            st["mfma_frac"] = round(ffn_flop / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)
        if n == "route":
            st["TFLOP/s"] = round(router_flop / (ms * 1e-3) / 1e12, 1)
        stages[n] = st

    ffn_achieved = ffn_flop / (stage_ms[2] * 1e-3) / 1e12
    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        tf = json.load(open(TRAFFIC_FILE))
        if tf.get("source_hash") == ffn_source_hash() and tf.get("workload") == a.workload and not a.tokens:
            traffic = tf.get("hbm_bytes_per_launch")
    # The bound is the larger of the two roofline times, flop / MFMA peak and
    # algorithmic bytes / HBM peak; the other fraction is reported beside it.
    # Algorithmic bytes: the minimal bytes of the layer's roofline -- every
    # weight once, x read once, the output written once (bf16) -- which the
    # grouped FFN cannot go below; the bytes this design moves per launch
    # (each dispatched row read, bf16 y written) ride alongside as io_bytes.
    ffn_io_bytes = bytes_["grouped_ffn"]
    ffn_bytes = w_bytes + T * H * 2 + T * H * 2
    t_mfma = ffn_flop / (PEAK_BF16_TFLOPS * 1e12)
    t_hbm = ffn_bytes / (PEAK_HBM_GBS * 1e9)
    ffn_gbs = ffn_bytes / (stage_ms[2] * 1e-3) / 1e9
    if t_hbm > t_mfma:
        roofline = {"bound": "hbm", "achieved": round(ffn_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                    "frac": round(ffn_gbs / PEAK_HBM_GBS, 4)}
    else:
        roofline = {"bound": "mfma", "achieved": round(ffn_achieved, 1), "peak": PEAK_BF16_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(ffn_achieved / PEAK_BF16_TFLOPS, 4)}
    roofline.update({
        "traffic": traffic,
        "kernel": "moe_grouped_ffn (ffn_gemm_bf16<0, ...> gate/up+SwiGLU, ffn_gemm_bf16<1, false> down, tile list)",
        "flop_per_launch": ffn_flop, "bytes_per_launch": ffn_bytes, "io_bytes_per_launch": ffn_io_bytes,
        "io_frac": round(ffn_io_bytes / (stage_ms[2] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
        "roofline_ms": round(max(t_mfma, t_hbm) * 1e3, 4),
        "mfma_frac": round(ffn_achieved / PEAK_BF16_TFLOPS, 4),
        "hbm_frac": round(ffn_gbs / PEAK_HBM_GBS, 4)})

    cpu = None if (a.no_cpu_baseline or extra) else cpu_baseline(s, x, w_r, a.cpu_seconds)
    # the clock under this load: from the committed counter run of the same
    # FFN sources (GRBM_GUI_ACTIVE per XCD over the kernel's duration), else null
    sclk = None
    if not extra and os.path.exists(CLOCK_FILE):
        cf = json.load(open(CLOCK_FILE))
        if cf.get("source_hash") == ffn_source_hash() and cf.get("workload") == a.workload and not a.tokens:
            sclk = {k: {"clock_ghz": v["clock_ghz"], "mfma_busy_frac": v.get("mfma_busy_frac")}
                    for k, v in cf["kernels"].items()}
            sclk["source"] = ("rocprofv3 --pmc GRBM_GUI_ACTIVE (one XCD's busy cycles) over the kernel's average "
                              "duration, SQ_VALU_MFMA_BUSY_CYCLES over those cycles x 1024 SIMDs; "
                              "profiles/clock_grouped_ffn_c3_dsv3_bf16.json")

    res = {
        "metric": METRIC, "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": a.steps,
        "warmup": a.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": s.name, "T": T, "H": H, "E": E, "k": k, "I": I, "shared_experts": int(s.shared),
                   "I_shared": I_sh, "router": s.score, "n_groups": s.n_groups, "topk_groups": s.topk_groups,
                   "routed_scale": s.routed_scale, "out_dtype": "bf16", "expert_out_dtype": "bf16",
                   "weight_layout": "row-major" if a.rowmajor_weights else "tiled",
                   **({"weight_table_layers": a.weight_table} if a.weight_table else {})},
        "tokens_per_s": round(T / (ms_step * 1e-3), 1),
        "mfma_peak_frac": round(tflops / PEAK_BF16_TFLOPS, 4),
        "layer_flop": layer_flop,
        "wall_s_timed": round(wall, 3),
        "stages": stages,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "sclk": sclk,
        **({"dispatch": dispatch} if dispatch else {}),
    }
    return res


def bench_fp8_ffn(a, s, dev):
    """c5: one GPU's expert-parallel share of a prefill layer -- the rows
    arrive dispatched (per-expert counts of the workload), so a step is one
    fp8 moe_grouped_ffn over them: e4m3 rows with 1x128 scales, e4m3 weights
    with 128x128 block scales, bf16 y."""
    import numpy as np
    import torch

    import expert_layer_amd as moe
    import synth

    if a.traffic_run:
        raise SystemExit("--traffic-run profiles the bf16 layer")
    t_gen = time.time()
    counts = synth.fp8_counts(s)
    f4 = a.fp4_weights
    gen = synth.mxfp4_expert_weights if f4 else synth.fp8_expert_weights
    wq = [gen(s, e, dev) for e in range(s.E)]
    wg, sg, wu, su, wd, sd = (torch.stack([w[i] for w in wq]) for i in range(6))
    del wq
    xq, xs = synth.fp8_rows(s, s.T, dev)
    offs = torch.tensor(np.concatenate([[0], np.cumsum(counts)]), dtype=torch.int32, device=dev)
    c = moe.make_cfg(T=s.T, H=s.H, E=s.E, k=1, I=s.I, act_dtype=moe.MOE_FP8_E4M3, y_dtype=moe.MOE_BF16,
                     w_dtype=moe.MOE_FP4_E2M1 if f4 else moe.MOE_FP8_E4M3)
    y = torch.empty((s.T, s.H), dtype=torch.bfloat16, device=dev)
    ws = moe.workspace(c, moe.MOE_STAGE_FFN, dev, n_rows_cap=s.T)
    w = moe.weights(wg, wu, wd, s_gate=sg, s_up=su, s_down=sd)
    wbuf = None
    if not f4:  # e4m3 weights in the tiled layout (rewritten once, at load time)
        w, wbuf = moe.tile_weights(c, w, dev)
        del wg, wu, wd
    torch.cuda.synchronize()
    print(f"[bench] inputs ready in {time.time() - t_gen:.1f}s", file=sys.stderr, flush=True)
    stream = torch.cuda.current_stream()

    def step():
        moe.moe_grouped_ffn(c, s.T, xq, xs, offs, w, None, y, None, ws, stream)

    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(a.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = ev0.elapsed_time(ev1) / a.steps
    flop = 6.0 * s.H * s.I * s.T
    tflops = flop / (ms * 1e-3) / 1e12
    # algorithmic bytes: the weights (e4m3 with 128x128 fp32 scales, or MXFP4
    # at half a byte with one E8M0 byte per 32), the rows and their scales read
    # once, bf16 y written once
    KB1, KB2 = s.H // 128, s.I // 128
    w_bytes = 3.0 * s.E * s.H * s.I * (0.5 + 1.0 / 32) if f4 else 3.0 * s.E * s.H * s.I + 3.0 * s.E * KB1 * KB2 * 4
    nbytes = w_bytes + s.T * s.H + s.T * KB1 * 4 + s.T * s.H * 2
    t_mfma = flop / (PEAK_FP8_TFLOPS * 1e12)
    t_hbm = nbytes / (PEAK_HBM_GBS * 1e9)
    assert t_mfma >= t_hbm, "the fp8 FFN workload is expected to be compute-bound"
    res = {
        "metric": "grouped FFN TFLOP/s (1 GPU, fp8 expert-parallel share of a DeepSeek-V3 prefill layer)",
        "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": a.steps, "warmup": a.warmup,
        "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8_e4m3 x mxfp4" if f4 else "fp8_e4m3", "data": "synthetic",
        "config": {"workload": s.name, "rows": s.T, "H": s.H, "E_local": s.E, "I": s.I,
                   "counts": [int(v) for v in counts],
                   "scales": "1x128 rows, E8M0 per 32 weights (MXFP4)" if f4 else "1x128 rows, 128x128 weights",
                   "out_dtype": "bf16"},
        "tokens_per_s": round(s.T / (ms * 1e-3), 1),
        "wall_s_timed": round(wall, 3),
        "roofline": {"bound": "mfma", "achieved": round(tflops, 1), "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / PEAK_FP8_TFLOPS, 4), "traffic": None,
                     "kernel": "moe_grouped_ffn (%s GEMM1+SwiGLU+requantise, GEMM2, tile list)"
                               % ("ffn_gemm_fp8" if f4 else "ffn_gemm_e4m3"),
                     "flop_per_launch": flop, "bytes_per_launch": nbytes,
                     "roofline_ms": round(max(t_mfma, t_hbm) * 1e3, 4),
                     "hbm_frac": round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)},
        "cpu_baseline": None,
    }
    return res


def bench_fp8_layer(a, s, dev):
    """The layer with e4m3 experts and bf16 activations: a step is one moe_layer
    call (route, per-token quantisation, dispatch of the e4m3 rows, the routed
    and shared fp8 grouped FFNs, combine); the stage breakdown makes the same
    calls one by one."""
    import numpy as np
    import torch

    import expert_layer_amd as moe
    import synth

    T, H, E, k, I = s.T, s.H, s.E, s.k, s.I
    I_sh = s.I_shared if s.shared else 0
    kw = dict(T=T, H=H, E=E, k=k, I=I, n_groups=s.n_groups, topk_groups=s.topk_groups,
              score_fn=moe.MOE_SCORE_SIGMOID if s.score == "sigmoid" else moe.MOE_SCORE_SOFTMAX,
              renormalize=s.renormalize, routed_scale=s.routed_scale, has_shared=s.shared, I_shared=I_sh,
              y_dtype=moe.MOE_BF16, out_dtype=moe.MOE_BF16)
    f4 = a.fp4_weights
    wdt = moe.MOE_FP4_E2M1 if f4 else moe.MOE_FP8_E4M3
    c = moe.make_cfg(**kw, act_dtype=moe.MOE_BF16, w_dtype=wdt)
    if a.traffic_run:
        # the route with its fused per-token quantisation alone
        x, w_r, bias = synth.router_inputs(s, dev)
        xq = torch.empty((T, H), dtype=torch.uint8, device=dev)
        xs = torch.empty((T, H // 128), device=dev)
        ids, tw = torch.empty((T, k), dtype=torch.int32, device=dev), torch.empty((T, k), device=dev)
        ws_r = moe.workspace(c, moe.MOE_STAGE_ROUTE, dev)
        for _ in range(a.warmup + a.steps):
            moe.moe_route_quantize(c, x, w_r, bias, None, ids, tw, xq, xs, ws_r)
        torch.cuda.synchronize()
        print(f"[bench] traffic run done: {a.warmup + a.steps} moe_route_quantize calls on bf16 x [{T}][{H}]",
              flush=True)
        return None
    t_gen = time.time()
    x, w_r, bias = synth.router_inputs(s, dev)
    gen = synth.mxfp4_expert_weights if f4 else synth.fp8_expert_weights
    if f4:
        wg = torch.empty((E, I, H // 2), dtype=torch.uint8, device=dev)
        wu, wd = torch.empty_like(wg), torch.empty((E, H, I // 2), dtype=torch.uint8, device=dev)
        sg = torch.empty((E, I, H // 32), dtype=torch.uint8, device=dev)
        su, sd = torch.empty_like(sg), torch.empty((E, H, I // 32), dtype=torch.uint8, device=dev)
    else:
        wg = torch.empty((E, I, H), dtype=torch.uint8, device=dev)
        wu, wd = torch.empty_like(wg), torch.empty((E, H, I), dtype=torch.uint8, device=dev)
        sg = torch.empty((E, I // 128, H // 128), device=dev)
        su, sd = torch.empty_like(sg), torch.empty((E, H // 128, I // 128), device=dev)
    for e in range(E):
        wg[e], sg[e], wu[e], su[e], wd[e], sd[e] = gen(s, e, dev)
    sh = gen(s.with_(I=I_sh), E, dev) if s.shared else (None,) * 6
    w = moe.weights(wg, wu, wd, s_gate=sg, s_up=su, s_down=sd, sh_gate=sh[0], sh_up=sh[2], sh_down=sh[4],
                    sh_s_gate=sh[1], sh_s_up=sh[3], sh_s_down=sh[5])
    wbuf = None
    if not f4:  # e4m3 weights in the tiled layout (rewritten once, at load time)
        w, wbuf = moe.tile_weights(c, w, dev)
        del wg, wu, wd
    out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    ws = moe.workspace(c, moe.MOE_STAGE_LAYER, dev)
    torch.cuda.synchronize()
    print(f"[bench] fp8 experts ready in {time.time() - t_gen:.1f}s", file=sys.stderr, flush=True)
    stream = torch.cuda.current_stream()

    def step():
        moe.moe_layer(c, w_r, bias, w, x, out, ws, stream)

    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(a.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = ev0.elapsed_time(ev1) / a.steps

    # ---- the same work as stage calls: route with the per-token quantisation
    # of x, permute (maps only, m_tile 16), the routed grouped FFN reading the
    # e4m3 token rows through row_src, the shared one (one group of T rows),
    # combine
    cq = moe.make_cfg(**dict(kw, has_shared=False, I_shared=0), act_dtype=moe.MOE_FP8_E4M3, w_dtype=wdt, m_tile=16,
                      x_layout=moe.MOE_LAYOUT_INDEXED)
    c1 = moe.make_cfg(**dict(kw, E=1, k=1, n_groups=1, topk_groups=1, I=max(I_sh, 128), has_shared=False,
                             I_shared=0), act_dtype=moe.MOE_FP8_E4M3, w_dtype=wdt)
    rows = moe.moe_max_rows(cq)
    i32 = dict(dtype=torch.int32, device=dev)
    ids, tw = torch.empty((T, k), **i32), torch.empty((T, k), dtype=torch.float32, device=dev)
    counts, offs, row_src, tok_row = (torch.empty(E, **i32), torch.empty(E + 1, **i32), torch.empty(rows, **i32),
                                      torch.empty((T, k), **i32))
    xq = torch.empty((T, H), dtype=torch.uint8, device=dev)
    xs = torch.empty((T, H // 128), device=dev)
    x_perm = xps = None  # indexed: the permute writes the maps only
    y_rows = torch.empty((rows, H), dtype=torch.bfloat16, device=dev)
    y_sh = torch.empty((T, H), dtype=torch.bfloat16, device=dev) if s.shared else None
    offs1 = torch.tensor([0, T], **i32)
    w1 = moe.moe_weights(w_gate=w.sh_gate, w_up=w.sh_up, w_down=w.sh_down, s_gate=w.sh_s_gate, s_up=w.sh_s_up,
                         s_down=w.sh_s_down, layout=w.layout) if s.shared else None
    ws_r = moe.workspace(c, moe.MOE_STAGE_ROUTE, dev)
    ws_p = moe.workspace(cq, moe.MOE_STAGE_PERMUTE, dev)
    ws_f = moe.workspace(cq, moe.MOE_STAGE_FFN, dev, n_rows_cap=rows)
    ws_1 = moe.workspace(c1, moe.MOE_STAGE_FFN, dev, n_rows_cap=T) if s.shared else None
    names = ["route_quantise", "permute", "grouped_ffn", "combine"]

    def stage_step(evs):
        evs[0].record(stream)
        moe.moe_route_quantize(c, x, w_r, bias, None, ids, tw, xq, xs, ws_r, stream)
        evs[1].record(stream)
        moe.moe_permute(cq, xq, xs, ids, counts, offs, row_src, tok_row, x_perm, xps, ws_p, stream)
        evs[2].record(stream)
        moe.moe_grouped_ffn(cq, rows, xq, xs, offs, w, None, y_rows, None, ws_f, stream, row_src=row_src)
        if s.shared:
            moe.moe_grouped_ffn(c1, T, xq, xs, offs1, w1, None, y_sh, None, ws_1, stream)
        evs[3].record(stream)
        moe.moe_combine(c, y_rows, tok_row, tw, y_sh, out, stream)
        evs[4].record(stream)

    ns = len(names)
    for _ in range(2):
        stage_step([torch.cuda.Event(enable_timing=True) for _ in range(ns + 1)])
    torch.cuda.synchronize()
    all_evs = [[torch.cuda.Event(enable_timing=True) for _ in range(ns + 1)] for _ in range(a.steps)]
    for evs in all_evs:
        stage_step(evs)
    torch.cuda.synchronize()
    stage_ms = np.mean([[evs[i].elapsed_time(evs[i + 1]) for i in range(ns)] for evs in all_evs], axis=0)

    R = T * k
    KB1, KB2 = H // 128, I // 128
    ffn_flop = 6.0 * H * I * R + 6.0 * H * I_sh * T
    layer_flop = ffn_flop + 2.0 * T * H * E
    if f4:
        w_bytes = (3.0 * E * H * I + 3.0 * H * I_sh) * (0.5 + 1.0 / 32)
    else:
        w_bytes = 3.0 * E * H * I + 3.0 * E * KB1 * KB2 * 4 + 3.0 * H * I_sh + 3.0 * KB1 * (I_sh // 128) * 4
    bytes_ = {
        "route_quantise": T * H * 2 + E * H * 2 + T * k * 8 + T * H + T * KB1 * 4,
        "permute": T * k * 4 + E * 8 + rows * 4 + T * k * 4,
        "grouped_ffn": w_bytes + (R + T * bool(s.shared)) * (H + KB1 * 4) + (R + T * bool(s.shared)) * H * 2,
        "combine": R * H * 2 + T * H * 2 * bool(s.shared) + T * H * 2 + T * k * 8,
    }
    stages = {}
    for i, n in enumerate(names):
        ms = float(stage_ms[i])
        st = {"ms": round(ms, 4), "GB/s": round(bytes_[n] / (ms * 1e-3) / 1e9, 1),
              "hbm_frac": round(bytes_[n] / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
        if n == "grouped_ffn":
            st["TFLOP/s"] = round(ffn_flop / (ms * 1e-3) / 1e12, 1)
            st["mfma_frac"] = round(ffn_flop / (ms * 1e-3) / 1e12 / PEAK_FP8_TFLOPS, 4)
        stages[n] = st
    ffn_ms = float(stage_ms[names.index("grouped_ffn")])
    t_mfma = ffn_flop / (PEAK_FP8_TFLOPS * 1e12)
    t_hbm = bytes_["grouped_ffn"] / (PEAK_HBM_GBS * 1e9)
    tf = ffn_flop / (ffn_ms * 1e-3) / 1e12
    gbs = bytes_["grouped_ffn"] / (ffn_ms * 1e-3) / 1e9
    if t_hbm > t_mfma:
        roofline = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                    "frac": round(gbs / PEAK_HBM_GBS, 4)}
    else:
        roofline = {"bound": "mfma", "achieved": round(tf, 1), "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(tf / PEAK_FP8_TFLOPS, 4)}
    roofline.update({"traffic": None, "kernel": "grouped FFN (%s routed + shared, tile lists)"
                     % ("ffn_gemm_fp8" if f4 else "ffn_gemm_e4m3"),
                     "flop_per_launch": ffn_flop, "bytes_per_launch": bytes_["grouped_ffn"],
                     "roofline_ms": round(max(t_mfma, t_hbm) * 1e3, 4),
                     "mfma_frac": round(tf / PEAK_FP8_TFLOPS, 4), "hbm_frac": round(gbs / PEAK_HBM_GBS, 4)})
    tflops = layer_flop / (ms_step * 1e-3) / 1e12
    res = {
        "metric": METRIC, "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": a.steps,
        "warmup": a.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": ("mxfp4" if f4 else "fp8_e4m3") + " experts, bf16 activations",
        "data": "synthetic",
        "config": {"workload": s.name, "T": T, "H": H, "E": E, "k": k, "I": I, "shared_experts": int(s.shared),
                   "I_shared": I_sh,
                   "experts": "MXFP4 (E2M1, E8M0 per 32), e4m3 rows" if f4 else "e4m3, 128x128 block scales",
                   "activations": "bf16, quantised per token (1x128)", "out_dtype": "bf16"},
        "tokens_per_s": round(T / (ms_step * 1e-3), 1),
        "wall_s_timed": round(wall, 3),
        "stages": stages,
        "roofline": roofline,
        "cpu_baseline": None,
    }
    return res


def cpu_baseline(s, x, w_r, target_s):
    """The oracle as it stands on the host cores: router logits + gating and one
    routed expert's SwiGLU FFN for a sample of token rows (the per-row
    arithmetic of the layer), sized to about target_s seconds; reported in
    TFLOP/s of that sample."""
    import numpy as np
    import torch

    import oracle

    def bits(t):
        return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)

    import synth

    wh = bits(w_r)
    g, u, d = (bits(t) for t in synth.expert_weights(s, 0, "cpu"))
    per_row = 2.0 * s.H * s.E + 6.0 * s.H * s.I

    def run(n):
        xr = bits(x[:n])
        t0 = time.perf_counter()
        lg = oracle.router_logits(xr, wh)
        oracle.route_select(lg, s.k, score=1 if s.score == "sigmoid" else 0, n_groups=s.n_groups,
                            topk_groups=s.topk_groups, renormalize=s.renormalize, routed_scale=s.routed_scale)
        oracle.expert_ffn(xr, g, u, d, h_bf16=True)
        return time.perf_counter() - t0

    n = 32
    dt = run(n)
    n = int(min(x.shape[0], max(32, n * target_s / max(dt, 1e-3))))  # at most every token row
    dt = run(n)
    threads = min(oracle.threads(), n)
    return {"value": round(n * per_row / dt / 1e12, 6), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{n} token rows: router logits + group-limited top-k over {s.E} experts and one routed "
                      f"SwiGLU expert (H={s.H}, I={s.I}), fp64, {dt:.1f} s",
            "seconds": round(dt, 2)}


if __name__ == "__main__":
    main()
