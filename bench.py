"""Benchmark of the weight-only quantized linear path on one MI355X.

Headline (`value`): decode GEMV weight GB/s of one decode step of a Qwen3-0.6B-shaped model
(28 layers x {q,k,v,o,gate,up,down} + lm_head = 197 projections, 595,984,384 weights, 4-bit
g64 affine with bf16 scales/biases, bf16 activations, batch 1): one step = one problem-list
launch over all 197 projections.  Weights are resident in HBM; three distinct weight copies
are used in rotation so that a repeat never finds the previous step's weights in the 256 MB
Infinity Cache.  The default warmup (1000 steps, about 60 ms) brings the clocks to their
sustained level before the timed steps.  Other legs in the same JSON line: 8-bit decode at
batch 1 and 8, 4-bit decode at batch 8, the prefill
GEMM of a 9B-class layer (M=2048), routed experts (32 x 5760x2880, 512 tokens, top-4) in MXFP4
and Q8_0, and the quantizer.  `roofline` is the decode kernel's achieved HBM GB/s (algorithmic
bytes / average kernel time measured with HIP events on the launch stream) against 8 TB/s;
`cpu_baseline` times the NumPy oracle on a bounded sample of the same decode workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-legs] [--no-cpu]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
METRIC = "qlinear GEMV weight GB/s (% HBM peak) + prefill GEMM TFLOP/s, 4-bit g64"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=1000)
    ap.add_argument("--copies", type=int, default=3)
    ap.add_argument("--no-legs", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--legs", default="all",
                    help="comma-separated legs to run (decode8, decode4m8, decode_breakdown, prefill, experts, "
                         "prefill6, decode_bits, quantize, blocks, transcode, kquant) or 'all'")
    ap.add_argument("--no-headline", action="store_true",
                    help="skip the headline decode step (for profiling single legs); prints the legs only")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain device copy of 1 GiB (4 times): the reference for the HBM byte "
                         "counters that the roofline traffic figure is scaled by")
    return ap.parse_args()


# Source files that define the decode GEMV kernel; the measured HBM traffic recorded under
# profiles/ is reported only while their contents hash to the value recorded with it.
GEMV_SOURCES = ["device_common.hpp", "launch.hpp", "gemv_impl.hpp", "gemv_mfma.hpp", "gemv.hip", "gemv_m1.hip",
                "qlinear_api.cpp"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_gemv_mf_kernel_qwen3_0.6b_decode_4bit_g64.txt")


def gemv_source_hash() -> str:
    import hashlib

    h = hashlib.sha256()
    for name in GEMV_SOURCES:
        with open(os.path.join(ROOT, "weight_only_quantized_affine_amd", "csrc", name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def recorded_traffic():
    """HBM bytes per decode launch from the committed counter runs (FETCH_SIZE + WRITE_SIZE, each
    scaled by the same counter's reading for a plain copy of known size), or None when the
    kernel sources changed since they were taken."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    vals = {}
    with open(TRAFFIC_FILE) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("source_sha256") != gemv_source_hash():
        return None
    try:
        return int(float(vals["traffic_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def copy_calibration():
    """A plain device-to-device copy of 1 GiB, four times (for the byte-counter calibration)."""
    import torch

    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(4):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "repeats": 4}), flush=True)


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU: --gpus {args.gpus} is not supported (the path runs on a single "
              "MI355X; the product shards along its output rows with no exchange)", file=sys.stderr)
        sys.exit(2)
    import torch

    import synth
    import weight_only_quantized_affine_amd as q

    q.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()

    def gen(seed):
        return torch.Generator(device=dev).manual_seed(seed)

    # ------------------------------------------------------------ decode workload
    def build_decode(bits, m, copies, seed_base):
        """`copies` independent weight sets of the 197 projections, GPU-quantized."""
        sets = []
        wbytes = 0
        for c in range(copies):
            probs = []
            for i, (name, k, n) in enumerate(synth.QWEN3_0_6B_DECODE):
                w = torch.randn((n, k), generator=gen(seed_base + 1000 * c + i), device=dev) * 0.02
                pk, sc, bi = q.qlinear_quantize(w, bits, 64, torch.bfloat16)
                del w
                x = torch.randn((m, k), generator=gen(seed_base + 500000 + 1000 * c + i), device=dev).to(torch.bfloat16)
                y = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
                probs.append(dict(x=x, packed=pk, scales=sc, biases=bi, y=y, bits=bits, group_size=64))
                if c == 0:
                    wbytes += pk.numel() * 4 + sc.numel() * 2 + bi.numel() * 2
            arr = q.qlinear_problem_list(probs)
            ws = torch.empty(q.qlinear_gemv_batched_workspace_size(arr), dtype=torch.uint8, device=dev)
            kw = dict(x_dtype=torch.bfloat16, param_dtype=torch.bfloat16, y_dtype=torch.bfloat16, workspace=ws)
            q.qlinear_gemv_batched(arr, upload=True, **kw)  # uploads the problem table once
            # the graphs below hold raw pointers: the tensors and the workspace with the problem
            # table must stay referenced for as long as they are replayed
            sets.append((probs, arr, kw))
        torch.cuda.synchronize()
        io_bytes = sum(p["x"].numel() * 2 + p["y"].numel() * 2 for p in sets[0][0])
        return sets, wbytes, io_bytes

    def step_graph(sets, count, first=0):
        """`count` decode steps (one problem-list launch each, weight copies in rotation) captured
        as one HIP graph, so that the timed region has no host work between steps."""
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(count):
                _, arr, kw = sets[(first + i) % len(sets)]
                q.qlinear_gemv_batched(arr, upload=False, **kw)
        torch.cuda.synchronize()
        return g

    def time_decode(sets, steps, warmup):
        """Wall seconds for exactly `steps` decode steps, and the average launch duration (ms) from
        HIP events recorded on the launch stream around them."""
        gw = step_graph(sets, warmup) if warmup > 0 else None
        gt = step_graph(sets, steps, warmup)
        if gw is not None:
            gw.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record(stream)
        gt.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        avg_ms = e0.elapsed_time(e1) / steps
        del gw, gt
        return wall, avg_ms

    if args.no_headline:
        legs = run_legs(q, torch, synth, dev, stream, gen, build_decode, time_decode, args.legs)
        print(json.dumps({"legs": legs}), flush=True)
        return
    log("building the 4-bit decode workload (3 weight copies)")
    sets4, wbytes4, io4 = build_decode(4, 1, args.copies, 20_000)
    log(f"weights per step {wbytes4} B; timing {args.steps} steps after {args.warmup} warmup")
    wall, avg_ms = time_decode(sets4, args.steps, args.warmup)
    ms_per_step = wall * 1e3 / args.steps
    value = wbytes4 * args.steps / wall / 1e9
    achieved = (wbytes4 + io4) / (avg_ms * 1e-3) / 1e9
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u4-affine-g64 x bf16 -> f32 accumulate",
        "data": "synthetic (seeded N(0,0.02) weights quantized on the GPU, N(0,1) bf16 activations)",
        "config": {
            "workload": "qwen3-0.6b-shaped decode step: 197 GEMVs (28 layers x q,k,v,o,gate,up,down + lm_head), "
                        "batch 1, 4-bit affine g64, bf16 scales/biases, bf16 in/out, one problem-list launch",
            "weights_bytes_per_step": wbytes4,
            "weights": 595984384,
            "weight_copies_rotated": args.copies,
            "launch": "the K timed steps (one problem-list launch each) replayed as one HIP graph; problem "
                      "tables uploaded once",
            "pct_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
            "kernel_ms_avg": round(avg_ms, 5),
            "tokens_per_s_gemv_only": round(1e3 / avg_ms, 1),
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": recorded_traffic(),
            "kernel": "gemv_mf_kernel<1,64,bf16,bf16> (one launch per step)",
            "bytes_per_launch": wbytes4 + io4,
        },
    }
    del sets4
    torch.cuda.empty_cache()

    legs = {}
    if not args.no_legs:
        legs = run_legs(q, torch, synth, dev, stream, gen, build_decode, time_decode, args.legs)
    result["legs"] = legs
    if "prefill_gemm_9b_layer" in legs:
        result["prefill_gemm_tflops"] = legs["prefill_gemm_9b_layer"]["tflops"]
    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline()
    print(json.dumps(result), flush=True)


def _time_launches(fn, reps, warmup, stream):
    import torch

    for _ in range(warmup):
        fn(0)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for i in range(reps):
        ev[i][0].record(stream)
        fn(i)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    ms = [a.elapsed_time(b) for a, b in ev]
    return sum(ms) / len(ms), sorted(ms)[len(ms) // 2]


def _time_graph(fn, reps, warmup):
    """Average milliseconds per call of `reps` calls fn(0) .. fn(reps - 1) captured as one HIP graph
    (no host work between calls, as in the decode step), after `warmup` eager calls and three
    replays; HIP events on the replaying stream around a fourth replay."""
    import torch

    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(reps):
            fn(i)
    torch.cuda.synchronize()
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(s)
    g.replay()
    e1.record(s)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del g
    return ms


def run_legs(q, torch, synth, dev, stream, gen, build_decode, time_decode, which="all"):
    selected = frozenset(which.split(",")) if which != "all" else None

    def want(name):
        return selected is None or name in selected

    legs = {}
    # ---------------- 8-bit decode at batch 1 and 8, 4-bit decode at batch 8
    for bits, m in ((8, 1), (8, 8), (4, 8)):
        if not want("decode4m8" if bits == 4 else "decode8"):
            continue
        log(f"leg: {bits}-bit decode m={m}")
        sets_b, wb, io = build_decode(bits, m, 2, 30_000 + 100 * bits + m)
        wall, avg = time_decode(sets_b, 200, 300)
        legs[f"decode_{bits}bit_m{m}"] = {
            "weight_gbs": round(wb / (avg * 1e-3) / 1e9, 2),
            "kernel_ms": round(avg, 5),
            "pct_hbm_peak": round(100 * (wb + io) / (avg * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
            "weights_bytes": wb,
        }
        del sets_b
        torch.cuda.empty_cache()

    # ---------------- where the decode step's time goes: lm_head alone, the 196 layer projections
    # alone (one list launch each), and all 197 as separate qlinear_gemv launches in one graph
    if want("decode_breakdown"):
        log("leg: decode breakdown")
        sets_b, wb, io = build_decode(4, 1, 3, 20_000)
        out = {}
        for label, pick in (("lm_head_alone", lambda pr: pr[-1:]), ("layers_alone", lambda pr: pr[:-1])):
            sub = []
            for probs, _, kw in sets_b:
                picked = pick(probs)
                arr = q.qlinear_problem_list(picked)
                ws = torch.empty(q.qlinear_gemv_batched_workspace_size(arr), dtype=torch.uint8, device=dev)
                kw2 = dict(kw, workspace=ws)
                q.qlinear_gemv_batched(arr, upload=True, **kw2)
                sub.append((picked, arr, kw2))
            byts = sum(p_["packed"].numel() * 4 + p_["scales"].numel() * 4 for p_ in sub[0][0])
            _, avg = time_decode(sub, 200, 300)
            out[label] = {"kernel_ms": round(avg, 5), "weight_gbs": round(byts / (avg * 1e-3) / 1e9, 1),
                          "weights_bytes": byts}
            del sub
        # per-projection launches (qlinear_gemv each), 197 per step, captured as one graph
        torch.cuda.synchronize()
        gsteps = 20
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(gsteps):
                probs, _, _ = sets_b[i % len(sets_b)]
                for p_ in probs:
                    q.qlinear_gemv(p_["x"], p_["packed"], p_["scales"], p_["biases"], bits=4, group_size=64, y=p_["y"])
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        avg = e0.elapsed_time(e1) / gsteps
        out["per_projection_launches_graph"] = {"step_ms": round(avg, 5), "weight_gbs": round(wb / (avg * 1e-3) / 1e9, 1)}
        del g, sets_b
        torch.cuda.empty_cache()
        legs["decode_4bit_breakdown"] = out

    # ---------------- prefill GEMM, 9B-class layer at M = 2048: the layer's four inputs, each through
    # one call (q|k|v and gate|up as grouped calls over the weights that read the same x), plus each
    # projection alone through qlinear_gemm
    if want("prefill"):
        log("leg: prefill GEMM 9B layer, M=2048")
        m = 2048
        wts = {}
        for i, (name, k, n) in enumerate(synth.PREFILL_9B_LAYER):
            w = torch.randn((n, k), generator=gen(40_000 + i), device=dev) * 0.02
            pk, sc, bi = q.qlinear_quantize(w, 4, 64, torch.bfloat16)
            del w
            wts[name] = dict(packed=pk, scales=sc, biases=bi, y=torch.empty((m, n), dtype=torch.bfloat16, device=dev),
                             k=k, n=n)
        calls = [("qkv", ["q", "k", "v"]), ("o", ["o"]), ("gate_up", ["gate", "up"]), ("down", ["down"])]
        per_call = {}
        tot_flop = tot_ms = 0.0
        for ci, (cname, members) in enumerate(calls):
            k = wts[members[0]]["k"]
            x = torch.randn((m, k), generator=gen(41_000 + ci), device=dev).to(torch.bfloat16)
            ws_list = [dict(packed=wts[nm]["packed"], scales=wts[nm]["scales"], biases=wts[nm]["biases"], y=wts[nm]["y"])
                       for nm in members]
            ws = torch.empty(q.qlinear_gemm_grouped_workspace_size(m, k, ws_list, 4, 64), dtype=torch.uint8,
                             device=dev)
            avg, _ = _time_launches(lambda _i: q.qlinear_gemm_grouped(x, ws_list, bits=4, group_size=64, workspace=ws),
                                    20, 60, stream)
            flop = sum(2.0 * m * wts[nm]["n"] * k for nm in members)
            per_call[cname] = {"ms": round(avg, 4), "tflops": round(flop / (avg * 1e-3) / 1e12, 1)}
            tot_flop += flop
            tot_ms += avg
            # each projection alone (qlinear_gemm)
            for nm in members:
                w_ = wts[nm]
                ws1 = torch.empty(q.qlinear_gemm_workspace_size(m, w_["n"], k, 4, 64), dtype=torch.uint8, device=dev)
                a1, _ = _time_launches(lambda _i: q.qlinear_gemm(x, w_["packed"], w_["scales"], w_["biases"], bits=4,
                                                                 group_size=64, y=w_["y"], workspace=ws1), 20, 30,
                                       stream)
                w_["single"] = {"ms": round(a1, 4), "tflops": round(2.0 * m * w_["n"] * k / (a1 * 1e-3) / 1e12, 1)}
                del ws1
            del x, ws
        torch.cuda.empty_cache()
        tflops = tot_flop / (tot_ms * 1e-3) / 1e12
        legs["prefill_gemm_9b_layer"] = {
            "tflops": round(tflops, 1),
            "layer_ms": round(tot_ms, 4),
            "gflop": round(tot_flop / 1e9, 1),
            "prefill_tokens_per_s_per_layer": round(m / (tot_ms * 1e-3), 0),
            "per_call": per_call,
            "per_projection_single_call": {nm: wts[nm]["single"] for nm in wts},
            "roofline": {"bound": "mfma", "achieved": round(tflops, 1), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tflops / BF16_PEAK_TFLOPS, 4), "traffic": None,
                         "kernel": "prep_pp + gemm_pp_kernel<4,64,128> (q|k|v and gate|up grouped; o, down alone)"},
        }
        del wts

    # ---------------- routed experts, MXFP4 and Q8_0
    if want("experts"):
        cfg = synth.EXPERTS_32x5760x2880
        e, n, k, tokens, top = cfg["e"], cfg["n"], cfg["k"], cfg["tokens"], cfg["top"]
        ids = torch.from_numpy(synth.topk_ids(synth.seed_for(5, part=2), tokens, top, e).reshape(-1)).to(dev)
        x = torch.randn((tokens, k), generator=gen(50_000), device=dev).to(torch.bfloat16)
        y = torch.empty((tokens * top, n), dtype=torch.bfloat16, device=dev)
        ws = torch.empty(q.qlinear_apply_experts_workspace_size(tokens * top, e), dtype=torch.uint8, device=dev)
        flop = 2.0 * tokens * top * n * k
        for fmt, fname in ((q.QL_MXFP4, "mxfp4"), (q.QL_Q8_0, "q8_0")):
            log(f"leg: experts {fname}")
            copies = []
            for c in range(3):
                if fmt == q.QL_MXFP4:
                    codes = torch.randint(0, 256, (e, n, k // 2), generator=gen(51_000 + c), device=dev,
                                          dtype=torch.int32).to(torch.uint8)
                    scales = torch.randint(118, 131, (e, n, k // 32), generator=gen(52_000 + c), device=dev,
                                           dtype=torch.int32).to(torch.uint8)
                    copies.append((codes, scales))
                    wb = codes.numel() + scales.numel()
                else:
                    nb = k // 32
                    d = torch.exp2(torch.empty((e, n, nb), device=dev).uniform_(-14, -9, generator=gen(53_000 + c)))
                    d = d.to(torch.float16).view(torch.uint8).view(e, n, nb, 2)
                    qv = torch.randint(-127, 128, (e, n, nb, 32), generator=gen(54_000 + c), device=dev,
                                       dtype=torch.int32).to(torch.int8).view(torch.uint8)
                    blocks = torch.cat([d, qv], dim=3).reshape(e, n, nb * 34).contiguous()
                    copies.append((blocks, None))
                    wb = blocks.numel()
            # calls captured in a graph: each one is the routing launch and the products launch
            avg = _time_graph(
                lambda i: q.qlinear_apply_experts(fmt, copies[i % 3][0], copies[i % 3][1], ids, x, n=n, k=k,
                                                  pos_per_row=top, y=y, workspace=ws), 30, 10)
            byts = wb + x.numel() * 2 + y.numel() * 2
            gbs = byts / (avg * 1e-3) / 1e9
            legs[f"experts_{fname}"] = {
                "ms": round(avg, 4),
                "gbs": round(gbs, 1),
                "tflops": round(flop / (avg * 1e-3) / 1e12, 1),
                "weights_bytes": wb,
                "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                             "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
                             "kernel": "route_kernel + " + ("experts_mx_kernel" if fname == "mxfp4" else "experts_q8_kernel")},
            }
            del copies
            torch.cuda.empty_cache()

    # ---------------- Q4_K / Q6_K routed experts: the same expert stack and routing with k = 2816
    # (11 blocks of 256 values: the nearest multiple of 256 to 2880)
    if want("kquant"):
        cfg = synth.EXPERTS_32x5760x2880
        e, n, tokens, top = cfg["e"], cfg["n"], cfg["tokens"], cfg["top"]
        k = 2816
        ids = torch.from_numpy(synth.topk_ids(synth.seed_for(5, part=2), tokens, top, e).reshape(-1)).to(dev)
        x = torch.randn((tokens, k), generator=gen(56_000), device=dev).to(torch.bfloat16)
        y = torch.empty((tokens * top, n), dtype=torch.bfloat16, device=dev)
        ws = torch.empty(q.qlinear_apply_experts_workspace_size(tokens * top, e), dtype=torch.uint8, device=dev)
        flop = 2.0 * tokens * top * n * k
        for fmt, fname, nbytes, dat, lo, hi in ((q.QL_Q4_K, "q4_k", 144, 0, -16.0, -11.0),
                                                (q.QL_Q6_K, "q6_k", 210, 208, -17.0, -12.0)):
            log(f"leg: experts {fname}")
            copies = []
            nb = k // 256
            for c in range(3):
                blocks = torch.randint(0, 256, (e, n, nb, nbytes), generator=gen(57_000 + 10 * c + fmt), device=dev,
                                       dtype=torch.int32).to(torch.uint8)
                nd = 2 if fmt == q.QL_Q4_K else 1  # fp16 fields: d, dmin (Q4_K) or d (Q6_K)
                d = torch.exp2(torch.empty((e, n, nb, nd), device=dev).uniform_(lo, hi, generator=gen(58_000 + c)))
                blocks[..., dat:dat + 2 * nd] = d.to(torch.float16).view(torch.uint8).view(e, n, nb, 2 * nd)
                copies.append(blocks.reshape(e, n, nb * nbytes).contiguous())
            wb = copies[0].numel()
            avg = _time_graph(
                lambda i: q.qlinear_apply_experts(fmt, copies[i % 3], None, ids, x, n=n, k=k, pos_per_row=top, y=y,
                                                  workspace=ws), 20, 10)
            byts = wb + x.numel() * 2 + y.numel() * 2
            gbs = byts / (avg * 1e-3) / 1e9
            legs[f"experts_{fname}"] = {
                "ms": round(avg, 4), "gbs": round(gbs, 1), "tflops": round(flop / (avg * 1e-3) / 1e12, 1),
                "weights_bytes": wb, "k": k,
                "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                             "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
                             "kernel": f"route_kernel + experts_kq_kernel<{fmt}>"},
            }
            del copies
            torch.cuda.empty_cache()

    # ---------------- prefill GEMM at 6 bits (bitstream rows: codes re-packed as bytes, then the 8-bit
    # kernel), same layer and M
    if want("prefill6"):
        log("leg: prefill GEMM 9B layer, M=2048, 6-bit")
        m = 2048
        wts = {}
        for i, (name, k, n) in enumerate(synth.PREFILL_9B_LAYER):
            w = torch.randn((n, k), generator=gen(45_000 + i), device=dev) * 0.02
            pk, sc, bi = q.qlinear_quantize(w, 6, 64, torch.bfloat16)
            del w
            wts[name] = dict(packed=pk, scales=sc, biases=bi, y=torch.empty((m, n), dtype=torch.bfloat16, device=dev),
                             k=k, n=n)
        calls = [("qkv", ["q", "k", "v"]), ("o", ["o"]), ("gate_up", ["gate", "up"]), ("down", ["down"])]
        tot_flop = tot_ms = 0.0
        per6 = {}
        for ci, (cname, members) in enumerate(calls):
            k = wts[members[0]]["k"]
            x = torch.randn((m, k), generator=gen(46_000 + ci), device=dev).to(torch.bfloat16)
            ws_list = [dict(packed=wts[nm]["packed"], scales=wts[nm]["scales"], biases=wts[nm]["biases"], y=wts[nm]["y"])
                       for nm in members]
            ws = torch.empty(q.qlinear_gemm_grouped_workspace_size(m, k, ws_list, 6, 64), dtype=torch.uint8,
                             device=dev)
            avg, _ = _time_launches(lambda _i: q.qlinear_gemm_grouped(x, ws_list, bits=6, group_size=64, workspace=ws),
                                    10, 20, stream)
            flop = sum(2.0 * m * wts[nm]["n"] * k for nm in members)
            per6[cname] = {"ms": round(avg, 4), "tflops": round(flop / (avg * 1e-3) / 1e12, 1)}
            tot_flop += flop
            tot_ms += avg
            del x, ws
        del wts
        torch.cuda.empty_cache()
        legs["prefill_gemm_9b_layer_6bit"] = {
            "tflops": round(tot_flop / (tot_ms * 1e-3) / 1e12, 1),
            "layer_ms": round(tot_ms, 4),
            "per_call": per6,
            "kernel": "stream_to_bytes (per weight) + prep_pp + gemm_pp_kernel<8,64,128> (q|k|v and gate|up grouped; "
                      "o, down alone)",
        }

    # ---------------- bitstream widths (2, 3, 5, 6 bits): the decode step at batch 1, one problem-list
    # launch per step as above
    if want("decode_bits"):
        for bits in (2, 3, 5, 6):
            log(f"leg: {bits}-bit decode m=1")
            sets_b, wb, io = build_decode(bits, 1, 2, 70_000 + 100 * bits)
            wall, avg = time_decode(sets_b, 200, 300)
            legs[f"decode_{bits}bit_m1"] = {
                "weight_gbs": round(wb / (avg * 1e-3) / 1e9, 2),
                "kernel_ms": round(avg, 5),
                "pct_hbm_peak": round(100 * (wb + io) / (avg * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
                "weights_bytes": wb,
                "kernel": f"gemv_mf_kernel<1, 64, bf16, bf16, {bits}> (one problem-list launch per step)",
            }
            del sets_b
            torch.cuda.empty_cache()

    # ---------------- quantizer on the lm_head-sized matrix (151936 x 1024)
    if want("quantize"):
        log("leg: quantize")
        w = torch.randn((151936, 1024), generator=gen(60_000), device=dev) * 0.02
        pk = torch.empty((151936, 128), dtype=torch.int32, device=dev)
        sc = torch.empty((151936, 16), dtype=torch.bfloat16, device=dev)
        bi = torch.empty_like(sc)
        avg, _ = _time_launches(lambda _i: q.qlinear_quantize(w, 4, 64, torch.bfloat16, pk, sc, bi), 10, 2, stream)
        byts = w.numel() * 4 + pk.numel() * 4 + sc.numel() * 4
        legs["quantize_4bit_g64_151936x1024"] = {"ms": round(avg, 4), "gbs": round(byts / (avg * 1e-3) / 1e9, 1),
                                                 "pct_hbm_peak": round(100 * byts / (avg * 1e-3) / 1e9 / HBM_PEAK_GBS, 2)}
        out = torch.empty((151936, 1024), dtype=torch.bfloat16, device=dev)
        avg, _ = _time_launches(lambda _i: q.qlinear_dequant(q.QL_AFFINE, pk, sc, bi, rows=151936, k=1024, bits=4,
                                                             group_size=64, out=out), 10, 2, stream)
        byts = out.numel() * 2 + pk.numel() * 4 + sc.numel() * 4
        legs["dequant_4bit_g64_151936x1024_bf16"] = {"ms": round(avg, 4), "gbs": round(byts / (avg * 1e-3) / 1e9, 1)}
        del pk, sc, bi, out

    # ---------------- quantize_q8_0, MXFP4 in GGUF blocks, take (HBM-bound byte movers)
    if want("blocks"):
        log("leg: quantize_q8_0, MXFP4 blocks dequant, take")
        blocks = torch.empty((151936, 1024 // 32 * 34), dtype=torch.uint8, device=dev)
        avg, _ = _time_launches(lambda _i: q.qlinear_quantize_q8_0(w, blocks), 10, 2, stream)
        byts = w.numel() * 4 + blocks.numel()
        legs["quantize_q8_0_151936x1024"] = {"ms": round(avg, 4), "gbs": round(byts / (avg * 1e-3) / 1e9, 1),
                                             "pct_hbm_peak": round(100 * byts / (avg * 1e-3) / 1e9 / HBM_PEAK_GBS, 2)}
        del w, blocks
        e_, n_, k_ = 32, 5760, 2880
        mxb = torch.randint(0, 256, (e_ * n_, k_ // 32 * 17), generator=gen(61_000), device=dev,
                            dtype=torch.int32).to(torch.uint8)
        mxb.view(e_ * n_, k_ // 32, 17)[:, :, 0] = 127
        out = torch.empty((e_ * n_, k_), dtype=torch.bfloat16, device=dev)
        avg, _ = _time_launches(lambda _i: q.qlinear_dequant(q.QL_MXFP4_BLOCKS, mxb, rows=e_ * n_, k=k_, out=out),
                                10, 2, stream)
        byts = mxb.numel() + out.numel() * 2
        legs["dequant_mxfp4_blocks_32x5760x2880_bf16"] = {"ms": round(avg, 4), "gbs": round(byts / (avg * 1e-3) / 1e9, 1),
                                                          "pct_hbm_peak": round(100 * byts / (avg * 1e-3) / 1e9 / HBM_PEAK_GBS, 2)}
        del out
        stack = mxb.view(e_, n_, k_ // 32 * 17)
        pos = torch.tensor([3, 17, 30, 8], dtype=torch.int64, device=dev)
        got = torch.empty((4, n_, k_ // 32 * 17), dtype=torch.uint8, device=dev)
        avg, _ = _time_launches(lambda _i: q.qlinear_take(pos, stack, got), 20, 5, stream)
        byts = 2 * got.numel()
        legs["take_4_experts_mxfp4_blocks"] = {"ms": round(avg, 4), "gbs": round(byts / (avg * 1e-3) / 1e9, 1),
                                               "pct_hbm_peak": round(100 * byts / (avg * 1e-3) / 1e9 / HBM_PEAK_GBS, 2)}
        del mxb, stack, got

    # ---------------- GPTQ -> affine transcode of a 4096 -> 12288 layer (4-bit g128)
    if want("transcode"):
        log("leg: GPTQ transcode")
        K, N = 4096, 12288
        qw = torch.randint(-2**31, 2**31 - 1, (K * 4 // 32, N), generator=gen(62_000), device=dev, dtype=torch.int32)
        qz = torch.randint(-2**31, 2**31 - 1, (K // 128, N * 4 // 32), generator=gen(62_001), device=dev,
                           dtype=torch.int32)
        sc = (torch.rand((K // 128, N), generator=gen(62_002), device=dev) * 0.02 + 1e-3).to(torch.float16)
        pk_o, so_o, bo_o = q.qlinear_transcode_gptq(qw, qz, sc, bits=4, group_size=128)
        torch.cuda.synchronize()
        g_tc = torch.cuda.CUDAGraph()  # 20 calls replayed as one graph: GPU time, not host pacing
        with torch.cuda.graph(g_tc):
            for _ in range(20):
                q.qlinear_transcode_gptq(qw, qz, sc, bits=4, group_size=128, packed=pk_o, scales_out=so_o,
                                         biases_out=bo_o)
        g_tc.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        g_tc.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        avg = e0.elapsed_time(e1) / 20
        del g_tc, pk_o, so_o, bo_o
        byts = 2 * qw.numel() * 4 + qz.numel() * 4 + sc.numel() * 2 * 3
        legs["transcode_gptq_4096x12288_4bit_g128"] = {
            "ms": round(avg, 4), "gbs": round(byts / (avg * 1e-3) / 1e9, 1),
            "pct_hbm_peak": round(100 * byts / (avg * 1e-3) / 1e9 / HBM_PEAK_GBS, 2)}
        del qw, qz, sc
        torch.cuda.empty_cache()

        # AWQ GEMM of the same layer: codes packed along the outputs, transposed code by code
        log("leg: AWQ transcode")
        qw = torch.randint(-2**31, 2**31 - 1, (K, N * 4 // 32), generator=gen(62_010), device=dev, dtype=torch.int32)
        qz = torch.randint(-2**31, 2**31 - 1, (K // 128, N * 4 // 32), generator=gen(62_011), device=dev,
                           dtype=torch.int32)
        sc = (torch.rand((K // 128, N), generator=gen(62_012), device=dev) * 0.02 + 1e-3).to(torch.float16)
        pk_o, so_o, bo_o = q.qlinear_transcode_awq(qw, qz, sc, bits=4, group_size=128)
        torch.cuda.synchronize()
        g_tc = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g_tc):
            for _ in range(20):
                q.qlinear_transcode_awq(qw, qz, sc, bits=4, group_size=128, packed=pk_o, scales_out=so_o,
                                        biases_out=bo_o)
        g_tc.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        g_tc.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        avg = e0.elapsed_time(e1) / 20
        del g_tc, pk_o, so_o, bo_o
        byts = 2 * qw.numel() * 4 + qz.numel() * 4 + sc.numel() * 2 * 3
        legs["transcode_awq_4096x12288_4bit_g128"] = {
            "ms": round(avg, 4), "gbs": round(byts / (avg * 1e-3) / 1e9, 1),
            "pct_hbm_peak": round(100 * byts / (avg * 1e-3) / 1e9 / HBM_PEAK_GBS, 2)}
        del qw, qz, sc
        torch.cuda.empty_cache()
    return legs


def cpu_baseline(min_seconds: float = 8.0):
    """The NumPy oracle (unpack + fp64 dequant + matmul) timed on the host over whole decode steps
    of the same Qwen3-0.6B-shaped workload (all 197 projections, batch 1, 4-bit g64 bf16), with
    synthetic packed words and parameters; passes repeat until `min_seconds` have elapsed."""
    import numpy as np

    import oracle as O
    import synth

    threads, blas = 1, "unknown"
    try:
        from threadpoolctl import threadpool_info, threadpool_limits

        info = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        threads = max([i.get("num_threads", 1) for i in info] or [1])
        blas = ", ".join(f"{i.get('internal_api')} {i.get('version')} ({os.path.basename(i.get('filepath', ''))})"
                         for i in info) or "unknown"
    except Exception:  # noqa: BLE001
        threadpool_limits = None
    cpu_model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    log("cpu baseline: oracle over whole decode steps")
    g = np.random.default_rng(990)
    prepared = []
    for (_, k, n) in synth.QWEN3_0_6B_DECODE:
        pk = g.integers(0, 2**32, size=(n, k // 8), dtype=np.uint64).astype(np.uint32)
        sb = O.to_bits("bf16", (0.006 + 0.001 * g.random((n, k // 64))).astype(np.float32))
        bb = O.to_bits("bf16", (-0.048 + 0.005 * g.standard_normal((n, k // 64))).astype(np.float32))
        xb = O.bits_to_f64("bf16", synth.acts_bits(991, 1, k, "bf16"))
        prepared.append((pk, sb, bb, xb, k))
    wbytes = sum(pk.nbytes + sb.nbytes + bb.nbytes for (pk, sb, bb, _, _) in prepared)

    def timed(limit_s):
        passes = 0
        t0 = time.perf_counter()
        while True:
            for (pk, sb, bb, x, k) in prepared:
                D = O.affine_dequant_f32(pk, sb, bb, 4, 64, "bf16", k)
                O.apply(x, D)
            passes += 1
            dt = time.perf_counter() - t0
            if dt >= limit_s or passes >= 5:
                return passes, dt

    passes, dt = timed(min_seconds)
    one = None
    if threadpool_limits is not None:
        log("cpu baseline: the same on one BLAS thread")
        with threadpool_limits(limits=1, user_api="blas"):
            p1, d1 = timed(min_seconds / 2)
        one = {"value": round(wbytes * p1 / d1 / 1e9, 4), "unit": "GB/s", "cores": 1, "seconds": round(d1, 2),
               "passes": p1}
    return {"value": round(wbytes * passes / dt / 1e9, 4), "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{passes} whole decode step(s) of the qwen3-0.6b-shaped workload (197 projections, "
                      f"{wbytes} weight bytes each, batch 1, 4-bit g64 bf16, synthetic packed words) in {dt:.2f} s: "
                      f"unpack + fp64 dequant (single-threaded NumPy) + matmul ({threads} BLAS threads)",
            "seconds": round(dt, 2), "tokens_per_s": round(passes / dt, 3), "one_thread": one,
            "cpu_model": cpu_model, "host_threads": os.cpu_count(), "blas": blas}


if __name__ == "__main__":
    main()
