"""Benchmark of the fused NF4 dequantise-and-multiply path on one MI355X.

A step is one pass of the hot path over the Llama-3.1-8B-shaped stack at
batch 1, S = 512 (M = 512): for each of 32 layers and each of the 7
projections (q, k, v, o, gate, up, down), the fused forward y = x . W^T, then
the fused input gradient grad_x = grad_y . W (layers in reverse), all from
nested NF4 weights resident in HBM (224 distinct weights, 3.6 GB packed).
The metric is TFLOP/s of algorithmic work (2 M N K per GEMM) and its fraction
of the bf16 dense MFMA peak.

Prints ONE JSON line.  Secondary workloads (decode-size M over the same 224
weights, the Qwen-32B-shaped layer at M = 2048, OLMoE grouped experts) are
measured after the main step and reported inside the line under "extra";
the oracle's CPU time on a bounded sample is under "cpu_baseline".
"""

from __future__ import annotations

import argparse
import json
import os
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6       # 256 CU x 4096 flop/clk x 2.4 GHz, dense
PEAK_HBM_GBS = 8000.0
METRIC = "NF4 fused GEMM TFLOP/s (fwd + bwd_input) at M=512/2048; % of bf16 MFMA peak"


def log(msg):
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--no-extra", action="store_true", help="skip the secondary workloads")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--only", default=None, metavar="[FAMILY:]DIR_PROJ",
                    help="time one shape and nothing else, for profiling: fwd_gate (the 32 layers' "
                         "forward gate projections of the step), qwen:bwd_down, olmoe:fwd_gate")
    ap.add_argument("--m", type=int, default=0,
                    help="with --only: rows of x (default: the workload's M, 512 or 2048)")
    ap.add_argument("--code", default="nf4", choices=("nf4", "fp4", "int8", "fp8_e4m3"),
                    help="with --only: the code table the weights are quantised with (int8 and fp8_e4m3 "
                         "are the 8-bit blockwise formats)")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="with --only: then run one plain device copy of this many bytes "
                         "(calibrates rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    return ap.parse_args()


def traffic_file(direction, proj, M):
    return os.path.join(ROOT, "profiles", f"traffic_fused_gemm_{direction}_{proj}_m{M}.md")


def clocks():
    try:
        r = subprocess.run(["rocm-smi", "--showclocks"], capture_output=True, text=True, timeout=20)
        out = {}
        for ln in r.stdout.splitlines():
            low = ln.lower()
            for key in ("sclk", "mclk", "fclk"):
                if f"({key})" in low or f" {key} " in low:
                    out[key] = ln.split(":")[-1].strip()
        return out or None
    except Exception:
        return None


def timed(torch, stream, fn, steps, warmup):
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def filler_copy(torch, dev, nbytes=1 << 30):
    """A device copy of 1 GiB (~0.4 ms) enqueued before each timed sample: the
    GPU works through it while the host enqueues the sample's calls, so the
    sample measures GPU time even where one call launches slower from Python
    than it runs, and every sample starts with the caches refilled by
    unrelated data."""
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    return lambda: dst.copy_(src)


def interleaved(torch, stream, arms, filler, rounds=21, reps=5, warmup=2):
    """Median time per call of each arm.  Every round runs each arm once (reps
    calls between two HIP events on the launch stream, after the filler), in
    an order rotated from round to round, so slow drift of clocks or
    temperature falls on all arms alike."""
    names = list(arms)
    for _ in range(warmup):
        for n in names:
            arms[n]()
    pairs = {n: [] for n in names}
    for r in range(rounds):
        k = r % len(names)
        for n in names[k:] + names[:k]:
            filler()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _ in range(reps):
                arms[n]()
            b.record(stream)
            pairs[n].append((a, b))
    torch.cuda.synchronize()
    out = {}
    for n in names:
        t = sorted(a.elapsed_time(b) * 1e3 / reps for a, b in pairs[n])
        out[n] = {"median_us": round(t[len(t) // 2], 2), "p10_us": round(t[len(t) // 10], 2),
                  "p90_us": round(t[(9 * len(t)) // 10], 2), "samples": len(t)}
    return out


def copy_ceiling(torch, stream, dev, nbytes=2 << 30, rounds=21):
    """Same-session HBM ceiling: median of `rounds` device-to-device copies of
    2 GiB (read + write = 4 GiB moved each)."""
    src = torch.ones(nbytes, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    pairs = []
    for _ in range(rounds):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        dst.copy_(src)
        b.record(stream)
        pairs.append((a, b))
    torch.cuda.synchronize()
    t = sorted(a.elapsed_time(b) * 1e-3 for a, b in pairs)
    med = t[len(t) // 2]
    gbs = 2 * nbytes / med / 1e9
    del src, dst
    return {"copy_bytes": nbytes, "bytes_moved": 2 * nbytes, "median_us": round(med * 1e6, 1),
            "GBps": round(gbs, 1), "frac_of_8TBps": round(gbs / PEAK_HBM_GBS, 4), "samples": rounds}


def build_stack(torch, api, WL, projs, layers, code, ncode, dev, seed0):
    weights = []
    for l in range(layers):
        row = []
        for i, p in enumerate(projs):
            w = WL.gpu_weight_f32(p.N, p.K, seed=WL.stack_weight_seed(seed0, l, i), device=dev)
            row.append(api.nf4_quantize(w, code, ncode))
            del w
        weights.append(row)
    torch.cuda.synchronize()
    return weights


def layer_inputs(torch, WL, projs, layers, M, dev, seed0):
    """One input per producer inside a layer (q/k/v share, gate/up share), a
    grad_y per projection."""
    xs, gys = [], []
    kdim = {}
    for i, p in enumerate(projs):
        kdim.setdefault(WL.X_SLOT[i], p.K)
    for l in range(layers):
        ins = {s: WL.gpu_normal_bf16(M, k, seed=WL.stack_x_seed(seed0, l, s), device=dev)
               for s, k in kdim.items()}
        xs.append([ins[WL.X_SLOT[i]] for i in range(len(projs))])
        gys.append([WL.gpu_normal_bf16(M, p.N, seed=WL.stack_gy_seed(seed0, l, i), device=dev)
                    for i, p in enumerate(projs)])
    return xs, gys


def run_stack_step(api, weights, xs, gys, ys, gxs, ws):
    """One step: every layer's 7 fused forwards, then every layer's 7 fused
    input gradients in reverse order."""
    L, P = len(weights), len(weights[0])
    for l in range(L):
        for i in range(P):
            api.nf4_matmul_fwd(xs[l][i], weights[l][i], out=ys[i], ws=ws)
    for l in reversed(range(L)):
        for i in reversed(range(P)):
            api.nf4_matmul_bwd_input(gys[l][i], weights[l][i], out=gxs[i], ws=ws)


def workspace_for(torch, api, projs, Ms, dev):
    need = 16
    for M in Ms:
        for p in projs:
            # forward / input gradient, NF4 and 8-bit plans
            need = max(need, *(api.nf4_workspace_bytes(op, M, p.N, p.K) for op in (1, 2, 5, 6)))
    return torch.empty(need, dtype=torch.uint8, device=dev)


# ---------------------------------------------------------------------------
def run_extra(torch, api, WL, code, ncode, dev, llama_weights, stream):
    extra = {}
    projs = WL.LLAMA_8B
    L = len(llama_weights)
    wbytes = sum(w.nbytes() for row in llama_weights for w in row)

    # same-session HBM ceiling, measured first so the decode passes can be set
    # against it as well as against the 8 TB/s peak
    ceil = copy_ceiling(torch, stream, dev)
    extra["hbm_copy_ceiling"] = ceil
    log(f"copy ceiling: {ceil}")

    # decode-size M: forward only over the same 224 weights (3.6 GB, beyond the
    # 256 MB last-level cache)
    dec = {}
    for M in WL.DECODE_MS:
        xs = [WL.gpu_normal_bf16(M, p.K, seed=40_000 + 7 * M + i, device=dev) for i, p in enumerate(projs)]
        ys = [torch.empty((M, p.N), dtype=torch.bfloat16, device=dev) for p in projs]
        ws = workspace_for(torch, api, projs, [M], dev)

        def one_pass():
            for l in range(L):
                for i in range(len(projs)):
                    api.nf4_matmul_fwd(xs[i], llama_weights[l][i], out=ys[i], ws=ws)

        # 224 back-to-back launches of a few microseconds each: issuing them
        # from Python costs more than running them, so the pass is captured
        # once into a HIP graph and replayed; the replay's outputs must equal
        # the eager pass bit for bit.
        one_pass()
        torch.cuda.synchronize()
        eager = [y.clone() for y in ys]
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            one_pass()
        for y in ys:
            y.zero_()
        graph.replay()
        torch.cuda.synchronize()
        same = all(torch.equal(a.view(torch.int16), b.view(torch.int16)) for a, b in zip(eager, ys))
        ms = timed(torch, stream, graph.replay, steps=10, warmup=3)
        ms_eager = timed(torch, stream, one_pass, steps=3, warmup=1)
        gbs = wbytes / (ms * 1e-3) / 1e9
        dec[f"M={M}"] = {"us_per_pass": round(ms * 1e3, 1), "weight_GBps": round(gbs, 1),
                         "frac_of_8TBps": round(gbs / PEAK_HBM_GBS, 4),
                         "frac_of_copy_ceiling": round(gbs / ceil["GBps"], 4),
                         "graph_replay_bitwise_equal": same,
                         "us_per_pass_eager_launches": round(ms_eager * 1e3, 1)}
        del graph
        del xs, ys, ws
    extra["decode_llama8b_fwd"] = dec

    log(f"decode done: {dec}")

    # Today's path as the comparator: dequantise every visit, then the dense
    # bf16 GEMM (hipBLASLt through torch), per Llama projection at M = 512 on
    # layer 0's weights; and the dense GEMM alone on a resident dequantised
    # weight (the same-session dense ceiling).  The three arms are interleaved
    # round by round (medians of 21 rounds of 5 calls).  Outputs are compared
    # with the fused ones: same exact product, different accumulation order.
    import torch.nn.functional as F
    filler = filler_copy(torch, dev)
    arm_names = ("fused", "dequant_plus_dense", "dense_only")
    M = WL.LLAMA_M
    comp = {}
    tot = {f"{n}_us": 0.0 for n in arm_names}
    for i, p in enumerate(projs):
        w = llama_weights[0][i]
        x = WL.gpu_normal_bf16(M, p.K, seed=90_000 + i, device=dev)
        gy = WL.gpu_normal_bf16(M, p.N, seed=91_000 + i, device=dev)
        ws_c = workspace_for(torch, api, [p], [M], dev)
        wd = torch.empty((p.N, p.K), dtype=torch.bfloat16, device=dev)
        wd_r = torch.empty((p.N, p.K), dtype=torch.bfloat16, device=dev)
        y_f = torch.empty((M, p.N), dtype=torch.bfloat16, device=dev)
        g_f = torch.empty((M, p.K), dtype=torch.bfloat16, device=dev)

        def fused():
            api.nf4_matmul_fwd(x, w, out=y_f, ws=ws_c)
            api.nf4_matmul_bwd_input(gy, w, out=g_f, ws=ws_c)

        def today():
            api.nf4_dequantize(w, out=wd)
            y = F.linear(x, wd)
            api.nf4_dequantize(w, out=wd)
            g = torch.matmul(gy, wd)
            return y, g

        api.nf4_dequantize(w, out=wd_r)

        def dense():
            return F.linear(x, wd_r), torch.matmul(gy, wd_r)

        med = interleaved(torch, stream, dict(zip(arm_names, (fused, today, dense))), filler)
        t_f, t_t, t_d = (med[n]["median_us"] for n in arm_names)
        api.nf4_reset_path_counts()
        fused()
        torch.cuda.synchronize()
        pc = api.nf4_path_counts()
        ran_fused = pc["fwd_tiled"] == 1 and pc["bwd_tiled"] == 1
        y_c, g_c = dense()
        torch.cuda.synchronize()

        def diff(a, b):
            a, b = a.float(), b.float()
            rel = float((a - b).norm().item() / max(b.norm().item(), 1e-30))
            same = float((a.view(torch.int32) == b.view(torch.int32)).float().mean().item())
            return rel, same

        ry, ey = diff(y_f, y_c)
        rg, eg = diff(g_f, g_c)
        comp[p.name] = {"fused_us": t_f, "dequant_plus_dense_us": t_t,
                        "dense_only_us": t_d, "speedup_vs_today": round(t_t / t_f, 2),
                        "p10_p90_us": {n: [med[n]["p10_us"], med[n]["p90_us"]] for n in arm_names},
                        "fwd_rel_fro_diff": float(f"{ry:.3g}"), "fwd_identical_frac": round(ey, 4),
                        "bwd_rel_fro_diff": float(f"{rg:.3g}"), "bwd_identical_frac": round(eg, 4),
                        "fused_kernels_ran": ran_fused}
        for n, t in zip(arm_names, (t_f, t_t, t_d)):
            tot[f"{n}_us"] += t
        del x, gy, ws_c, wd, wd_r, y_f, g_f, y_c, g_c
    flops_layer = 2 * sum(2.0 * M * p.N * p.K for p in projs)
    comp["timing"] = "per arm: median over 21 interleaved rounds of 5 calls, each round after a 1 GiB filler copy"
    comp["layer_total"] = {k: round(v, 1) for k, v in tot.items()}
    comp["layer_total"]["fused_tflops"] = round(flops_layer / (tot["fused_us"] * 1e-6) / 1e12, 1)
    comp["layer_total"]["dense_only_tflops"] = round(flops_layer / (tot["dense_only_us"] * 1e-6) / 1e12, 1)
    comp["layer_total"]["today_tflops"] = round(flops_layer / (tot["dequant_plus_dense_us"] * 1e-6) / 1e12, 1)
    # decode sizes, forward only: the fused forward (the streaming kernels, or
    # the 64-row staged tiles for the large products above M = 16) against
    # dequantise + dense GEMV/GEMM, summed over layer 0's seven projections
    for Md in WL.DECODE_MS:
        t = {f"{n}_us": 0.0 for n in arm_names}
        rels, ran = [], True
        for i, p in enumerate(projs):
            w = llama_weights[0][i]
            x = WL.gpu_normal_bf16(Md, p.K, seed=92_000 + i, device=dev)
            ws_c = workspace_for(torch, api, [p], [Md], dev)
            wd = torch.empty((p.N, p.K), dtype=torch.bfloat16, device=dev)
            wd_r = torch.empty((p.N, p.K), dtype=torch.bfloat16, device=dev)
            api.nf4_dequantize(w, out=wd_r)
            y_f = torch.empty((Md, p.N), dtype=torch.bfloat16, device=dev)
            med = interleaved(torch, stream, {
                "fused": lambda: api.nf4_matmul_fwd(x, w, out=y_f, ws=ws_c),
                "dequant_plus_dense": lambda: F.linear(x, api.nf4_dequantize(w, out=wd)),
                "dense_only": lambda: F.linear(x, wd_r)}, filler)
            for n in arm_names:
                t[f"{n}_us"] += med[n]["median_us"]
            api.nf4_reset_path_counts()
            api.nf4_matmul_fwd(x, w, out=y_f, ws=ws_c)
            y_c = F.linear(x, wd_r)
            torch.cuda.synchronize()
            pc = api.nf4_path_counts()
            ran = ran and pc["fwd_small_m"] + pc["fwd_tiled"] == 1
            rels.append(float((y_f.float() - y_c.float()).norm().item() / max(y_c.float().norm().item(), 1e-30)))
            del x, ws_c, wd, wd_r, y_f, y_c
        comp[f"decode_M={Md}_fwd"] = {k: round(v, 1) for k, v in t.items()}
        comp[f"decode_M={Md}_fwd"].update({
            "speedup_vs_today": round(t["dequant_plus_dense_us"] / t["fused_us"], 2),
            "max_rel_fro_diff": float(f"{max(rels):.3g}"), "fused_kernels_ran": ran})
    extra["comparator_llama8b_layer0"] = comp
    log(f"comparator done: {comp['layer_total']}")

    extra["code_tables_llama8b_layer0"] = run_code_tables(torch, api, WL, ncode, dev, stream, filler, ceil)
    del filler
    log(f"code tables done: {extra['code_tables_llama8b_layer0']['summary']}")

    extra["layer_streaming_llama8b_m512"] = run_streaming(torch, api, WL, dev, llama_weights, stream)
    log(f"streaming done: {extra['layer_streaming_llama8b_m512']}")
    # Qwen-32B-shaped layer at M = 2048: two layer copies, rotated
    qp = WL.QWEN_32B
    M = WL.QWEN_M
    qw = build_stack(torch, api, WL, qp, 2, code, ncode, dev, seed0=50_000)
    xs, gys = layer_inputs(torch, WL, qp, 2, M, dev, seed0=60_000)
    ys = [torch.empty((M, p.N), dtype=torch.bfloat16, device=dev) for p in qp]
    gxs = [torch.empty((M, p.K), dtype=torch.bfloat16, device=dev) for p in qp]
    ws = workspace_for(torch, api, qp, [M], dev)
    ms = timed(torch, stream, lambda: run_stack_step(api, qw, xs, gys, ys, gxs, ws), steps=3, warmup=1)
    flops = 2 * 2 * sum(2.0 * M * p.N * p.K for p in qp)
    # bitwise repeatability of the last layer's outputs
    run_stack_step(api, qw, xs, gys, ys, gxs, ws)
    y_a, g_a = ys[6].clone(), gxs[0].clone()
    run_stack_step(api, qw, xs, gys, ys, gxs, ws)
    same = bool(torch.equal(ys[6].view(torch.int16), y_a.view(torch.int16)) and
                torch.equal(gxs[0].view(torch.int16), g_a.view(torch.int16)))
    tf = flops / (ms * 1e-3) / 1e12
    extra["qwen32b_m2048_fwd_bwd"] = {"ms_per_layer": round(ms / 2, 3), "tflops": round(tf, 1),
                                      "frac_of_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4),
                                      "bitwise_repeat": same}
    del qw, xs, gys, ys, gxs, ws

    log(f"qwen done: {extra['qwen32b_m2048_fwd_bwd']}")
    # OLMoE grouped experts: 512 tokens, top-8 of 64; gate/up [64,1024,2048], down [64,2048,1024]
    E, H, I = WL.OLMOE_E, WL.OLMOE_HIDDEN, WL.OLMOE_INTER
    _, _, offsets = WL.olmoe_routing()
    T = int(offsets[-1])
    off = torch.from_numpy(offsets).to(dev)
    stacks = {}
    for j, (name, N, K) in enumerate((("gate", I, H), ("up", I, H), ("down", H, I))):
        w = WL.gpu_weight_f32(E * N, K, seed=70_000 + j, device=dev)
        stacks[name] = (api.nf4_quantize(w, code, ncode).per_expert(E), N, K)
        del w
    xin = {n: WL.gpu_normal_bf16(T, K, seed=71_000 + j, device=dev) for j, (n, (_, N, K)) in enumerate(stacks.items())}
    gin = {n: WL.gpu_normal_bf16(T, N, seed=72_000 + j, device=dev) for j, (n, (_, N, K)) in enumerate(stacks.items())}
    outs = {n: torch.empty((T, N), dtype=torch.bfloat16, device=dev) for n, (_, N, K) in stacks.items()}
    gouts = {n: torch.empty((T, K), dtype=torch.bfloat16, device=dev) for n, (_, N, K) in stacks.items()}

    def moe_fwd():
        for n, (wq, N, K) in stacks.items():
            api.nf4_grouped_matmul_fwd(xin[n], off, wq, E, out=outs[n])

    def moe_bwd():
        for n, (wq, N, K) in stacks.items():
            api.nf4_grouped_matmul_bwd_input(gin[n], off, wq, E, out=gouts[n])

    # medians of interleaved rounds: a sample is 5 passes over the three
    # stacks after a 1 GiB copy (the first pass reads the 208 MB of packed
    # stacks from HBM; they fit the 256 MB last-level cache for the others)
    med = interleaved(torch, stream, {"fwd": moe_fwd, "bwd": moe_bwd}, filler_copy(torch, dev))
    ms_f, ms_b = med["fwd"]["median_us"] * 1e-3, med["bwd"]["median_us"] * 1e-3
    fl = sum(2.0 * T * N * K for (_, N, K) in stacks.values())
    wb = sum(wq.nbytes() for (wq, _, _) in stacks.values())
    extra["olmoe_grouped"] = {
        "fwd_us": round(ms_f * 1e3, 1), "bwd_us": round(ms_b * 1e3, 1),
        "p10_p90_us": {d: [med[d]["p10_us"], med[d]["p90_us"]] for d in ("fwd", "bwd")},
        "fwd_tflops": round(fl / (ms_f * 1e-3) / 1e12, 1),
        "bwd_tflops": round(fl / (ms_b * 1e-3) / 1e12, 1),
        "fwd_weight_GBps": round(wb / (ms_f * 1e-3) / 1e9, 1),
        "rows": T,
        "timing": "per direction: median over 21 interleaved rounds of 5 passes over the three stacks",
    }
    return extra


def run_code_tables(torch, api, WL, ncode, dev, stream, filler, ceil):
    """The code-table variants of the same calls (Experts PR, "Commit 1",
    quant_type table): nf4 and fp4 (16-entry tables, the same kernels) and the
    8-bit blockwise int8 and fp8 e4m3 formats (one byte per weight, 256-entry
    tables, the 8-bit register-staged tiles).  Layer 0's seven Llama-3.1-8B
    projections are quantised from the same fp32 weights in each format (all
    nested); per projection the four formats are interleaved round by round:
    forward + input gradient at M = 512, forward at M = 1.  Figures are sums
    over the projections.  Every call is also compared with the dense product
    of its own dequantised weight, and the path counters with its kernels."""
    import torch.nn.functional as F
    tables = {"nf4": (WL.nf4_code_np(), 4), "fp4": (WL.fp4_code_np(), 4),
              "int8": (WL.int8_code_np(), 8), "fp8_e4m3": (WL.fp8_e4m3_code_np(), 8)}
    codes = {f: (torch.from_numpy(t).to(dev), b) for f, (t, b) in tables.items()}
    M, projs = WL.LLAMA_M, WL.LLAMA_8B
    res = {f: {"m512_fwd_bwd_us": 0.0, "m1_fwd_us": 0.0, "weight_bytes": 0, "max_rel_fro_diff": 0.0,
               "kernels_ran": True} for f in tables}
    for i, p in enumerate(projs):
        wf = WL.gpu_weight_f32(p.N, p.K, seed=WL.stack_weight_seed(WL.LLAMA_STACK_W_SEED, 0, i), device=dev)
        wq = {f: api.nf4_quantize(wf, c, ncode, bits=b) for f, (c, b) in codes.items()}
        del wf
        x = WL.gpu_normal_bf16(M, p.K, seed=93_000 + i, device=dev)
        gy = WL.gpu_normal_bf16(M, p.N, seed=94_000 + i, device=dev)
        x1 = WL.gpu_normal_bf16(1, p.K, seed=95_000 + i, device=dev)
        wsb = workspace_for(torch, api, [p], [M, 1], dev)
        y = torch.empty((M, p.N), dtype=torch.bfloat16, device=dev)
        g = torch.empty((M, p.K), dtype=torch.bfloat16, device=dev)
        y1 = torch.empty((1, p.N), dtype=torch.bfloat16, device=dev)

        def fwd_bwd(w):
            return lambda: (api.nf4_matmul_fwd(x, w, out=y, ws=wsb), api.nf4_matmul_bwd_input(gy, w, out=g, ws=wsb))

        def fwd1(w):
            return lambda: api.nf4_matmul_fwd(x1, w, out=y1, ws=wsb)

        m512 = interleaved(torch, stream, {f: fwd_bwd(w) for f, w in wq.items()}, filler, rounds=11)
        m1 = interleaved(torch, stream, {f: fwd1(w) for f, w in wq.items()}, filler, rounds=11)
        for f, w in wq.items():
            r = res[f]
            r["m512_fwd_bwd_us"] += m512[f]["median_us"]
            r["m1_fwd_us"] += m1[f]["median_us"]
            r["weight_bytes"] += w.nbytes()
            api.nf4_reset_path_counts()
            fwd_bwd(w)()
            fwd1(w)()
            torch.cuda.synchronize()
            pc = api.nf4_path_counts()
            if w.bits == 8:
                ok = pc["fwd_8bit"] == 2 and pc["bwd_8bit"] == 1
            else:
                ok = pc["fwd_tiled"] + pc["fwd_small_m"] == 2 and pc["bwd_tiled"] == 1
            r["kernels_ran"] = r["kernels_ran"] and ok
            wd = api.nf4_dequantize(w)
            for got, ref in ((y, F.linear(x, wd)), (g, torch.matmul(gy, wd)), (y1, F.linear(x1, wd))):
                rel = float((got.float() - ref.float()).norm().item() / max(ref.float().norm().item(), 1e-30))
                r["max_rel_fro_diff"] = max(r["max_rel_fro_diff"], rel)
            del wd
        del wq, x, gy, x1, wsb, y, g, y1
    flops = 2 * sum(2.0 * M * p.N * p.K for p in projs)
    nweights = sum(p.N * p.K for p in projs)
    out = {}
    for f, r in res.items():
        t5, t1 = r["m512_fwd_bwd_us"], r["m1_fwd_us"]
        gbs = r["weight_bytes"] / (t1 * 1e-6) / 1e9
        out[f] = {"m512_fwd_bwd_us": round(t5, 1), "m512_tflops": round(flops / (t5 * 1e-6) / 1e12, 1),
                  "m512_frac_of_bf16_peak": round(flops / (t5 * 1e-6) / 1e12 / PEAK_BF16_TFLOPS, 4),
                  "m1_fwd_us": round(t1, 1), "m1_weight_GBps": round(gbs, 1),
                  "m1_frac_of_copy_ceiling": round(gbs / ceil["GBps"], 4),
                  "bytes_per_weight": round(r["weight_bytes"] / nweights, 4),
                  "max_rel_fro_diff": float(f"{r['max_rel_fro_diff']:.3g}"), "kernels_ran": r["kernels_ran"]}
    out["timing"] = ("per projection, the four formats interleaved: median over 11 rounds of 5 calls, each round "
                     "after a 1 GiB filler copy; figures summed over the seven projections")
    out["summary"] = {f: [out[f]["m512_tflops"], out[f]["m1_weight_GBps"]] for f in tables}
    return out


def run_streaming(torch, api, WL, dev, llama_weights, stream, slots=3):
    """The 32-layer step with every layer's NF4 fields copied from page-locked
    host memory into a ring of device slots on each visit (forward in order,
    input gradients in reverse: 64 visits), against the same step on resident
    weights.  Reports tokens/s and the arm's device bytes (persistent weights
    or slots, plus the step's transient peak) together, the copy-only time of
    the same visit sequence, and whether the outputs are bit-identical."""
    from nf4_bit_weight_amd.streaming import LayerBuffer, SlotStreamer
    projs = WL.LLAMA_8B
    names = [p.name for p in projs]
    L, M = len(llama_weights), WL.LLAMA_M
    host = [LayerBuffer(names, row, pin_memory=True) for row in llama_weights]
    xs = [WL.gpu_normal_bf16(M, p.K, seed=93_000 + i, device=dev) for i, p in enumerate(projs)]
    gys = [WL.gpu_normal_bf16(M, p.N, seed=94_000 + i, device=dev) for i, p in enumerate(projs)]
    ys = [torch.empty((M, p.N), dtype=torch.bfloat16, device=dev) for p in projs]
    gxs = [torch.empty((M, p.K), dtype=torch.bfloat16, device=dev) for p in projs]
    ws = workspace_for(torch, api, projs, [M], dev)
    visits = list(range(L)) + list(reversed(range(L)))

    def fn(v, layer, w):
        for i, n in enumerate(names):
            if v < L:
                api.nf4_matmul_fwd(xs[i], w[n], out=ys[i], ws=ws)
            else:
                api.nf4_matmul_bwd_input(gys[i], w[n], out=gxs[i], ws=ws)

    def resident():
        for v, layer in enumerate(visits):
            fn(v, layer, dict(zip(names, llama_weights[layer])))

    st = SlotStreamer(host, slots, dev)

    def measure(run, persistent):
        torch.cuda.synchronize()
        base = torch.cuda.memory_allocated()
        torch.cuda.reset_peak_memory_stats()
        ms = timed(torch, stream, run, steps=3, warmup=1)
        peak = torch.cuda.max_memory_allocated() - base
        return ms, persistent + peak

    wbytes = sum(w.nbytes() for row in llama_weights for w in row)
    ms_r, mem_r = measure(resident, wbytes)
    resident()
    y_r, g_r = ys[6].clone(), gxs[0].clone()
    ms_s, mem_s = measure(lambda: st.run(visits, fn), st.device_bytes)
    st.run(visits, fn)
    torch.cuda.synchronize()
    same = bool(torch.equal(ys[6].view(torch.int16), y_r.view(torch.int16)) and
                torch.equal(gxs[0].view(torch.int16), g_r.view(torch.int16)))
    ms_c = timed(torch, stream, lambda: st.run(visits, lambda v, l, w: None), steps=3, warmup=1)
    copied = 2 * sum(h.nbytes for h in host)
    out = {
        "slots": slots, "layer_MiB": round(host[0].nbytes / 2 ** 20, 1),
        "resident_ms_per_step": round(ms_r, 2), "resident_tokens_per_s": round(M / (ms_r * 1e-3), 1),
        "resident_device_MiB": round(mem_r / 2 ** 20, 1),
        "streamed_ms_per_step": round(ms_s, 2), "streamed_tokens_per_s": round(M / (ms_s * 1e-3), 1),
        "streamed_device_MiB": round(mem_s / 2 ** 20, 1),
        "copy_only_ms_per_step": round(ms_c, 2),
        "h2d_GBps": round(copied / (ms_c * 1e-3) / 1e9, 1),
        "bitwise_equal_to_resident": same,
    }
    del host, st
    return out


# ---------------------------------------------------------------------------
def _repeat(fn, min_s, max_reps):
    """Run fn until at least min_s seconds have passed (at most max_reps times)."""
    reps = 0
    t0 = time.perf_counter()
    while reps < max_reps and (reps == 0 or time.perf_counter() - t0 < min_s):
        fn()
        reps += 1
    return reps, time.perf_counter() - t0


def cpu_baseline(WL):
    """The CPU oracle, as it stands, on bounded samples of the workloads:
    the headline figure is layer 0 of the Llama-3.1-8B stack at M = 512, all 7
    projections, each dequantised from its packed NF4 form and multiplied
    forward and backward (the oracle's fp64 matmul); "breadth" times the same
    oracle on the tiny linear, on decode (M = 1), on one Qwen-32B projection
    at M = 2048 and on 8 of the 64 OLMoE experts.  Quantisation is set-up and
    not timed."""
    import numpy as np
    from oracle import nf4_oracle as O

    threads = None
    try:
        from threadpoolctl import threadpool_info
        threads = max((d.get("num_threads") or 0) for d in threadpool_info()) or None
    except Exception:
        pass
    code, ncode = WL.nf4_code_np(), WL.nested_code_np()

    def deq(q, shape, nested=True):
        return O.dequantize_nf4_bf16_bits(q["packed"], q["absmax"], q["nested_absmax"] if nested else None,
                                          q["nested_offset"] if nested else None, code,
                                          ncode if nested else None).reshape(shape)

    projs = WL.LLAMA_8B
    M = WL.LLAMA_M
    qs = []
    for i, p in enumerate(projs):
        w = WL.weight_f32(p.N, p.K, WL.W_LLAMA, 0, i)
        qs.append(O.quantize_nf4(w, code, ncode, nested=True))
        del w
    x = {p.K: WL.bf16_bits(WL.x_bf16(M, p.K, WL.W_LLAMA, 0)) for p in projs}
    gy = [WL.bf16_bits(WL.grad_y_bf16(M, p.N, WL.W_LLAMA, 0, i)) for i, p in enumerate(projs)]

    def layer_pass():
        for i, p in enumerate(projs):
            wb = deq(qs[i], (p.N, p.K))
            O.matmul_fwd(x[p.K], wb)
            O.matmul_bwd_input(gy[i], wb)

    passes, dt = _repeat(layer_pass, 6.0, 8)
    flops = passes * 2 * sum(2.0 * M * p.N * p.K for p in projs)
    breadth = {}

    # tiny linear: M = 64, N = 128, K = 256, plain NF4
    wt = WL.weight_f32(WL.TINY_N, WL.TINY_K, WL.W_TINY, 0)
    qt = O.quantize_nf4(wt, code)
    xt = WL.bf16_bits(WL.x_bf16(WL.TINY_M, WL.TINY_K, WL.W_TINY, 0))
    gt = WL.bf16_bits(WL.grad_y_bf16(WL.TINY_M, WL.TINY_N, WL.W_TINY, 0))

    def tiny():
        wb = deq(qt, (WL.TINY_N, WL.TINY_K), nested=False)
        O.matmul_fwd(xt, wb)
        O.matmul_bwd_input(gt, wb)

    n, t = _repeat(tiny, 0.5, 10_000)
    breadth["tiny_linear"] = {"value": round(n * 2 * 2.0 * WL.TINY_M * WL.TINY_N * WL.TINY_K / t / 1e9, 4),
                              "unit": "GFLOP/s", "seconds": round(t, 2),
                              "sample": f"M=64 N=128 K=256 plain NF4, {n} passes of dequantise + fwd + bwd_input"}

    # decode: layer 0's attention projections (q, k, v, o) forward at M = 1,
    # rated on their packed weight bytes
    x1 = {p.K: WL.bf16_bits(WL.x_bf16(1, p.K, WL.W_DECODE, 0)) for p in projs[:4]}

    def decode():
        for i, p in enumerate(projs[:4]):
            O.matmul_fwd(x1[p.K], deq(qs[i], (p.N, p.K)))

    n, t = _repeat(decode, 0.0, 1)
    wbytes = sum(O.storage_bytes(p.N * p.K, True) for p in projs[:4])
    breadth["decode_m1"] = {"value": round(n * wbytes / t / 1e9, 4), "unit": "GB/s of packed weights",
                            "seconds": round(t, 2),
                            "sample": "Llama-3.1-8B layer 0 q/k/v/o at M=1, 1 pass of dequantise + fwd"}

    # Qwen-32B q projection (5120 x 5120) at M = 2048, forward and backward
    qp = WL.QWEN_32B[0]
    wq = WL.weight_f32(qp.N, qp.K, WL.W_QWEN, 0, 0)
    qq = O.quantize_nf4(wq, code, ncode, nested=True)
    del wq
    xq = WL.bf16_bits(WL.x_bf16(WL.QWEN_M, qp.K, WL.W_QWEN, 0))
    gq = WL.bf16_bits(WL.grad_y_bf16(WL.QWEN_M, qp.N, WL.W_QWEN, 0, 0))

    def qwen():
        wb = deq(qq, (qp.N, qp.K))
        O.matmul_fwd(xq, wb)
        O.matmul_bwd_input(gq, wb)

    n, t = _repeat(qwen, 0.0, 1)
    breadth["qwen32b_q_m2048"] = {"value": round(n * 2 * 2.0 * WL.QWEN_M * qp.N * qp.K / t / 1e12, 5),
                                  "unit": "TFLOP/s", "seconds": round(t, 2),
                                  "sample": "Qwen-32B q projection at M=2048, 1 pass of dequantise + fwd + bwd_input"}

    # OLMoE: experts 0..7 of the gate, up and down stacks with their routed rows
    E8, H, I = 8, WL.OLMOE_HIDDEN, WL.OLMOE_INTER
    _, _, offsets = WL.olmoe_routing()
    off8 = offsets[:E8 + 1].astype(np.int32)
    T8 = int(off8[-1])
    stacks = []
    for j, (N, K) in enumerate(((I, H), (I, H), (H, I))):
        w8 = WL.weight_f32(E8 * N, K, WL.W_OLMOE, 0, j)
        stacks.append((O.quantize_nf4(w8, code, ncode, nested=True), N, K,
                       WL.bf16_bits(WL.x_bf16(T8, K, WL.W_OLMOE, 0, j)),
                       WL.bf16_bits(WL.grad_y_bf16(T8, N, WL.W_OLMOE, 0, j))))
        del w8

    def olmoe():
        for q, N, K, xe, ge in stacks:
            wb = deq(q, (E8, N, K))
            O.grouped_matmul_fwd(xe, off8, wb)
            O.grouped_matmul_bwd_input(ge, off8, wb)

    n, t = _repeat(olmoe, 0.0, 1)
    fl = sum(2 * 2.0 * T8 * N * K for _, N, K, _, _ in stacks)
    breadth["olmoe_8_experts"] = {"value": round(n * fl / t / 1e12, 5), "unit": "TFLOP/s",
                                  "seconds": round(t, 2),
                                  "sample": f"OLMoE gate/up/down experts 0-7 ({T8} routed rows), 1 pass of "
                                            f"dequantise + grouped fwd + grouped bwd_input"}
    return {"value": round(flops / dt / 1e12, 5), "unit": "TFLOP/s",
            "cores": threads or len(os.sched_getaffinity(0)), "kind": "oracle",
            "sample": f"Llama-3.1-8B layer 0 (7 projections) at M=512, {passes} pass(es): dequantise "
                      f"+ fwd + bwd_input, NumPy oracle (fp64 matmul)",
            "seconds": round(dt, 2), "host_cpus": len(os.sched_getaffinity(0)),
            "breadth": breadth}


# ---------------------------------------------------------------------------
def run_only(args):
    """One shape of a workload, launched with distinct weights per call as in
    the step, `steps` times.  FAMILY:DIR_PROJ names it: llama:fwd_gate (the
    32 layers' forward gate projections of the M = 512 step; "llama:" may be
    left out), qwen:bwd_down (8 distinct Qwen-32B down weights at M = 2048),
    olmoe:fwd_gate (4 distinct copies of the OLMoE gate expert stack, grouped
    call over the 4096 routed rows)."""
    import torch

    import workloads as WL
    from nf4_bit_weight_amd import api

    family, _, shape = args.only.rpartition(":")
    family = family or "llama"
    d, name = shape.split("_", 1)
    if d not in ("fwd", "bwd") or family not in ("llama", "qwen", "olmoe"):
        raise SystemExit(f"--only {args.only}: expected [llama:|qwen:|olmoe:](fwd|bwd)_<projection>")
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    tab = {"nf4": WL.nf4_code_np, "fp4": WL.fp4_code_np, "int8": WL.int8_code_np,
           "fp8_e4m3": WL.fp8_e4m3_code_np}[args.code]()
    bits = 8 if args.code in ("int8", "fp8_e4m3") else 4
    code = torch.from_numpy(tab).to(dev)
    ncode = torch.from_numpy(WL.nested_code_np()).to(dev)
    off = None
    if family == "olmoe":
        E, H, I = WL.OLMOE_E, WL.OLMOE_HIDDEN, WL.OLMOE_INTER
        dims = {"gate": (I, H), "up": (I, H), "down": (H, I)}
        N, K = dims[name]
        j = list(dims).index(name)
        _, _, offsets = WL.olmoe_routing()
        off = torch.from_numpy(offsets).to(dev)
        M, L = int(offsets[-1]), 4
        wts = []
        for l in range(L):
            w = WL.gpu_weight_f32(E * N, K, seed=70_000 + 16 * l + j, device=dev)
            wts.append(api.nf4_quantize(w, code, ncode, bits=bits).per_expert(E))
            del w
    else:
        projs = WL.LLAMA_8B if family == "llama" else WL.QWEN_32B
        i = [p.name for p in projs].index(name)
        N, K = projs[i].N, projs[i].K
        if family == "llama":
            M, L, seed0 = (args.m or WL.LLAMA_M), WL.LLAMA_LAYERS, 10_000
        else:
            M, L, seed0 = (args.m or WL.QWEN_M), 8, 50_000
        wts = []
        for l in range(L):
            w = WL.gpu_weight_f32(N, K, seed=WL.stack_weight_seed(seed0, l, i), device=dev)
            wts.append(api.nf4_quantize(w, code, ncode, bits=bits))
            del w
    ins = [WL.gpu_normal_bf16(M, K if d == "fwd" else N, seed=30_000 + l, device=dev) for l in range(L)]
    out = torch.empty((M, N if d == "fwd" else K), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(max(16, *(api.nf4_workspace_bytes(op, M, N, K) for op in (1, 2, 5, 6))),
                     dtype=torch.uint8, device=dev)

    def one():
        for l in range(L):
            if off is not None:
                if d == "fwd":
                    api.nf4_grouped_matmul_fwd(ins[l], off, wts[l], WL.OLMOE_E, out=out)
                else:
                    api.nf4_grouped_matmul_bwd_input(ins[l], off, wts[l], WL.OLMOE_E, out=out)
            elif d == "fwd":
                api.nf4_matmul_fwd(ins[l], wts[l], out=out, ws=ws)
            else:
                api.nf4_matmul_bwd_input(ins[l], wts[l], out=out, ws=ws)

    ms = timed(torch, stream, one, args.steps, args.warmup) / L
    flops = 2.0 * M * N * K
    wbytes = wts[0].nbytes()
    if args.copy_bytes > 0:
        src = torch.ones(args.copy_bytes, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
    print(json.dumps({"shape": f"{family}:{shape}", "code": args.code, "M": M, "N": N, "K": K,
                      "experts": WL.OLMOE_E if off is not None else None,
                      "ops": L * (args.steps + args.warmup), "avg_us": round(ms * 1e3, 2),
                      "tflops": round(flops / (ms * 1e-3) / 1e12, 1),
                      "weight_GBps": round(wbytes / (ms * 1e-3) / 1e9, 1),
                      "copy_bytes": args.copy_bytes}), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU; --gpus {args.gpus} is not supported here.  The "
              f"data-parallel path needs no collective (each GPU runs this step on its own rows "
              f"of x and grad_y against a replica of the frozen packed weights).", file=sys.stderr)
        sys.exit(2)

    if args.only:
        run_only(args)
        return

    import torch

    import workloads as WL
    from nf4_bit_weight_amd import api
    from nf4_bit_weight_amd import profiling

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    clk_before = clocks()
    code = torch.from_numpy(WL.nf4_code_np()).to(dev)
    ncode = torch.from_numpy(WL.nested_code_np()).to(dev)

    M, L, projs = WL.LLAMA_M, WL.LLAMA_LAYERS, WL.LLAMA_8B
    t0 = time.time()
    log("building the 32-layer Llama-3.1-8B NF4 stack")
    weights = build_stack(torch, api, WL, projs, L, code, ncode, dev, seed0=WL.LLAMA_STACK_W_SEED)
    xs, gys = layer_inputs(torch, WL, projs, L, M, dev, seed0=WL.LLAMA_STACK_IN_SEED)
    ys = [torch.empty((M, p.N), dtype=torch.bfloat16, device=dev) for p in projs]
    gxs = [torch.empty((M, p.K), dtype=torch.bfloat16, device=dev) for p in projs]
    ws = workspace_for(torch, api, projs, [M], dev)
    torch.cuda.synchronize()
    setup_s = time.time() - t0
    weight_bytes = sum(w.nbytes() for row in weights for w in row)

    flops_gemm = {i: 2.0 * M * p.N * p.K for i, p in enumerate(projs)}
    flops_step = 2 * L * sum(flops_gemm.values())

    log(f"stack ready in {time.time() - t0:.1f}s; timing {args.steps} steps")
    wall0 = time.perf_counter()
    ms_step = timed(torch, stream, lambda: run_stack_step(api, weights, xs, gys, ys, gxs, ws),
                    args.steps, args.warmup)
    wall = time.perf_counter() - wall0
    tflops = flops_step / (ms_step * 1e-3) / 1e12

    log(f"{ms_step:.3f} ms/step = {tflops:.1f} TFLOP/s; per-shape timing")
    # Per-shape timing for the roofline: for each (direction, projection) the
    # 32 launches of one step (one per layer, distinct weights) run back to
    # back between two HIP events on the launch stream; avg = span / 32.
    per = {}
    for d in ("fwd", "bwd"):
        for i, p in enumerate(projs):
            def one(i=i, d=d):
                for l in range(L):
                    if d == "fwd":
                        api.nf4_matmul_fwd(xs[l][i], weights[l][i], out=ys[i], ws=ws)
                    else:
                        api.nf4_matmul_bwd_input(gys[l][i], weights[l][i], out=gxs[i], ws=ws)
            per[(d, i)] = timed(torch, stream, one, steps=3, warmup=1) / L       # ms per launch
    per_kernel = {}
    for (d, i), avg in sorted(per.items()):
        per_kernel[f"{d}_{projs[i].name}"] = {"avg_us": round(avg * 1e3, 2),
                                              "tflops": round(flops_gemm[i] / (avg * 1e-3) / 1e12, 1)}
    dom = max(per, key=lambda k: per[k])                 # largest share of the step
    dom_avg_s = per[dom] * 1e-3
    achieved = flops_gemm[dom[1]] / dom_avg_s / 1e12
    p = projs[dom[1]]
    roofline = {
        "bound": "mfma",
        "kernel": f"fused NF4 {'forward' if dom[0] == 'fwd' else 'input gradient'} "
                  f"{p.name} (M={M}, N={p.N}, K={p.K})",
        "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
        "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": None,
        "avg_launch_us": round(dom_avg_s * 1e6, 2),
    }
    # HBM bytes per launch from the committed rocprofv3 counter summary of this
    # shape, if it was measured on the kernel sources built here
    fig = profiling.read_traffic(traffic_file(dom[0], p.name, M))
    if fig is not None:
        roofline["traffic"] = fig["bytes_per_op"]
        roofline["traffic_source"] = os.path.relpath(traffic_file(dom[0], p.name, M), ROOT)

    extra = {}
    if not args.no_extra:
        log("secondary workloads")
        del xs, gys, ys, gxs
        extra = run_extra(torch, api, WL, code, ncode, dev, weights, stream)
    if not args.no_cpu:
        log("oracle CPU baseline")
    cpu = None if args.no_cpu else cpu_baseline(WL)

    line = {
        "metric": METRIC, "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic: seeded N(0,1) bf16 activations, 0.02*N(0,1) weights quantised to nested NF4 on the GPU",
        "config": {
            "workload": "Llama-3.1-8B NF4 projections, batch 1 x S=512 (M=512), 32 layers x 7 "
                        "projections, fused forward then fused input gradient",
            "M": M, "layers": L, "projections": {q.name: [q.N, q.K] for q in projs},
            "nested": True, "weight_bytes": weight_bytes,
            "tflop_per_step": round(flops_step / 1e12, 3),
        },
        "pct_of_bf16_peak": round(100 * tflops / PEAK_BF16_TFLOPS, 2),
        "roofline": roofline,
        "cpu_baseline": cpu,
        "per_kernel": per_kernel,
        "extra": extra,
        "clocks": {"before": clk_before, "after": clocks()},
        "setup_s": round(setup_s, 1),
        "timed_wall_s": round(wall, 3),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
