"""Summaries of rocprofv3 output for the fused NF4 kernels.

Turns the CSV files rocprofv3 writes (``--kernel-trace --stats`` and
``--pmc``) into the short text summaries kept with the project, and reads the
HBM-traffic figure back for the benchmark line.  Needs no GPU.

    python -m nf4_bit_weight_amd.profiling stats  <kernel_stats.csv> <out.md> "<command>"
    python -m nf4_bit_weight_amd.profiling traffic <fetch_counter_collection.csv>
           <write_counter_collection.csv> <copy_bytes> <ops> <out.md> "<shape>" "<command>"
    python -m nf4_bit_weight_amd.profiling mfma <counter_collection.csv> <flops_per_op>
           <out.md> "<shape>" "<command>"
    python -m nf4_bit_weight_amd.profiling lds <counter_collection.csv> <out.md> "<shape>" "<command>"
    python -m nf4_bit_weight_amd.profiling counters <counter_collection.csv> <copy_bytes> <ops>
           <bytes_per_op> <out.md> "<shape>" "<command>"

MFMA: one rocprofv3 run collecting the derived MfmaUtil and VALUBusy metrics
(percent of the dispatch's active cycles in which the MFMA unit, resp. the
vector ALU, was busy, averaged over SIMDs / CUs) and SQ_INSTS_VALU_MFMA_MOPS_BF16
(bf16 MFMA work in units of 512 flops), averaged over the fused matmul
dispatches; the counted flops are checked against 2 M N K.

Counters: every counter of one run summed over the fused dispatches and
divided by the operations; FETCH_SIZE / WRITE_SIZE also in bytes, scaled by
the calibration copy as below, and set against the algorithmic bytes of one
operation (the decode runs: FETCH_SIZE with SQ_INSTS_VALU and GRBM_GUI_ACTIVE).

Traffic: FETCH_SIZE and WRITE_SIZE (KiB per dispatch, one rocprofv3 run
each) summed over the dispatches of the measured operation (the fused GEMM
and, when the contraction is split, its reduction), divided by the number of
operations, each scaled by the factor that maps the same counter onto the
known byte count of a plain device-to-device copy measured in the same run.
"""

from __future__ import annotations

import csv
import hashlib
import json
import os
import re
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
KERNEL_SOURCES = ("csrc/nf4_gemm.hip", "csrc/nf4_gemv.hip", "csrc/nf4_device.hpp")
COPY_KERNEL = "__amd_rocclr_copyBuffer"
FUSED_KERNELS = ("k_gemm<", "k_pp<", "k_rb<", "k_gemv<", "k_gemv_ln<", "k_gemmt<", "k_splitk_reduce")
MFMA_KERNELS = ("k_gemm<", "k_pp<", "k_rb<", "k_gemv<", "k_gemv_ln<", "k_gemmt<")


def _code_only(text: str) -> str:
    """C++ source with comments removed and whitespace collapsed (string and
    character literals kept), so that a comment edit keeps the hash."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c == "/" and i + 1 < n and text[i + 1] == "/":
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif c == "/" and i + 1 < n and text[i + 1] == "*":
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        elif c in "\"'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def kernel_source_sha256() -> str:
    """Hash of the code (comments and layout excluded) the fused kernels are
    built from: a traffic figure taken from counters is valid only for the
    kernel it was measured on."""
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(PKG, rel), encoding="utf-8") as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()


def _short(name: str, width: int = 96) -> str:
    name = name.replace("nf4::(anonymous namespace)::", "").replace("(GemmParams)", "")
    name = re.sub(r"^void ", "", name)
    return name if len(name) <= width else name[: width - 3] + "..."


def summarize_stats(stats_csv: str, out_md: str, command: str, top: int = 12) -> None:
    rows = list(csv.DictReader(open(stats_csv)))
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    lines = [
        "# rocprofv3 kernel statistics",
        "",
        "Command (run from the repository root on one MI355X):",
        "",
        "```",
        command,
        "```",
        "",
        "| kernel | calls | total ms | avg us | min us | max us | % |",
        "|---|---:|---:|---:|---:|---:|---:|",
    ]
    for r in rows[:top]:
        lines.append(
            f"| `{_short(r['Name'])}` | {r['Calls']} | {float(r['TotalDurationNs']) / 1e6:.3f} | "
            f"{float(r['AverageNs']) / 1e3:.2f} | {float(r['MinNs']) / 1e3:.2f} | "
            f"{float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.2f} |")
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")


def _per_dispatch(pmc_csv: str, counter: str):
    """{dispatch_id: (kernel_name, value)} for one counter."""
    out = {}
    for r in csv.DictReader(open(pmc_csv)):
        if r["Counter_Name"] != counter:
            continue
        d = int(r["Dispatch_Id"])
        name, val = r["Kernel_Name"], float(r["Counter_Value"])
        if d in out:
            out[d] = (name, out[d][1] + val)
        else:
            out[d] = (name, val)
    return out


def traffic_figures(fetch_csv: str, write_csv: str, copy_bytes: int, ops: int) -> dict:
    res = {}
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        disp = _per_dispatch(path, counter)
        copies = [v for (n, v) in disp.values() if COPY_KERNEL in n]
        fused = [v for (n, v) in disp.values() if any(k in n for k in FUSED_KERNELS)]
        if not copies or not fused:
            raise RuntimeError(f"{path}: no copy or no fused-kernel dispatches for {counter}")
        copy_kib = max(copies)                     # the calibration copy is the largest one
        factor = (copy_bytes / 1024.0) / copy_kib
        res[counter] = {
            "copy_kib": round(copy_kib, 1), "factor": round(factor, 4),
            "fused_dispatches": len(fused),
            "kib_per_op_raw": round(sum(fused) / ops, 1),
            "bytes_per_op": round(sum(fused) / ops * 1024.0 * factor),
        }
    res["bytes_per_op"] = res["FETCH_SIZE"]["bytes_per_op"] + res["WRITE_SIZE"]["bytes_per_op"]
    return res


def summarize_traffic(fetch_csv, write_csv, copy_bytes, ops, out_md, shape, command) -> dict:
    fig = traffic_figures(fetch_csv, write_csv, int(copy_bytes), int(ops))
    fig["shape"] = shape
    fig["ops"] = int(ops)
    fig["copy_bytes"] = int(copy_bytes)
    fig["kernel_source_sha256"] = kernel_source_sha256()
    lines = [
        f"# HBM traffic of the fused NF4 GEMM: {shape}",
        "",
        "Two rocprofv3 counter runs (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch) of:",
        "",
        "```",
        command,
        "```",
        "",
        f"Each counter is scaled by the factor that maps it onto a plain {copy_bytes} B "
        f"device-to-device copy (`{COPY_KERNEL}`) measured in the same run; the sum over the "
        f"fused GEMM and split-K reduction dispatches is divided by the {ops} operations.",
        "",
        "```json",
        json.dumps(fig, indent=1),
        "```",
    ]
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")
    return fig


def mfma_figures(pmc_csv: str, flops_per_op: float) -> dict:
    util = _per_dispatch(pmc_csv, "MfmaUtil")
    valu = _per_dispatch(pmc_csv, "VALUBusy")
    mops = _per_dispatch(pmc_csv, "SQ_INSTS_VALU_MFMA_MOPS_BF16")
    ids = [d for d, (n, _) in util.items() if any(k in n for k in MFMA_KERNELS)]
    if not ids:
        raise RuntimeError(f"{pmc_csv}: no fused matmul dispatches")
    names = sorted({_short(util[d][0]) for d in ids})
    avg = lambda m: sum(m[d][1] for d in ids if d in m) / max(1, sum(1 for d in ids if d in m))
    flops = avg(mops) * 512.0
    return {
        "kernels": names, "dispatches": len(ids),
        "MfmaUtil_pct": round(avg(util), 2), "VALUBusy_pct": round(avg(valu), 2),
        "bf16_mfma_flops_per_dispatch": round(flops),
        "algorithmic_flops_per_op": round(flops_per_op),
        "counted_over_algorithmic": round(flops / flops_per_op, 4) if flops_per_op else None,
    }


def summarize_mfma(pmc_csv, flops_per_op, out_md, shape, command) -> dict:
    fig = mfma_figures(pmc_csv, float(flops_per_op))
    fig["shape"] = shape
    fig["kernel_source_sha256"] = kernel_source_sha256()
    lines = [
        f"# MFMA utilisation of the fused NF4 GEMM: {shape}",
        "",
        "One rocprofv3 counter run (MfmaUtil, VALUBusy, SQ_INSTS_VALU_MFMA_MOPS_BF16, GRBM_GUI_ACTIVE) of:",
        "",
        "```",
        command,
        "```",
        "",
        "MfmaUtil is the share of the dispatch's active cycles in which a SIMD's MFMA unit was "
        "busy, averaged over all SIMDs; it is the counter form of the fraction of the bf16 dense "
        "peak reached while the kernel runs. Counter runs serialise dispatches, so durations are "
        "taken from the kernel-trace statistics, not from this run. A split contraction runs "
        "inside the one fused dispatch (its fixed-order reduction is a separate, MFMA-free dispatch), "
        "so each fused dispatch counts the whole 2 M N K.",
        "",
        "```json",
        json.dumps(fig, indent=1),
        "```",
    ]
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")
    return fig


def lds_figures(pmc_csv: str) -> dict:
    """LDS counters averaged over the fused matmul dispatches, and the derived
    bank-conflict ratio (conflict cycles over conflict-free active cycles, the
    form of rocprofv3's LdsBankConflict metric)."""
    names = ("SQ_LDS_IDX_ACTIVE", "SQ_LDS_BANK_CONFLICT", "SQ_LDS_ADDR_CONFLICT",
             "SQ_LDS_UNALIGNED_STALL", "SQ_INSTS_LDS", "SQ_WAIT_INST_LDS")
    per = {c: _per_dispatch(pmc_csv, c) for c in names}
    ids = [d for d, (n, _) in per["SQ_LDS_IDX_ACTIVE"].items() if any(k in n for k in MFMA_KERNELS)]
    if not ids:
        raise RuntimeError(f"{pmc_csv}: no fused matmul dispatches")
    avg = {c: sum(per[c][d][1] for d in ids if d in per[c]) / len(ids) for c in names}
    act, bc = avg["SQ_LDS_IDX_ACTIVE"], avg["SQ_LDS_BANK_CONFLICT"]
    return {
        "kernels": sorted({_short(per["SQ_LDS_IDX_ACTIVE"][d][0]) for d in ids}),
        "dispatches": len(ids),
        **{c: round(v) for c, v in avg.items()},
        "bank_conflict_ratio": round(bc / (act - bc), 4) if act > bc else None,
    }


def summarize_lds(pmc_csv, out_md, shape, command) -> dict:
    fig = lds_figures(pmc_csv)
    fig["shape"] = shape
    fig["kernel_source_sha256"] = kernel_source_sha256()
    lines = [
        f"# LDS counters of the fused NF4 GEMM: {shape}",
        "",
        "One rocprofv3 counter run of:",
        "",
        "```",
        command,
        "```",
        "",
        "Per-dispatch averages over the fused matmul dispatches. bank_conflict_ratio is "
        "SQ_LDS_BANK_CONFLICT / (SQ_LDS_IDX_ACTIVE - SQ_LDS_BANK_CONFLICT): extra LDS cycles "
        "spent on bank conflicts per conflict-free LDS cycle.",
        "",
        "```json",
        json.dumps(fig, indent=1),
        "```",
    ]
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")
    return fig


def counter_figures(pmc_csv: str, copy_bytes: int, ops: int, bytes_per_op: float) -> dict:
    names = sorted({r["Counter_Name"] for r in csv.DictReader(open(pmc_csv))})
    res = {"per_op": {}}
    kernels = set()
    for c in names:
        disp = _per_dispatch(pmc_csv, c)
        fused = [(n, v) for (n, v) in disp.values() if any(k in n for k in FUSED_KERNELS)]
        if not fused:
            raise RuntimeError(f"{pmc_csv}: no fused-kernel dispatches for {c}")
        kernels.update(_short(n) for n, _ in fused)
        res["fused_dispatches"] = len(fused)
        res["per_op"][c] = round(sum(v for _, v in fused) / ops, 1)
        if c in ("FETCH_SIZE", "WRITE_SIZE"):
            copies = [v for (n, v) in disp.values() if COPY_KERNEL in n]
            if not copies:
                raise RuntimeError(f"{pmc_csv}: no calibration copy for {c}")
            factor = (copy_bytes / 1024.0) / max(copies)
            res[f"{c}_factor"] = round(factor, 4)
            res[f"{c}_bytes_per_op"] = round(res["per_op"][c] * 1024.0 * factor)
            if bytes_per_op:
                res[f"{c}_over_algorithmic"] = round(res[f"{c}_bytes_per_op"] / bytes_per_op, 4)
    res["kernels"] = sorted(kernels)
    res["algorithmic_bytes_per_op"] = round(bytes_per_op)
    return res


def summarize_counters(pmc_csv, copy_bytes, ops, bytes_per_op, out_md, shape, command) -> dict:
    fig = counter_figures(pmc_csv, int(copy_bytes), int(ops), float(bytes_per_op))
    fig["shape"] = shape
    fig["ops"] = int(ops)
    fig["copy_bytes"] = int(copy_bytes)
    fig["kernel_source_sha256"] = kernel_source_sha256()
    lines = [
        f"# Counters of the fused NF4 kernels: {shape}",
        "",
        "One rocprofv3 counter run of:",
        "",
        "```",
        command,
        "```",
        "",
        f"per_op: each counter summed over the fused dispatches and divided by the {ops} operations. "
        f"FETCH_SIZE (KiB) is scaled to bytes by the factor that maps it onto a plain {copy_bytes} B "
        f"device copy (`{COPY_KERNEL}`) in the same run. SQ_INSTS_VALU counts wave-level VALU "
        "instructions (MFMA included); GRBM_GUI_ACTIVE counts GPU-busy cycles of the dispatches.",
        "",
        "```json",
        json.dumps(fig, indent=1),
        "```",
    ]
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")
    return fig


def read_traffic(md_path: str):
    """The figures of a traffic summary, or None when the file is missing or
    was measured on other kernel sources."""
    try:
        text = open(md_path).read()
    except OSError:
        return None
    m = re.search(r"```json\n(.*?)\n```", text, re.S)
    if not m:
        return None
    fig = json.loads(m.group(1))
    if fig.get("kernel_source_sha256") != kernel_source_sha256():
        return None
    return fig


def main(argv):
    if len(argv) >= 4 and argv[0] == "stats":
        summarize_stats(argv[1], argv[2], argv[3])
    elif len(argv) >= 5 and argv[0] == "lds":
        print(json.dumps(summarize_lds(argv[1], argv[2], argv[3], argv[4])))
    elif len(argv) >= 6 and argv[0] == "mfma":
        print(json.dumps(summarize_mfma(argv[1], float(argv[2]), argv[3], argv[4], argv[5])))
    elif len(argv) >= 8 and argv[0] == "counters":
        print(json.dumps(summarize_counters(argv[1], int(argv[2]), int(argv[3]), float(argv[4]),
                                            argv[5], argv[6], argv[7])))
    elif len(argv) >= 8 and argv[0] == "traffic":
        fig = summarize_traffic(argv[1], argv[2], int(argv[3]), int(argv[4]), argv[5], argv[6], argv[7])
        print(json.dumps(fig))
    else:
        print(__doc__)
        return 2
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
