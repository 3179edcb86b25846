"""Summaries of rocprofv3 output for the decode kernel (measurement helper,
not the decode path).

`python -m moe_decode_02_amd.profiling stats <dir> <out.txt> <command...>`
    writes a text summary of a `rocprofv3 --kernel-trace --stats
    --output-format csv` run: per kernel, calls and average / median / min /
    max duration.

`python -m moe_decode_02_amd.profiling traffic <fetch_dir> <write_dir> <out.txt> <command...>`
    combines two `rocprofv3 --pmc FETCH_SIZE` and `--pmc WRITE_SIZE` runs of
    the benchmark: per dispatch of the decode kernel, the counters (KiB) are
    scaled by the ratio the same counters show for the benchmark's copy kernel
    of known size, giving HBM bytes read and written per launch. The summary
    records the SHA-256 of the kernel source it was taken on, so that the
    benchmark reports the figure only while the kernel is unchanged.

`python -m moe_decode_02_amd.profiling mfma <pmc_dir> <trace_dir> <out.txt> <command...>`
    summarises a `rocprofv3 --pmc SQ_INSTS_VALU_MFMA_MOPS_BF16
    SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE` run of the decode kernel with
    the kernel durations of a kernel-trace run of the same command: MFMA
    work per dispatch (the MOPS counter counts units of 512 flops), the
    achieved MFMA rate against the 2.5 PFLOP/s dense bf16 peak, and the
    fraction of the kernel's active cycles in which MFMA units were busy.

`python -m moe_decode_02_amd.profiling counters <pmc_dir> <out.txt> <command...>`
    the mean per dispatch of every counter of a `rocprofv3 --pmc` run, for
    the decode kernel (for example LDS bank conflicts against LDS
    instructions, or L2 hits against misses).

`python -m moe_decode_02_amd.profiling unfused <fetch_dir> <write_dir> <out.txt> <command...>`
    the same two runs for the multi-launch path: per kernel of that path
    (the `uf_` kernels), dispatches and HBM bytes read and written per
    dispatch, and the totals per layer (the dispatches of its combine kernel
    count the layers), scaled by the copy kernel as above.

`<command...>` is the profiled command line, copied into the summary.
"""
from __future__ import annotations

import csv
import glob
import hashlib
import os
import statistics
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
KERNEL_SOURCE = os.path.join(HERE, "csrc", "moedecode.hip")
DECODE_KERNEL = "::moe_kernel<"
COPY_KERNEL = "::copy_kernel("
UNFUSED_KERNEL = "::uf_"
UNFUSED_LAYER_END = "::uf_combine<"
# bytes the benchmark's calibration copy reads (and writes)
COPY_BYTES = 1 << 30


def kernel_source_sha() -> str:
    with open(KERNEL_SOURCE, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def _find(d: str, suffix: str) -> str:
    hits = sorted(glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True))
    if not hits:
        raise FileNotFoundError(f"no *{suffix} under {d}")
    return hits[0]


def kernel_durations(trace_dir: str):
    """{kernel name: [durations in us]} from a kernel-trace CSV."""
    path = _find(trace_dir, "kernel_trace.csv")
    out = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            d = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0
            out.setdefault(r["Kernel_Name"], []).append(d)
    return out


def write_stats(trace_dir: str, out_txt: str, command: str) -> None:
    durs = kernel_durations(trace_dir)
    lines = [f"# rocprofv3 kernel trace summary", f"# command: {command}",
             f"# kernel source sha256: {kernel_source_sha()}",
             f"{'kernel':60s} {'calls':>6s} {'avg_us':>9s} {'median_us':>10s} {'min_us':>9s} {'max_us':>9s}"]
    for name, v in sorted(durs.items(), key=lambda kv: -sum(kv[1])):
        short = name if len(name) <= 60 else name[:57] + "..."
        lines.append(f"{short:60s} {len(v):6d} {statistics.mean(v):9.2f} {statistics.median(v):10.2f} "
                     f"{min(v):9.2f} {max(v):9.2f}")
    with open(out_txt, "w") as f:
        f.write("\n".join(lines) + "\n")


def _counter_per_dispatch(pmc_dir: str, counter: str):
    """{kernel name: [counter value per dispatch]} from a --pmc CSV."""
    path = _find(pmc_dir, "counter_collection.csv")
    out = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            out.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return out


def _pick(d, needle):
    for k, v in d.items():
        if needle in k:
            return v
    raise KeyError(needle)


def write_traffic(fetch_dir: str, write_dir: str, out_txt: str, command: str) -> None:
    fetch = _counter_per_dispatch(fetch_dir, "FETCH_SIZE")
    write = _counter_per_dispatch(write_dir, "WRITE_SIZE")
    kf, kw = _pick(fetch, DECODE_KERNEL), _pick(write, DECODE_KERNEL)
    cf, cw = _pick(fetch, COPY_KERNEL), _pick(write, COPY_KERNEL)
    # counters are KiB per dispatch; the copy reads and writes COPY_BYTES
    fetch_scale = COPY_BYTES / (statistics.mean(cf) * 1024.0)
    write_scale = COPY_BYTES / (statistics.mean(cw) * 1024.0)
    fb = statistics.mean(kf) * 1024.0 * fetch_scale
    wb = statistics.mean(kw) * 1024.0 * write_scale
    lines = ["# HBM traffic of the decode kernel from rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE",
             f"# command: {command}",
             f"# copy calibration: {COPY_BYTES} B copied; FETCH_SIZE {statistics.mean(cf):.0f} KiB, "
             f"WRITE_SIZE {statistics.mean(cw):.0f} KiB per dispatch",
             f"kernel_source_sha256 = {kernel_source_sha()}",
             f"dispatches = {len(kf)}",
             f"fetch_kib_per_dispatch = {statistics.mean(kf):.1f}",
             f"write_kib_per_dispatch = {statistics.mean(kw):.1f}",
             f"fetch_scale = {fetch_scale:.4f}",
             f"write_scale = {write_scale:.4f}",
             f"hbm_read_bytes_per_launch = {fb:.0f}",
             f"hbm_write_bytes_per_launch = {wb:.0f}",
             f"hbm_bytes_per_launch = {fb + wb:.0f}"]
    with open(out_txt, "w") as f:
        f.write("\n".join(lines) + "\n")


def write_unfused_traffic(fetch_dir: str, write_dir: str, out_txt: str, command: str) -> None:
    fetch = _counter_per_dispatch(fetch_dir, "FETCH_SIZE")
    write = _counter_per_dispatch(write_dir, "WRITE_SIZE")
    cf, cw = _pick(fetch, COPY_KERNEL), _pick(write, COPY_KERNEL)
    fetch_scale = COPY_BYTES / (statistics.mean(cf) * 1024.0)
    write_scale = COPY_BYTES / (statistics.mean(cw) * 1024.0)
    layers = len(_pick(fetch, UNFUSED_LAYER_END))
    lines = ["# HBM traffic of the multi-launch path from rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE",
             f"# command: {command}",
             f"# copy calibration: fetch_scale {fetch_scale:.4f}, write_scale {write_scale:.4f}",
             f"kernel_source_sha256 = {kernel_source_sha()}",
             f"layers = {layers}",
             f"{'kernel':60s} {'calls':>6s} {'read_MB_per_call':>17s} {'write_MB_per_call':>18s}"]
    tr = tw = 0.0
    for name in sorted(k for k in fetch if UNFUSED_KERNEL in k):
        fv, wv = fetch[name], write.get(name, [0.0])
        rb = statistics.mean(fv) * 1024.0 * fetch_scale
        wb = statistics.mean(wv) * 1024.0 * write_scale
        tr += sum(fv) * 1024.0 * fetch_scale
        tw += sum(wv) * 1024.0 * write_scale
        short = name if len(name) <= 60 else name[:57] + "..."
        lines.append(f"{short:60s} {len(fv):6d} {rb / 1e6:17.3f} {wb / 1e6:18.3f}")
    lines += [f"hbm_read_bytes_per_layer = {tr / layers:.0f}", f"hbm_write_bytes_per_layer = {tw / layers:.0f}"]
    with open(out_txt, "w") as f:
        f.write("\n".join(lines) + "\n")


def read_traffic(path: str):
    """HBM bytes per launch from a traffic summary, or None when the summary is
    missing or was taken on a different kernel source."""
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if "=" in line and not line.startswith("#"):
                k, v = line.split("=", 1)
                kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha256") != kernel_source_sha():
        return None
    return {"read": float(kv["hbm_read_bytes_per_launch"]), "write": float(kv["hbm_write_bytes_per_launch"])}


def write_mfma(pmc_dir: str, trace_dir: str, out_txt: str, command: str) -> None:
    mops = _pick(_counter_per_dispatch(pmc_dir, "SQ_INSTS_VALU_MFMA_MOPS_BF16"), DECODE_KERNEL)
    busy = _pick(_counter_per_dispatch(pmc_dir, "SQ_VALU_MFMA_BUSY_CYCLES"), DECODE_KERNEL)
    active = _pick(_counter_per_dispatch(pmc_dir, "GRBM_GUI_ACTIVE"), DECODE_KERNEL)
    durs = _pick(kernel_durations(trace_dir), DECODE_KERNEL)
    flops = statistics.mean(mops) * 512.0
    t = statistics.mean(durs) * 1e-6
    # SQ_VALU_MFMA_BUSY_CYCLES sums over the chip's SIMDs (4 per CU, 256 CUs);
    # GRBM_GUI_ACTIVE counts cycles of the graphics block per XCD (8 XCDs)
    simds, xcds = 4 * 256, 8
    frac = statistics.mean(busy) / (statistics.mean(active) / xcds * simds)
    lines = ["# MFMA use of the decode kernel from rocprofv3 --pmc (one pass) and --kernel-trace",
             f"# command: {command}",
             f"kernel_source_sha256 = {kernel_source_sha()}",
             f"dispatches = {len(mops)}",
             f"mfma_mops_bf16_per_dispatch = {statistics.mean(mops):.0f}",
             f"mfma_flops_per_dispatch = {flops:.4g}",
             f"kernel_avg_us = {statistics.mean(durs):.2f}",
             f"mfma_tflops = {flops / t / 1e12:.2f}",
             f"mfma_fraction_of_2500_tflops = {flops / t / 2.5e15:.5f}",
             f"mfma_busy_cycles_per_dispatch = {statistics.mean(busy):.0f}",
             f"gui_active_cycles_per_dispatch = {statistics.mean(active):.0f}",
             f"mfma_busy_fraction_of_simd_cycles = {frac:.5f}"]
    with open(out_txt, "w") as f:
        f.write("\n".join(lines) + "\n")


def write_counters(pmc_dir: str, out_txt: str, command: str) -> None:
    path = _find(pmc_dir, "counter_collection.csv")
    per = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            if DECODE_KERNEL in r["Kernel_Name"]:
                per.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    lines = ["# counters of the decode kernel from rocprofv3 --pmc (mean per dispatch)",
             f"# command: {command}",
             f"kernel_source_sha256 = {kernel_source_sha()}"]
    for name in sorted(per):
        lines.append(f"{name} = {statistics.mean(per[name]):.6g}   (dispatches {len(per[name])})")
    with open(out_txt, "w") as f:
        f.write("\n".join(lines) + "\n")


def main(argv) -> int:
    if len(argv) >= 4 and argv[1] == "stats":
        write_stats(argv[2], argv[3], " ".join(argv[4:]))
        return 0
    if len(argv) >= 5 and argv[1] == "traffic":
        write_traffic(argv[2], argv[3], argv[4], " ".join(argv[5:]))
        return 0
    if len(argv) >= 4 and argv[1] == "counters":
        write_counters(argv[2], argv[3], " ".join(argv[4:]))
        return 0
    if len(argv) >= 5 and argv[1] == "unfused":
        write_unfused_traffic(argv[2], argv[3], argv[4], " ".join(argv[5:]))
        return 0
    if len(argv) >= 5 and argv[1] == "mfma":
        write_mfma(argv[2], argv[3], argv[4], " ".join(argv[5:]))
        return 0
    print(__doc__, file=sys.stderr)
    return 2


if __name__ == "__main__":
    sys.exit(main(sys.argv))
