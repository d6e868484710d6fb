"""rocprofv3 summaries for the committed profiles: per-kernel duration statistics and HBM traffic per launch.

Used by hand after a profiled run of ``bench.py``; reads only rocprofv3's CSV output (``--output-format csv
-o run``) and writes short text summaries.  Nothing here runs a kernel except ``copy_probe``, the plain
device-to-device copy of known size that calibrates the FETCH_SIZE / WRITE_SIZE counters, and
``measured_peaks``, which times the library's achievable-rate probes (int8 MFMA on random and on constant
operands, HBM read through LDS DMA) for ``bench.py``.

    python -m w8a8_rotated_int8_amd.profiling stats <run_dir> <out.txt> "<command>"
    python -m w8a8_rotated_int8_amd.profiling copy <MiB> <iters>
    python -m w8a8_rotated_int8_amd.profiling traffic <fetch_dir> <write_dir> <copy_fetch_dir> <copy_write_dir>
        <copy_MiB> <kernel_substring> <out.txt> "<commands>"
    python -m w8a8_rotated_int8_amd.profiling pmc <out.txt> "<commands>" <label=kernel_substring>,... <run_dir>...
"""
from __future__ import annotations

import collections
import csv
import hashlib
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GEMM_SRC = os.path.join(ROOT, "w8a8_rotated_int8_amd", "csrc", "gemm.hip")


def gemm_code_digest(path: str = GEMM_SRC) -> str:
    """First 16 hex digits of the SHA-256 of the GEMM source's code: every line with its // comment, trailing
    blanks and blank lines dropped, so that a change of comments alone keeps the committed counter summaries
    valid while any change of code invalidates them."""
    lines = []
    for line in open(path, encoding="utf-8").read().splitlines():
        code = line.split("//", 1)[0].rstrip()
        if code:
            lines.append(code)
    return hashlib.sha256("\n".join(lines).encode()).hexdigest()[:16]


def _csv(run_dir: str, suffix: str):
    path = os.path.join(run_dir, f"run_{suffix}.csv")
    if not os.path.exists(path):
        cands = [os.path.join(dp, f) for dp, _, fs in os.walk(run_dir) for f in fs if f.endswith(f"_{suffix}.csv")]
        if not cands:
            raise FileNotFoundError(f"no *_{suffix}.csv under {run_dir}")
        path = sorted(cands)[0]
    with open(path) as fh:
        return list(csv.DictReader(fh))


def short_name(name: str) -> str:
    name = name.replace("crk::(anonymous namespace)::", "").replace("(anonymous namespace)::", "")
    return name if len(name) <= 110 else name[:107] + "..."


def stats_summary(run_dir: str, out_txt: str, command: str) -> None:
    rows = _csv(run_dir, "kernel_stats")
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    lines = [f"command: {command}", "source: rocprofv3 --kernel-trace --stats (kernel_stats.csv)", "",
             f"{'calls':>6} {'avg_us':>9} {'min_us':>9} {'max_us':>9} {'total%':>7}  kernel"]
    for r in rows:
        lines.append(f"{int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:9.2f} {float(r['MinNs']) / 1e3:9.2f} "
                     f"{float(r['MaxNs']) / 1e3:9.2f} {float(r['Percentage']):7.2f}  {short_name(r['Name'])}")
    with open(out_txt, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def measured_peaks(stream=None, mfma_iters: int = 4096, hbm_bytes: int = 4 << 30) -> dict:
    """What the chip sustains, measured with the library's probes on the current device (best of 3 timed
    launches each, HIP events on `stream`): int8 MFMA TOPS on random and on constant operand bytes, and HBM
    read GB/s through non-temporal LDS DMA over `hbm_bytes` (well above the 256 MB memory-side cache)."""
    import torch
    from . import binding as cr
    dev = torch.device("cuda")
    st = stream or torch.cuda.current_stream()
    out = torch.empty(cr.lib().convrot_probe_out_words(), dtype=torch.int32, device=dev)
    g = torch.Generator(device=dev)
    g.manual_seed(12345)
    pool_rand = torch.randint(-128, 128, (256 * 1024,), dtype=torch.int8, device=dev, generator=g)
    pool_const = torch.full((256 * 1024,), 0x11, dtype=torch.int8, device=dev)
    src = torch.empty(hbm_bytes, dtype=torch.int8, device=dev)

    def best(fn):
        fn()
        times = []
        for _ in range(3):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(st)
            work = fn()
            b.record(st)
            torch.cuda.synchronize()
            times.append(a.elapsed_time(b) * 1e-3)
        return work / min(times)

    res = {
        "int8_mfma_random_tops": best(lambda: cr.convrot_probe_mfma_i8(pool_rand, mfma_iters, out, st)) / 1e12,
        "int8_mfma_const_tops": best(lambda: cr.convrot_probe_mfma_i8(pool_const, mfma_iters, out, st)) / 1e12,
        "hbm_read_gbs": best(lambda: cr.convrot_probe_hbm_read(src, out, st)) / 1e9,
    }
    del src
    return {k: round(v, 1) for k, v in res.items()}


def counter_per_dispatch(run_dir: str, counter: str, pattern: str, skip: int = 1):
    """Mean value of `counter` over the dispatches whose kernel name contains `pattern` (the first `skip`
    dispatches are dropped as warm-up)."""
    rows = [r for r in _csv(run_dir, "counter_collection") if pattern in r["Kernel_Name"]
            and r["Counter_Name"] == counter]
    per = collections.defaultdict(float)
    for r in rows:
        per[int(r["Dispatch_Id"])] += float(r["Counter_Value"])
    ids = sorted(per)
    if len(ids) > skip:
        ids = ids[skip:]
    if not ids:
        raise ValueError(f"no dispatch of a kernel matching {pattern!r} with counter {counter}")
    return sum(per[i] for i in ids) / len(ids), len(ids)


N_XCD = 8          # GRBM_GUI_ACTIVE comes summed over the XCDs
N_SIMD = 256 * 4   # MFMA units: 4 SIMDs in each of the 256 compute units


def _dispatches(run_dir: str, pattern: str, skip: int = 1):
    """{dispatch id: {counter: value summed over its dimensions}} and the durations in us, for the dispatches
    whose kernel name contains `pattern` (the first `skip` dropped as warm-up)."""
    per = collections.defaultdict(lambda: collections.defaultdict(float))
    dur = {}
    for r in _csv(run_dir, "counter_collection"):
        if pattern not in r["Kernel_Name"]:
            continue
        k = int(r["Dispatch_Id"])
        per[k][r["Counter_Name"]] += float(r["Counter_Value"])
        dur[k] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-3
    ids = sorted(per)
    if len(ids) > skip:
        ids = ids[skip:]
    return {k: per[k] for k in ids}, [dur[k] for k in ids]


def pmc_summary(out_txt: str, command: str, kernels: str, run_dirs) -> None:
    """Counters of the named kernels, one collection pass per run directory, averaged per dispatch, with the
    derived figures: clock (GRBM_GUI_ACTIVE per XCD over the dispatch time), MFMA busy fraction (MFMA busy
    cycles over all SIMDs' cycles), per-cycle rates of the SQ / TA / TD counters and the mean L2 read latency
    seen by the vector caches."""
    lines = [f"command: {command}", "source: rocprofv3 --pmc (counter_collection.csv), one pass per counter set;",
             "  values are means per dispatch after the first; the profiler serialises dispatches, so the clock",
             "  here is the unthrottled one", f"gemm_code_sha256_16: {gemm_code_digest()}", ""]
    for spec in kernels.split(","):
        label, pattern = spec.split("=", 1)
        lines.append(f"== {label} (kernel name contains {pattern!r})")
        for d in run_dirs:
            disp, durs = _dispatches(d, pattern)
            if not disp:
                lines.append(f"  pass {os.path.basename(d.rstrip('/'))}: no dispatch")
                continue
            names = sorted({c for v in disp.values() for c in v})
            avg = {c: sum(v.get(c, 0.0) for v in disp.values()) / len(disp) for c in names}
            us = sum(durs) / len(durs)
            lines.append(f"  pass {os.path.basename(d.rstrip('/'))}: {len(disp)} dispatches, {us:.1f} us each")
            grbm = avg.get("GRBM_GUI_ACTIVE", 0.0)
            cyc = grbm / N_XCD
            if cyc > 0:
                lines.append(f"    clock: {cyc / us * 1e-3:.2f} GHz ({cyc:.4g} cycles per XCD)")
            for c in names:
                if c == "GRBM_GUI_ACTIVE":
                    continue
                rate = f"  ({avg[c] / cyc:.4g} per cycle)" if cyc > 0 else ""
                lines.append(f"    {c}: {avg[c]:.4g}{rate}")
            if cyc > 0 and "SQ_VALU_MFMA_BUSY_CYCLES" in avg:
                lines.append(f"    MFMA busy: {100.0 * avg['SQ_VALU_MFMA_BUSY_CYCLES'] / (cyc * N_SIMD):.1f} % "
                             f"of {N_SIMD} SIMDs")
            if avg.get("TCP_TCC_READ_REQ_sum", 0.0) > 0:
                lines.append(f"    L2 read latency: {avg['TCP_TCC_READ_REQ_LATENCY_sum'] / avg['TCP_TCC_READ_REQ_sum']:.0f}"
                             " cycles per request")
            if avg.get("SQ_LDS_IDX_ACTIVE", 0.0) > avg.get("SQ_LDS_BANK_CONFLICT", 0.0) > 0:
                lines.append(f"    LDS bank conflict ratio: {avg['SQ_LDS_BANK_CONFLICT'] / (avg['SQ_LDS_IDX_ACTIVE'] - avg['SQ_LDS_BANK_CONFLICT']):.3f}")
        lines.append("")
    with open(out_txt, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def copy_probe(mib: int, iters: int) -> None:
    """Plain device-to-device copy of `mib` MiB, `iters` times (counter calibration)."""
    import torch
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(iters):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(f"copy probe: {iters} copies of {mib} MiB", flush=True)


def traffic_summary(fetch_dir, write_dir, copy_fetch_dir, copy_write_dir, copy_mib, pattern, out_txt, command):
    nbytes = copy_mib << 20
    cf, _ = counter_per_dispatch(copy_fetch_dir, "FETCH_SIZE", "copy", skip=1)
    cw, _ = counter_per_dispatch(copy_write_dir, "WRITE_SIZE", "copy", skip=1)
    f_scale = nbytes / (cf * 1024.0)
    w_scale = nbytes / (cw * 1024.0)
    kf, nf = counter_per_dispatch(fetch_dir, "FETCH_SIZE", pattern)
    kw, nw = counter_per_dispatch(write_dir, "WRITE_SIZE", pattern)
    fetch_b = kf * 1024.0 * f_scale
    write_b = kw * 1024.0 * w_scale
    sha = gemm_code_digest()
    lines = [f"command: {command}",
             f"kernel: dispatches whose name contains {pattern!r} ({nf} FETCH, {nw} WRITE dispatches after warm-up)",
             f"gemm_code_sha256_16: {sha}",
             f"copy calibration: {copy_mib} MiB device copy reads FETCH_SIZE {cf:.1f} KiB, WRITE_SIZE {cw:.1f} KiB",
             f"fetch_scale: {f_scale:.4f}", f"write_scale: {w_scale:.4f}",
             f"fetch_kib_raw: {kf:.1f}", f"write_kib_raw: {kw:.1f}",
             f"fetch_bytes_per_launch: {fetch_b:.6g}", f"write_bytes_per_launch: {write_b:.6g}",
             f"traffic_bytes_per_launch: {fetch_b + write_b:.6g}"]
    with open(out_txt, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


if __name__ == "__main__":
    cmd = sys.argv[1] if len(sys.argv) > 1 else ""
    if cmd == "stats":
        stats_summary(sys.argv[2], sys.argv[3], sys.argv[4])
    elif cmd == "copy":
        copy_probe(int(sys.argv[2]), int(sys.argv[3]))
    elif cmd == "traffic":
        traffic_summary(*sys.argv[2:6], int(sys.argv[6]), sys.argv[7], sys.argv[8], sys.argv[9])
    elif cmd == "pmc":
        pmc_summary(sys.argv[2], sys.argv[3], sys.argv[4], sys.argv[5:])
    else:
        sys.exit(__doc__)
