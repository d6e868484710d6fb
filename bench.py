"""Benchmark: one expert-choice W8A8 ConvRot MoE layer (routed experts) on one MI355X.

A step is one full pass of the hot path over one batch: router softmax + per-expert top-C, rotate+quantise of
the tokens, grouped INT8 gate/up GEMM with SwiGLU, rotate+quantise of the hidden rows, grouped INT8 down GEMM,
probability-weighted combine.  Weights are converted once before timing (offline in the method).  Inputs are
resident in HBM when the timed region starts.

--workload dense times one dense W8A8 ConvRot linear over the same 8192 tokens instead (rotate+quantise of the
tokens + INT8 GEMM with dequant to bf16; --dense-shape picks the projection); --workload g16 the same linear
with 4- or 6-bit weights and an E4M3 scale per group of 16 (--g16-bits).  --workload lora times the load-time
LoRA patch of the layer's quantised gate/up weights (64 x [3072, 2048], rank 32), re-quantised with random
rounding into the layout the GEMM streams.

Prints one JSON line (see --help for options).  --gpus above 1 is refused: the library runs on one GPU.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "effective INT8 TOPS + tokens/s per MoE layer, % of INT8 MFMA / HBM peak"
PEAK_INT8_TOPS = 5000.0      # MI355X dense INT8 MFMA, TOPS
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E, GB/s
GEMM_SRC = os.path.join(ROOT, "w8a8_rotated_int8_amd", "csrc", "gemm.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gateup_gemm_T8192_C256_traffic.txt")


def layer_ops(s) -> float:
    """INT8 ops of one layer: 2 * E*C * (2I*d + d*I)."""
    return 6.0 * s.E * s.C * s.I * s.d


def layer_bytes(s, wbits=8) -> int:
    """Algorithmic HBM bytes of one layer: weights and scales once, x in, logits in, out written."""
    wb = (2 * s.I * s.d + s.d * s.I) * s.E * wbits // 8
    scales = (2 * s.I + s.d) * s.E * 4
    return wb + scales + s.T * s.d * 2 + s.T * s.E * 4 + s.T * s.d * 2


def gateup_bytes(s, wbits=8) -> int:
    """Algorithmic bytes of one gate/up GEMM launch: weights + scales, the quantised tokens and their scales,
    the routing indices, and the bf16 hidden rows written."""
    return (s.E * 2 * s.I * s.d * wbits // 8 + s.E * 2 * s.I * 4 + s.T * s.d + s.T * 4 + s.E * s.C * 4
            + s.E * s.C * s.I * 2)


def gateup_ops(s) -> float:
    return 2.0 * s.E * s.C * 2 * s.I * s.d


def src_hash(path) -> str:
    """The GEMM source's code digest, as the counter summaries record it (comments do not count)."""
    from w8a8_rotated_int8_amd.profiling import gemm_code_digest
    return gemm_code_digest(path)


def read_traffic():
    """HBM bytes per gate/up launch from the committed rocprofv3 counter summary, or None if absent or taken on
    another version of the kernel source."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    text = open(TRAFFIC_FILE).read()
    m = re.search(r"gemm_code_sha256_16:\s*(\w+)", text)
    t = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m or not t or m.group(1) != src_hash(GEMM_SRC):
        return None
    return float(t.group(1))


def cpu_model() -> str:
    """The host CPU's model name (from /proc/cpuinfo), for the CPU-baseline record."""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_cores() -> int:
    n = len(os.sched_getaffinity(0))
    omp = os.environ.get("OMP_NUM_THREADS")
    return min(n, int(omp)) if omp and omp.isdigit() else n


def cpu_baseline(x, lg, w_gu, w_dn, s, n_experts: int, min_seconds: float = 10.0):
    """Time the CPU oracle (as it stands) on a bounded sample: the same T-token layer restricted to its first
    n_experts experts (same per-expert work: C tokens each through gate/up, SwiGLU, rotate+quantise, down,
    combine), repeated until about `min_seconds` of CPU time.  Weight conversion is not timed, as on the GPU."""
    import oracle
    q_gu, s_gu = oracle.quantize_weights(w_gu[:n_experts], s.g_gu)
    q_dn, s_dn = oracle.quantize_weights(w_dn[:n_experts], s.g_dn)
    lg_s = np.ascontiguousarray(lg[:, :n_experts])
    reps, dt = 0, 0.0
    while reps == 0 or (dt < min_seconds and reps < 64):
        t0 = time.perf_counter()
        oracle.moe_forward(x, lg_s, s.C, q_gu, s_gu, s.g_gu, q_dn, s_dn, s.g_dn)
        dt += time.perf_counter() - t0
        reps += 1
    ops = 6.0 * n_experts * s.C * s.I * s.d * reps
    return {"value": ops / dt / 1e12, "unit": "TOPS", "cores": cpu_cores(), "kind": "oracle", "cpu": cpu_model(),
            "sample": f"T={s.T} layer restricted to experts 0..{n_experts - 1} (each C={s.C} tokens, full per-expert "
                      f"work), run {reps} times: {ops / 1e9:.1f} GOP in {dt:.2f} s, scaled to TOPS"}


def dense_cpu_baseline(x, q, s, g, b, M, K, N, min_seconds: float = 10.0):
    """Time the CPU oracle's linear (as it stands) on the same [M, K] tokens, repeated until about `min_seconds`
    of CPU time; weight conversion not timed."""
    import oracle
    reps, dt = 0, 0.0
    while reps == 0 or (dt < min_seconds and reps < 64):
        t0 = time.perf_counter()
        oracle.linear_w8a8(x, q, s, g, b)
        dt += time.perf_counter() - t0
        reps += 1
    ops = 2.0 * M * N * K * reps
    return {"value": ops / dt / 1e12, "unit": "TOPS", "cores": cpu_cores(), "kind": "oracle", "cpu": cpu_model(),
            "sample": f"the whole linear (M={M}, K={K}, N={N}), run {reps} times: {ops / 1e9:.1f} GOP in {dt:.2f} s"}


def add_measured_peaks(line, stream, mfma_tops=None, hbm_gbs=None):
    """What the chip sustains (the library's probes, timed in this run), beside the datasheet peaks the roofline
    uses: the dominant kernel's rate as a fraction of each."""
    from w8a8_rotated_int8_amd import profiling
    pk = profiling.measured_peaks(stream)
    print(f"bench: measured peaks {pk}", file=sys.stderr, flush=True)
    line["measured_peaks"] = pk
    if mfma_tops is not None:
        line["roofline"]["frac_of_measured_int8_mfma_random"] = round(mfma_tops / pk["int8_mfma_random_tops"], 4)
    if hbm_gbs is not None:
        line["roofline"]["frac_of_measured_hbm_read"] = round(hbm_gbs / pk["hbm_read_gbs"], 4)


def run_dense(args):
    import torch
    from w8a8_rotated_int8_amd import binding as cr
    from w8a8_rotated_int8_amd import synth

    dev = torch.device("cuda:0")
    name = args.dense_shape
    M, K, N, g = synth.DENSE_SHAPES[name]
    with_bias = name == "out"
    print(f"bench: dense {name} M={M} K={K} N={N} g={g} bias={with_bias}", file=sys.stderr, flush=True)
    x, w, b = synth.dense_linear_inputs(M, K, N, with_bias)

    def bf16_dev(a):
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)

    xd, bd = bf16_dev(x), (None if b is None else bf16_dev(b))
    qw, sw = cr.convrot_quantize_weights(bf16_dev(w), g, 8)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(cr.convrot_linear_workspace_bytes(M, K), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step():
        cr.convrot_linear_w8a8(xd, qw, sw, g, bias=bd, y=y, ws=ws, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / args.steps

    # dominant kernel: the GEMM stage on the step's token codes, HIP events on its stream
    qx, sx, _ = cr.convrot_rotq_rows(xd, g)
    for _ in range(3):
        cr.convrot_gemm_w8a8_bf16(qx, sx, qw, sw, bias=bd, y=y, stream=stream)
    k0, k1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    k0.record(stream)
    for _ in range(args.kernel_iters):
        cr.convrot_gemm_w8a8_bf16(qx, sx, qw, sw, bias=bd, y=y, stream=stream)
    k1.record(stream)
    torch.cuda.synchronize()
    k_us = k0.elapsed_time(k1) / args.kernel_iters * 1e3
    ops = 2.0 * M * N * K
    gemm_tops = ops / (k_us * 1e-6) / 1e12
    gemm_bytes = M * K + N * K + M * 4 + N * 4 + (N * 2 if with_bias else 0) + M * N * 2
    print(f"bench: {args.steps} steps, {ms * 1e3:.1f} us/step; GEMM {k_us:.1f} us/launch, {gemm_tops:.0f} TOPS",
          file=sys.stderr, flush=True)
    line = {
        "metric": "effective INT8 TOPS of one dense W8A8 ConvRot linear (rotate+quantise + GEMM + dequant)",
        "value": round(ops / (ms * 1e-3) / 1e12, 2),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic (seeded N(0,1) activations with 1% outlier channels x20, N(0,0.02) weights"
                + (" and bias" if with_bias else "") + ")",
        "config": {"workload": f"dense W8A8 ConvRot linear ({name}) M={M} K={K} N={N} group={g}"
                               + (" with bias" if with_bias else ""), "M": M, "K": K, "N": N, "group": g},
        "tokens_per_s": round(M / (ms * 1e-3), 1),
        "roofline": {"kernel": "dense INT8 GEMM + dequant (convrot_gemm_w8a8_bf16)", "bound": "mfma",
                     "achieved": round(gemm_tops, 1), "peak": PEAK_INT8_TOPS, "unit": "TOPS",
                     "frac": round(gemm_tops / PEAK_INT8_TOPS, 4), "traffic": None, "launch_us": round(k_us, 2),
                     "hbm_frac": round(gemm_bytes / (k_us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)},
        "cpu_baseline": None,
    }
    if args.peaks:
        add_measured_peaks(line, stream, mfma_tops=gemm_tops)
    if args.cpu_experts > 0:
        import oracle
        q, s = oracle.quantize_weights(w, g, 8)
        print("bench: timing the CPU oracle", file=sys.stderr, flush=True)
        line["cpu_baseline"] = dense_cpu_baseline(x, q, s, g, b, M, K, N)
    print(json.dumps(line), flush=True)


PEAK_FP16_TFLOPS = 2500.0   # MI355X dense fp16 MFMA, TFLOP/s


def run_g16(args):
    """The W6A8 / W4A8 dense linear (E4M3 scale per group of 16): rotate+quantise of the tokens + the GEMM
    whose matrix cores multiply exact fp16 products."""
    import torch
    from w8a8_rotated_int8_amd import binding as cr
    from w8a8_rotated_int8_amd import synth

    dev = torch.device("cuda:0")
    name, bits = args.dense_shape, args.g16_bits
    M, K, N, g = synth.DENSE_SHAPES[name]
    with_bias = name == "out"
    print(f"bench: g16 {name} M={M} K={K} N={N} g={g} bits={bits} bias={with_bias}", file=sys.stderr, flush=True)
    x, w, b = synth.dense_linear_inputs(M, K, N, with_bias)

    def bf16_dev(a):
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)

    xd, bd = bf16_dev(x), (None if b is None else bf16_dev(b))
    q, f8, s = cr.convrot_quantize_weights_g16(bf16_dev(w), g, bits)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(cr.convrot_linear_workspace_bytes(M, K), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step():
        cr.convrot_linear_g16(xd, q, f8, s, g, bits, bias=bd, y=y, ws=ws, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / args.steps

    qx, sx, _ = cr.convrot_rotq_rows(xd, g)
    for _ in range(3):
        cr.convrot_gemm_g16_bf16(qx, sx, q, f8, s, bits, bias=bd, y=y, stream=stream)
    k0, k1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    k0.record(stream)
    for _ in range(args.kernel_iters):
        cr.convrot_gemm_g16_bf16(qx, sx, q, f8, s, bits, bias=bd, y=y, stream=stream)
    k1.record(stream)
    torch.cuda.synchronize()
    k_us = k0.elapsed_time(k1) / args.kernel_iters * 1e3
    ops = 2.0 * M * N * K
    gemm_tflops = ops / (k_us * 1e-6) / 1e12
    gemm_bytes = M * K + N * K * bits // 8 + N * K // 16 + M * 4 + N * 4 + (N * 2 if with_bias else 0) + M * N * 2
    print(f"bench: {args.steps} steps, {ms * 1e3:.1f} us/step; GEMM {k_us:.1f} us/launch, {gemm_tflops:.0f} TFLOP/s",
          file=sys.stderr, flush=True)
    line = {
        "metric": f"effective TOPS of one dense W{bits}A8 linear with E4M3 group-16 scales (rotate+quantise + GEMM)",
        "value": round(ops / (ms * 1e-3) / 1e12, 2),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": f"int{bits}w-int8a (fp16 MFMA, fp32 accumulate)",
        "data": "synthetic (seeded N(0,1) activations with 1% outlier channels x20, N(0,0.02) weights"
                + (" and bias" if with_bias else "") + ")",
        "config": {"workload": f"dense W{bits}A8 linear, E4M3 scale per 16 ({name}) M={M} K={K} N={N} group={g}"
                               + (" with bias" if with_bias else ""), "M": M, "K": K, "N": N, "group": g,
                   "bits": bits},
        "tokens_per_s": round(M / (ms * 1e-3), 1),
        "roofline": {"kernel": "group-16 GEMM + dequant (convrot_gemm_g16_bf16)", "bound": "mfma",
                     "achieved": round(gemm_tflops, 1), "peak": PEAK_FP16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(gemm_tflops / PEAK_FP16_TFLOPS, 4), "traffic": None, "launch_us": round(k_us, 2),
                     "hbm_frac": round(gemm_bytes / (k_us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)},
        "cpu_baseline": None,
    }
    if args.cpu_experts > 0:
        import oracle
        rq, rf, rs, codes = oracle.quantize_g16(w, g, bits)
        rows = 64
        reps, dt = 0, 0.0
        print("bench: timing the CPU oracle", file=sys.stderr, flush=True)
        while reps == 0 or (dt < 10.0 and reps < 64):
            t0 = time.perf_counter()
            oracle.linear_g16(x[:rows], g, codes, rf, rs, b)
            dt += time.perf_counter() - t0
            reps += 1
        line["cpu_baseline"] = {"value": 2.0 * rows * N * K * reps / dt / 1e12, "unit": "TOPS",
                                "cores": cpu_cores(), "kind": "oracle", "cpu": cpu_model(),
                                "sample": f"the linear on the first {rows} of the {M} token rows (all {N} outputs), "
                                          f"run {reps} times in {dt:.2f} s"}
    print(json.dumps(line), flush=True)


PEAK_VALU_OPS = 256 * 64 * 2.4e9 / 1e12  # fp32 VALU operations (no FMA) per second, T: 256 CUs x 64 lanes x 2.4 GHz


def run_lora(args):
    import torch
    from w8a8_rotated_int8_amd import binding as cr
    from w8a8_rotated_int8_amd import synth

    dev = torch.device("cuda:0")
    s3 = synth.CONFIGS[3]
    E, N, K, g, rank, alpha = s3.E, 2 * s3.I, s3.d, s3.g_gu, 32, 0.5
    print(f"bench: lora E={E} N={N} K={K} g={g} rank={rank}", file=sys.stderr, flush=True)
    gen = torch.Generator(device=dev).manual_seed(3000)
    w = (torch.randn((E, N, K), generator=gen, device=dev) * synth.W_STD).to(torch.bfloat16)
    q, s = cr.convrot_quantize_weights(w, g, 8, layout=cr.LAYOUT_ROWMAJOR)
    del w
    lb = (torch.randn((E, N, rank), generator=gen, device=dev) * 0.02).to(torch.bfloat16)
    la = (torch.randn((E, rank, K), generator=gen, device=dev) * 0.02).to(torch.bfloat16)
    qo = torch.empty(cr.convrot_weight_bytes(E, N, K, 8, cr.LAYOUT_MFMA), dtype=torch.int8, device=dev)
    so = torch.empty((E, N), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    def step():
        cr.convrot_requantize_lora(q, s, g, lb, la, alpha, 7, q_out=qo, s_out=so, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / args.steps
    elems = E * N * K
    nbytes = elems * 2 + E * N * 8 + E * N * rank * 2 + E * rank * K * 2  # codes in and out, scales, factors
    # fp32 operations per weight the method specifies: rank products and sums, alpha, log2(g) butterfly stages
    # and the scaling, the dequantising multiply and the add, the division
    ops = (2 * rank + 1 + int(np.log2(g)) + 1 + 2 + 1) * elems
    achieved = ops / (ms * 1e-3) / 1e12
    print(f"bench: {ms * 1e3:.1f} us per conversion", file=sys.stderr, flush=True)
    line = {
        "metric": "LoRA patch + random-rounding re-quantisation of quantised weights, GB of int8 weights per second",
        "value": round(elems / (ms * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (weights N(0,0.02) drawn on the GPU with torch's generator, LoRA factors N(0,0.02))",
        "config": {"workload": f"LoRA rank {rank} on quantised gate/up weights E={E} N={N} K={K} group={g}",
                   "E": E, "N": N, "K": K, "group": g, "rank": rank},
        "roofline": {"kernel": "lora_requant_kernel", "bound": "alu", "achieved": round(achieved, 2),
                     "peak": round(PEAK_VALU_OPS, 1), "unit": "T fp32 ops/s", "frac": round(achieved / PEAK_VALU_OPS, 4),
                     "traffic": None, "launch_us": round(ms * 1e3, 2),
                     "hbm_frac": round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)},
        "cpu_baseline": None,
    }
    if args.cpu_experts > 0:
        import oracle
        qh, sh = q[:1].cpu().numpy(), s[:1].cpu().numpy()
        lbh = lb[:1].view(torch.int16).cpu().numpy().view(np.uint16)
        lah = la[:1].view(torch.int16).cpu().numpy().view(np.uint16)
        reps, dt = 0, 0.0
        while reps == 0 or (dt < 10.0 and reps < 64):
            t0 = time.perf_counter()
            oracle.requantize_lora(qh, sh, g, lbh, lah, alpha, 7)
            dt += time.perf_counter() - t0
            reps += 1
        line["cpu_baseline"] = {"value": N * K * reps / dt / 1e9, "unit": "GB/s", "cores": cpu_cores(),
                                "kind": "oracle", "cpu": cpu_model(),
                                "sample": f"expert 0 of the set ({N} x {K}), run {reps} times in {dt:.2f} s"}
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=3, choices=[2, 3, 4],
                    help="2: T=2048 C=64; 3: T=8192 C=256; 4: the T=8192 layer stacked --layers times, each layer "
                         "with its own weights and logits (weights drawn on the GPU), a step being the whole stack")
    ap.add_argument("--layers", type=int, default=29, help="layers of the config-4 stack")
    ap.add_argument("--wbits", type=int, default=8, choices=[8, 4])
    ap.add_argument("--cpu-experts", type=int, default=64,
                    help="experts in the CPU-oracle sample of the MoE workload; 0 skips the CPU baseline (either workload)")
    ap.add_argument("--kernel-iters", type=int, default=50, help="timed launches of the dominant kernel")
    ap.add_argument("--workload", default="moe", choices=["moe", "dense", "lora", "g16"])
    ap.add_argument("--g16-bits", type=int, default=4, choices=[4, 6],
                    help="weight bits of the group-16 workload (W4A8 or W6A8)")
    ap.add_argument("--no-peaks", dest="peaks", action="store_false",
                    help="skip the achievable-rate probes (int8 MFMA, HBM read) reported beside the roofline")
    ap.add_argument("--dense-shape", default="qkv", choices=["qkv", "ffn_down", "out"])
    ap.add_argument("--cold-steps", type=int, default=20,
                    help="single-layer workloads: steps timed one by one after a 1 GiB scratch write (0 skips)")
    ap.add_argument("--fused-rounds", type=int, default=4,
                    help="rounds of the one-launch expert path against the default (0: skip)")
    ap.add_argument("--stack-layers", type=int, default=29,
                    help="config 3: also time the weight-streaming stack of this many layers with 8- and 4-bit "
                         "weights (0 skips)")
    args = ap.parse_args()
    if args.gpus != 1:
        sys.exit(f"bench.py: the library runs on exactly one GPU; --gpus {args.gpus} is not supported "
                 "(sharding the experts over several GPUs is not built)")
    if args.workload == "dense":
        return run_dense(args)
    if args.workload == "lora":
        return run_lora(args)
    if args.workload == "g16":
        return run_g16(args)

    return run_moe(args)


def _events(n):
    import torch
    return [torch.cuda.Event(enable_timing=True) for _ in range(n)]


def time_launches(fn, iters, stream, warm=3):
    """Mean duration in microseconds of `iters` back-to-back calls of fn (HIP events on `stream`)."""
    import torch
    for _ in range(warm):
        fn()
    k0, k1 = _events(2)
    k0.record(stream)
    for _ in range(iters):
        fn()
    k1.record(stream)
    torch.cuda.synchronize()
    return k0.elapsed_time(k1) / iters * 1e3


def stack_sweep(cr, synth, s, n_layers, wbits, stream, dev, warm=2, sweeps=5):
    """The weight-streaming regime: n_layers layers of the T-token shape, each with its own seeded weights and
    logits drawn on the GPU, the same tokens; one sweep runs every layer once.  Returns (us per layer,
    gate/up launch us with successive layers' weights)."""
    import torch
    layers = []
    for li in range(n_layers):
        lgd, w_gu_d, w_dn_d = synth.stack_layer_device(li, s, dev)
        layers.append((lgd, cr.quantize_moe_weights(w_gu_d, w_dn_d, s.g_gu, s.g_dn, wbits)))
        del w_gu_d, w_dn_d
    x = torch.from_numpy(synth.stack_x(s).view(np.int16)).view(torch.bfloat16).to(dev)
    out = torch.empty((s.T, s.d), dtype=torch.bfloat16, device=dev)
    idx = torch.empty((s.E, s.C), dtype=torch.int32, device=dev)
    wt = torch.empty((s.E, s.C), dtype=torch.float32, device=dev)
    ws = torch.empty(cr.moe_expert_choice_workspace_bytes(s.T, s.C, layers[0][1]), dtype=torch.uint8, device=dev)

    def sweep():
        for lgd, w in layers:
            cr.moe_expert_choice_forward(x, lgd, s.C, w, out=out, idx_out=idx, wt_out=wt, ws=ws, stream=stream)

    us_sweep = time_launches(sweep, sweeps, stream, warm=warm)
    qx, sx, _ = cr.convrot_rotq_rows(x, s.g_gu)
    a = torch.empty((s.E * s.C, s.I), dtype=torch.bfloat16, device=dev)
    it = iter(range(1 << 30))
    gu_us = time_launches(lambda: cr.moe_gateup_swiglu(qx, sx, idx, layers[next(it) % n_layers][1], a_out=a,
                                                       stream=stream), 2 * n_layers, stream)
    del layers, ws
    torch.cuda.empty_cache()
    return us_sweep / n_layers, gu_us


def run_moe(args):
    import torch
    from w8a8_rotated_int8_amd import binding as cr
    from w8a8_rotated_int8_amd import synth

    dev = torch.device("cuda:0")
    s = synth.CONFIGS[args.config]
    n_layers = args.layers if args.config == 4 else 1
    print(f"bench: config {args.config} T={s.T} d={s.d} E={s.E} I={s.I} C={s.C} wbits={args.wbits} "
          f"layers={n_layers}", file=sys.stderr, flush=True)

    def bf16_dev(a):
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)

    def host_bf16(t):
        return t.view(torch.int16).cpu().numpy().view(np.uint16)

    # layers: (router logits on the device, converted weights); the CPU sample takes layer 0's first experts
    layers = []
    if args.config == 4:
        if n_layers < 1:
            sys.exit("bench.py: --layers must be at least 1")
        x = synth.stack_x(s)
        for li in range(n_layers):
            lgd_l, w_gu_d, w_dn_d = synth.stack_layer_device(li, s, dev)
            if li == 0:
                lg = lgd_l.cpu().numpy()
                n_cpu = max(args.cpu_experts, 1)
                w_gu, w_dn = host_bf16(w_gu_d[:n_cpu]), host_bf16(w_dn_d[:n_cpu])
            layers.append((lgd_l, cr.quantize_moe_weights(w_gu_d, w_dn_d, s.g_gu, s.g_dn, args.wbits)))
            del w_gu_d, w_dn_d
        print(f"bench: {n_layers} layers converted", file=sys.stderr, flush=True)
    else:
        x, lg, w_gu, w_dn = synth.moe_inputs(args.config)
        layers.append((torch.from_numpy(lg).to(dev),
                       cr.quantize_moe_weights(bf16_dev(w_gu), bf16_dev(w_dn), s.g_gu, s.g_dn, args.wbits)))
    xd = bf16_dev(x)
    w = layers[0][1]
    out = torch.empty((s.T, s.d), dtype=torch.bfloat16, device=dev)
    idx = torch.empty((s.E, s.C), dtype=torch.int32, device=dev)
    wt = torch.empty((s.E, s.C), dtype=torch.float32, device=dev)
    ws = torch.empty(cr.moe_expert_choice_workspace_bytes(s.T, s.C, w), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step():
        for lgd_l, w_l in layers:
            cr.moe_expert_choice_forward(xd, lgd_l, s.C, w_l, out=out, idx_out=idx, wt_out=wt, ws=ws, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev0, ev1 = _events(2)
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = ev0.elapsed_time(ev1) / args.steps
    print(f"bench: {args.steps} steps, {ms * 1e3:.1f} us/step (events), wall {wall / args.steps * 1e6:.1f} us/step",
          file=sys.stderr, flush=True)

    # Dominant kernel: the grouped gate/up GEMM, timed on its own stage entry point (same kernel, same inputs,
    # the routing of the last step) with HIP events on the stream it is launched on.  In the stack, successive
    # launches take successive layers' weights, so each launch streams weights the previous ones did not touch.
    qx, sx, _ = cr.convrot_rotq_rows(xd, s.g_gu)
    a = torch.empty((s.E * s.C, s.I), dtype=torch.bfloat16, device=dev)
    it = iter(range(1 << 30))
    k_us = time_launches(lambda: cr.moe_gateup_swiglu(qx, sx, idx, layers[next(it) % n_layers][1], a_out=a,
                                                      stream=stream), args.kernel_iters, stream)
    # the down GEMM on the hidden rows of that launch, for the GEMM-only MFMA fraction
    qa, sa, _ = cr.convrot_rotq_rows(a, s.g_dn)
    z = torch.empty((s.E * s.C, s.d), dtype=torch.bfloat16, device=dev)
    it = iter(range(1 << 30))
    dn_us = time_launches(lambda: cr.moe_down_proj(qa, sa, s.C, layers[next(it) % n_layers][1], z_out=z,
                                                   stream=stream), args.kernel_iters, stream)
    gb = gateup_bytes(s, args.wbits)
    achieved = gb / (k_us * 1e-6) / 1e9
    gemm_tops = gateup_ops(s) / (k_us * 1e-6) / 1e12
    gemm_only_tops = layer_ops(s) / ((k_us + dn_us) * 1e-6) / 1e12
    print(f"bench: gate/up GEMM {k_us:.1f} us/launch, {achieved:.0f} GB/s algorithmic, {gemm_tops:.0f} TOPS; down "
          f"GEMM {dn_us:.1f} us; both GEMMs {gemm_only_tops:.0f} TOPS", file=sys.stderr, flush=True)

    sec = ms * 1e-3 / n_layers  # one layer
    tops = layer_ops(s) / sec / 1e12
    workload = (f"expert-choice W{args.wbits}A8 ConvRot MoE layer T={s.T} d={s.d} E={s.E} I={s.I} C={s.C} "
                f"(g_gu={s.g_gu}, g_dn={s.g_dn}, {args.wbits}-bit weights)")
    if n_layers > 1:
        workload = f"{n_layers} stacked {workload.replace('layer', 'layers', 1)}, each with its own weights and logits"
    # the committed counter summary covers the 8-bit gate/up launch at T=8192, C=256
    traffic = read_traffic() if (s.T, s.C, args.wbits) == (8192, 256, 8) else None
    lbytes = layer_bytes(s, args.wbits)
    line = {
        "metric": METRIC,
        "value": round(tops, 2),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8" if args.wbits == 8 else "int4w-int8a",
        "data": "synthetic (seeded N(0,1) activations with 1% outlier channels x20, N(0,0.02) weights, "
                "N(0,1) router logits)",
        "config": {"workload": workload, "T": s.T, "d": s.d, "E": s.E, "I": s.I, "C": s.C, "wbits": args.wbits,
                   "layers": n_layers},
        "us_per_layer": round(sec * 1e6, 2),
        "tokens_per_s": round(s.T / sec, 1),
        "frac_int8_mfma_peak": round(tops / PEAK_INT8_TOPS, 4),
        "frac_hbm_peak": round(lbytes / sec / 1e9 / PEAK_HBM_GBS, 4),
        "gemm_only": {"gateup_us": round(k_us, 2), "down_us": round(dn_us, 2), "tops": round(gemm_only_tops, 1),
                      "frac_int8_mfma_peak": round(gemm_only_tops / PEAK_INT8_TOPS, 4)},
        "roofline": {"kernel": "grouped gate/up INT8 GEMM + SwiGLU", "bound": "hbm", "achieved": round(achieved, 1),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": traffic, "launch_us": round(k_us, 2),
                     "mfma_frac": round(gemm_tops / PEAK_INT8_TOPS, 4)},
        "cpu_baseline": None,
    }
    if n_layers == 1 and args.cold_steps > 0:
        # cold: a 1 GiB write between steps evicts the 256 MB memory-side cache and the L2s; each step is timed
        # by its own event pair
        scratch = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        cold = []
        for i in range(args.cold_steps):
            scratch.fill_(i & 255)
            e0, e1 = _events(2)
            e0.record(stream)
            step()
            e1.record(stream)
            torch.cuda.synchronize()
            cold.append(e0.elapsed_time(e1) * 1e3)
        del scratch
        cu = float(np.median(cold))
        line["cold"] = {"us_per_layer": round(cu, 2), "tops": round(layer_ops(s) / (cu * 1e-6) / 1e12, 2),
                        "tokens_per_s": round(s.T / (cu * 1e-6), 1),
                        "frac_hbm_peak": round(lbytes / (cu * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
                        "steps": args.cold_steps, "note": "median over steps, each after a 1 GiB scratch write"}
        print(f"bench: cold {cu:.1f} us/layer (median of {args.cold_steps})", file=sys.stderr, flush=True)
    if n_layers == 1 and args.fused_rounds > 0 and cr.moe_expert_choice_fused(w, s.C):
        # the one-launch expert path against the default three launches, alternating blocks of 10 steps so that
        # both see the same clock
        def block(fused):
            e0, e1 = _events(2)
            e0.record(stream)
            for _ in range(10):
                cr.moe_expert_choice_forward(xd, layers[0][0], s.C, w, out=out, idx_out=idx, wt_out=wt, ws=ws,
                                             stream=stream, fused=fused)
            e1.record(stream)
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) * 1e3 / 10
        res = {False: [], True: []}
        block(True)
        for r in range(args.fused_rounds):
            for fz in ((False, True) if r % 2 == 0 else (True, False)):
                res[fz].append(block(fz))
        f_us, t_us = float(np.median(res[True])), float(np.median(res[False]))
        line["fused_experts"] = {"us_per_layer": round(f_us, 2), "three_launches_us_per_layer": round(t_us, 2),
                                 "note": "moe_expert_choice_forward_fused against moe_expert_choice_forward, "
                                         "median of alternating 10-step blocks"}
        print(f"bench: one-launch experts {f_us:.1f} us/layer, three launches {t_us:.1f} us/layer",
              file=sys.stderr, flush=True)
    if args.config == 3 and args.stack_layers > 0:
        st4 = synth.CONFIGS[4]
        line["stack"] = {"layers": args.stack_layers,
                         "workload": f"{args.stack_layers} stacked T={st4.T} layers, each with its own weights "
                                     "and logits (weights drawn on the GPU), a sweep timed as a whole"}
        for wbits in (8, 4):
            lu, gu = stack_sweep(cr, synth, st4, args.stack_layers, wbits, stream, dev)
            sb = layer_bytes(st4, wbits)
            line["stack"][f"w{wbits}a8"] = {
                "us_per_layer": round(lu, 2), "tops": round(layer_ops(st4) / (lu * 1e-6) / 1e12, 2),
                "frac_hbm_peak": round(sb / (lu * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
                "gateup_us": round(gu, 2),
                "gateup_frac_hbm_peak": round(gateup_bytes(st4, wbits) / (gu * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)}
            print(f"bench: stack of {args.stack_layers} layers, {wbits}-bit weights: {lu:.1f} us/layer, gate/up "
                  f"{gu:.1f} us", file=sys.stderr, flush=True)
    if args.peaks:
        add_measured_peaks(line, stream, mfma_tops=gemm_tops, hbm_gbs=achieved)
        line["gemm_only"]["frac_of_measured_int8_mfma_random"] = round(
            gemm_only_tops / line["measured_peaks"]["int8_mfma_random_tops"], 4)
    if args.cpu_experts > 0:
        print(f"bench: timing the CPU oracle on {args.cpu_experts} experts", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(x, lg, w_gu, w_dn, s, args.cpu_experts)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
