"""W6A8 / W4A8 with an FP8 (E4M3) scale per group of 16 on the GPU, against the oracle.

The converter is compared bit for bit (packed codes, E4M3 scales, fp32 row scales).  The GEMM multiplies exact
fp16 products and accumulates them in fp32, where the oracle sums them exactly: its BF16 outputs must be within
1e-2 relative of the oracle's, plus the fp32 accumulation bound K * 2^-23 * sum|terms| * sx * s_row."""
import numpy as np
import pytest
import torch

import oracle
from w8a8_rotated_int8_amd import binding as cr
from w8a8_rotated_int8_amd import synth

from helpers import DEV, assert_bf16_within, dev, dev_bf16, host, host_bf16, say

pytestmark = pytest.mark.gpu


def _weights(N, K, seed):
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    if N > 3:
        w[1] = 0.0  # all-zero row
        w[2, :16] *= 1e-5  # a group far below its row's largest: tiny or zero FP8 scale
    return oracle.bf16_round(w)


@pytest.mark.parametrize("N,K,g,bits", [(37, 512, 256, 6), (64, 2048, 256, 4), (33, 1536, 64, 6),
                                        (16, 256, 64, 4), (5, 8192, 256, 6)])
def test_converter_bit_exact(N, K, g, bits):
    say(f"g16 converter N={N} K={K} g={g} bits={bits}")
    w = _weights(N, K, 100 + N)
    rq, rf, rs, _ = oracle.quantize_g16(w, g, bits)
    q, f8, s = cr.convrot_quantize_weights_g16(dev_bf16(w), g, bits)
    torch.cuda.synchronize()
    assert np.array_equal(host(q), rq), "packed codes"
    assert np.array_equal(host(f8), rf), "E4M3 group scales"
    assert np.array_equal(host(s).view(np.uint32), rs.view(np.uint32)), "row scales"


def _check_y(y, ref, aabs, sx, s_row, K, what):
    floor = K * 2.0 ** -23 * aabs * np.abs(sx)[:, None].astype(np.float64) * np.abs(s_row)[None, :]
    exact = assert_bf16_within(host_bf16(y), ref, rel=1e-2, floor=floor, what=what)
    say(f"{what}: {exact * 100:.2f}% bit-identical")


@pytest.mark.parametrize("M,K,N,bits,with_bias", [(96, 512, 160, 6, False), (130, 2048, 257, 4, True),
                                                  (64, 1536, 128, 6, True), (1, 256, 3, 4, False),
                                                  (300, 8192, 96, 4, False), (257, 256, 513, 6, True)])
def test_gemm_stage_within_tolerance(M, K, N, bits, with_bias):
    say(f"g16 GEMM M={M} K={K} N={N} bits={bits} bias={with_bias}")
    g = 256 if K % 256 == 0 else 64
    x, w = synth.linear_inputs(0, M=M, K=K, N=N, n_outlier=max(1, K // 100))
    rng = np.random.default_rng(M + N)
    bias = oracle.bf16_round(rng.standard_normal(N).astype(np.float32)) if with_bias else None
    q, f8, s, codes = oracle.quantize_g16(w, g, bits)
    qx, sx = oracle.rotq_rows(x, g, 127)
    ref, acc, aabs = oracle.gemm_g16(qx, sx, codes, f8, s, bias)
    y = cr.convrot_gemm_g16_bf16(dev(qx), dev(sx), dev(q), dev(f8), dev(s), bits,
                                 bias=None if bias is None else dev_bf16(bias))
    torch.cuda.synchronize()
    _check_y(y, ref, aabs, sx, s, K, "GEMM stage")


@pytest.mark.parametrize("bits", [6, 4])
def test_linear_end_to_end(bits):
    M, K, N, g = 200, 2048, 384, 256
    say(f"g16 linear M={M} K={K} N={N} bits={bits}")
    x, w = synth.linear_inputs(0, M=M, K=K, N=N, n_outlier=K // 100)
    q, f8, s = cr.convrot_quantize_weights_g16(dev_bf16(w), g, bits)
    y = cr.convrot_linear_g16(dev_bf16(x), q, f8, s, g, bits)
    torch.cuda.synchronize()
    codes = oracle.unpack_g16(host(q), K, bits)
    ref, qx, sx, acc, aabs = oracle.linear_g16(x, g, codes, host(f8), host(s))
    _check_y(y, ref, aabs, sx, host(s), K, "linear")


@pytest.mark.parametrize("name,bits", [("qkv", 6), ("qkv", 4), ("out", 4)])
def test_full_size(name, bits):
    """Dense projections over 8192 tokens (qkv: K = 2048, N = 6144; out: K = N = 2048, group 64, bias):
    converter bit for bit in full, the linear's output on 64 sampled token rows (all columns) against the
    oracle."""
    M, K, N, g = synth.DENSE_SHAPES[name]
    with_bias = name == "out"
    say(f"g16 full-size {name} M={M} K={K} N={N} g={g} bits={bits}")
    x, w, b = synth.dense_linear_inputs(M, K, N, with_bias)
    q, f8, s = cr.convrot_quantize_weights_g16(dev_bf16(w), g, bits)
    y = cr.convrot_linear_g16(dev_bf16(x), q, f8, s, g, bits, bias=None if b is None else dev_bf16(b))
    torch.cuda.synchronize()
    rq, rf, rs, codes = oracle.quantize_g16(w, g, bits)
    assert np.array_equal(host(q), rq) and np.array_equal(host(f8), rf)
    assert np.array_equal(host(s).view(np.uint32), rs.view(np.uint32))
    rows = np.sort(np.random.default_rng(9).choice(M, 64, replace=False))
    ref, qx, sx, acc, aabs = oracle.linear_g16(x[rows], g, codes, rf, rs, b)
    _check_y(y[torch.from_numpy(rows).to(DEV)], ref, aabs, sx, rs, K, "full-size linear (sampled rows)")
