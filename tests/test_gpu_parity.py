"""GPU parity: every stage of the HIP path against the CPU oracle on the same seeded inputs, through the C ABI.

Bar: codes, scales, rotated fp32 values, INT32 accumulators and routing bit-exact; BF16 outputs within 1e-2
relative elementwise.  Because every fp32 step is specified (order, no contraction, the fixed exponential), the
BF16 outputs are also expected bit-identical, and the tests assert that too.
"""
import numpy as np
import pytest
import torch

import oracle
from w8a8_rotated_int8_amd import binding as cr
from w8a8_rotated_int8_amd import synth

from helpers import DEV, assert_bf16_within, dev, dev_bf16, host, host_bf16, say, untile_codes

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _setup():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    cr.lib()
    oracle.load()


# ----------------------------------------------------------------------------------------------------------
# INT32 product (MFMA main loop)
# ----------------------------------------------------------------------------------------------------------

@pytest.mark.parametrize("M,N,K", [(1, 1, 16), (5, 7, 32), (33, 70, 48), (64, 128, 512), (100, 200, 272),
                                   (257, 129, 1536), (300, 130, 2048), (64, 256, 4096)])
def test_gemm_i8_i32_bit_exact(M, N, K):
    say(f"gemm_i8_i32 M={M} N={N} K={K}")
    rng = np.random.default_rng(M * 7 + N * 3 + K)
    a = rng.integers(-127, 128, (M, K)).astype(np.int8)
    b = rng.integers(-127, 128, (N, K)).astype(np.int8)
    got = host(cr.convrot_gemm_i8_i32(dev(a), dev(b)))
    assert np.array_equal(got, oracle.gemm_i8_i32(a, b))


def test_gemm_i8_i32_extremes():
    say("gemm_i8_i32 extremes K=8192")
    K = 8192
    a = np.full((40, K), 127, np.int8)
    a[1::2] = -127
    b = np.full((70, K), -127, np.int8)
    b[::3] = 127
    got = host(cr.convrot_gemm_i8_i32(dev(a), dev(b)))
    ref = oracle.gemm_i8_i32(a, b)
    assert np.array_equal(got, ref) and np.abs(ref).max() == K * 127 * 127


# ----------------------------------------------------------------------------------------------------------
# Rotate + quantise
# ----------------------------------------------------------------------------------------------------------

def _special_rows(rows, K, seed):
    x = synth.activations(seed, rows, K, max(1, K // 100))
    f = synth.bf16_bits_to_f32(x).copy()
    if rows >= 5:
        f[0] = 0.0                              # all-zero row: scale 0, codes 0
        f[1] = 0.0
        f[1, K // 3] = -3.0                     # one-hot
        f[2] *= np.float32(1e-38)               # subnormal-range values
        f[3] *= np.float32(1e30)                # large values
        f[4] = np.float32(0.5)                  # constant row
    return synth.to_bf16_bits(f)


@pytest.mark.parametrize("g", [64, 256])
@pytest.mark.parametrize("K", [256, 512, 1536, 2048, 8192])
@pytest.mark.parametrize("rows", [1, 7, 37])
def test_rotq_bit_exact(g, K, rows):
    if K % g:
        pytest.skip("K must be a multiple of the group")
    say(f"rotq g={g} K={K} rows={rows}")
    x = _special_rows(rows, K, 5000 + K + rows)
    q, s, rot = cr.convrot_rotq_rows(dev_bf16(x), g, want_rot=True)
    rq, rs, rrot = oracle.rotq_rows(x, g, return_rot=True)
    assert np.array_equal(host(rot).view(np.uint32), rrot.view(np.uint32))
    assert np.array_equal(host(s).view(np.uint32), rs.view(np.uint32))
    assert np.array_equal(host(q), rq)


@pytest.mark.parametrize("g,K", [(64, 512), (64, 1024), (64, 1536), (64, 3072), (64, 4096), (256, 2048),
                                 (256, 4096), (256, 8192)])
@pytest.mark.parametrize("rows", [1, 7, 37])
def test_rotq_codes_only_bit_exact(g, K, rows):
    """The codes-only path (no rotated values requested; the layer's own path), including rows whose scale
    falls below and just above the threshold of the reciprocal-based division, and a row whose scale is below
    2^-96 while 2^k times it (the unnormalised transform's scale) is not."""
    say(f"rotq codes g={g} K={K} rows={rows}")
    x = _special_rows(rows, K, 7000 + K + rows)
    if rows >= 7:
        f = synth.bf16_bits_to_f32(x).copy()
        f[5] *= np.float32(2.0 ** -100)         # scale near 2^-107: IEEE division
        f[6] *= np.float32(2.0 ** -80)          # scale near 2^-87: reciprocal-based division
        if rows >= 8:
            f[7] *= np.float32(2.0 ** -93)      # scale near 2^-97, unnormalised scale near 2^-94 (g 64) or 2^-93
        x = synth.to_bf16_bits(f)
    q, s, _ = cr.convrot_rotq_rows(dev_bf16(x), g)
    rq, rs = oracle.rotq_rows(x, g)
    assert np.array_equal(host(s).view(np.uint32), rs.view(np.uint32))
    assert np.array_equal(host(q), rq)


def test_rotq_zero_rows_is_noop():
    x = torch.zeros((0, 512), dtype=torch.bfloat16, device=DEV)
    q, s, _ = cr.convrot_rotq_rows(x, 64)
    assert q.shape == (0, 512) and s.shape == (0,)


def test_quantize_prerotated_ties_and_subnormals():
    import json
    import os
    fx = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "quantizer_ties.json")))
    for key, bits in (("rows", 8), ("rows4", 4)):
        r = np.zeros((len(fx[key]), 16), np.float32)
        for i, row in enumerate(fx[key]):
            r[i, :len(row["r"])] = row["r"]
        q, s = cr.convrot_quantize_prerotated(dev(r), bits)
        q, s = host(q), host(s)
        for i, row in enumerate(fx[key]):
            assert s[i] == row["scale"] and q[i, :len(row["codes"])].tolist() == row["codes"]
    tiny = np.float32(2.0 ** -149)
    rng = np.random.default_rng(3)
    r = (rng.standard_normal((64, 64)) * 10.0 ** rng.integers(-40, 30, (64, 1))).astype(np.float32)
    r[0, :4] = [190 * tiny, -100 * tiny, 3 * tiny, 0.0]
    r[0, 4:] = 0
    for bits, qmax in ((8, 127), (4, 7)):
        q, s = cr.convrot_quantize_prerotated(dev(r), bits)
        rq, rs = oracle.quantize_rows(r, qmax)
        assert np.array_equal(host(q), rq) and np.array_equal(host(s).view(np.uint32), rs.view(np.uint32))


# ----------------------------------------------------------------------------------------------------------
# Weight converter
# ----------------------------------------------------------------------------------------------------------

@pytest.mark.parametrize("bits", [8, 4])
@pytest.mark.parametrize("g,shape", [(64, (3, 40, 512)), (256, (2, 33, 1536)), (64, (1, 5, 8192)), (256, (2, 64, 256))])
def test_weight_converter_bit_exact(bits, g, shape):
    say(f"convert bits={bits} g={g} shape={shape}")
    w = synth.weights(900 + g + bits, shape)
    rq, rs = oracle.quantize_weights(w, g, bits)
    q, s = cr.convrot_quantize_weights(dev_bf16(w), g, bits, layout=cr.LAYOUT_ROWMAJOR)
    assert np.array_equal(host(q), rq)
    assert np.array_equal(host(s).view(np.uint32), rs.view(np.uint32))
    qt, st = cr.convrot_quantize_weights(dev_bf16(w), g, bits, layout=cr.LAYOUT_MFMA)
    E, N, K = shape
    assert qt.numel() == cr.convrot_weight_bytes(E, N, K, bits, cr.LAYOUT_MFMA) == E * ((N + 31) // 32) * 32 * K * bits // 8
    codes = rq if bits == 8 else oracle.unpack_int4(rq, K)
    assert np.array_equal(untile_codes(host(qt), E, N, K, bits), codes)
    # rows past N in the last block are zero
    NB = (N + 31) // 32
    full = untile_codes(host(qt), E, NB * 32, K, bits)
    assert not full[:, N:, :].any()
    assert np.array_equal(host(st).view(np.uint32), rs.view(np.uint32))


def test_weight_converter_rejects_nonfinite():
    w = synth.weights(5, (2, 8, 256))
    w[1, 3, 17] = 0x7F80  # +inf
    with pytest.raises(cr.ConvrotError) as ei:
        cr.convrot_quantize_weights(dev_bf16(w), 64, 8)
    assert ei.value.status == 7


# ----------------------------------------------------------------------------------------------------------
# Single W8A8 ConvRot linear (config 0 and ragged shapes)
# ----------------------------------------------------------------------------------------------------------

@pytest.mark.parametrize("M,K,N,g,with_bias", [(64, 512, 256, 64, False), (64, 512, 256, 64, True),
                                               (37, 768, 77, 256, False), (1, 256, 1, 64, True),
                                               (300, 2048, 300, 256, True),
                                               # 65..128 rows: the GEMM's 128-row tile
                                               (100, 512, 300, 64, True), (128, 1024, 256, 256, False)])
def test_linear_bit_exact(M, K, N, g, with_bias):
    say(f"linear M={M} K={K} N={N} g={g} bias={with_bias}")
    x, w = synth.linear_inputs(0, M=M, K=K, N=N, n_outlier=max(1, K // 128))
    bias = synth.to_bf16_bits(np.random.default_rng(1).standard_normal(N).astype(np.float32)) if with_bias else None
    qw, sw = cr.convrot_quantize_weights(dev_bf16(w), g, 8)
    y = cr.convrot_linear_w8a8(dev_bf16(x), qw, sw, g, bias=None if bias is None else dev_bf16(bias))
    rqw, rsw = oracle.quantize_weights(w, g, 8)
    ry, _, _ = oracle.linear_w8a8(x, rqw, rsw, g, bias)
    got = host_bf16(y)
    exact = assert_bf16_within(got, ry, what="linear")
    assert exact == 1.0


# ----------------------------------------------------------------------------------------------------------
# LoRA patch of quantised weights, re-quantised with random rounding
# ----------------------------------------------------------------------------------------------------------

def _lora_case(E, N, K, g, rank, seed):
    rng = np.random.default_rng(seed)
    w = synth.weights(seed, (E, N, K))
    q, s = oracle.quantize_weights(w, g, 8)
    lb = synth.to_bf16_bits((rng.standard_normal((E, N, rank)) * 0.05).astype(np.float32))
    la = synth.to_bf16_bits((rng.standard_normal((E, rank, K)) * 0.05).astype(np.float32))
    return q, s, lb, la


@pytest.mark.parametrize("E,N,K,g,rank,alpha", [(2, 37, 512, 64, 8, 0.5), (1, 64, 2048, 256, 16, 1.0),
                                                (3, 5, 256, 64, 0, 1.0), (2, 33, 1536, 64, 4, -0.75),
                                                (1, 32, 8192, 256, 2, 2.0)])
def test_lora_requant_bit_exact(E, N, K, g, rank, alpha):
    say(f"lora requant E={E} N={N} K={K} g={g} rank={rank} alpha={alpha}")
    q, s, lb, la = _lora_case(E, N, K, g, rank, 900 + N + K)
    rq, rs = oracle.requantize_lora(q, s, g, lb, la, alpha, seed=77)
    qd, sd = dev(q), dev(s)
    lbd = dev_bf16(lb) if rank else None
    lad = dev_bf16(la) if rank else None
    q_row, s_row = cr.convrot_requantize_lora(qd, sd, g, lbd, lad, alpha, 77, layout=cr.LAYOUT_ROWMAJOR)
    assert np.array_equal(host(s_row).view(np.uint32), rs.view(np.uint32)), "scales"
    assert np.array_equal(host(q_row), rq), "codes (row-major)"
    q_t, s_t = cr.convrot_requantize_lora(qd, sd, g, lbd, lad, alpha, 77, layout=cr.LAYOUT_MFMA)
    assert np.array_equal(untile_codes(host(q_t), E, N, K, 8), rq), "codes (MFMA layout)"
    assert np.array_equal(host(s_t), host(s_row))
    if rank:  # without a delta the quotients are (nearly always) whole numbers: nothing random to round
        q_o, _ = cr.convrot_requantize_lora(qd, sd, g, lbd, lad, alpha, 78, layout=cr.LAYOUT_ROWMAJOR)
        assert not np.array_equal(host(q_o), rq), "another seed draws other roundings"
    # the re-quantising mode: nearest rounding of the same patched values
    rqn, rsn = oracle.requantize_lora(q, s, g, lb, la, alpha, seed=77, nearest=True)
    for layout in (cr.LAYOUT_ROWMAJOR, cr.LAYOUT_MFMA):
        q_n, s_n = cr.convrot_requantize_lora(qd, sd, g, lbd, lad, alpha, 5, layout=layout, rounding=cr.ROUND_NEAREST)
        got = host(q_n) if layout == cr.LAYOUT_ROWMAJOR else untile_codes(host(q_n), E, N, K, 8)
        assert np.array_equal(got, rqn), f"nearest codes (layout {layout})"
        assert np.array_equal(host(s_n).view(np.uint32), rsn.view(np.uint32)), "nearest scales"


# ----------------------------------------------------------------------------------------------------------
# Routing
# ----------------------------------------------------------------------------------------------------------

@pytest.mark.parametrize("T,E,C", [(300, 16, 1), (300, 16, 17), (300, 16, 300), (2048, 64, 64), (5000, 8, 1234),
                                   (1001, 48, 100), (8192, 64, 256), (13000, 16, 777), (20000, 8, 5000),
                                   # more than 64 experts: the one-thread-per-token softmax
                                   (500, 96, 50), (70, 80, 70),
                                   # more than 32768 tokens: the selection that re-reads its keys each pass
                                   (40000, 4, 3000), (33000, 2, 1)])
def test_route_from_logits_bit_exact(T, E, C):
    say(f"route T={T} E={E} C={C}")
    lg = synth.logits(T + E, T, E)
    lg[7] = lg[3]  # exact ties between tokens
    idx, wt, p = cr.moe_route_expert_choice(dev(lg), C, want_probs=True)
    ridx, rwt, rp = oracle.route(lg, C)
    assert np.array_equal(host(p).view(np.uint32), rp.view(np.uint32))
    assert np.array_equal(host(idx), ridx)
    assert np.array_equal(host(wt).view(np.uint32), rwt.view(np.uint32))


@pytest.mark.parametrize("T,E,C", [(96, 4, 10), (300, 8, 37), (5000, 64, 100), (40000, 4, 999), (400, 72, 40)])
def test_route_large_logit_gaps_bit_exact(T, E, C):
    """Gaps of 86 to 100 nats to the token's maximum: the exponential underflows into the subnormals, the
    divisions take subnormal numerators, and the selection ranks subnormal probabilities."""
    say(f"route large gaps T={T} E={E} C={C}")
    lg = synth.large_gap_logits(T, E, 40 + T + E)
    idx, wt, p = cr.moe_route_expert_choice(dev(lg), C, want_probs=True)
    ridx, rwt, rp = oracle.route(lg, C)
    assert np.array_equal(host(p).view(np.uint32), rp.view(np.uint32))
    assert np.array_equal(host(idx), ridx)
    assert np.array_equal(host(wt).view(np.uint32), rwt.view(np.uint32))
    assert np.count_nonzero((rp[:, 1:] > 0) & (rp[:, 1:] < np.finfo(np.float32).tiny)) > T  # subnormals hit


def test_route_from_probs_with_heavy_ties():
    say("route from probs with ties")
    rng = np.random.default_rng(8)
    T, E = 3000, 12
    p = rng.choice(np.float32([0.0, -0.0, 0.25, 0.5, 0.125, 1e-30, 3e-41]), size=(T, E)).astype(np.float32)
    for C in (1, 5, 700, 2999, 3000):
        idx, wt, _ = cr.moe_route_expert_choice(dev(p), C, is_probs=True)
        ridx, rwt = oracle.route_from_probs(p, C)
        assert np.array_equal(host(idx), ridx)
        assert np.array_equal(host(wt).view(np.uint32), rwt.view(np.uint32))


@pytest.mark.parametrize("n_bin,tie", [(1, False), (7, True), (64, False), (64, True), (65, False), (65, True),
                                       (300, True)])
def test_route_few_keys_left_after_first_pass(n_bin, tie):
    """After the first 11-bit radix pass the threshold's bin holds n_bin keys (0.5 (1 + k 2^-20): same exponent and
    top mantissa bits, apart from the 0.9 above and the [1e-3, 2e-3) below).  Up to 64 such keys are ranked by one
    wavefront, more take the further passes; both must give the oracle's list, equal keys in the bin included."""
    say(f"route few keys left n_bin={n_bin} tie={tie}")
    rng = np.random.default_rng(100 + n_bin + tie)
    T, E, n_top = 4096, 2, 37
    p = np.empty((T, E), np.float32)
    k = np.arange(n_bin) // (2 if tie else 1)
    cluster = (np.float32(0.5) * (np.float32(1) + k.astype(np.float32) * np.float32(2.0 ** -20))).astype(np.float32)
    for e in range(E):
        col = ((rng.random(T) + 1.0) * 1e-3).astype(np.float32)
        perm = rng.permutation(T)
        col[perm[:n_top]] = np.float32(0.9)
        col[perm[n_top:n_top + n_bin]] = cluster
        p[:, e] = col
    for r in sorted({1, n_bin // 2 + 1, n_bin}):
        C = n_top + r
        idx, wt, _ = cr.moe_route_expert_choice(dev(p), C, is_probs=True)
        ridx, rwt = oracle.route_from_probs(p, C)
        assert np.array_equal(host(idx), ridx), f"C={C}"
        assert np.array_equal(host(wt).view(np.uint32), rwt.view(np.uint32)), f"C={C}"


@pytest.mark.parametrize("mix", [(1, 1, 1, 1, 1, 1, 1), (48, 48, 4, 0, 0, 0, 0)])
def test_route_from_probs_with_zero_ties_long(mix):
    """T > 16384: the selection keeps only keys and recovers a selected token's weight from its key, with one
    bit per key for the sign of zero.  Selected +0 and -0 must come back as they were, for C below the LDS
    staging limit (1024) and above it."""
    say(f"route from probs with zero ties, T=20000, mix={mix}")
    rng = np.random.default_rng(sum(mix))
    T, E = 20000, 4
    vals = np.float32([0.0, -0.0, 0.25, 0.5, 0.125, 1e-30, 3e-41])
    w = np.float64(mix) / np.sum(mix)
    p = rng.choice(vals, size=(T, E), p=w).astype(np.float32)
    for C in (3, 1000, 5000, 19999):
        idx, wt, _ = cr.moe_route_expert_choice(dev(p), C, is_probs=True)
        ridx, rwt = oracle.route_from_probs(p, C)
        assert np.array_equal(host(idx), ridx), f"C={C}"
        assert np.array_equal(host(wt).view(np.uint32), rwt.view(np.uint32)), f"C={C}"
        sel = rwt.view(np.uint32)
        if C == 1000 and mix[0] == 48:
            assert np.any(sel == 0x80000000) and np.any(sel == 0), "both signs of zero selected"


# ----------------------------------------------------------------------------------------------------------
# MoE stages given identical inputs, and the whole layer
# ----------------------------------------------------------------------------------------------------------

SMALL = [
    synth.MoEShape(T=96, d=512, E=4, I=128, C=24),
    synth.MoEShape(T=200, d=768, E=5, I=192, C=37, g_gu=256, g_dn=64),
    synth.MoEShape(T=64, d=256, E=3, I=64, C=64, g_gu=64, g_dn=64),
    synth.MoEShape(T=333, d=512, E=6, I=256, C=1, g_gu=256, g_dn=256),
    synth.MoEShape(T=400, d=512, E=2, I=128, C=300),
    # d a multiple of 8 g_gu: the token rotate+quantise rides in the routing launches (rows split between them)
    synth.MoEShape(T=300, d=512, E=8, I=128, C=50, g_gu=64, g_dn=64),
    synth.MoEShape(T=3, d=512, E=2, I=64, C=2, g_gu=64, g_dn=64),
    # 65..128 slots per expert: the GEMMs' 128-row tile (both epilogues, both weight widths)
    synth.MoEShape(T=300, d=512, E=4, I=128, C=100),
    synth.MoEShape(T=256, d=512, E=3, I=192, C=128, g_gu=64, g_dn=64),
    # the routing launches' rotate+quantise with 4 and 2 register rounds per lane, and the selection with 2 and 8
    # key rounds per lane (T up to 4096, up to 16384)
    synth.MoEShape(T=3000, d=2048, E=4, I=64, C=20, g_gu=64, g_dn=64),
    synth.MoEShape(T=10000, d=1024, E=4, I=64, C=50, g_gu=64, g_dn=64),
    synth.MoEShape(T=500, d=4096, E=2, I=64, C=10, g_gu=256, g_dn=64),
    # more than 64 experts: softmax, rotate+quantise and selection as separate launches
    synth.MoEShape(T=200, d=256, E=80, I=64, C=5, g_gu=64, g_dn=64),
    # one expert taking every token (all probabilities 1: ties throughout, one slot-table column)
    synth.MoEShape(T=50, d=512, E=1, I=64, C=50, g_gu=64, g_dn=64),
    # 64 experts (the softmax tile compiled for E = 64) with a ragged last tile of 4 tokens
    synth.MoEShape(T=100, d=512, E=64, I=64, C=10, g_gu=64, g_dn=64),
]


def _layer(shape, bits, seed):
    x, lg, w_gu, w_dn = synth.moe_inputs(2, shape, seed_base=seed)
    q_gu, s_gu = oracle.quantize_weights(w_gu, shape.g_gu, bits)
    q_dn, s_dn = oracle.quantize_weights(w_dn, shape.g_dn, bits)
    ref = oracle.moe_forward(x, lg, shape.C, q_gu, s_gu, shape.g_gu, q_dn, s_dn, shape.g_dn, bits,
                             intermediates=True)
    w = cr.quantize_moe_weights(dev_bf16(w_gu), dev_bf16(w_dn), shape.g_gu, shape.g_dn, bits)
    cg = q_gu if bits == 8 else oracle.unpack_int4(q_gu, shape.d)
    cd = q_dn if bits == 8 else oracle.unpack_int4(q_dn, shape.I)
    assert np.array_equal(untile_codes(host(w.q_gu), shape.E, 2 * shape.I, shape.d, bits), cg)
    assert np.array_equal(untile_codes(host(w.q_dn), shape.E, shape.d, shape.I, bits), cd)
    return x, lg, w, ref


@pytest.mark.parametrize("bits", [8, 4])
@pytest.mark.parametrize("si", range(len(SMALL)))
def test_moe_stages_bit_exact(si, bits):
    shape = SMALL[si]
    say(f"moe stages {shape} bits={bits}")
    x, lg, w, ref = _layer(shape, bits, 10000 + si)
    idx = dev(ref["idx"])
    a = cr.moe_gateup_swiglu(dev(ref["qx"]), dev(ref["sx"]), idx, w)
    assert np.array_equal(host_bf16(a), ref["a"]), "gate/up + SwiGLU stage"
    qa, sa, _ = cr.convrot_rotq_rows(dev_bf16(ref["a"]), shape.g_dn)
    assert np.array_equal(host(qa), ref["qa"]) and np.array_equal(host(sa), ref["sa"])
    z = cr.moe_down_proj(dev(ref["qa"]), dev(ref["sa"]), shape.C, w)
    assert np.array_equal(host_bf16(z), ref["z"]), "down stage"
    out = cr.moe_combine(dev_bf16(ref["z"]), idx, dev(ref["wt"]), shape.T)
    assert np.array_equal(host_bf16(out), ref["out"]), "combine stage"


@pytest.mark.parametrize("bits", [8, 4])
@pytest.mark.parametrize("si", range(len(SMALL)))
def test_moe_forward_end_to_end(si, bits):
    shape = SMALL[si]
    say(f"moe forward {shape} bits={bits}")
    x, lg, w, ref = _layer(shape, bits, 20000 + si)
    out, idx, wt = cr.moe_expert_choice_forward(dev_bf16(x), dev(lg), shape.C, w)
    assert np.array_equal(host(idx), ref["idx"])
    assert np.array_equal(host(wt).view(np.uint32), ref["wt"].view(np.uint32))
    got = host_bf16(out)
    exact = assert_bf16_within(got, ref["out"], what="moe out")
    assert exact == 1.0
    # determinism: a second call gives the same bits
    out2, _, _ = cr.moe_expert_choice_forward(dev_bf16(x), dev(lg), shape.C, w)
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))


# Shapes that the one-launch expert path (gate/up, hidden-row rotate+quantise, down) takes: each rotation variant
# of the hidden rows (group 64 with I / 512 = 1, 2, 3, 4; group 256 with I = 2048), the three tile heights
# (C <= 64, <= 128, > 128, and two M-blocks per expert), an expert count that the 8 XCDs do not divide, and a
# grid of fewer than 8 workgroups.
FUSED = [
    synth.MoEShape(T=300, d=512, E=6, I=512, C=37, g_gu=256, g_dn=64),
    synth.MoEShape(T=400, d=256, E=5, I=1024, C=100, g_gu=256, g_dn=64),
    synth.MoEShape(T=64, d=512, E=9, I=1536, C=8, g_gu=64, g_dn=64),
    synth.MoEShape(T=600, d=512, E=3, I=2048, C=300, g_gu=256, g_dn=256),
    synth.MoEShape(T=200, d=256, E=2, I=2048, C=130, g_gu=64, g_dn=64),
    synth.MoEShape(T=2, d=512, E=1, I=512, C=1, g_gu=256, g_dn=64),
]


@pytest.mark.parametrize("bits", [8, 4])
@pytest.mark.parametrize("si", range(len(FUSED)))
def test_moe_forward_fused_bit_exact(si, bits):
    shape = FUSED[si]
    say(f"moe forward, one expert launch {shape} bits={bits}")
    x, lg, w, ref = _layer(shape, bits, 30000 + si)
    assert cr.moe_expert_choice_fused(w, shape.C)
    out, idx, wt = cr.moe_expert_choice_forward(dev_bf16(x), dev(lg), shape.C, w, fused=True)
    assert np.array_equal(host(idx), ref["idx"])
    assert np.array_equal(host(wt).view(np.uint32), ref["wt"].view(np.uint32))
    assert np.array_equal(host_bf16(out), ref["out"]), "moe out"
    # the counters are cleared by every call's selection: further calls, also after a three-launch forward on
    # the same workspace, give the same bits
    ws = torch.empty(cr.moe_expert_choice_workspace_bytes(shape.T, shape.C, w), dtype=torch.uint8, device=DEV)
    for fused in (True, False, True):
        o, _, _ = cr.moe_expert_choice_forward(dev_bf16(x), dev(lg), shape.C, w, ws=ws, fused=fused)
        assert torch.equal(out.view(torch.int16), o.view(torch.int16)), f"repeat (fused={fused})"


def test_single_expert_ffn_config1():
    """One routed-expert SwiGLU FFN without routing (E = 1, C = T = 1024, d = 2048, I = 1536)."""
    shape = synth.CONFIGS[1]
    say(f"config 1 {shape}")
    x, lg, w_gu, w_dn = synth.moe_inputs(1)
    w = cr.quantize_moe_weights(dev_bf16(w_gu), dev_bf16(w_dn), 256, 64, 8)
    out, idx, wt = cr.moe_expert_choice_forward(dev_bf16(x), dev(lg), shape.C, w)
    q_gu, s_gu = oracle.quantize_weights(w_gu, 256)
    q_dn, s_dn = oracle.quantize_weights(w_dn, 64)
    assert np.array_equal(untile_codes(host(w.q_gu), 1, 3072, 2048, 8), q_gu)
    assert np.array_equal(host(w.s_dn), s_dn)
    ref = oracle.moe_forward(x, lg, shape.C, q_gu, s_gu, 256, q_dn, s_dn, 64)
    assert np.array_equal(host(idx), ref["idx"]) and np.all(host(wt) == 1.0)
    exact = assert_bf16_within(host_bf16(out), ref["out"], what="config 1 out")
    assert exact == 1.0


def test_moe_forward_fused_without_routing_outputs():
    shape = FUSED[0]
    say(f"moe forward, one expert launch, NULL routing outputs {shape}")
    x, lg, w, ref = _layer(shape, 8, 30100)
    out, idx, wt = cr.moe_expert_choice_forward(dev_bf16(x), dev(lg), shape.C, w, want_routing=False, fused=True)
    assert idx is None and wt is None
    assert np.array_equal(host_bf16(out), ref["out"]), "moe out"


def test_moe_forward_fused_rejects_other_shapes():
    shape = SMALL[0]  # I = 128: rows too short for the one-launch path
    x, lg, w_gu, w_dn = synth.moe_inputs(2, shape, seed_base=40000)
    w = cr.quantize_moe_weights(dev_bf16(w_gu), dev_bf16(w_dn), shape.g_gu, shape.g_dn, 8)
    assert not cr.moe_expert_choice_fused(w, shape.C)
    with pytest.raises(cr.ConvrotError, match="SHAPE"):
        cr.moe_expert_choice_forward(dev_bf16(x), dev(lg), shape.C, w, fused=True)


def test_moe_forward_without_routing_outputs():
    """idx_out / wt_out NULL: the forward keeps the routing in its workspace."""
    shape = SMALL[5]
    say(f"moe forward, routing outputs NULL {shape}")
    x, lg, w, ref = _layer(shape, 8, 30000)
    out, idx, wt = cr.moe_expert_choice_forward(dev_bf16(x), dev(lg), shape.C, w, want_routing=False)
    assert idx is None and wt is None
    assert np.array_equal(host_bf16(out), ref["out"])


def test_moe_forward_large_logit_gaps():
    """The whole layer with router logits 86 to 100 nats below each token's maximum (subnormal probabilities
    weight the combine)."""
    shape = SMALL[5]
    say(f"moe forward, large logit gaps {shape}")
    x, _, w_gu, w_dn = synth.moe_inputs(2, shape, seed_base=31000)
    lg = synth.large_gap_logits(shape.T, shape.E, 31004)
    q_gu, s_gu = oracle.quantize_weights(w_gu, shape.g_gu, 8)
    q_dn, s_dn = oracle.quantize_weights(w_dn, shape.g_dn, 8)
    ref = oracle.moe_forward(x, lg, shape.C, q_gu, s_gu, shape.g_gu, q_dn, s_dn, shape.g_dn, 8)
    w = cr.quantize_moe_weights(dev_bf16(w_gu), dev_bf16(w_dn), shape.g_gu, shape.g_dn, 8)
    out, idx, wt = cr.moe_expert_choice_forward(dev_bf16(x), dev(lg), shape.C, w)
    assert np.array_equal(host(idx), ref["idx"])
    assert np.array_equal(host(wt).view(np.uint32), ref["wt"].view(np.uint32))
    assert np.array_equal(host_bf16(out), ref["out"])


@pytest.mark.parametrize("bits", [8, 4])
def test_gateup_swiglu_far_gates(bits):
    """Gate scales stretched so the dequantised gates reach +-1e4: the epilogue evaluates silu for every gate
    outside its LDS window, including gates below -64 (silu as g * E(g)), below -88.7 (where E(-g) overflows)
    and below -104 (silu underflows to -0)."""
    shape = synth.MoEShape(T=96, d=512, E=4, I=128, C=24)
    say(f"gate/up far gates {shape} bits={bits}")
    x, lg, w_gu, w_dn = synth.moe_inputs(2, shape, seed_base=32000)
    w = cr.quantize_moe_weights(dev_bf16(w_gu), dev_bf16(w_dn), shape.g_gu, shape.g_dn, bits)
    rng = np.random.default_rng(5)
    s_gu = host(w.s_gu).copy()
    s_gu[:, :shape.I] *= (10.0 ** rng.uniform(0.0, 4.5, (shape.E, shape.I))).astype(np.float32)
    w.s_gu = dev(s_gu)
    q_gu = untile_codes(host(w.q_gu), shape.E, 2 * shape.I, shape.d, bits)
    qx, sx = oracle.rotq_rows(x, shape.g_gu)
    idx, _, _ = oracle.route(lg, shape.C)
    packed = q_gu if bits == 8 else oracle.pack_int4(q_gu)
    ref = oracle.moe_gateup(qx, sx, idx, packed, s_gu, bits)
    a = cr.moe_gateup_swiglu(dev(qx), dev(sx), dev(idx), w)
    assert np.array_equal(host_bf16(a), ref)
    # the gates really reach the far ranges
    g = np.concatenate([oracle.gemm_i8_i32(qx[idx[e]], q_gu[e, :shape.I]).astype(np.float64)
                        * sx[idx[e]][:, None] * s_gu[e, :shape.I][None, :] for e in range(shape.E)])
    for lo, hi in ((-np.inf, -104.0), (-104.0, -88.8), (-88.7, -64.0), (88.8, np.inf)):
        assert np.count_nonzero((g > lo) & (g < hi)) > 10, (lo, hi)
