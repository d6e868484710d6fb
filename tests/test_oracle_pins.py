"""Pins for the CPU oracle: each check ties the oracle to something other than itself (hand-derived fixtures,
library routines, closed forms, invariants, brute force), chosen so that a dropped term, a wrong sign or index,
or a transposed operand anywhere in the oracle fails at least one of them."""
import json
import math
import os

import numpy as np
import pytest
import scipy.linalg
import torch

from w8a8_rotated_int8_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _ulp_diff_f32(a, b):
    """Distance in fp32 units in the last place between two fp32 arrays (finite, same sign region)."""
    ai = np.asarray(a, np.float32).view(np.int32).astype(np.int64)
    bi = np.asarray(b, np.float32).view(np.int32).astype(np.int64)
    ai = np.where(ai < 0, np.int64(-2**31) - ai, ai)
    bi = np.where(bi < 0, np.int64(-2**31) - bi, bi)
    return np.abs(ai - bi)


# ---------------------------------------------------------------------------------------------------------
# bf16 rounding and the fixed exponential
# ---------------------------------------------------------------------------------------------------------

def test_bf16_round_matches_torch(orc):
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10.0 ** rng.integers(-30, 30, 100000),
                        np.array([0.0, -0.0, 1.0, 3.4e38, -3.4e38, 1e-45, 1.00390625, 1.01171875, np.inf, -np.inf],
                                 np.float32)]).astype(np.float32)
    ours = orc.bf16_round(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def _all_finite_bf16_as_f32():
    bits = np.arange(65536, dtype=np.uint32)
    f = (bits << 16).view(np.float32)
    return f[np.isfinite(f)]


def test_exp_within_two_ulp_of_libm(orc):
    # Every fp32 result, normal and subnormal, is within 2 units in the last place of e^x rounded from
    # float64: a dense sweep from where e^x rounds to 0 to where it overflows, and every finite bf16 input.
    x = np.concatenate([np.linspace(-110.0, 95.0, 4_000_001, dtype=np.float32), _all_finite_bf16_as_f32()])
    ours = orc.exp(x)
    with np.errstate(over="ignore"):
        ref = np.exp(x.astype(np.float64)).astype(np.float32)
    fin = np.isfinite(ref)
    assert np.array_equal(ours[~fin], ref[~fin])  # +inf exactly where e^x overflows fp32
    assert _ulp_diff_f32(ours[fin], ref[fin]).max() <= 2
    assert orc.exp(np.float32([0.0]))[0] == 1.0
    # underflow through the subnormals: e^-100 is about 3.7e-44, representable only as a subnormal
    e100 = orc.exp(np.float32([-100.0]))[0]
    assert 0.0 < e100 < np.finfo(np.float32).tiny and abs(float(e100) - math.exp(-100.0)) <= 2.0 ** -148
    # the ends: exactly 0 below about -103.97, +inf above about 88.72, also for infinite arguments
    assert np.all(orc.exp(np.float32([-104.0, -150.0, -1000.0, -np.inf])) == 0.0)
    assert np.all(np.isposinf(orc.exp(np.float32([88.73, 100.0, 1e30, np.inf]))))
    assert np.isfinite(orc.exp(np.float32([88.72]))[0])


def _silu_fp64(g):
    g = np.asarray(g, np.float64)
    with np.errstate(over="ignore", under="ignore"):
        e = np.exp(-np.abs(g))  # never overflows
    return np.where(g >= 0, g / (1.0 + e), g * e / (1.0 + e))


def test_silu_close_to_fp64(orc):
    # within a few ulp of fp64 silu, with an absolute floor for subnormal results: there e^g carries up to
    # 2 subnormal ulps and the product with g scales that by |g| (plus one rounding of the product)
    g = np.concatenate([np.linspace(-160.0, 160.0, 800001, dtype=np.float32), _all_finite_bf16_as_f32()])
    ours = orc.silu(g).astype(np.float64)
    ref = _silu_fp64(g)
    floor = (2.0 * np.abs(g.astype(np.float64)) + 2.0) * 2.0 ** -149
    assert np.all(np.abs(ours - ref) <= 5e-7 * np.abs(ref) + floor)
    assert orc.silu(np.float32([0.0]))[0] == 0.0
    # far negative gates stay on the curve instead of saturating: silu(-90) is about -7.3e-38
    v = orc.silu(np.float32([-90.0, -100.0]))
    assert v[0] < 0 and abs(v[0] / (-90.0 * math.exp(-90.0)) - 1.0) < 1e-6
    assert v[1] < 0 and abs(float(v[1]) + 100.0 * math.exp(-100.0)) <= 202 * 2.0 ** -149
    assert np.all(orc.silu(np.float32([-120.0, -np.finfo(np.float32).max])) == 0.0)
    big = np.float32([100.0, 3.0e38])
    assert np.array_equal(orc.silu(big), big)


# ---------------------------------------------------------------------------------------------------------
# Rotation
# ---------------------------------------------------------------------------------------------------------

def test_hadamard_fixture_g4(orc):
    fx = json.load(open(os.path.join(GOLDEN, "hadamard_g4.json")))
    H = orc.rotate_rows_f32(np.eye(4, dtype=np.float32), 4)
    assert np.array_equal(H, np.array(fx["H_normalised"], np.float32))
    for ex in fx["examples"]:
        v = np.array(ex["v"], np.float32)[None]
        assert np.array_equal(orc.rotate_rows_f32(v, 4)[0], np.array(ex["rotated"], np.float32))


@pytest.mark.parametrize("g", [64, 256])
def test_hadamard_is_sylvester_and_orthonormal(orc, g):
    # Rotating the identity yields the matrix itself (one-hot e_i -> row i of H / sqrt(g)); entries are
    # +-2^-k so every check below is exact.
    H = orc.rotate_rows_f32(np.eye(g, dtype=np.float32), g).astype(np.float64)
    assert np.array_equal(H, scipy.linalg.hadamard(g) / math.sqrt(g))
    assert np.array_equal(H, H.T)
    assert np.array_equal(H @ H.T, np.eye(g))


@pytest.mark.parametrize("g", [64, 256])
def test_rotation_is_block_diagonal_fwht(orc, g):
    rng = np.random.default_rng(g)
    K = 3 * g
    x = rng.standard_normal((5, K)).astype(np.float32)
    r = orc.rotate_rows_f32(x, g).astype(np.float64)
    Hn = scipy.linalg.hadamard(g) / math.sqrt(g)
    ref = np.concatenate([x[:, b:b + g].astype(np.float64) @ Hn for b in range(0, K, g)], axis=1)
    # fp32 butterflies: each output is a sum of g terms, error below log2(g) roundings of the partial sums
    assert np.abs(r - ref).max() <= np.abs(x).max() * math.sqrt(g) * 8 * 2.0 ** -24 * 8


def test_rotation_of_bf16_input_equals_fp32_path(orc):
    x = synth.activations(77, 4, 512, 4)
    assert np.array_equal(orc.rotate_rows_bf16(x, 64), orc.rotate_rows_f32(synth.bf16_bits_to_f32(x), 64))


@pytest.mark.parametrize("g", [64, 256])
def test_rotation_invariance_of_product(orc, g):
    # x . W^T == (x R)(W R)^T because R is orthogonal and symmetric; here R is applied by the oracle in fp32.
    rng = np.random.default_rng(1 + g)
    x = rng.standard_normal((16, 2 * g)).astype(np.float32)
    w = (0.02 * rng.standard_normal((24, 2 * g))).astype(np.float32)
    xr = orc.rotate_rows_f32(x, g).astype(np.float64)
    wr = orc.rotate_rows_f32(w, g).astype(np.float64)
    ref = x.astype(np.float64) @ w.astype(np.float64).T
    got = xr @ wr.T
    assert np.linalg.norm(got - ref) / np.linalg.norm(ref) < 1e-6


# ---------------------------------------------------------------------------------------------------------
# Quantiser
# ---------------------------------------------------------------------------------------------------------

def test_quantizer_ties_fixture(orc):
    fx = json.load(open(os.path.join(GOLDEN, "quantizer_ties.json")))
    for key, qkey in (("rows", "qmax"), ("rows4", "qmax4")):
        for row in fx[key]:
            q, s = orc.quantize_rows(np.array(row["r"], np.float32)[None], fx[qkey])
            assert s[0] == row["scale"]
            assert q[0].tolist() == row["codes"]


def test_quantizer_invariants(orc):
    rng = np.random.default_rng(5)
    r = (rng.standard_normal((200, 512)) * 10.0 ** rng.integers(-20, 20, (200, 1))).astype(np.float32)
    r[3] = 0.0
    q, s = orc.quantize_rows(r, 127)
    assert q.min() >= -127 and q.max() <= 127
    assert s[3] == 0 and not q[3].any()
    amax = np.abs(r).max(axis=1)
    assert np.array_equal(s, (amax / np.float32(127)).astype(np.float32))
    for i in range(r.shape[0]):
        if amax[i] > 0:
            j = np.argmax(np.abs(r[i]))
            assert abs(int(q[i, j])) == 127
    err = np.abs(r.astype(np.float64) - q.astype(np.float64) * s[:, None])
    assert np.all(err <= s[:, None].astype(np.float64) * (0.5 + 1e-5))
    # quantise -> dequantise -> quantise returns the same codes
    r2 = (q.astype(np.float32) * s[:, None]).astype(np.float32)
    q2, _ = orc.quantize_rows(r2, 127)
    assert np.array_equal(q, q2)


def test_quantizer_clamps_when_scale_is_subnormal(orc):
    # amax = 190 * 2^-149: amax / 127 rounds to the smallest subnormal 2^-149, so amax / scale = 190 and only
    # the clamp keeps the code at 127; the other elements code exactly.
    tiny = np.float32(2.0 ** -149)
    r = np.array([[190 * tiny, -100 * tiny, 3 * tiny, 0.0]], np.float32)
    q, s = orc.quantize_rows(r, 127)
    assert s[0] == tiny
    assert q[0].tolist() == [127, -100, 3, 0]


def test_int4_pack_roundtrip_and_range(orc):
    rng = np.random.default_rng(9)
    q = rng.integers(-7, 8, (6, 64)).astype(np.int8)
    p = orc.pack_int4(q)
    assert p.shape == (6, 32)
    assert np.array_equal(orc.unpack_int4(p, 64), q)
    # nibble order: even k in the low nibble
    assert (p[0, 0] & 0xF) == (q[0, 0] & 0xF) and (p[0, 0] >> 4) == (q[0, 1] & 0xF)
    w = synth.weights(123, (2, 8, 128))
    qq, s = orc.quantize_weights(w, 64, bits=4)
    codes = orc.unpack_int4(qq, 128)
    assert codes.min() >= -7 and codes.max() <= 7
    r = orc.rotate_rows_bf16(w.reshape(16, 128), 64).reshape(2, 8, 128)
    assert np.array_equal(s, (np.abs(r).max(axis=2) / np.float32(7)).astype(np.float32))


def test_weight_converter_is_rotate_then_quantize_per_row(orc):
    w = synth.weights(321, (3, 16, 512))
    q, s = orc.quantize_weights(w, 256, bits=8)
    r = orc.rotate_rows_bf16(w.reshape(48, 512), 256)
    q2, s2 = orc.quantize_rows(r, 127)
    assert np.array_equal(q.reshape(48, 512), q2) and np.array_equal(s.reshape(48), s2)
    # dequantised rotated weights approximate the rotated weights to half a step
    assert np.all(np.abs(q2 * s2[:, None].astype(np.float64) - r) <= s2[:, None] * (0.5 + 1e-5))


# ---------------------------------------------------------------------------------------------------------
# Integer product and dequantisation
# ---------------------------------------------------------------------------------------------------------

def test_gemm_brute_force_int64(orc):
    rng = np.random.default_rng(11)
    for (M, N, K) in [(1, 1, 1), (3, 5, 7), (17, 33, 64), (64, 48, 40)]:
        a = rng.integers(-127, 128, (M, K)).astype(np.int8)
        b = rng.integers(-127, 128, (N, K)).astype(np.int8)
        ref = np.zeros((M, N), np.int64)
        for m in range(M):
            for n in range(N):
                ref[m, n] = sum(int(a[m, k]) * int(b[n, k]) for k in range(K))
        assert np.array_equal(orc.gemm_i8_i32(a, b), ref)


def test_gemm_extremes_exact_via_fp64(orc):
    # all partial sums are integers below 2^53, so an fp64 product is exact; |acc| reaches K * 127^2
    rng = np.random.default_rng(12)
    a = rng.integers(-127, 128, (64, 2048)).astype(np.int8)
    b = rng.integers(-127, 128, (96, 2048)).astype(np.int8)
    a[0] = 127
    b[0] = 127
    b[1] = -127
    ref = a.astype(np.float64) @ b.astype(np.float64).T
    got = orc.gemm_i8_i32(a, b)
    assert np.array_equal(got.astype(np.float64), ref)
    assert got[0, 0] == 2048 * 127 * 127 and got[0, 1] == -2048 * 127 * 127


def test_dequant_exact_with_power_of_two_scales(orc):
    rng = np.random.default_rng(13)
    acc = rng.integers(-2**20, 2**20, (8, 12)).astype(np.int32)
    sa = np.float32(2.0) ** rng.integers(-12, -2, 8).astype(np.float32)
    sb = np.float32(2.0) ** rng.integers(-10, -1, 12).astype(np.float32)
    exact = acc.astype(np.float64) * sa[:, None] * sb[None, :]
    ref = torch.from_numpy(exact).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(orc.dequant_bf16(acc, sa, sb), ref)
    bias = synth.to_bf16_bits(np.float32(2.0) ** rng.integers(-6, 0, 12).astype(np.float32))
    exact_b = exact + synth.bf16_bits_to_f32(bias)[None, :]
    ref_b = torch.from_numpy(exact_b).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(orc.dequant_bf16(acc, sa, sb, bias), ref_b)


def _linear_rel_err(orc, x, w, g):
    qw, sw = orc.quantize_weights(w, g, 8)
    y, _, _ = orc.linear_w8a8(x, qw, sw, g)
    ref = synth.bf16_bits_to_f32(x).astype(np.float64) @ synth.bf16_bits_to_f32(w).astype(np.float64).T
    got = synth.bf16_bits_to_f32(y).astype(np.float64)
    return np.linalg.norm(got - ref) / np.linalg.norm(ref), got, ref


def test_linear_close_to_unquantized_product(orc):
    x, w = synth.linear_inputs(0)
    rel, got, ref = _linear_rel_err(orc, x, w, 64)
    assert rel < 0.02
    # a transposed or mis-scaled operand would not track the reference this closely
    assert np.corrcoef(got.ravel(), ref.ravel())[0, 1] > 0.999


def test_method_sanity_rotation_beats_plain_int8_on_outliers(orc):
    # ConvRot's purpose: with outlier channels, rotated W8A8 is closer to the unquantised product than
    # W8A8 without rotation (group 1 = identity rotation).
    x, w = synth.linear_inputs(0)
    rel_rot, _, _ = _linear_rel_err(orc, x, w, 64)
    rel_plain, _, _ = _linear_rel_err(orc, x, w, 1)
    assert rel_rot < 0.5 * rel_plain


# ---------------------------------------------------------------------------------------------------------
# Routing
# ---------------------------------------------------------------------------------------------------------

def test_softmax_against_fp64(orc):
    lg = synth.logits(2000, 512, 64)
    p = orc.softmax_experts(lg)
    l64 = lg.astype(np.float64)
    ref = np.exp(l64 - l64.max(axis=1, keepdims=True))
    ref /= ref.sum(axis=1, keepdims=True)
    assert np.max(np.abs(p - ref) / ref) < 2e-6
    assert np.allclose(p.sum(axis=1), 1.0, atol=1e-6)
    assert np.all(orc.softmax_experts(np.zeros((4, 1), np.float32)) == 1.0)


@pytest.mark.parametrize("T,E,C", [(1, 1, 1), (8, 3, 3), (40, 5, 7), (64, 8, 64), (33, 4, 1)])
def test_routing_brute_force_stable_sort(orc, T, E, C):
    rng = np.random.default_rng(T * 100 + E * 10 + C)
    p = rng.random((T, E)).astype(np.float32)
    p[rng.random((T, E)) < 0.3] = 0.5  # plenty of exact ties
    idx, wt = orc.route_from_probs(p, C)
    for e in range(E):
        order = sorted(range(T), key=lambda t: (-float(p[t, e]), t))
        assert idx[e].tolist() == sorted(order[:C])
        assert np.array_equal(wt[e], p[idx[e], e])


def test_routing_invariants_and_ties(orc):
    lg = synth.logits(3000, 256, 16)
    lg[10] = lg[3]   # duplicate rows give bit-identical probabilities: the lower index must win
    lg[200] = lg[3]
    idx, wt, p = orc.route(lg, 20)
    for e in range(16):
        sel = idx[e]
        assert len(set(sel.tolist())) == 20 and np.all(np.diff(sel) > 0)
        mask = np.zeros(256, bool)
        mask[sel] = True
        assert p[mask, e].min() >= p[~mask, e].max()
        if mask[10]:
            assert mask[3]
        if mask[200]:
            assert mask[3] and mask[10]
    assert idx.size == 16 * 20
    all_idx, _, _ = orc.route(lg, 256)
    assert np.array_equal(all_idx, np.tile(np.arange(256, dtype=np.int32), (16, 1)))


@pytest.mark.parametrize("T,E,C", [(96, 4, 10), (300, 8, 37)])
def test_routing_resolves_logit_gaps_beyond_86_nats(orc, T, E, C):
    # Expert choice ranks tokens by their probabilities: each expert's list must be the C highest of the
    # exact (float64) softmax probabilities rounded to fp32, ties to the lower token index; a saturating
    # exponential would make every such token tie.
    lg = synth.large_gap_logits(T, E, T + E)
    idx, wt, p = orc.route(lg, C)
    l64 = lg.astype(np.float64)
    p64 = np.exp(l64 - l64.max(axis=1, keepdims=True))
    p64 /= p64.sum(axis=1, keepdims=True)
    ref32 = p64.astype(np.float32)
    assert np.all(ref32[:, 1:] < np.finfo(np.float32).tiny * 2 ** 24) and np.all(ref32[:, 1:] > 0)
    for e in range(E):
        order = sorted(range(T), key=lambda t: (-float(ref32[t, e]), t))
        assert idx[e].tolist() == sorted(order[:C])
        # and the probabilities themselves follow the exact ones into the subnormal range
        assert np.all(np.abs(p[:, e].astype(np.float64) - p64[:, e]) <= 4e-7 * p64[:, e] + 2.0 ** -148)


# ---------------------------------------------------------------------------------------------------------
# Expert FFN, combine, layer
# ---------------------------------------------------------------------------------------------------------

def test_swiglu_against_fp64(orc):
    rng = np.random.default_rng(21)
    gu = synth.to_bf16_bits(rng.standard_normal((64, 2 * 96)).astype(np.float32) * 3)
    a = synth.bf16_bits_to_f32(orc.swiglu(gu)).astype(np.float64)
    g = synth.bf16_bits_to_f32(gu[:, :96]).astype(np.float64)
    u = synth.bf16_bits_to_f32(gu[:, 96:]).astype(np.float64)
    ref = g / (1.0 + np.exp(-g)) * u      # first half is the gate, second half the up projection
    assert np.all(np.abs(a - ref) <= np.abs(ref) * 2.0 ** -8 * 1.01 + 1e-30)


def test_combine_dense_when_every_expert_takes_every_token(orc):
    rng = np.random.default_rng(22)
    T, E, d = 24, 5, 32
    lg = rng.standard_normal((T, E)).astype(np.float32)
    idx, wt, p = orc.route(lg, T)
    z = synth.to_bf16_bits(rng.standard_normal((E * T, d)).astype(np.float32))
    out = synth.bf16_bits_to_f32(orc.combine(z, idx, wt, T)).astype(np.float64)
    zf = synth.bf16_bits_to_f32(z).reshape(E, T, d).astype(np.float64)
    ref = np.einsum("te,etd->td", p.astype(np.float64), zf)
    bound = np.einsum("te,etd->td", p.astype(np.float64), np.abs(zf))
    assert np.all(np.abs(out - ref) <= np.abs(ref) * 2.0 ** -8 + bound * 2.0 ** -20)


def test_combine_untaken_tokens_are_zero(orc):
    idx = np.array([[1, 4]], np.int32)
    wt = np.array([[0.5, 0.25]], np.float32)
    z = synth.to_bf16_bits(np.ones((2, 8), np.float32))
    out = orc.combine(z, idx, wt, 6)
    f = synth.bf16_bits_to_f32(out)
    assert np.all(f[[0, 2, 3, 5]] == 0) and np.all(out[[0, 2, 3, 5]] == 0)
    assert np.all(f[1] == 0.5) and np.all(f[4] == 0.25)


def _small_moe(T=96, d=512, E=4, I=128, C=24, seed=31, bits=8):
    s = synth.MoEShape(T=T, d=d, E=E, I=I, C=C, g_gu=256, g_dn=64)
    return s, synth.moe_inputs(2, s, seed_base=seed * 1000)


def test_moe_single_expert_all_tokens_equals_dense_ffn(orc):
    # E = 1, C = T: softmax of one logit is exactly 1, every token is taken once, so the layer must equal the
    # plain FFN: W8A8 linear gate/up -> SwiGLU -> W8A8 linear down, bit for bit.
    s, (x, _, w_gu, w_dn) = _small_moe(E=1, C=96)
    lg = np.random.default_rng(0).standard_normal((s.T, 1)).astype(np.float32)
    q_gu, s_gu = orc.quantize_weights(w_gu, 256)
    q_dn, s_dn = orc.quantize_weights(w_dn, 64)
    r = orc.moe_forward(x, lg, s.T, q_gu, s_gu, 256, q_dn, s_dn, 64)
    gu, _, _ = orc.linear_w8a8(x, q_gu[0], s_gu[0], 256)
    a = orc.swiglu(gu)
    y, _, _ = orc.linear_w8a8(a, q_dn[0], s_dn[0], 64)
    assert np.array_equal(r["out"], y)
    assert np.array_equal(r["wt"], np.ones((1, s.T), np.float32))


@pytest.mark.parametrize("bits", [8, 4])
def test_moe_close_to_unquantized_expert_choice_layer(orc, bits):
    s, (x, lg, w_gu, w_dn) = _small_moe()
    q_gu, s_gu = orc.quantize_weights(w_gu, 256, bits)
    q_dn, s_dn = orc.quantize_weights(w_dn, 64, bits)
    r = orc.moe_forward(x, lg, s.C, q_gu, s_gu, 256, q_dn, s_dn, 64, bits, intermediates=True)
    # fp64 expert-choice layer from the unquantised weights, same routing
    xf = synth.bf16_bits_to_f32(x).astype(np.float64)
    wg = synth.bf16_bits_to_f32(w_gu).astype(np.float64)
    wd = synth.bf16_bits_to_f32(w_dn).astype(np.float64)
    ref = np.zeros((s.T, s.d))
    for e in range(s.E):
        t = r["idx"][e]
        h = xf[t] @ wg[e].T
        g, u = h[:, :s.I], h[:, s.I:]
        a = g / (1 + np.exp(-g)) * u
        ref[t] += r["wt"][e][:, None].astype(np.float64) * (a @ wd[e].T)
    got = synth.bf16_bits_to_f32(r["out"]).astype(np.float64)
    rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    assert rel < (0.05 if bits == 8 else 0.5)
    assert np.corrcoef(got.ravel(), ref.ravel())[0, 1] > (0.998 if bits == 8 else 0.8)
    # staged intermediates are consistent with the routing
    assert np.array_equal(r["sx"], orc.rotq_rows(x, 256)[1])
    assert r["z"].shape == (s.E * s.C, s.d)


def test_moe_rows_equals_full_layer_at_every_token(orc):
    s, (x, lg, w_gu, w_dn) = _small_moe(C=30)
    q_gu, s_gu = orc.quantize_weights(w_gu, 256)
    q_dn, s_dn = orc.quantize_weights(w_dn, 64)
    r = orc.moe_forward(x, lg, s.C, q_gu, s_gu, 256, q_dn, s_dn, 64, intermediates=True)
    rows = orc.moe_rows(r["qx"], r["sx"], r["idx"], r["wt"], q_gu, s_gu, q_dn, s_dn, 64, np.arange(s.T))
    assert np.array_equal(rows, r["out"])


# ----------------------------------------------------------------------------------------------------------
# LoRA re-quantisation with random rounding (NitroFusion2 page, "Why a step-1 file"; XB loader, lora_mode)
# ----------------------------------------------------------------------------------------------------------

def _np_philox(ctr, key):
    """numpy's own Philox4x64-10 bit generator, which advances its counter by one before each block."""
    c = [int(v) for v in ctr]
    c[0] = (c[0] - 1) % (1 << 64)  # every test counter has word 0 >= 1: no borrow
    bg = np.random.Philox(key=np.array(key, dtype=np.uint64), counter=np.array(c, dtype=np.uint64))
    return bg.random_raw(4)


@pytest.mark.parametrize("seed", [0, 1, 12345])
def test_philox_matches_numpy_bit_generator(orc, seed):
    rng = np.random.default_rng(seed)
    for _ in range(20):
        ctr = [int(rng.integers(1, 1 << 63)), int(rng.integers(0, 1 << 63)), int(rng.integers(0, 1 << 63)),
               int(rng.integers(0, 1 << 63))]
        key = [int(rng.integers(0, 1 << 63)), int(rng.integers(0, 1 << 63))]
        assert np.array_equal(orc.philox4x64_10(ctr, key), _np_philox(ctr, key))


def _quantised_rows(rng, E, N, K, pow2_scales=False):
    q = rng.integers(-127, 128, (E, N, K)).astype(np.int8)
    q[..., 1] = 127  # every row reaches qmax
    if pow2_scales:
        s = np.ldexp(np.float32(1.0), rng.integers(-12, -4, (E, N))).astype(np.float32)
    else:
        s = (rng.random((E, N)) * 1e-3 + 1e-4).astype(np.float32)
    return q, s


def test_lora_requant_without_delta_keeps_codes(orc):
    """No delta and power-of-two scales: every value is exactly code * scale, the fresh scale is the old one and
    every quotient an integer, so the random rounding returns the codes unchanged."""
    rng = np.random.default_rng(3)
    q, s = _quantised_rows(rng, 2, 8, 512, pow2_scales=True)
    lb = synth.to_bf16_bits(rng.standard_normal((2, 8, 4)).astype(np.float32))
    la = synth.to_bf16_bits(rng.standard_normal((2, 4, 512)).astype(np.float32))
    for rank_b, rank_a, alpha in [(lb[..., :0], la[:, :0], 1.0), (lb, la, 0.0)]:
        q2, s2 = orc.requantize_lora(q, s, 64, rank_b, rank_a, alpha, seed=7)
        assert np.array_equal(q2, q) and np.array_equal(s2, s)


def test_lora_requant_follows_the_rotated_patch(orc):
    """Codes are floor or ceil of V / scale with V = R + rotate(alpha B A) computed in fp64 here, and the
    scale is max|V| / 127 (a dropped term, a wrong sign or a transposed factor moves V far beyond this)."""
    rng = np.random.default_rng(4)
    E, N, K, r, g = 2, 6, 512, 8, 64
    q, s = _quantised_rows(rng, E, N, K)
    lb = synth.to_bf16_bits((rng.standard_normal((E, N, r)) * 0.05).astype(np.float32))
    la = synth.to_bf16_bits((rng.standard_normal((E, r, K)) * 0.05).astype(np.float32))
    alpha = 0.5
    q2, s2 = orc.requantize_lora(q, s, g, lb, la, alpha, seed=11)
    bf = synth.bf16_bits_to_f32
    delta = alpha * np.einsum("enr,erk->enk", bf(lb).astype(np.float64), bf(la).astype(np.float64))
    h = scipy.linalg.hadamard(g).astype(np.float64) / math.sqrt(g)
    drot = (delta.reshape(E, N, K // g, g) @ h.T).reshape(E, N, K)
    v = q.astype(np.float64) * s[..., None].astype(np.float64) + drot
    sc = np.abs(v).max(axis=-1) / 127
    np.testing.assert_allclose(s2, sc, rtol=1e-5)
    t = v / s2[..., None].astype(np.float64)
    c = q2.astype(np.float64)
    assert np.all(c >= np.floor(t) - 1e-3 - 1) and np.all(c <= np.ceil(t) + 1e-3)
    assert np.all((c == np.floor(t + 1e-4)) | (c == np.ceil(t - 1e-4)) | (np.abs(t) > 126.9))
    assert np.abs(q2.astype(int) - q.astype(int)).max() > 0  # the patch changed something


def test_lora_requant_rounding_is_unbiased_and_seeded(orc):
    """A rank-1 delta constant over a rotation block rotates into one element per block: c * sqrt(g).  With
    scale 1 that element's quotient is code + 0.3, so it rounds up in about 30 % of the rows; the rest
    stay exact.  The same seed gives the same codes, another seed other codes."""
    rng = np.random.default_rng(5)
    E, N, K, g = 1, 4096, 256, 256
    q = rng.integers(-100, 100, (E, N, K)).astype(np.int8)
    q[..., 1] = 127
    s = np.ones((E, N), np.float32)
    c = np.float32(0.3 / 16)  # rotate(c * ones) = 16 c at k = 0 (g = 256), bf16-exact? no: use its bf16 value
    cb = synth.to_bf16_bits(np.array([c], np.float32))
    cf = float(synth.bf16_bits_to_f32(cb)[0])
    lb = synth.to_bf16_bits(np.ones((E, N, 1), np.float32))
    la = np.tile(cb, (E, 1, K)).reshape(E, 1, K)
    q2, s2 = orc.requantize_lora(q, s, g, lb, la, 1.0, seed=21)
    assert np.array_equal(s2, s)
    frac = 16 * cf
    up = q2[..., 0].astype(int) - q[..., 0].astype(int)
    assert set(np.unique(up)) <= {0, 1}
    assert abs(up.mean() - frac) < 0.03, (up.mean(), frac)
    assert np.array_equal(q2[..., 1:], q[..., 1:])
    q3, _ = orc.requantize_lora(q, s, g, lb, la, 1.0, seed=21)
    q4, _ = orc.requantize_lora(q, s, g, lb, la, 1.0, seed=22)
    assert np.array_equal(q3, q2) and not np.array_equal(q4, q2)


def test_lora_requant_nearest_mode(orc):
    """The re-quantising mode rounds to nearest: without a delta it keeps the codes; with one, every code is the
    nearest integer to V / scale for an fp64 reference of the rotated patch (away from half-integers), whatever
    the seed; and a quotient of code + 0.3 (+ 0.7) always rounds down (up) where random rounding moves ~30 %."""
    rng = np.random.default_rng(6)
    q, s = _quantised_rows(rng, 2, 8, 512, pow2_scales=True)
    lb0 = synth.to_bf16_bits(rng.standard_normal((2, 8, 0)).astype(np.float32))
    la0 = synth.to_bf16_bits(rng.standard_normal((2, 0, 512)).astype(np.float32))
    q2, s2 = orc.requantize_lora(q, s, 64, lb0, la0, 1.0, seed=7, nearest=True)
    assert np.array_equal(q2, q) and np.array_equal(s2, s)

    E, N, K, r, g = 2, 6, 512, 8, 64
    q, s = _quantised_rows(rng, E, N, K)
    lb = synth.to_bf16_bits((rng.standard_normal((E, N, r)) * 0.05).astype(np.float32))
    la = synth.to_bf16_bits((rng.standard_normal((E, r, K)) * 0.05).astype(np.float32))
    qn, sn = orc.requantize_lora(q, s, g, lb, la, 0.5, seed=11, nearest=True)
    qn2, sn2 = orc.requantize_lora(q, s, g, lb, la, 0.5, seed=12, nearest=True)
    assert np.array_equal(qn, qn2) and np.array_equal(sn, sn2)
    _, sr = orc.requantize_lora(q, s, g, lb, la, 0.5, seed=11)
    assert np.array_equal(sn, sr)  # same patched values, same fresh scale
    bf = synth.bf16_bits_to_f32
    delta = 0.5 * np.einsum("enr,erk->enk", bf(lb).astype(np.float64), bf(la).astype(np.float64))
    h = scipy.linalg.hadamard(g).astype(np.float64) / math.sqrt(g)
    v = q.astype(np.float64) * s[..., None] + (delta.reshape(E, N, K // g, g) @ h.T).reshape(E, N, K)
    t = v / sn[..., None].astype(np.float64)
    away = np.abs(np.abs(t - np.floor(t)) - 0.5) > 1e-3
    assert np.array_equal(qn[away], np.clip(np.round(t[away]), -127, 127).astype(np.int8))
    assert np.abs(qn.astype(np.float64) - t).max() <= 0.5 + 1e-3

    E, N, K, g = 1, 512, 256, 256
    q = rng.integers(-100, 100, (E, N, K)).astype(np.int8)
    q[..., 1] = 127
    s = np.ones((E, N), np.float32)
    ones = synth.to_bf16_bits(np.ones((E, N, 1), np.float32))
    for frac, want in ((0.3, 0), (0.7, 1)):
        cb = synth.to_bf16_bits(np.array([frac / 16], np.float32))
        la = np.tile(cb, (E, 1, K)).reshape(E, 1, K)
        qn, _ = orc.requantize_lora(q, s, g, ones, la, 1.0, seed=21, nearest=True)
        assert np.all(qn[..., 0].astype(int) - q[..., 0].astype(int) == want)
        assert np.array_equal(qn[..., 1:], q[..., 1:])


# ----------------------------------------------------------------------------------------------------------
# W6A8 / W4A8: FP8 (E4M3) scale per group of 16 (NitroFusion2 page, "How they were made")
# ----------------------------------------------------------------------------------------------------------

def test_e4m3_decode_fixed_points():
    import oracle
    got = oracle.e4m3_decode(np.array([0x00, 0x01, 0x07, 0x08, 0x38, 0x39, 0x7e, 0x80, 0xb8], np.uint8))
    want = np.array([0.0, 2.0 ** -9, 7 * 2.0 ** -9, 2.0 ** -6, 1.0, 1.125, 448.0, -0.0, -1.0], np.float32)
    assert np.array_equal(got, want) and np.signbit(got[7])
    assert np.isnan(oracle.e4m3_decode(np.array([0x7f, 0xff], np.uint8))).all()


def test_e4m3_encode_matches_torch_cast():
    """Nearest-even rounding onto the E4M3 grid, against torch's float8_e4m3fn conversion (values up to 448,
    where the two agree by definition; above it the oracle saturates)."""
    import oracle
    import torch
    grid = oracle.e4m3_decode(np.arange(0x7f, dtype=np.uint8))  # every non-negative finite value
    mids = (grid[:-1] + grid[1:]) / 2  # exact ties
    rng = np.random.default_rng(7)
    rnd = np.concatenate([rng.uniform(0, 448, 20000), np.exp2(rng.uniform(-12, 8.8, 20000))]).astype(np.float32)
    x = np.concatenate([grid, mids.astype(np.float32), np.nextafter(mids, 0).astype(np.float32),
                        np.nextafter(mids, 1000).astype(np.float32), rnd[rnd <= 448]])
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(oracle.e4m3_encode(x), ref)
    assert np.array_equal(oracle.e4m3_encode(grid), np.arange(0x7f, dtype=np.uint8))
    assert oracle.e4m3_encode(np.array([500.0, 1e9], np.float32)).tolist() == [0x7e, 0x7e]


def test_int6_packing_layout():
    import oracle
    q = np.array([[1, -1, 31, -32, 0, 5, -7, 30]], np.int8)
    p = oracle.pack_int6(q)
    w0 = 1 | (63 << 6) | (31 << 12) | (32 << 18)
    w1 = 0 | (5 << 6) | ((64 - 7) << 12) | (30 << 18)
    assert p.tolist() == [[w0 & 255, (w0 >> 8) & 255, w0 >> 16, w1 & 255, (w1 >> 8) & 255, w1 >> 16]]
    rng = np.random.default_rng(3)
    r = rng.integers(-32, 32, (5, 64)).astype(np.int8)
    assert np.array_equal(oracle.unpack_int6(oracle.pack_int6(r), 64), r)


@pytest.mark.parametrize("bits", [6, 4])
def test_quantize_g16_properties(bits):
    """Codes within +-qmax and, where not clamped, within half a group step of the rotated value (a group
    scale rounded down onto the E4M3 grid can push its largest values past qmax: those clamp, off by at most
    the scale's rounding, 2^-4 relative); the largest group's FP8 scale is 448; an all-zero row quantises to
    zero; finer codes approximate better."""
    import oracle
    qmax = 31 if bits == 6 else 7
    rng = np.random.default_rng(11)
    w = (rng.standard_normal((6, 512)) * 0.02).astype(np.float32)
    w[2] = 0.0
    w[4, :16] *= 1e-4  # one group far below the row's largest
    wb = oracle.bf16_round(w)
    q, f8, s, codes = oracle.quantize_g16(wb, 256, bits)
    assert np.array_equal(oracle.unpack_g16(q, 512, bits), codes)
    r = oracle.rotate_rows_bf16(wb, 256).astype(np.float64)
    S = s[:, None].astype(np.float64) * np.repeat(oracle.e4m3_decode(f8), 16, axis=1)
    assert np.abs(codes).max() <= qmax
    nz = S > 0
    inner = nz & (np.abs(codes) < qmax)
    clamped = nz & (np.abs(codes) == qmax)
    assert (np.abs(r - codes * S)[inner] <= S[inner] / 2 * (1 + 1e-6)).all()
    assert (np.abs(r)[clamped] >= (qmax - 0.5) * S[clamped] * (1 - 1e-6)).all()
    assert (np.abs(r - codes * S)[clamped] <= 2.0 ** -4 * np.abs(r)[clamped] + S[clamped] / 2).all()
    assert (codes[~nz] == 0).all()
    assert not codes[2].any() and s[2] == 0 and not f8[2].any()
    for i in (0, 1, 3, 4, 5):
        assert f8[i].max() == 0x7e and np.isclose(s[i], np.abs(r[i]).max() / (qmax * 448), rtol=1e-6)
    err = np.linalg.norm(r - codes * S) / np.linalg.norm(r)
    assert err < (0.03 if bits == 6 else 0.15)


@pytest.mark.parametrize("bits", [6, 4])
def test_linear_g16_exact_sum_and_rotation_invariance(bits):
    """The oracle's A is the exact dot product of the token codes with the decoded weights (checked by a
    float64 matmul, exact here), and y approximates x W^T (rotation invariance) within quantisation error."""
    import oracle
    rng = np.random.default_rng(5)
    M, K, N = 7, 512, 9
    x = oracle.bf16_round(rng.standard_normal((M, K)).astype(np.float32))
    w = oracle.bf16_round((rng.standard_normal((N, K)) * 0.02).astype(np.float32))
    q, f8, s, codes = oracle.quantize_g16(w, 256, bits)
    y, qx, sx, acc, aabs = oracle.linear_g16(x, 256, codes, f8, s)
    wdec = codes.astype(np.float64) * np.repeat(oracle.e4m3_decode(f8), 16, axis=1)
    assert np.array_equal(acc, qx.astype(np.float64) @ wdec.T)
    assert np.array_equal(aabs, np.abs(qx.astype(np.float64)) @ np.abs(wdec).T)
    ref = oracle.bf16_to_f32(x).astype(np.float64) @ oracle.bf16_to_f32(w).astype(np.float64).T
    got = oracle.bf16_to_f32(y).astype(np.float64)
    rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    assert rel < (0.05 if bits == 6 else 0.2)
