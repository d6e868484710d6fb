"""GPU parity at the benchmark sizes, in the launch configuration the benchmark times.

Every configuration is checked in full against the oracle (the oracle finishes one T = 8192 layer in seconds on
the host cores): converted weight codes and scales, token codes and scales, routing indices and weights, the
gate/up + SwiGLU rows, the hidden-row codes, the down rows and the combined output.  Each stage is also run on
its own from the oracle's inputs, so a mismatch names the stage.  Bar: bit-exact for codes, scales and routing;
BF16 within 1e-2 relative (and, the arithmetic being fully specified, expected bit-identical).

  * T = 2048, C = 64, T = 4096, C = 128 and T = 8192, C = 256 layers (64 experts, d = 2048, I = 1536),
    host-generated inputs;
  * the 29-layer stack: layers 0 and 28 with 8-bit weights and layer 0 with 4-bit weights (weights drawn on the
    GPU by torch's generator, copied to the host for the oracle);
  * dense W8A8 ConvRot linears over the same T = 8192 tokens (fused qkv, an FFN-down-like [2048, 8192] and the
    attention output projection with group 64 and a bias), through the linear entry point and through its GEMM
    stage from the oracle's token codes;
  * a rank-16 LoRA patched onto the 64 quantised down projections [2048, 1536] (group 64) and re-quantised with
    random rounding, in the layout the GEMM streams.
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


def _check_layer(x, lg, w_gu_d, w_dn_d, w_gu, w_dn, shape, bits, what):
    """x, lg, w_gu, w_dn: host arrays (bf16 bits / fp32); w_gu_d, w_dn_d: the same weights on the GPU."""
    s = shape
    say(f"{what}: converting weights (bits={bits})")
    w = cr.quantize_moe_weights(w_gu_d, w_dn_d, s.g_gu, s.g_dn, bits)
    q_gu, s_gu = oracle.quantize_weights(w_gu, s.g_gu, bits)
    q_dn, s_dn = oracle.quantize_weights(w_dn, s.g_dn, bits)
    cg = q_gu if bits == 8 else oracle.unpack_int4(q_gu, s.d)
    cd = q_dn if bits == 8 else oracle.unpack_int4(q_dn, s.I)
    assert np.array_equal(untile_codes(host(w.q_gu), s.E, 2 * s.I, s.d, bits), cg), "gate/up weight codes"
    assert np.array_equal(untile_codes(host(w.q_dn), s.E, s.d, s.I, bits), cd), "down weight codes"
    assert np.array_equal(host(w.s_gu).view(np.uint32), s_gu.view(np.uint32)), "gate/up weight scales"
    assert np.array_equal(host(w.s_dn).view(np.uint32), s_dn.view(np.uint32)), "down weight scales"
    del cg, cd

    say(f"{what}: oracle layer")
    ref = oracle.moe_forward(x, lg, s.C, q_gu, s_gu, s.g_gu, q_dn, s_dn, s.g_dn, bits, intermediates=True)

    say(f"{what}: GPU layer")
    xd, lgd = dev_bf16(x), dev(lg)
    out, idx, wt = cr.moe_expert_choice_forward(xd, lgd, s.C, w)
    torch.cuda.synchronize()
    assert np.array_equal(host(idx), ref["idx"]), "routing indices"
    assert np.array_equal(host(wt).view(np.uint32), ref["wt"].view(np.uint32)), "routing weights"
    exact = assert_bf16_within(host_bf16(out), ref["out"], what=f"{what} out")
    say(f"{what}: layer output {exact * 100:.3f}% bit-identical")
    assert exact == 1.0
    if cr.moe_expert_choice_fused(w, s.C):
        say(f"{what}: GPU layer, one-launch expert path")
        out_f, _, _ = cr.moe_expert_choice_forward(xd, lgd, s.C, w, fused=True)
        assert torch.equal(out_f.view(torch.int16), out.view(torch.int16)), "one-launch layer output"
        del out_f

    say(f"{what}: stages from the oracle's inputs")
    qx, sx, _ = cr.convrot_rotq_rows(xd, s.g_gu)
    assert np.array_equal(host(qx), ref["qx"]) and np.array_equal(host(sx).view(np.uint32),
                                                                   ref["sx"].view(np.uint32)), "token codes"
    idx_d = dev(ref["idx"])
    a = cr.moe_gateup_swiglu(dev(ref["qx"]), dev(ref["sx"]), idx_d, w)
    assert np.array_equal(host_bf16(a), ref["a"]), "gate/up + SwiGLU rows"
    qa, sa, _ = cr.convrot_rotq_rows(dev_bf16(ref["a"]), s.g_dn)
    assert np.array_equal(host(qa), ref["qa"]) and np.array_equal(host(sa).view(np.uint32),
                                                                   ref["sa"].view(np.uint32)), "hidden codes"
    z = cr.moe_down_proj(dev(ref["qa"]), dev(ref["sa"]), s.C, w)
    assert np.array_equal(host_bf16(z), ref["z"]), "down rows"
    o2 = cr.moe_combine(dev_bf16(ref["z"]), idx_d, dev(ref["wt"]), s.T)
    assert np.array_equal(host_bf16(o2), ref["out"]), "combine"


@pytest.mark.parametrize("cfg,bits", [(2, 8), (3, 8), (3, 4)])
def test_full_size_layer(cfg, bits):
    s = synth.CONFIGS[cfg]
    what = f"config {cfg} T={s.T} C={s.C} bits={bits}"
    say(f"{what}: generating inputs")
    x, lg, w_gu, w_dn = synth.moe_inputs(cfg)
    _check_layer(x, lg, dev_bf16(w_gu), dev_bf16(w_dn), w_gu, w_dn, s, bits, what)


@pytest.mark.parametrize("bits", [8, 4])
def test_layer_T4096_C128(bits):
    """A 724x724-image-sized layer at capacity factor 2 (T = 4096, C = 128): the GEMMs' 128-row tile at full
    expert shapes."""
    s = synth.MoEShape(T=4096, d=2048, E=64, I=1536, C=128)
    what = f"T={s.T} C={s.C} bits={bits}"
    say(f"{what}: generating inputs")
    x, lg, w_gu, w_dn = synth.moe_inputs(2, s, seed_base=6000)
    _check_layer(x, lg, dev_bf16(w_gu), dev_bf16(w_dn), w_gu, w_dn, s, bits, what)


@pytest.mark.parametrize("layer,bits", [(0, 8), (28, 8), (0, 4)])
def test_layer_stack(layer, bits):
    s = synth.CONFIGS[4]
    what = f"stack layer {layer} bits={bits}"
    say(f"{what}: drawing weights on the GPU")
    lgd, w_gu_d, w_dn_d = synth.stack_layer_device(layer, s, DEV)
    x = synth.stack_x(s)
    lg = host(lgd)
    w_gu = host_bf16(w_gu_d)
    w_dn = host_bf16(w_dn_d)
    _check_layer(x, lg, w_gu_d, w_dn_d, w_gu, w_dn, s, bits, what)


@pytest.mark.parametrize("name", list(synth.DENSE_SHAPES))
def test_dense_linear_full_size(name):
    M, K, N, g = synth.DENSE_SHAPES[name]
    with_bias = name == "out"
    say(f"dense {name}: M={M} K={K} N={N} g={g} bias={with_bias}")
    x, w, b = synth.dense_linear_inputs(M, K, N, with_bias)
    qw, sw = cr.convrot_quantize_weights(dev_bf16(w), g, 8)
    rqw, rsw = oracle.quantize_weights(w, g, 8)
    assert np.array_equal(untile_codes(host(qw), 1, N, K, 8)[0], rqw), "weight codes"
    assert np.array_equal(host(sw).view(np.uint32), rsw.view(np.uint32)), "weight scales"
    bd = None if b is None else dev_bf16(b)
    y = cr.convrot_linear_w8a8(dev_bf16(x), qw, sw, g, bias=bd)
    say(f"dense {name}: oracle")
    ry, rqx, rsx = oracle.linear_w8a8(x, rqw, rsw, g, b)
    exact = assert_bf16_within(host_bf16(y), ry, what=f"dense {name}")
    say(f"dense {name}: {exact * 100:.3f}% bit-identical")
    assert exact == 1.0
    y2 = cr.convrot_gemm_w8a8_bf16(dev(rqx), dev(rsx), qw, sw, bias=bd)
    assert np.array_equal(host_bf16(y2), ry), "GEMM stage"


def test_lora_requant_full_size_down_weights():
    E, N, K, g, rank = 64, 2048, 1536, 64, 16
    say(f"lora requant full size E={E} N={N} K={K} rank={rank}")
    w = synth.weights(3000 + synth.ROLE_WDN, (E, N, K))
    q, s = oracle.quantize_weights(w, g, 8)
    rng = np.random.default_rng(31)
    lb = synth.to_bf16_bits((rng.standard_normal((E, N, rank)) * 0.02).astype(np.float32))
    la = synth.to_bf16_bits((rng.standard_normal((E, rank, K)) * 0.02).astype(np.float32))
    qt, st = cr.convrot_requantize_lora(dev(q), dev(s), g, dev_bf16(lb), dev_bf16(la), 0.5, 2024)
    torch.cuda.synchronize()
    say("lora requant: oracle")
    rq, rs = oracle.requantize_lora(q, s, g, lb, la, 0.5, 2024)
    assert np.array_equal(host(st).view(np.uint32), rs.view(np.uint32)), "scales"
    assert np.array_equal(untile_codes(host(qt), E, N, K, 8), rq), "codes"
    say("lora requant, nearest rounding")
    qn, sn = cr.convrot_requantize_lora(dev(q), dev(s), g, dev_bf16(lb), dev_bf16(la), 0.5, 0,
                                        rounding=cr.ROUND_NEAREST)
    torch.cuda.synchronize()
    rqn, rsn = oracle.requantize_lora(q, s, g, lb, la, 0.5, 0, nearest=True)
    assert np.array_equal(host(sn).view(np.uint32), rsn.view(np.uint32)), "nearest scales"
    assert np.array_equal(untile_codes(host(qn), E, N, K, 8), rqn), "nearest codes"
