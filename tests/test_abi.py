"""The C ABI on the host, no GPU needed: the library loads, exports every function include/convrot.h and
include/convrot_probes.h declare, and rejects invalid arguments (validation runs before anything touches the
GPU)."""
import ctypes

import pytest

from w8a8_rotated_int8_amd import binding as cr

OK, NULL, SHAPE, GROUP, BITS, ALIGN, WS = 0, 1, 2, 3, 4, 5, 6
P = 0x10000  # a 16-byte aligned stand-in pointer: never dereferenced, validation rejects first


@pytest.fixture(scope="module")
def L():
    return cr.lib()


def test_exports_every_declared_function(L):
    names = cr.header_functions()
    assert len(names) == 28
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(cr._SIGS)


def test_g16_validation(L):
    assert L.convrot_weight_g16_bytes(3, 512, 6) == 3 * 384 and L.convrot_weight_g16_bytes(3, 512, 4) == 3 * 256
    assert L.convrot_weight_g16_bytes(3, 512, 5) == 0
    f = L.convrot_quantize_weights_g16
    assert f(None, 4, 512, 256, 6, P, P, P, None) == NULL
    assert f(P, 4, 512, 256, 5, P, P, P, None) == BITS
    assert f(P, 4, 500, 256, 6, P, P, P, None) == GROUP
    assert f(P, 4, 128, 256, 6, P, P, P, None) == GROUP
    assert f(P, 0, 512, 256, 6, P, P, P, None) == SHAPE
    assert f(P, 4, 16384, 256, 6, P, P, P, None) == SHAPE
    assert f(P + 2, 4, 512, 256, 6, P, P, P, None) == ALIGN
    g = L.convrot_gemm_g16_bf16
    assert g(P, P, 8, 512, P, P, P, 16, 8, None, P, None) == BITS
    assert g(P, P, 8, 48, P, P, P, 16, 4, None, P, None) == SHAPE
    assert g(P, P, 8, 96, P, P, P, 16, 4, None, P, None) == SHAPE  # K a multiple of 64
    assert g(P, P, 0, 512, P, P, P, 16, 4, None, P, None) == SHAPE
    assert g(P, P, 8, 512, P, P, P, 16, 4, P + 4, P, None) == ALIGN
    lin = L.convrot_linear_g16
    need = L.convrot_linear_workspace_bytes(8, 512)
    assert lin(P, 8, 512, P, P, P, 16, 256, 6, None, P, P, need - 1, None) == WS
    assert lin(P, 8, 500, P, P, P, 16, 256, 6, None, P, P, need, None) == GROUP
    assert lin(P, 8, 512, None, P, P, 16, 256, 6, None, P, P, need, None) == NULL


def test_probe_validation(L):
    d = ctypes.c_double(0.0)
    assert L.convrot_probe_mfma_i8(None, 1 << 18, 1, P, 1 << 20, ctypes.byref(d), None) == NULL
    assert L.convrot_probe_mfma_i8(P, 1 << 18, 1, P, 1 << 20, None, None) == NULL
    assert L.convrot_probe_hbm_read(P, 1 << 30, None, 1 << 20, ctypes.byref(d), None) == NULL


def test_status_strings(L):
    for code, name in cr.STATUS.items():
        assert cr.convrot_status_str(code).startswith(name)


def _weights(**kw):
    base = dict(E=64, d=2048, I=1536, group_gu=256, group_dn=64, wbits=8, q_gu=P, s_gu=P, q_dn=P, s_dn=P)
    base.update(kw)
    return cr.ConvrotMoeWeightsC(*[base[f] for f, _ in cr.ConvrotMoeWeightsC._fields_])


def test_quantize_weights_validation(L):
    f = L.convrot_quantize_weights
    assert f(None, 1, 1, 64, 64, 8, 1, P, P, None) == NULL
    assert f(P, 1, 1, 64, 64, 5, 1, P, P, None) == BITS
    assert f(P, 1, 1, 100, 64, 8, 1, P, P, None) == GROUP
    assert f(P, 1, 1, 256, 128, 8, 0, P, P, None) == GROUP
    assert f(P, 0, 1, 64, 64, 8, 1, P, P, None) == SHAPE
    assert f(P, 1, 1, 16384, 256, 8, 1, P, P, None) == SHAPE
    assert f(P, 1, 1, 256, 256, 8, 2, P, P, None) == SHAPE
    assert f(P + 2, 1, 1, 64, 64, 8, 1, P, P, None) == ALIGN
    # MFMA layout pads rows to blocks of 32; int4 halves the bytes
    assert L.convrot_weight_bytes(64, 3072, 2048, 8, 1) == 64 * 3072 * 2048
    assert L.convrot_weight_bytes(2, 33, 512, 8, 1) == 2 * 64 * 512
    assert L.convrot_weight_bytes(2, 33, 512, 4, 1) == 2 * 64 * 256
    assert L.convrot_weight_bytes(2, 33, 512, 8, 0) == 2 * 33 * 512


def test_linear_validation(L):
    f = L.convrot_linear_w8a8
    need = L.convrot_linear_workspace_bytes(64, 512)
    assert need >= 64 * 512 + 64 * 4
    assert f(P, 64, 512, P, P, 256, 64, None, P, P, need - 1, None) == WS
    assert f(P, 64, 512, P, P, 256, 64, None, P, None, need, None) == WS
    assert f(P, 64, 500, P, P, 256, 64, None, P, P, need, None) == GROUP
    assert f(P, 0, 512, P, P, 256, 64, None, P, P, need, None) == SHAPE
    assert f(P, 64, 512, None, P, 256, 64, None, P, P, need, None) == NULL
    assert f(P, 64, 512, P, P, 256, 64, P + 8, P, P, need, None) == ALIGN


def test_moe_forward_validation(L):
    f = L.moe_expert_choice_forward
    w = _weights()
    need = L.moe_expert_choice_workspace_bytes(8192, 256, ctypes.byref(w))
    # probs^T + slot table (E*T*4 each), qx + sx, idx + wt, a (bf16) + qa + sa, z (bf16)
    S = 64 * 256
    assert need >= 2 * 64 * 8192 * 4 + 8192 * 2048 + 8192 * 4 + 2 * S * 4 + S * 1536 * 3 + S * 4 + S * 2048 * 2
    args = lambda T=8192, C=256, ww=w, ws=P, nb=need: (P, T, P, C, ctypes.byref(ww), P, None, None, ws, nb, None)
    assert f(*args(C=8193)) == SHAPE
    assert f(*args(C=0)) == SHAPE
    assert f(*args(nb=need - 1)) == WS
    assert f(*args(ww=_weights(group_gu=128))) == GROUP
    assert f(*args(ww=_weights(d=2000))) == GROUP
    assert f(*args(ww=_weights(wbits=3))) == BITS
    assert f(*args(ww=_weights(q_dn=None))) == NULL
    assert f(*args(ww=_weights(s_gu=P + 4))) == ALIGN
    assert f(*args(ww=_weights(I=1568))) == GROUP  # 1568 is not a multiple of the down group 64
    assert f(None, 8192, P, 256, ctypes.byref(w), P, None, None, P, need, None) == NULL


def test_moe_fused_query(L):
    """Which layers the one-launch forward (gate/up, the hidden rows' rotate+quantise, down) takes."""
    f = L.moe_expert_choice_fused
    for bits in (8, 4):
        assert f(ctypes.byref(_weights(wbits=bits)), 256) == 1  # T = 8192 layer: I = 1536, group 64
        assert f(ctypes.byref(_weights(wbits=bits)), 1024) == 1  # several M-blocks per expert
    assert f(ctypes.byref(_weights(I=512)), 37) == 1
    assert f(ctypes.byref(_weights(I=2048, group_dn=256)), 8) == 1
    assert f(ctypes.byref(_weights(I=1024, group_dn=256)), 8) == 0  # group 256 only with I = 2048
    assert f(ctypes.byref(_weights(I=128)), 24) == 0   # rows too short: three launches
    assert f(ctypes.byref(_weights(I=2560)), 24) == 0  # five 512-element rounds: three launches
    assert f(ctypes.byref(_weights(wbits=3)), 24) == 0
    assert f(ctypes.byref(_weights()), 0) == 0
    assert f(None, 256) == 0
    g = L.moe_expert_choice_forward_fused
    w = _weights()
    need = L.moe_expert_choice_workspace_bytes(8192, 256, ctypes.byref(w))
    args = lambda C=256, ww=w, nb=need: (P, 8192, P, C, ctypes.byref(ww), P, None, None, P, nb, None)
    assert g(*args(ww=_weights(I=128))) == SHAPE
    assert g(*args(nb=need - 1)) == WS
    assert g(*args(C=0)) == SHAPE
    assert g(None, 8192, P, 256, ctypes.byref(w), P, None, None, P, need, None) == NULL


def test_stage_validation(L):
    assert L.convrot_rotq_rows(P, 4, 300, 64, P, P, None, None) == GROUP
    assert L.convrot_rotq_rows(P, -1, 512, 64, P, P, None, None) == SHAPE
    assert L.convrot_quantize_prerotated(P, 4, 12, 8, P, P, None) == SHAPE
    assert L.convrot_quantize_prerotated(P, 4, 16, 6, P, P, None) == BITS
    assert L.convrot_gemm_i8_i32(P, P, 4, 4, 24, P, None) == SHAPE
    assert L.convrot_gemm_i8_i32(P, P, 4, 4, 140000, P, None) == SHAPE
    assert L.convrot_gemm_i8_i32(P, P, 4, 4, 131072, P, None) == SHAPE  # K * 128^2 reaches 2^31
    assert L.convrot_gemm_i8_i32(P, None, 4, 4, 32, P, None) == NULL
    assert L.convrot_gemm_w8a8_bf16(P, P, 4, 96, P, P, 8, None, P, None) == SHAPE  # K % 64
    assert L.convrot_gemm_w8a8_bf16(P, P, 0, 128, P, P, 8, None, P, None) == SHAPE
    assert L.convrot_gemm_w8a8_bf16(P, None, 4, 128, P, P, 8, None, P, None) == NULL
    assert L.convrot_requantize_lora(P, P, 1, 8, 512, 64, None, None, 4, 1.0, 1, 0, 1, P, P, None) == NULL
    assert L.convrot_requantize_lora(P, P, 1, 8, 512, 64, P, P, -1, 1.0, 1, 0, 1, P, P, None) == SHAPE
    assert L.convrot_requantize_lora(P, P, 1, 8, 500, 64, P, P, 4, 1.0, 1, 0, 1, P, P, None) == GROUP
    assert L.convrot_requantize_lora(P, P, 1, 8, 512, 64, P, P, 4, float("inf"), 1, 0, 1, P, P, None) == SHAPE
    assert L.convrot_requantize_lora(P, P, 1, 8, 512, 64, P, P, 4, 1.0, 1, 0, 2, P, P, None) == SHAPE  # layout
    assert L.convrot_requantize_lora(P, P, 1, 8, 512, 64, P, P, 4, 1.0, 1, 2, 1, P, P, None) == SHAPE  # rounding
    nb = L.moe_route_workspace_bytes(100, 8)
    assert nb >= 100 * 8 * 4
    assert L.moe_route_expert_choice(P, 0, 100, 8, 101, P, P, None, P, nb, None) == SHAPE
    assert L.moe_route_expert_choice(P, 0, 100, 8, 10, P, P, None, P, nb - 4, None) == WS
    w = _weights()
    assert L.moe_gateup_swiglu(P, P, 100, P, 200, ctypes.byref(w), P, None) == SHAPE
    assert L.moe_down_proj(P, P, 0, ctypes.byref(w), P, None) == SHAPE
    nb = L.moe_combine_workspace_bytes(100, 8)
    assert L.moe_combine(P, P, P, 100, 8, 10, 12, P, P, nb, None) == SHAPE
    assert L.moe_combine(P, P, P, 100, 8, 10, 64, P, P, nb - 1, None) == WS


def test_moe_forward_noalloc_validation(L):
    """The allocation-free forward validates like the forward and rejects workspaces beyond its static
    scratch before any HIP call."""
    f = L.moe_expert_choice_forward_noalloc
    w = _weights()
    need = L.moe_expert_choice_workspace_bytes(8192, 256, ctypes.byref(w))
    assert need <= cr.NOALLOC_SCRATCH_BYTES < L.moe_expert_choice_workspace_bytes(8192, 512, ctypes.byref(w))
    assert f(P, 8192, P, 512, ctypes.byref(w), P, None, None, None) == WS
    assert f(None, 8192, P, 256, ctypes.byref(w), P, None, None, None) == NULL
    assert f(P, 8192, P, 8193, ctypes.byref(w), P, None, None, None) == SHAPE
    assert f(P, 8192, P, 256, ctypes.byref(_weights(group_gu=128)), P, None, None, None) == GROUP
    assert f(P, 8192, P, 256, ctypes.byref(w), P + 4, None, None, None) == ALIGN
