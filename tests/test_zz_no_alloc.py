"""The allocation-free forward (moe_expert_choice_forward_noalloc) against the forward with a caller workspace,
through the C ABI: two calls in a row, the second on a smaller layer, then the first shape again.  Both entry
points run the same kernels, so routing and outputs must agree bit for bit."""
import numpy as np
import pytest
import torch

from w8a8_rotated_int8_amd import binding as cr
from w8a8_rotated_int8_amd import synth

from helpers import DEV, dev, dev_bf16, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _setup():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    cr.lib()


def _full_layer():
    s = synth.CONFIGS[3]
    lgd, w_gu_d, w_dn_d = synth.stack_layer_device(0, s, DEV)
    w = cr.quantize_moe_weights(w_gu_d, w_dn_d, s.g_gu, s.g_dn, 8)
    return s, dev_bf16(synth.stack_x(s)), lgd, w


def _small_layer():
    s = synth.MoEShape(T=300, d=512, E=8, I=128, C=50, g_gu=64, g_dn=64)
    x, lg, w_gu, w_dn = synth.moe_inputs(2, s, seed_base=41000)
    w = cr.quantize_moe_weights(dev_bf16(w_gu), dev_bf16(w_dn), s.g_gu, s.g_dn, 8)
    return s, dev_bf16(x), dev(lg), w


def _compare(s, x, lg, w, what):
    say(f"noalloc {what}: T={s.T} d={s.d} E={s.E} I={s.I} C={s.C}")
    need = cr.moe_expert_choice_workspace_bytes(s.T, s.C, w)
    assert need <= cr.NOALLOC_SCRATCH_BYTES
    ref, ridx, rwt = cr.moe_expert_choice_forward(x, lg, s.C, w)
    out = torch.full((s.T, s.d), 7.0, dtype=torch.bfloat16, device=DEV)
    idx = torch.full((s.E, s.C), -5, dtype=torch.int32, device=DEV)
    wt = torch.full((s.E, s.C), -1.0, dtype=torch.float32, device=DEV)
    cr.moe_expert_choice_forward_noalloc(x, lg, s.C, w, out, idx, wt)
    torch.cuda.synchronize()
    assert torch.equal(idx, ridx), f"{what}: routing indices"
    assert torch.equal(wt.view(torch.int32), rwt.view(torch.int32)), f"{what}: routing weights"
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), f"{what}: layer output"
    # routing outputs NULL: the scratch keeps them
    out2 = torch.empty_like(out)
    cr.moe_expert_choice_forward_noalloc(x, lg, s.C, w, out2)
    torch.cuda.synchronize()
    assert torch.equal(out2.view(torch.int16), ref.view(torch.int16)), f"{what}: layer output, routing NULL"


def test_noalloc_matches_forward_large_then_small():
    big = _full_layer()
    _compare(*big, "T=8192 layer")
    _compare(*_small_layer(), "smaller layer after it")
    _compare(*big, "T=8192 layer again")


def test_noalloc_rejects_beyond_scratch():
    s = synth.MoEShape(T=8192, d=2048, E=64, I=1536, C=512)
    w = cr.MoeWeights(torch.zeros(16, dtype=torch.int8, device=DEV), torch.zeros(16, device=DEV),
                      torch.zeros(16, dtype=torch.int8, device=DEV), torch.zeros(16, device=DEV), s.E, s.d, s.I)
    assert cr.moe_expert_choice_workspace_bytes(s.T, s.C, w) > cr.NOALLOC_SCRATCH_BYTES
    x = torch.zeros((s.T, s.d), dtype=torch.bfloat16, device=DEV)
    lg = torch.zeros((s.T, s.E), device=DEV)
    out = torch.zeros_like(x)
    with pytest.raises(cr.ConvrotError) as ei:
        cr.moe_expert_choice_forward_noalloc(x, lg, s.C, w, out)
    assert ei.value.status == 6
