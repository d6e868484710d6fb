"""Thin Python binding of libconvrot_amd (the C ABI declared in include/convrot.h).

Argument marshalling only: every function takes torch tensors that live on the GPU, passes their device
pointers and sizes to the C entry point of the same name on torch's current HIP stream, and raises
``ConvrotError`` on a non-OK status.  Outputs that are not supplied are allocated with torch (device memory is
torch's job here); all arithmetic happens in the HIP kernels.  There is no fallback: if the shared library is
missing or was built for another GPU the call fails.
"""
from __future__ import annotations

import ctypes
import os
import re
import threading
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# CONVROT_AMD_LIB names another build of the same sources (the host-sanitizer build of tests/sanitize.py)
LIB_PATH = os.environ.get("CONVROT_AMD_LIB") or os.path.join(_HERE, "libconvrot_amd.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "convrot.h")
PROBES_HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "convrot_probes.h")

STATUS = {0: "CONVROT_OK", 1: "CONVROT_ERR_NULL", 2: "CONVROT_ERR_SHAPE", 3: "CONVROT_ERR_GROUP",
          4: "CONVROT_ERR_BITS", 5: "CONVROT_ERR_ALIGN", 6: "CONVROT_ERR_WORKSPACE", 7: "CONVROT_ERR_NONFINITE",
          8: "CONVROT_ERR_HIP"}


class ConvrotError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} returned {STATUS.get(status, status)}")


class ConvrotMoeWeightsC(ctypes.Structure):
    _fields_ = [("E", ctypes.c_int), ("d", ctypes.c_int), ("I", ctypes.c_int), ("group_gu", ctypes.c_int),
                ("group_dn", ctypes.c_int), ("wbits", ctypes.c_int), ("q_gu", ctypes.c_void_p),
                ("s_gu", ctypes.c_void_p), ("q_dn", ctypes.c_void_p), ("s_dn", ctypes.c_void_p)]


_p, _i, _i64, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
_SIGS = {
    "convrot_status_str": (ctypes.c_char_p, [_i]),
    "convrot_weight_bytes": (_sz, [_i, _i, _i, _i, _i]),
    "convrot_quantize_weights": (_i, [_p, _i, _i, _i, _i, _i, _i, _p, _p, _p]),
    "convrot_linear_workspace_bytes": (_sz, [_i, _i]),
    "convrot_linear_w8a8": (_i, [_p, _i, _i, _p, _p, _i, _i, _p, _p, _p, _sz, _p]),
    "moe_expert_choice_workspace_bytes": (_sz, [_i, _i, ctypes.POINTER(ConvrotMoeWeightsC)]),
    "moe_expert_choice_fused": (_i, [ctypes.POINTER(ConvrotMoeWeightsC), _i]),
    "moe_expert_choice_forward_fused": (_i, [_p, _i, _p, _i, ctypes.POINTER(ConvrotMoeWeightsC), _p, _p, _p, _p, _sz, _p]),
    "moe_expert_choice_forward": (_i, [_p, _i, _p, _i, ctypes.POINTER(ConvrotMoeWeightsC), _p, _p, _p, _p, _sz, _p]),
    "moe_expert_choice_forward_noalloc": (_i, [_p, _i, _p, _i, ctypes.POINTER(ConvrotMoeWeightsC), _p, _p, _p, _p]),
    "convrot_rotq_rows": (_i, [_p, _i64, _i, _i, _p, _p, _p, _p]),
    "convrot_quantize_prerotated": (_i, [_p, _i64, _i, _i, _p, _p, _p]),
    "convrot_gemm_i8_i32": (_i, [_p, _p, _i, _i, _i, _p, _p]),
    "convrot_gemm_w8a8_bf16": (_i, [_p, _p, _i, _i, _p, _p, _i, _p, _p, _p]),
    "convrot_requantize_lora": (_i, [_p, _p, _i, _i, _i, _i, _p, _p, _i, ctypes.c_float, ctypes.c_uint64, _i, _i, _p, _p,
                                     _p]),
    "moe_route_workspace_bytes": (_sz, [_i, _i]),
    "moe_route_expert_choice": (_i, [_p, _i, _i, _i, _i, _p, _p, _p, _p, _sz, _p]),
    "moe_gateup_swiglu": (_i, [_p, _p, _i, _p, _i, ctypes.POINTER(ConvrotMoeWeightsC), _p, _p]),
    "moe_down_proj": (_i, [_p, _p, _i, ctypes.POINTER(ConvrotMoeWeightsC), _p, _p]),
    "moe_combine_workspace_bytes": (_sz, [_i, _i]),
    "moe_combine": (_i, [_p, _p, _p, _i, _i, _i, _i, _p, _p, _sz, _p]),
    "convrot_weight_g16_bytes": (_sz, [_i, _i, _i]),
    "convrot_quantize_weights_g16": (_i, [_p, _i, _i, _i, _i, _p, _p, _p, _p]),
    "convrot_gemm_g16_bf16": (_i, [_p, _p, _i, _i, _p, _p, _p, _i, _i, _p, _p, _p]),
    "convrot_linear_g16": (_i, [_p, _i, _i, _p, _p, _p, _i, _i, _i, _p, _p, _p, _sz, _p]),
    "convrot_probe_out_words": (_sz, []),
    "convrot_probe_mfma_i8": (_i, [_p, _sz, _i, _p, _sz, ctypes.POINTER(ctypes.c_double), _p]),
    "convrot_probe_hbm_read": (_i, [_p, _sz, _p, _sz, ctypes.POINTER(ctypes.c_double), _p]),
}

_lock = threading.Lock()
_lib = None


def lib():
    """Load libconvrot_amd.so (raises if it has not been built)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m w8a8_rotated_int8_amd.build` "
                                   "(there is no non-HIP fallback)")
            handle = ctypes.CDLL(LIB_PATH)
            for name, (res, args) in _SIGS.items():
                fn = getattr(handle, name)
                fn.restype = res
                fn.argtypes = args
            _lib = handle
    return _lib


def header_functions() -> list[str]:
    """Names of the functions declared in include/convrot.h and include/convrot_probes.h."""
    text = open(HEADER_PATH).read() + open(PROBES_HEADER_PATH).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\**(\w+)\(", text, flags=re.M)))


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _ptr(t) -> int | None:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("libconvrot_amd takes device tensors")
    if not t.is_contiguous():
        raise ValueError("libconvrot_amd takes contiguous tensors")
    return t.data_ptr()


def _check(name: str, st: int):
    if st != 0:
        raise ConvrotError(name, st)


def _empty(shape, dtype, like):
    return torch.empty(shape, dtype=dtype, device=like.device)


def _workspace(nbytes: int, like, ws):
    if ws is not None:
        return ws
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=like.device)


# ------------------------------------------------------------------------------------------------------
# Weights
# ------------------------------------------------------------------------------------------------------

@dataclass
class MoeWeights:
    """Quantised routed-expert weights of one layer (device tensors) and their shape/format."""
    q_gu: torch.Tensor
    s_gu: torch.Tensor
    q_dn: torch.Tensor
    s_dn: torch.Tensor
    E: int
    d: int
    I: int
    group_gu: int = 256
    group_dn: int = 64
    wbits: int = 8

    def c_struct(self) -> ConvrotMoeWeightsC:
        return ConvrotMoeWeightsC(self.E, self.d, self.I, self.group_gu, self.group_dn, self.wbits,
                                  _ptr(self.q_gu), _ptr(self.s_gu), _ptr(self.q_dn), _ptr(self.s_dn))


def convrot_status_str(status: int) -> str:
    return lib().convrot_status_str(status).decode()


LAYOUT_ROWMAJOR, LAYOUT_MFMA = 0, 1


def convrot_weight_bytes(E: int, N: int, K: int, bits: int = 8, layout: int = LAYOUT_MFMA) -> int:
    return lib().convrot_weight_bytes(E, N, K, bits, layout)


def convrot_quantize_weights(w: torch.Tensor, group: int, bits: int = 8, layout: int = LAYOUT_MFMA, q_out=None,
                             scale_out=None, stream=None):
    """w [E, N, K] (or [N, K]) bf16 -> (codes as a flat uint8/int8 buffer in `layout`, scales fp32 [.., N]).
    Row-major codes come back shaped [.., N, K] (int8) or [.., N, K/2] (uint8, packed int4)."""
    shape = w.shape
    E, N, K = (1, *shape) if w.dim() == 2 else shape
    if q_out is None:
        if layout == LAYOUT_ROWMAJOR:
            q_out = _empty((*shape[:-1], K if bits == 8 else K // 2), torch.int8 if bits == 8 else torch.uint8, w)
        else:
            q_out = _empty((convrot_weight_bytes(E, N, K, bits, layout),), torch.int8 if bits == 8 else torch.uint8, w)
    if scale_out is None:
        scale_out = _empty(shape[:-1], torch.float32, w)
    _check("convrot_quantize_weights", lib().convrot_quantize_weights(
        _ptr(w), E, N, K, group, bits, layout, _ptr(q_out), _ptr(scale_out), _stream(stream)))
    return q_out, scale_out


def quantize_moe_weights(w_gu: torch.Tensor, w_dn: torch.Tensor, group_gu: int = 256, group_dn: int = 64,
                         bits: int = 8, stream=None) -> MoeWeights:
    """Offline conversion of one layer: W_gu [E, 2I, d] and W_dn [E, d, I] (bf16, device) -> MoeWeights."""
    E, two_i, d = w_gu.shape
    q_gu, s_gu = convrot_quantize_weights(w_gu, group_gu, bits, stream=stream)
    q_dn, s_dn = convrot_quantize_weights(w_dn, group_dn, bits, stream=stream)
    return MoeWeights(q_gu, s_gu, q_dn, s_dn, E, d, two_i // 2, group_gu, group_dn, bits)


# ------------------------------------------------------------------------------------------------------
# Linear and layer
# ------------------------------------------------------------------------------------------------------

def convrot_linear_workspace_bytes(M: int, K: int) -> int:
    return lib().convrot_linear_workspace_bytes(M, K)


def convrot_linear_w8a8(x, qw, sw, group: int, bias=None, y=None, ws=None, stream=None):
    """qw: codes in the MFMA layout (from convrot_quantize_weights); N is taken from the scales sw [N]."""
    M, K = x.shape
    N = sw.shape[0]
    if y is None:
        y = _empty((M, N), torch.bfloat16, x)
    nbytes = convrot_linear_workspace_bytes(M, K)
    ws = _workspace(nbytes, x, ws)
    _check("convrot_linear_w8a8", lib().convrot_linear_w8a8(
        _ptr(x), M, K, _ptr(qw), _ptr(sw), N, group, _ptr(bias), _ptr(y), _ptr(ws), ws.numel() * ws.element_size(),
        _stream(stream)))
    return y


def moe_expert_choice_workspace_bytes(T: int, C: int, w: MoeWeights) -> int:
    cw = w.c_struct()
    return lib().moe_expert_choice_workspace_bytes(T, C, ctypes.byref(cw))


def moe_expert_choice_fused(w: MoeWeights, C: int) -> bool:
    """Whether moe_expert_choice_forward_fused takes this layer."""
    cw = w.c_struct()
    return bool(lib().moe_expert_choice_fused(ctypes.byref(cw), C))


def moe_expert_choice_forward(x, router_logits, C: int, w: MoeWeights, out=None, idx_out=None, wt_out=None,
                              ws=None, stream=None, want_routing: bool = True, fused: bool = False):
    """Routed-expert MoE layer.  Returns (out [T, d] bf16, idx [E, C] int32, wt [E, C] fp32); with
    want_routing=False and no idx_out / wt_out given, the routing outputs are not written (NULL) and come back
    as None.  fused=True calls moe_expert_choice_forward_fused (the expert GEMMs and the hidden rows'
    rotate+quantise in one launch; same results)."""
    T, d = x.shape
    if out is None:
        out = _empty((T, d), torch.bfloat16, x)
    if idx_out is None and want_routing:
        idx_out = _empty((w.E, C), torch.int32, x)
    if wt_out is None and want_routing:
        wt_out = _empty((w.E, C), torch.float32, x)
    cw = w.c_struct()
    nbytes = lib().moe_expert_choice_workspace_bytes(T, C, ctypes.byref(cw))
    ws = _workspace(nbytes, x, ws)
    name = "moe_expert_choice_forward_fused" if fused else "moe_expert_choice_forward"
    _check(name, getattr(lib(), name)(
        _ptr(x), T, _ptr(router_logits), C, ctypes.byref(cw), _ptr(out), _ptr(idx_out), _ptr(wt_out), _ptr(ws),
        ws.numel() * ws.element_size(), _stream(stream)))
    return out, idx_out, wt_out


NOALLOC_SCRATCH_BYTES = 192 << 20  # CONVROT_NOALLOC_SCRATCH_BYTES


def moe_expert_choice_forward_noalloc(x, router_logits, C: int, w: MoeWeights, out, idx_out=None, wt_out=None,
                                      stream=None):
    """The forward with the library's static per-GPU scratch as its workspace (the C entry point allocates
    nothing; `out` and the optional routing outputs are the caller's)."""
    T, _ = x.shape
    cw = w.c_struct()
    _check("moe_expert_choice_forward_noalloc", lib().moe_expert_choice_forward_noalloc(
        _ptr(x), T, _ptr(router_logits), C, ctypes.byref(cw), _ptr(out), _ptr(idx_out), _ptr(wt_out),
        _stream(stream)))
    return out, idx_out, wt_out


# ------------------------------------------------------------------------------------------------------
# Stage entry points
# ------------------------------------------------------------------------------------------------------

def convrot_rotq_rows(x, group: int, want_rot: bool = False, q_out=None, s_out=None, rot_out=None, stream=None):
    K = x.shape[-1]
    rows = x.numel() // K
    if q_out is None:
        q_out = _empty(x.shape, torch.int8, x)
    if s_out is None:
        s_out = _empty(x.shape[:-1], torch.float32, x)
    if rot_out is None and want_rot:
        rot_out = _empty(x.shape, torch.float32, x)
    _check("convrot_rotq_rows", lib().convrot_rotq_rows(
        _ptr(x), rows, K, group, _ptr(q_out), _ptr(s_out), _ptr(rot_out), _stream(stream)))
    return q_out, s_out, rot_out


def convrot_quantize_prerotated(r, bits: int = 8, q_out=None, s_out=None, stream=None):
    K = r.shape[-1]
    rows = r.numel() // K
    if q_out is None:
        q_out = _empty(r.shape, torch.int8, r)
    if s_out is None:
        s_out = _empty(r.shape[:-1], torch.float32, r)
    _check("convrot_quantize_prerotated", lib().convrot_quantize_prerotated(
        _ptr(r), rows, K, bits, _ptr(q_out), _ptr(s_out), _stream(stream)))
    return q_out, s_out


ROUND_RANDOM, ROUND_NEAREST = 0, 1


def convrot_requantize_lora(q, s, group: int, lora_b, lora_a, alpha: float, seed: int, layout: int = LAYOUT_MFMA,
                            q_out=None, s_out=None, stream=None, rounding: int = ROUND_RANDOM):
    """q int8 [E, N, K] (or [N, K]) row-major codes, s [E, N]; lora_b bf16 [E, N, r], lora_a bf16 [E, r, K]
    (r = 0: both may be None).  rounding: ROUND_RANDOM (stochastic mode) or ROUND_NEAREST (re-quantising
    mode).  Returns (codes in `layout`, scales fp32 [.., N])."""
    shape = q.shape
    E, N, K = (1, *shape) if q.dim() == 2 else shape
    r = 0 if lora_b is None else lora_b.shape[-1]
    if q_out is None:
        if layout == LAYOUT_ROWMAJOR:
            q_out = _empty(shape, torch.int8, q)
        else:
            q_out = _empty((convrot_weight_bytes(E, N, K, 8, layout),), torch.int8, q)
    if s_out is None:
        s_out = _empty(shape[:-1], torch.float32, q)
    _check("convrot_requantize_lora", lib().convrot_requantize_lora(
        _ptr(q), _ptr(s), E, N, K, group, _ptr(lora_b), _ptr(lora_a), r, float(alpha), int(seed), int(rounding), layout,
        _ptr(q_out), _ptr(s_out), _stream(stream)))
    return q_out, s_out


def convrot_gemm_w8a8_bf16(qx, sx, qw, sw, bias=None, y=None, stream=None):
    """The linear's GEMM + dequant on quantised tokens qx [M, K] int8, sx [M]; qw in the MFMA layout."""
    M, K = qx.shape
    N = sw.shape[0]
    if y is None:
        y = _empty((M, N), torch.bfloat16, qx)
    _check("convrot_gemm_w8a8_bf16", lib().convrot_gemm_w8a8_bf16(
        _ptr(qx), _ptr(sx), M, K, _ptr(qw), _ptr(sw), N, _ptr(bias), _ptr(y), _stream(stream)))
    return y


def convrot_quantize_weights_g16(w, group: int, bits: int, stream=None):
    """w: bf16 [N, K].  Returns (packed codes u8 [N, K*bits/8], E4M3 group scales u8 [N, K/16], row scales
    fp32 [N]) in the W6A8 / W4A8 format."""
    N, K = w.shape
    q = _empty((N, K * bits // 8), torch.uint8, w)
    f8 = _empty((N, K // 16), torch.uint8, w)
    s = _empty((N,), torch.float32, w)
    _check("convrot_quantize_weights_g16", lib().convrot_quantize_weights_g16(
        _ptr(w), N, K, group, bits, _ptr(q), _ptr(f8), _ptr(s), _stream(stream)))
    return q, f8, s


def convrot_gemm_g16_bf16(qx, sx, q, f8, s_row, bits: int, bias=None, y=None, stream=None):
    M, K = qx.shape
    N = s_row.shape[0]
    if y is None:
        y = _empty((M, N), torch.bfloat16, qx)
    _check("convrot_gemm_g16_bf16", lib().convrot_gemm_g16_bf16(
        _ptr(qx), _ptr(sx), M, K, _ptr(q), _ptr(f8), _ptr(s_row), N, bits, _ptr(bias), _ptr(y), _stream(stream)))
    return y


def convrot_linear_g16(x, q, f8, s_row, group: int, bits: int, bias=None, y=None, ws=None, stream=None):
    M, K = x.shape
    N = s_row.shape[0]
    if y is None:
        y = _empty((M, N), torch.bfloat16, x)
    ws = _workspace(lib().convrot_linear_workspace_bytes(M, K), x, ws)
    _check("convrot_linear_g16", lib().convrot_linear_g16(
        _ptr(x), M, K, _ptr(q), _ptr(f8), _ptr(s_row), N, group, bits, _ptr(bias), _ptr(y), _ptr(ws), ws.numel(),
        _stream(stream)))
    return y


def convrot_probe_mfma_i8(src, iters: int, out, stream=None) -> float:
    """Enqueue the int8 MFMA rate probe (src: >= 256 KiB int8 operand pool; out: convrot_probe_out_words()
    int32); returns the int8 operations the launch performs."""
    ops = ctypes.c_double(0.0)
    _check("convrot_probe_mfma_i8", lib().convrot_probe_mfma_i8(
        _ptr(src), src.numel() * src.element_size(), iters, _ptr(out), out.numel(), ctypes.byref(ops),
        _stream(stream)))
    return ops.value


def convrot_probe_hbm_read(src, out, stream=None) -> float:
    """Enqueue the HBM read probe over src (device bytes); returns the bytes the launch reads."""
    nbytes = ctypes.c_double(0.0)
    _check("convrot_probe_hbm_read", lib().convrot_probe_hbm_read(
        _ptr(src), src.numel() * src.element_size(), _ptr(out), out.numel(), ctypes.byref(nbytes),
        _stream(stream)))
    return nbytes.value


def convrot_gemm_i8_i32(a, b, acc_out=None, stream=None):
    M, K = a.shape
    N = b.shape[0]
    if acc_out is None:
        acc_out = _empty((M, N), torch.int32, a)
    _check("convrot_gemm_i8_i32", lib().convrot_gemm_i8_i32(
        _ptr(a), _ptr(b), M, N, K, _ptr(acc_out), _stream(stream)))
    return acc_out


def moe_route_expert_choice(inp, C: int, is_probs: bool = False, want_probs: bool = False, idx_out=None,
                            wt_out=None, probs_out=None, ws=None, stream=None):
    T, E = inp.shape
    if idx_out is None:
        idx_out = _empty((E, C), torch.int32, inp)
    if wt_out is None:
        wt_out = _empty((E, C), torch.float32, inp)
    if probs_out is None and want_probs:
        probs_out = _empty((T, E), torch.float32, inp)
    ws = _workspace(lib().moe_route_workspace_bytes(T, E), inp, ws)
    _check("moe_route_expert_choice", lib().moe_route_expert_choice(
        _ptr(inp), int(is_probs), T, E, C, _ptr(idx_out), _ptr(wt_out), _ptr(probs_out), _ptr(ws),
        ws.numel() * ws.element_size(), _stream(stream)))
    return idx_out, wt_out, probs_out


def moe_gateup_swiglu(qx, sx, idx, w: MoeWeights, a_out=None, stream=None):
    T = qx.shape[0]
    E, C = idx.shape
    if a_out is None:
        a_out = _empty((E * C, w.I), torch.bfloat16, qx)
    cw = w.c_struct()
    _check("moe_gateup_swiglu", lib().moe_gateup_swiglu(
        _ptr(qx), _ptr(sx), T, _ptr(idx), C, ctypes.byref(cw), _ptr(a_out), _stream(stream)))
    return a_out


def moe_down_proj(qa, sa, C: int, w: MoeWeights, z_out=None, stream=None):
    if z_out is None:
        z_out = _empty((w.E * C, w.d), torch.bfloat16, qa)
    cw = w.c_struct()
    _check("moe_down_proj", lib().moe_down_proj(_ptr(qa), _ptr(sa), C, ctypes.byref(cw), _ptr(z_out),
                                                _stream(stream)))
    return z_out


def moe_combine(z, idx, wt, T: int, out=None, ws=None, stream=None):
    E, C = idx.shape
    d = z.shape[-1]
    if out is None:
        out = _empty((T, d), torch.bfloat16, z)
    ws = _workspace(lib().moe_combine_workspace_bytes(T, E), z, ws)
    _check("moe_combine", lib().moe_combine(
        _ptr(z), _ptr(idx), _ptr(wt), T, E, C, d, _ptr(out), _ptr(ws), ws.numel() * ws.element_size(),
        _stream(stream)))
    return out
