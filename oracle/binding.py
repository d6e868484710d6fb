"""numpy wrapper around the C oracle (test infrastructure only; see ``convrot_oracle.c``).

bf16 tensors cross this wrapper as ``numpy.uint16`` arrays holding the raw bf16 bits.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

__all__ = [
    "build", "load", "bf16_round", "bf16_to_f32", "exp", "silu", "rotate_rows_f32", "rotate_rows_bf16",
    "quantize_rows", "rotq_rows", "pack_int4", "unpack_int4", "quantize_weights", "gemm_i8_i32",
    "dequant_bf16", "linear_w8a8", "softmax_experts", "route_from_probs", "route", "swiglu", "combine",
    "moe_gateup", "moe_down", "moe_forward", "moe_rows", "philox4x64_10", "requantize_lora",
    "e4m3_encode", "e4m3_decode", "pack_int6", "unpack_int6", "quantize_g16", "unpack_g16", "gemm_g16",
    "linear_g16",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "convrot_oracle.c")
# CONVROT_ORACLE_LIB names another build of the same source (the sanitizer pass in tests/sanitize.py)
_LIB = os.environ.get("CONVROT_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

# -ffp-contract=off: no fused multiply-add anywhere; -fno-fast-math: IEEE semantics (gcc's default, stated).
CFLAGS = ["-O3", "-std=gnu11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off", "-fno-fast-math"]


def build(force: bool = True) -> str:
    """Compile the oracle with gcc into ``oracle/liboracle.so`` and return its path."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.run(["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


def load():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB):
                build(force=False)
            _lib = _declare(ctypes.CDLL(_LIB))
    return _lib


_p = ctypes.c_void_p
_i = ctypes.c_int
_i64 = ctypes.c_int64


def _declare(lib):
    sig = {
        "oracle_bf16_round": (None, [_p, _i64, _p]),
        "oracle_exp": (ctypes.c_float, [ctypes.c_float]),
        "oracle_exp_array": (None, [_p, _i64, _p]),
        "oracle_silu_array": (None, [_p, _i64, _p]),
        "oracle_rotate_rows_f32": (_i, [_p, _i64, _i, _i, _p]),
        "oracle_rotate_rows_bf16": (_i, [_p, _i64, _i, _i, _p]),
        "oracle_quantize_rows": (None, [_p, _i64, _i, _i, _p, _p]),
        "oracle_rotq_rows": (_i, [_p, _i64, _i, _i, _i, _p, _p, _p]),
        "oracle_pack_int4": (None, [_p, _i64, _i, _p]),
        "oracle_unpack_int4": (None, [_p, _i64, _i, _p]),
        "oracle_quantize_weights": (_i, [_p, _i, _i, _i, _i, _i, _p, _p]),
        "oracle_philox4x64_10": (None, [_p, _p, _p]),
        "oracle_requantize_lora": (_i, [_p, _p, _i, _i, _i, _i, _p, _p, _i, ctypes.c_float, ctypes.c_uint64, _i, _p,
                                        _p]),
        "oracle_gemm_i8_i32": (None, [_p, _p, _i, _i, _i, _p]),
        "oracle_dequant_bf16": (None, [_p, _p, _p, _p, _i, _i, _p]),
        "oracle_linear_w8a8": (_i, [_p, _i, _i, _p, _p, _i, _i, _p, _p, _p, _p]),
        "oracle_softmax_experts": (None, [_p, _i, _i, _p]),
        "oracle_route_from_probs": (_i, [_p, _i, _i, _i, _p, _p]),
        "oracle_route": (_i, [_p, _i, _i, _i, _p, _p, _p]),
        "oracle_swiglu": (None, [_p, _i64, _i, _p]),
        "oracle_combine": (None, [_p, _p, _p, _i, _i, _i, _i, _p]),
        "oracle_moe_gateup": (None, [_p, _p, _i, _p, _i, _i, _i, _p, _p, _i, _p]),
        "oracle_moe_down": (None, [_p, _p, _i, _i, _i, _i, _p, _p, _i, _p]),
        "oracle_moe_forward": (_i, [_p, _i, _i, _p, _i, _i, _i, _p, _p, _i, _p, _p, _i, _i,
                                    _p, _p, _p, _p, _p, _p, _p, _p, _p, _p]),
        "oracle_moe_rows": (_i, [_p, _p, _i, _p, _p, _i, _i, _i, _p, _p, _p, _p, _i, _i, _p, _i, _p]),
        "oracle_e4m3_encode_array": (None, [_p, _i64, _p]),
        "oracle_e4m3_decode_array": (None, [_p, _i64, _p]),
        "oracle_pack_int6": (None, [_p, _i64, _i, _p]),
        "oracle_unpack_int6": (None, [_p, _i64, _i, _p]),
        "oracle_quantize_g16_rows": (None, [_p, _i64, _i, _i, _p, _p, _p]),
        "oracle_quantize_g16": (_i, [_p, _i, _i, _i, _i, _p, _p, _p, _p]),
        "oracle_gemm_g16": (None, [_p, _p, _i, _i, _p, _p, _p, _i, _p, _p, _p, _p]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a


def _ptr(a):
    return None if a is None else a.ctypes.data


def _check(st, what):
    if st != 0:
        raise ValueError(f"oracle {what} rejected its arguments (status {st})")


# --------------------------------------------------------------------------------------------------
# Elementwise helpers
# --------------------------------------------------------------------------------------------------

def bf16_round(x) -> np.ndarray:
    """fp32 -> bf16 bits, nearest-even."""
    x = _c(x, np.float32)
    out = np.empty(x.shape, np.uint16)
    load().oracle_bf16_round(_ptr(x), x.size, _ptr(out))
    return out


def bf16_to_f32(h) -> np.ndarray:
    h = _c(h, np.uint16)
    return (h.astype(np.uint32) << 16).view(np.float32)


def exp(x) -> np.ndarray:
    x = _c(x, np.float32)
    out = np.empty_like(x)
    load().oracle_exp_array(_ptr(x), x.size, _ptr(out))
    return out


def silu(x) -> np.ndarray:
    x = _c(x, np.float32)
    out = np.empty_like(x)
    load().oracle_silu_array(_ptr(x), x.size, _ptr(out))
    return out


# --------------------------------------------------------------------------------------------------
# Rotation and quantisation
# --------------------------------------------------------------------------------------------------

def rotate_rows_f32(x, g: int) -> np.ndarray:
    x = _c(x, np.float32)
    K = x.shape[-1]
    out = np.empty_like(x)
    _check(load().oracle_rotate_rows_f32(_ptr(x), x.size // K, K, g, _ptr(out)), "rotate")
    return out


def rotate_rows_bf16(x, g: int) -> np.ndarray:
    x = _c(x, np.uint16)
    K = x.shape[-1]
    out = np.empty(x.shape, np.float32)
    _check(load().oracle_rotate_rows_bf16(_ptr(x), x.size // K, K, g, _ptr(out)), "rotate")
    return out


def quantize_rows(r, qmax: int = 127):
    r = _c(r, np.float32)
    K = r.shape[-1]
    q = np.empty(r.shape, np.int8)
    s = np.empty(r.shape[:-1], np.float32)
    load().oracle_quantize_rows(_ptr(r), r.size // K, K, qmax, _ptr(q), _ptr(s))
    return q, s


def rotq_rows(x, g: int, qmax: int = 127, return_rot: bool = False):
    x = _c(x, np.uint16)
    K = x.shape[-1]
    q = np.empty(x.shape, np.int8)
    s = np.empty(x.shape[:-1], np.float32)
    rot = np.empty(x.shape, np.float32) if return_rot else None
    _check(load().oracle_rotq_rows(_ptr(x), x.size // K, K, g, qmax, _ptr(q), _ptr(s), _ptr(rot)), "rotq")
    return (q, s, rot) if return_rot else (q, s)


def pack_int4(q) -> np.ndarray:
    q = _c(q, np.int8)
    K = q.shape[-1]
    out = np.empty(q.shape[:-1] + (K // 2,), np.uint8)
    load().oracle_pack_int4(_ptr(q), q.size // K, K, _ptr(out))
    return out


def unpack_int4(p, K: int) -> np.ndarray:
    p = _c(p, np.uint8)
    out = np.empty(p.shape[:-1] + (K,), np.int8)
    load().oracle_unpack_int4(_ptr(p), p.size // (K // 2), K, _ptr(out))
    return out


def philox4x64_10(ctr, key) -> np.ndarray:
    """The four 64-bit words of Philox4x64-10 at counter ctr (4 words) and key (2 words)."""
    c = np.ascontiguousarray(ctr, dtype=np.uint64)
    k = np.ascontiguousarray(key, dtype=np.uint64)
    out = np.empty(4, np.uint64)
    load().oracle_philox4x64_10(_ptr(c), _ptr(k), _ptr(out))
    return out


def requantize_lora(q, s, g: int, lb, la, alpha: float, seed: int, nearest: bool = False):
    """q int8 [E, N, K] (or [N, K]), s [E, N]; lb bf16 bits [E, N, r], la [E, r, K] (or without E).
    Returns (codes int8, scales fp32) of the LoRA-patched weights, re-quantised with random rounding, or with
    nearest rounding when `nearest` (then `seed` is unused)."""
    q = _c(q, np.int8)
    squeeze = q.ndim == 2
    if squeeze:
        q, s, lb, la = q[None], np.asarray(s)[None], np.asarray(lb)[None], np.asarray(la)[None]
    s, lb, la = _c(s, np.float32), _c(lb, np.uint16), _c(la, np.uint16)
    E, N, K = q.shape
    r = lb.shape[-1]
    qo = np.empty_like(q)
    so = np.empty((E, N), np.float32)
    _check(load().oracle_requantize_lora(_ptr(q), _ptr(s), E, N, K, g, _ptr(lb), _ptr(la), r, float(alpha),
                                         int(seed), int(bool(nearest)), _ptr(qo), _ptr(so)), "requantize_lora")
    return (qo[0], so[0]) if squeeze else (qo, so)


def quantize_weights(w, g: int, bits: int = 8):
    """w: bf16 bits [E, N, K] (or [N, K]).  Returns (codes int8 [.., K] or packed u8 [.., K/2], scales)."""
    w = _c(w, np.uint16)
    squeeze = w.ndim == 2
    if squeeze:
        w = w[None]
    E, N, K = w.shape
    q = np.empty((E, N, K if bits == 8 else K // 2), np.int8 if bits == 8 else np.uint8)
    s = np.empty((E, N), np.float32)
    _check(load().oracle_quantize_weights(_ptr(w), E, N, K, g, bits, _ptr(q), _ptr(s)), "quantize_weights")
    return (q[0], s[0]) if squeeze else (q, s)


# --------------------------------------------------------------------------------------------------
# Linear
# --------------------------------------------------------------------------------------------------

def gemm_i8_i32(a, b) -> np.ndarray:
    a = _c(a, np.int8)
    b = _c(b, np.int8)
    M, K = a.shape
    N = b.shape[0]
    acc = np.empty((M, N), np.int32)
    load().oracle_gemm_i8_i32(_ptr(a), _ptr(b), M, N, K, _ptr(acc))
    return acc


def dequant_bf16(acc, sa, sb, bias=None) -> np.ndarray:
    acc = _c(acc, np.int32)
    sa = _c(sa, np.float32)
    sb = _c(sb, np.float32)
    bias = None if bias is None else _c(bias, np.uint16)
    M, N = acc.shape
    y = np.empty((M, N), np.uint16)
    load().oracle_dequant_bf16(_ptr(acc), _ptr(sa), _ptr(sb), _ptr(bias), M, N, _ptr(y))
    return y


def linear_w8a8(x, qw, sw, g: int, bias=None):
    """Returns (y bf16 bits [M, N], qx [M, K], sx [M])."""
    x = _c(x, np.uint16)
    qw = _c(qw, np.int8)
    sw = _c(sw, np.float32)
    bias = None if bias is None else _c(bias, np.uint16)
    M, K = x.shape
    N = qw.shape[0]
    y = np.empty((M, N), np.uint16)
    qx = np.empty((M, K), np.int8)
    sx = np.empty(M, np.float32)
    _check(load().oracle_linear_w8a8(_ptr(x), M, K, _ptr(qw), _ptr(sw), N, g, _ptr(bias), _ptr(y),
                                     _ptr(qx), _ptr(sx)), "linear")
    return y, qx, sx


# --------------------------------------------------------------------------------------------------
# W6A8 / W4A8 with FP8 (E4M3) group-16 scales
# --------------------------------------------------------------------------------------------------

def e4m3_encode(x) -> np.ndarray:
    x = _c(x, np.float32)
    out = np.empty(x.shape, np.uint8)
    load().oracle_e4m3_encode_array(_ptr(x), x.size, _ptr(out))
    return out


def e4m3_decode(b) -> np.ndarray:
    b = _c(b, np.uint8)
    out = np.empty(b.shape, np.float32)
    load().oracle_e4m3_decode_array(_ptr(b), b.size, _ptr(out))
    return out


def pack_int6(q) -> np.ndarray:
    q = _c(q, np.int8)
    rows, K = q.shape
    out = np.empty((rows, K // 4 * 3), np.uint8)
    load().oracle_pack_int6(_ptr(q), rows, K, _ptr(out))
    return out


def unpack_int6(p, K: int) -> np.ndarray:
    p = _c(p, np.uint8)
    rows = p.shape[0]
    q = np.empty((rows, K), np.int8)
    load().oracle_unpack_int6(_ptr(p), rows, K, _ptr(q))
    return q


def quantize_g16(w, g: int, bits: int):
    """w: bf16 bits [N, K].  Returns (packed codes u8 [N, K*bits/8], E4M3 group scales u8 [N, K/16],
    row scales fp32 [N], codes int8 [N, K])."""
    w = _c(w, np.uint16)
    N, K = w.shape
    q = np.empty((N, K * bits // 8), np.uint8)
    f8 = np.empty((N, K // 16), np.uint8)
    s = np.empty(N, np.float32)
    codes = np.empty((N, K), np.int8)
    _check(load().oracle_quantize_g16(_ptr(w), N, K, g, bits, _ptr(q), _ptr(f8), _ptr(s), _ptr(codes)),
           "quantize_g16")
    return q, f8, s, codes


def unpack_g16(q, K: int, bits: int) -> np.ndarray:
    """Codes int8 [N, K] from the 6- or 4-bit packing."""
    if bits == 6:
        return unpack_int6(q, K)
    return unpack_int4(q, K)


def gemm_g16(qx, sx, codes, f8, s_row, bias=None):
    """Returns (y bf16 bits [M, N], A fp64 [M, N] (exact), sum of |terms| fp64 [M, N])."""
    qx = _c(qx, np.int8)
    sx = _c(sx, np.float32)
    codes = _c(codes, np.int8)
    f8 = _c(f8, np.uint8)
    s_row = _c(s_row, np.float32)
    bias = None if bias is None else _c(bias, np.uint16)
    M, K = qx.shape
    N = codes.shape[0]
    y = np.empty((M, N), np.uint16)
    acc = np.empty((M, N), np.float64)
    aabs = np.empty((M, N), np.float64)
    load().oracle_gemm_g16(_ptr(qx), _ptr(sx), M, K, _ptr(codes), _ptr(f8), _ptr(s_row), N, _ptr(bias), _ptr(y),
                           _ptr(acc), _ptr(aabs))
    return y, acc, aabs


def linear_g16(x, g: int, codes, f8, s_row, bias=None):
    """The W6A8 / W4A8 linear: tokens rotated and quantised to int8 per token (as W8A8), then gemm_g16.
    Returns (y, qx, sx, A, sum of |terms|)."""
    x = _c(x, np.uint16)
    M, K = x.shape
    qx, sx = rotq_rows(x, g, 127)[:2]
    y, acc, aabs = gemm_g16(qx, sx, codes, f8, s_row, bias)
    return y, qx, sx, acc, aabs


# --------------------------------------------------------------------------------------------------
# Routing, expert FFN, combine, whole layer
# --------------------------------------------------------------------------------------------------

def softmax_experts(logits) -> np.ndarray:
    logits = _c(logits, np.float32)
    T, E = logits.shape
    p = np.empty((T, E), np.float32)
    load().oracle_softmax_experts(_ptr(logits), T, E, _ptr(p))
    return p


def route_from_probs(p, C: int):
    p = _c(p, np.float32)
    T, E = p.shape
    idx = np.empty((E, C), np.int32)
    wt = np.empty((E, C), np.float32)
    _check(load().oracle_route_from_probs(_ptr(p), T, E, C, _ptr(idx), _ptr(wt)), "route")
    return idx, wt


def route(logits, C: int):
    logits = _c(logits, np.float32)
    T, E = logits.shape
    idx = np.empty((E, C), np.int32)
    wt = np.empty((E, C), np.float32)
    p = np.empty((T, E), np.float32)
    _check(load().oracle_route(_ptr(logits), T, E, C, _ptr(idx), _ptr(wt), _ptr(p)), "route")
    return idx, wt, p


def swiglu(gu) -> np.ndarray:
    gu = _c(gu, np.uint16)
    I = gu.shape[-1] // 2
    rows = gu.size // (2 * I)
    a = np.empty(gu.shape[:-1] + (I,), np.uint16)
    load().oracle_swiglu(_ptr(gu), rows, I, _ptr(a))
    return a


def combine(z, idx, wt, T: int) -> np.ndarray:
    idx = _c(idx, np.int32)
    wt = _c(wt, np.float32)
    E, C = idx.shape
    z = _c(z, np.uint16).reshape(E * C, -1)
    d = z.shape[1]
    out = np.empty((T, d), np.uint16)
    load().oracle_combine(_ptr(z), _ptr(idx), _ptr(wt), T, E, C, d, _ptr(out))
    return out


def moe_gateup(qx, sx, idx, q_gu, s_gu, wbits: int = 8) -> np.ndarray:
    qx = _c(qx, np.int8)
    sx = _c(sx, np.float32)
    idx = _c(idx, np.int32)
    q_gu = np.ascontiguousarray(q_gu)
    s_gu = _c(s_gu, np.float32)
    E, C = idx.shape
    d = qx.shape[1]
    I = s_gu.shape[1] // 2
    a = np.empty((E * C, I), np.uint16)
    load().oracle_moe_gateup(_ptr(qx), _ptr(sx), d, _ptr(idx), E, C, I, _ptr(q_gu), _ptr(s_gu), wbits, _ptr(a))
    return a


def moe_down(qa, sa, E: int, C: int, q_dn, s_dn, wbits: int = 8) -> np.ndarray:
    qa = _c(qa, np.int8)
    sa = _c(sa, np.float32)
    q_dn = np.ascontiguousarray(q_dn)
    s_dn = _c(s_dn, np.float32)
    I = qa.shape[1]
    d = s_dn.shape[1]
    z = np.empty((E * C, d), np.uint16)
    load().oracle_moe_down(_ptr(qa), _ptr(sa), E, C, I, d, _ptr(q_dn), _ptr(s_dn), wbits, _ptr(z))
    return z


def moe_forward(x, logits, C: int, q_gu, s_gu, g_gu: int, q_dn, s_dn, g_dn: int, wbits: int = 8,
                intermediates: bool = False) -> dict:
    """Whole routed-expert layer.  Returns a dict with out, idx, wt (and p, qx, sx, a, qa, sa, z)."""
    x = _c(x, np.uint16)
    logits = _c(logits, np.float32)
    q_gu = np.ascontiguousarray(q_gu)
    q_dn = np.ascontiguousarray(q_dn)
    s_gu = _c(s_gu, np.float32)
    s_dn = _c(s_dn, np.float32)
    T, d = x.shape
    E = logits.shape[1]
    I = s_gu.shape[1] // 2
    S = E * C
    r = {"out": np.empty((T, d), np.uint16), "idx": np.empty((E, C), np.int32),
         "wt": np.empty((E, C), np.float32)}
    if intermediates:
        r.update(p=np.empty((T, E), np.float32), qx=np.empty((T, d), np.int8), sx=np.empty(T, np.float32),
                 a=np.empty((S, I), np.uint16), qa=np.empty((S, I), np.int8), sa=np.empty(S, np.float32),
                 z=np.empty((S, d), np.uint16))
    g = r.get
    _check(load().oracle_moe_forward(
        _ptr(x), T, d, _ptr(logits), E, C, I, _ptr(q_gu), _ptr(s_gu), g_gu, _ptr(q_dn), _ptr(s_dn), g_dn, wbits,
        _ptr(r["out"]), _ptr(r["idx"]), _ptr(r["wt"]), _ptr(g("p")), _ptr(g("qx")), _ptr(g("sx")), _ptr(g("a")),
        _ptr(g("qa")), _ptr(g("sa")), _ptr(g("z"))), "moe_forward")
    return r


def moe_rows(qx, sx, idx, wt, q_gu, s_gu, q_dn, s_dn, g_dn: int, tokens, wbits: int = 8) -> np.ndarray:
    """Layer output rows (bf16 bits [len(tokens), d]) for the given tokens only."""
    qx = _c(qx, np.int8)
    sx = _c(sx, np.float32)
    idx = _c(idx, np.int32)
    wt = _c(wt, np.float32)
    q_gu = np.ascontiguousarray(q_gu)
    q_dn = np.ascontiguousarray(q_dn)
    s_gu = _c(s_gu, np.float32)
    s_dn = _c(s_dn, np.float32)
    tokens = _c(tokens, np.int32)
    E, C = idx.shape
    d = qx.shape[1]
    I = s_gu.shape[1] // 2
    out = np.empty((tokens.size, d), np.uint16)
    _check(load().oracle_moe_rows(_ptr(qx), _ptr(sx), d, _ptr(idx), _ptr(wt), E, C, I, _ptr(q_gu), _ptr(s_gu),
                                  _ptr(q_dn), _ptr(s_dn), g_dn, wbits, _ptr(tokens), tokens.size, _ptr(out)),
           "moe_rows")
    return out
