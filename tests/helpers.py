"""Small host<->device helpers for the GPU tests (bf16 travels as raw uint16 bits on the host side)."""
import numpy as np
import torch

DEV = "cuda:0"


def dev_bf16(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16)).view(torch.bfloat16).to(DEV)


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host_bf16(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def host(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().cpu().numpy()


def f32(bits: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def assert_bf16_within(got_bits, ref_bits, rel=1e-2, floor=None, what="output"):
    """Elementwise |got - ref| <= rel * |ref| (+ floor), the parity bar for BF16 outputs; returns the fraction of
    bit-identical elements."""
    g = f32(got_bits).astype(np.float64)
    r = f32(ref_bits).astype(np.float64)
    bound = rel * np.abs(r) + (0.0 if floor is None else floor)
    bad = np.abs(g - r) > bound
    assert not bad.any(), f"{what}: {int(bad.sum())} of {bad.size} elements outside tolerance; first at " \
                          f"{np.argwhere(bad)[0].tolist()}: got {g[bad][0]!r} ref {r[bad][0]!r}"
    return float(np.mean(np.asarray(got_bits) == np.asarray(ref_bits)))


def say(msg: str):
    print(msg, flush=True)


def untile_codes(buf: np.ndarray, E: int, N: int, K: int, bits: int) -> np.ndarray:
    """Row-major codes (int8 [E, N, K]) from a buffer in the MFMA-tiled layout documented in include/convrot.h:
    rows in blocks of 32 (padded), each (row block, K-block) tile 1 KiB; int8: lane L = r + 32*((k%32)/16)
    holding 16 consecutive k; int4: 8-byte entry 64*(r/16) + 16*((k%64)/16) + r%16 holding 16 consecutive k,
    in each 4-byte word the low nibbles 4 consecutive k and the high nibbles the next 4."""
    NB = (N + 31) // 32
    b = np.ascontiguousarray(buf).view(np.uint8)
    if bits == 8:
        t = b.view(np.int8).reshape(E, NB, K // 32, 2, 32, 16)        # e, nb, ks, half, r, j
        codes = t.transpose(0, 1, 4, 2, 3, 5).reshape(E, NB * 32, K)  # e, nb, r, ks, half, j
    else:
        t = b.reshape(E, NB, K // 64, 2, 4, 16, 2, 4)                  # e, nb, ks, r/16, (k%64)/16, r%16, word, byte
        lo = (t & 0xF).astype(np.int8)                                 # k%16 = 8 word + byte
        hi = (t >> 4).astype(np.int8)                                  # k%16 = 8 word + 4 + byte
        lo = np.where(lo >= 8, lo - 16, lo)
        hi = np.where(hi >= 8, hi - 16, hi)
        nib = np.stack([lo, hi], axis=-2).reshape(E, NB, K // 64, 2, 4, 16, 16)  # ..., k%16
        codes = nib.transpose(0, 1, 3, 5, 2, 4, 6).reshape(E, NB * 32, K)          # e, nb, r/16, r%16, ks, g, j
    return np.ascontiguousarray(codes[:, :N, :]).astype(np.int8)
