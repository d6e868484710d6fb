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
