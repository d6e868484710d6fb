"""Host-side tables of the library, no GPU needed.

The GEMM's SwiGLU epilogue looks the gate activation up instead of evaluating it: the gate is rounded to bf16
before the activation (Nucleus-Image MLX expert MLP), so silu has 65536 possible inputs.  The table comes from
the library's own host generator (w8a8_rotated_int8_amd/csrc/silu_table_gen.c); here every entry is checked
bit for bit against the oracle's silu of the same bf16 input, and the window the kernel keeps in LDS against
its index arithmetic."""
import numpy as np
import pytest

import oracle
from w8a8_rotated_int8_amd import build as hip_build


@pytest.fixture(scope="module")
def table():
    path = hip_build.silu_table("bin")
    t = np.fromfile(path, dtype=np.float32)
    assert t.size == 65536
    return t


def test_silu_table_matches_oracle_on_every_bf16_input(table):
    g = (np.arange(65536, dtype=np.uint32) << 16).view(np.float32)
    ref = oracle.silu(g)
    nan = np.isnan(g)
    assert np.array_equal(table.view(np.uint32)[~nan], ref.view(np.uint32)[~nan])
    assert np.isnan(table[nan]).all()


def test_silu_window_index_arithmetic(table):
    # the kernel's window: bf16 exponent fields 114..131 (|g| in [2^-13, 2^5)), both signs, 2 * 18 * 128 entries
    lo, span = 114 << 7, 18 << 7
    bits = np.arange(65536, dtype=np.uint32)
    off = ((bits & 0x7FFF) - lo) & 0xFFFFFFFF
    inside = off < span
    mag = np.abs((bits << 16).view(np.float32))
    finite = np.isfinite(mag)
    assert np.array_equal(inside[finite], ((mag >= 2.0 ** -13) & (mag < 32.0))[finite])
    window = np.empty(2 * span, dtype=np.float32)
    for k in range(2 * span):
        window[k] = table[(0 if k < span else 0x8000) + lo + (k % span)]
    idx = off[inside] + ((bits[inside] >> 15) & 1) * span
    assert np.array_equal(window[idx].view(np.uint32), table[bits[inside]].view(np.uint32))
