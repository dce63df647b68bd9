"""Integer arithmetic the kernels do in floating point, checked exhaustively
on the CPU in the same float32 operations.

The attention kernels split a token index t into (t / P, t mod P) with a
float32 reciprocal of the page size, a truncating conversion and one
correction step.  The host passes 1.0f / P; every length the library
accepts is below 2^22 (PGQA_MAX_SEQ_LEN).  Here the same steps run over
every t < 2^22 for a spread of page sizes and must give t // P and t % P."""
from __future__ import annotations

import numpy as np
import pytest

MAX_T = 1 << 22


@pytest.fixture(scope="module")
def tokens():
    t = np.arange(MAX_T, dtype=np.int64)
    return t, t.astype(np.float32)


@pytest.mark.parametrize("P", [1, 2, 3, 4, 5, 7, 16, 100, 128, 255, 256, 300, 784, 1000, 4095])
def test_page_division_exact(tokens, P):
    t, tf = tokens
    inv = np.float32(1.0) / np.float32(P)
    qt = (tf * inv).astype(np.int64)            # v_mul_f32 then v_cvt_i32_f32 (truncation)
    rem = t - qt * P
    adj = np.where(rem < 0, -1, np.where(rem >= P, 1, 0))
    assert np.array_equal(qt + adj, t // P)
    assert np.array_equal(rem - adj * P, t % P)
    assert np.abs(qt - t // P).max() <= 1       # one correction step suffices
