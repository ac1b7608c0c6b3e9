"""Pins of the rotated 8-bit cache oracle (``oracle/qsa_kv_q8.py``).

- the Sylvester matrix is a Hadamard matrix (H H = d I, entries +-1) and the
  float32 butterflies equal its product with the input within float32
  rounding (and exactly on small integers);
- quantization: codes in [-127, 127], every value within half a step of its
  code (the largest ones exactly at +-127 steps when the step is a power of
  two), exact round trips for values on the grid, zero rows to zero codes;
- attention over a cache whose rotated values lie on the quantization grid
  equals plain attention over the unrotated keys and values (the rotation
  is undone exactly).
"""
from __future__ import annotations

import numpy as np
import pytest

from oracle import qsa_kv_q8 as Q
from oracle import qsa_oracle as O


@pytest.mark.parametrize("d", [2, 8, 64, 128])
def test_sylvester_is_hadamard(d):
    H = Q.sylvester(d)
    assert set(np.unique(H)) == {-1.0, 1.0}
    assert np.array_equal(H @ H.T, d * np.eye(d))
    assert np.array_equal(H, H.T)


@pytest.mark.parametrize("d", [64, 128])
def test_butterflies_are_the_matrix_product(d):
    rng = np.random.default_rng(d)
    x = rng.standard_normal((10, d)).astype(np.float32)
    got = Q.fwht_f32(x).astype(np.float64)
    want = x.astype(np.float64) @ Q.sylvester(d).T
    bound = np.log2(d) * 2.0 ** -24 * (np.abs(x.astype(np.float64)) @ np.abs(Q.sylvester(d)).T)
    assert np.all(np.abs(got - want) <= bound + 1e-30)
    ints = rng.integers(-50, 50, size=(4, d)).astype(np.float32)
    assert np.array_equal(Q.fwht_f32(ints).astype(np.float64), ints.astype(np.float64) @ Q.sylvester(d).T)
    assert np.array_equal(Q.fwht_f32(Q.fwht_f32(ints)), d * ints)  # H H = d I, exactly on integers


def test_quantization_bounds_and_grid():
    rng = np.random.default_rng(7)
    r = (rng.standard_normal((50, 128)) * rng.uniform(0.01, 10, size=(50, 1))).astype(np.float32)
    codes, s16 = Q.quantize(r)
    assert codes.dtype == np.int8 and s16.dtype == np.float16 and s16.shape == (50, 4)
    assert np.abs(codes.astype(int)).max() <= 127
    back = Q.dequantize(codes, s16)
    step = np.repeat(s16.astype(np.float64), 32, axis=1)
    clipped = np.abs(codes.astype(int)) == 127
    err = np.abs(back - r.astype(np.float64))
    assert np.all(err[~clipped] <= step[~clipped] / 2 * (1 + 1e-12))
    # the largest magnitude of a group lands at 126 or 127 steps (the float16 scale may round either way)
    g = np.abs(codes.astype(int)).reshape(50, 4, 32).max(axis=2)
    assert np.all((g == 127) | (g == 126))
    # values on the grid of a power-of-two step, one of them at 127 steps: exact codes
    m = rng.integers(-127, 128, size=(6, 128))
    m[:, ::32] = 127
    step2 = 2.0 ** rng.integers(-10, 3, size=(6, 1))
    grid = (m * step2).astype(np.float32)
    c2, s2 = Q.quantize(grid)
    assert np.array_equal(c2.astype(int), m)
    assert np.array_equal(Q.dequantize(c2, s2), grid.astype(np.float64))
    c0, s0 = Q.quantize(np.zeros((2, 64), dtype=np.float32))
    assert not c0.any() and not s0.astype(np.float64).any()


def test_attention_on_the_grid_equals_plain_attention():
    rng = np.random.default_rng(11)
    d, N, G, bs, k = 64, 96, 4, 16, 4
    H = Q.sylvester(d)

    def on_grid(n):
        m = rng.integers(-127, 128, size=(n, d))
        m[:, ::32] = 127
        rot = m * 2.0 ** -6  # rotated rows exactly on the grid (step 2^-6)
        return H @ rot.T / d, rot  # unrotated rows (exact in float32: small integers / 2^12)

    Kt, Krot = on_grid(N)
    Vt, Vrot = on_grid(N)
    K, V = Kt.T.astype(np.float32), Vt.T.astype(np.float32)
    assert np.array_equal(Q.fwht_f32(K).astype(np.float64), Krot)  # the butterflies recover the grid exactly
    kq, ks = Q.quantize_cache(K)
    vq, vs = Q.quantize_cache(V)
    q = rng.standard_normal((G, d))
    scale = O.default_scale(d)
    for p in (5, 40, 95):
        kc = O.compress_keys(K[None].astype(np.float64), bs)[0]
        sel = O.select_blocks(O.block_scores(q, kc, p // bs, scale), p // bs, k)
        got = Q.attend_q8(q, kq, ks, vq, vs, sel, p, bs, scale)
        want = O.attend_given_selection(q, K.astype(np.float64), V.astype(np.float64), sel, p, bs, scale)
        assert np.allclose(got, want, rtol=1e-12, atol=1e-12)
