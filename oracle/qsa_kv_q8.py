"""CPU oracle of the rotated 8-bit K/V cache path (decode attention).

TEST INFRASTRUCTURE ONLY (like ``qsa_oracle``); shares no code with the HIP
implementation.

Source: [port] "Qwen4 in llama.cpp: Dissecting PR #27742" (ramgpt.org),
section "Quantized KV Exposed a Backend Storage Invariant": the K/V cache is
stored in a Hadamard-rotated basis and quantized, attention runs in that
basis and the output is rotated back, exactly, since the (scaled) Hadamard
matrix is its own inverse; the indexer cache is not rotated. The storage
format is this library's reading (the pages name a q8_0-like cache only):

* rotation of a row ``x`` (length d, a power of two): ``H x`` with ``H`` the
  unnormalised Sylvester Hadamard matrix (entries +-1), computed as the
  butterfly stages h = 1, 2, ..., d/2 in that order, pair ``(i, i+h)``
  (``i`` with bit h clear) becoming ``(x_i + x_{i+h}, x_i - x_{i+h})``, in
  float32;
* per 32 values of a rotated row: ``scale = float16(max|value| / 127)``
  (the division in float32), ``code = round_half_even(value / scale)``
  clamped to [-127, 127], 0 when the scale is 0; value = ``code * scale``;
* attention: scores ``scale_attn * (H q) . k_hat / d`` over the visible
  positions, softmax, ``o_rot = sum p v_hat``, output ``H o_rot / d``.

The rotation and the codes are integers decided by float32 arithmetic, so
they follow the stated float32 steps exactly (``fwht_f32``, ``quantize``);
the attention is float64 on the dequantized values. Every function has a
pin in ``tests/test_kv_q8_oracle.py``.
"""
from __future__ import annotations

import numpy as np

from oracle import qsa_oracle as O

GROUP = 32


def sylvester(d: int) -> np.ndarray:
    """The unnormalised Sylvester Hadamard matrix of order d (float64, entries +-1)."""
    h = np.ones((1, 1))
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    if h.shape[0] != d:
        raise ValueError("d must be a power of two")
    return h


def fwht_f32(x: np.ndarray) -> np.ndarray:
    """Rows of ``x`` (last axis, length d) rotated by the butterfly stages, in float32."""
    y = np.array(x, dtype=np.float32, copy=True)
    d = y.shape[-1]
    h = 1
    while h < d:
        v = y.reshape(y.shape[:-1] + (d // (2 * h), 2, h))
        a = v[..., 0, :].copy()
        b = v[..., 1, :].copy()
        v[..., 0, :] = a + b
        v[..., 1, :] = a - b
        h *= 2
    return y


def quantize(rot: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Codes (int8, same shape) and float16 scales (``[..., d/32]``) of rotated float32 rows."""
    r = np.asarray(rot, dtype=np.float32)
    d = r.shape[-1]
    g = r.reshape(r.shape[:-1] + (d // GROUP, GROUP))
    amax = np.abs(g).max(axis=-1)
    scales16 = (amax / np.float32(127.0)).astype(np.float16)
    s = scales16.astype(np.float32)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.where(s > 0, np.rint(g / np.where(s > 0, s, np.float32(1.0))), np.float32(0.0))
    codes = np.clip(q, -127, 127).astype(np.int8).reshape(r.shape)
    return codes, scales16


def dequantize(codes: np.ndarray, scales16: np.ndarray) -> np.ndarray:
    """Float64 values ``code * scale`` (exact)."""
    c = np.asarray(codes, dtype=np.float64)
    d = c.shape[-1]
    s = np.asarray(scales16, dtype=np.float64)
    return (c.reshape(c.shape[:-1] + (d // GROUP, GROUP)) * s[..., None]).reshape(c.shape)


def quantize_cache(X: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """The 8-bit cache of K or V rows ``[..., N, d]`` (stored values, widened exactly)."""
    return quantize(fwht_f32(X))


def attend_q8(q_group, kq, ks, vq, vs, selection, p, block_size, scale):
    """``[G][d]`` decode output of one token and KV head over the 8-bit cache.

    ``kq``/``vq``: codes ``[N][d]``; ``ks``/``vs``: float16 scales ``[N][d/32]``.
    """
    q_group = np.asarray(q_group, dtype=np.float64)
    d = q_group.shape[-1]
    H = sylvester(d)
    pos = O.visible_positions(selection, p, block_size)
    k_hat = dequantize(kq[pos], ks[pos])
    v_hat = dequantize(vq[pos], vs[pos])
    out = np.zeros_like(q_group)
    for j in range(q_group.shape[0]):
        q_rot = H @ q_group[j]
        logits = scale * (k_hat @ q_rot) / d
        wts = np.exp(logits - logits.max())
        o_rot = (wts @ v_hat) / wts.sum()
        out[j] = H @ o_rot / d
    return out
