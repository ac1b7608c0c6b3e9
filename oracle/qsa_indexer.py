"""Plain fp64 CPU oracle of the learned-indexer variant of QSA selection.

TEST INFRASTRUCTURE ONLY (like ``qsa_oracle``): used by the test-suite and
never by the product path; it shares no code with the HIP implementation.

Source: [port] "Qwen4 in llama.cpp: Dissecting PR #27742" (ramgpt.org),
section "QSA Is an Address-Selection Problem, Not a New Attention
Equation": the selector runs indexer projections, forms a compressed-block
representation, scores it and keeps the top-k blocks; the learned selector
is architecture-specific and the pages give neither its weights nor its
exact form. Readings taken here (each restated where it is used):

* the indexer space has its own dimension ``d_idx``; a key ``k`` (the
  cached attention key, ``[d]``) maps to ``k @ W_k`` and a query head ``q``
  to ``q @ W_q``, with ``W_k``, ``W_q`` of shape ``[d][d_idx]`` shared by all
  heads (synthetic, seeded weights: no trained ones exist here);
* a block's compressed indexer key is the mean of its projected keys;
* each query head ``j`` of a KV head's group scores candidate ``c`` with
  ``s_j(c) = scale * <q_j @ W_q, kidx_c>``, ``scale = 1/sqrt(d_idx)`` unless
  given;
* the group's score of a candidate aggregates its heads' scores by one of:
  ``sum`` (the default frame's reading, here in indexer space), ``max``
  (the best head decides), or ``softmax`` (each head's scores turned into a
  probability distribution over the row's candidates, then summed over the
  heads);
* the frame, the forced block, the tie rule and the output format are those
  of ``qsa_oracle.select_in_frame``.

Every function has an independent pin in ``tests/test_indexer_oracle.py``.
"""
from __future__ import annotations

import math

import numpy as np

AGG_SUM, AGG_MAX, AGG_SOFTMAX = 0, 1, 2
AGG_NAMES = {AGG_SUM: "sum", AGG_MAX: "max", AGG_SOFTMAX: "softmax"}


def default_indexer_scale(d_idx: int) -> float:
    return 1.0 / math.sqrt(d_idx)


def indexer_keys(K: np.ndarray, W_k: np.ndarray, block_size: int) -> np.ndarray:
    """Compressed indexer keys ``[..., nb, d_idx]`` of keys ``K`` ``[..., N, d]``.

    Each cached key is projected into the indexer space first, then the
    projected keys of every complete block ``[c*Bs, (c+1)*Bs)`` are averaged.
    """
    K = np.asarray(K, dtype=np.float64)
    W = np.asarray(W_k, dtype=np.float64)
    n_blocks = K.shape[-2] // block_size
    projected = K[..., : n_blocks * block_size, :] @ W
    out = np.zeros(K.shape[:-2] + (n_blocks, W.shape[1]), dtype=np.float64)
    for c in range(n_blocks):
        out[..., c, :] = projected[..., c * block_size:(c + 1) * block_size, :].sum(axis=-2) / block_size
    return out


def head_scores(q_group: np.ndarray, W_q: np.ndarray, k_idx: np.ndarray, n_candidates: int,
                scale: float) -> np.ndarray:
    """Per-head indexer scores ``[n_candidates][G]`` of one token and KV head.

    ``q_group``: ``[G, d]``; ``k_idx``: ``[n_blocks, d_idx]``.
    """
    qi = np.asarray(q_group, dtype=np.float64) @ np.asarray(W_q, dtype=np.float64)  # [G][d_idx]
    kc = np.asarray(k_idx[:n_candidates], dtype=np.float64)
    out = np.zeros((n_candidates, qi.shape[0]), dtype=np.float64)
    for j in range(qi.shape[0]):
        out[:, j] = scale * (kc @ qi[j])
    return out


def aggregate(per_head: np.ndarray, agg: int) -> np.ndarray:
    """Group score of every candidate from its per-head scores ``[n][G]``."""
    if per_head.shape[0] == 0:
        return np.zeros(0, dtype=np.float64)
    if agg == AGG_SUM:
        return per_head.sum(axis=1)
    if agg == AGG_MAX:
        return per_head.max(axis=1)
    if agg == AGG_SOFTMAX:
        total = np.zeros(per_head.shape[0], dtype=np.float64)
        for j in range(per_head.shape[1]):
            col = per_head[:, j]
            e = np.exp(col - col.max())
            total += e / e.sum()
        return total
    raise ValueError(f"unknown aggregation {agg}")


def indexer_scores(q_group, W_q, k_idx, n_candidates, scale, agg) -> np.ndarray:
    """Group scores ``[n_candidates]`` of one token and KV head under aggregation ``agg``."""
    return aggregate(head_scores(q_group, W_q, k_idx, n_candidates, scale), agg)
