"""Plain fp64 CPU oracle for Qwen Sparse Attention (QSA).

TEST INFRASTRUCTURE ONLY. It is imported by the test-suite, by the smoke
check and by the benchmark's CPU-baseline leg, never by the product path, and
it shares no code with the HIP implementation. Everything is computed in
float64 from the stored (bf16 or fp32) values, which widen exactly.

Sources, cited by page title and section:

[overview]  "Qwen4 architecture: QSA, GatedResidual, PLE" (codebridge-ai.com),
            section 1 "QSA: not looking at every token equally": keys are
            compressed into small blocks, the blocks are scored against the
            query, the best contiguous token blocks are kept and attention runs
            over those only.
[port]      "Qwen4 in llama.cpp: Dissecting PR #27742" (ramgpt.org), section
            "QSA Is an Address-Selection Problem, Not a New Attention
            Equation": compressed-block representation -> indexer scoring ->
            top-k -> cache-cell IDs -> ordinary attention over those cells;
            the visible-width bound and the dense regime below the budget.
[basics]    "Qwen Model Architecture: From Transformer to MoE, What Developers
            Should Understand" (exaiv.com), section "Attention: what the model
            is 'looking at'": dot-product relevance of Q against K, then a
            relevance-weighted sum of V.

Readings taken where the pages are silent (each restated where it is used):

* compression is the arithmetic mean of the raw keys of each aligned,
  complete block ``[c*Bs, (c+1)*Bs)``; there is no learned projection;
* the candidates of a query at absolute position ``p`` are the complete
  blocks strictly before its own block ``i = p // Bs``;
* a candidate's score is ``scale * sum_j <q_j, kc>`` over the query heads
  ``j`` of the KV head's group (shared selection per token and KV head),
  with ``scale = 1/sqrt(d)`` unless given;
* ``top_k`` counts the query's own block, which is always kept; the other
  ``min(top_k - 1, i)`` slots go to the best-scoring candidates, equal
  scores going to the smaller block index;
* optional ``keep_tail`` frame, the one behind the released configuration of
  [port] (visible width at most ``budget + ratio - 1`` with a budget of
  whole blocks): every complete block among the ``p + 1`` cached positions
  is a candidate, the own block included once it is complete, and only the
  positions not yet in a complete block are always visible; their block
  takes one of the ``top_k`` slots when it is not empty (so ``top_k >= 2``);
* the selection is reported as ascending block ids padded with -1;
* attention is exact softmax attention with the same scale over the keys of
  the selected complete blocks plus positions ``i*Bs .. p`` of the own block.

Every function here has an independent pin in the CPU test-suite (brute
force, dense causal attention from the library, closed forms, Hadamard
invariance, planted blocks, block size 1, the pages' printed regime).
"""
from __future__ import annotations

import math

import numpy as np


def default_scale(head_dim: int) -> float:
    return 1.0 / math.sqrt(head_dim)


def compress_keys(K: np.ndarray, block_size: int) -> np.ndarray:
    """Mean of every complete aligned block of keys ([overview] §1, [port] address selection).

    ``K``: ``[..., N, d]``. Returns float64 ``[..., N // block_size, d]``
    whose row ``c`` is the mean of keys ``c*Bs .. c*Bs+Bs-1``. A trailing
    partial block is not compressed.
    """
    K = np.asarray(K)
    n_blocks = K.shape[-2] // block_size
    out = np.zeros(K.shape[:-2] + (n_blocks, K.shape[-1]), dtype=np.float64)
    for c in range(n_blocks):
        block = K[..., c * block_size:(c + 1) * block_size, :].astype(np.float64)
        out[..., c, :] = block.sum(axis=-2) / block_size
    return out


def block_scores(q_group: np.ndarray, k_comp: np.ndarray, n_candidates: int, scale: float) -> np.ndarray:
    """Relevance of candidate blocks ``0 .. n_candidates-1`` for one token and KV head.

    ``q_group``: ``[G, d]``, the query heads that share the KV head.
    ``k_comp``: ``[n_blocks, d]``. Each head's dot products with the
    compressed keys are computed separately and then added ([basics] Q/K dot
    product; the per-group sum is the shared-selection reading).
    """
    q_group = np.asarray(q_group, dtype=np.float64)
    kc = np.asarray(k_comp[:n_candidates], dtype=np.float64)
    total = np.zeros(n_candidates, dtype=np.float64)
    for j in range(q_group.shape[0]):
        total += kc @ q_group[j]
    return scale * total


def selection_frame(p: int, block_size: int, keep_tail: bool = False) -> tuple[int, int | None]:
    """``(n_candidates, forced)`` for a query at absolute position ``p``.

    Default: the candidates are the complete blocks ``0 .. i-1`` before the
    own block ``i = p // Bs`` and block ``i`` is always kept.
    ``keep_tail`` ([port], released budget and the bound
    ``min(n_kv, budget + ratio - 1)``): the candidates are all
    ``(p + 1) // Bs`` complete blocks; the block holding the positions past
    the last complete block is always kept when there are such positions,
    else nothing is forced.
    """
    if not keep_tail:
        own = p // block_size
        return own, own
    n_complete = (p + 1) // block_size
    return n_complete, (n_complete if (p + 1) % block_size else None)


def select_in_frame(scores: np.ndarray, n_candidates: int, forced: int | None, top_k: int) -> list[int]:
    """Kept block ids for one token and KV head ([port] top-k selection -> cache-cell IDs).

    ``scores[c]`` for candidates ``c < n_candidates``. One of the ``top_k``
    slots is reserved for the forced block; ``min(top_k - 1, n_candidates)``
    slots take the best-scoring candidates (ties to the smaller id). Returns
    ``top_k`` ids, ascending, padded with -1.
    """
    if forced is None and top_k < 2:
        raise ValueError("a frame without a forced block needs top_k >= 2 (else nothing is visible)")
    slots = min(top_k - 1, n_candidates)
    ranked = sorted(range(n_candidates), key=lambda c: (-float(scores[c]), c))
    kept = sorted(ranked[:slots] + ([] if forced is None else [forced]))
    return kept + [-1] * (top_k - len(kept))


def select_blocks(scores: np.ndarray, own_block: int, top_k: int) -> list[int]:
    """Default frame: candidates ``c < own_block``, the own block always kept and counted in ``top_k``."""
    return select_in_frame(scores, own_block, own_block, top_k)


def visible_positions(selection, p: int, block_size: int) -> np.ndarray:
    """Absolute key positions one query at position ``p`` attends to.

    Complete selected blocks contribute all their positions; the own block
    contributes ``i*Bs .. p`` (causal inside the block), which is the whole
    block once ``p`` is its last position.
    """
    own = p // block_size
    positions: list[int] = []
    for c in selection:
        if c < 0:
            continue
        if c < own:
            positions.extend(range(c * block_size, (c + 1) * block_size))
        elif c == own:
            positions.extend(range(own * block_size, p + 1))
        else:
            raise ValueError(f"block {c} lies after the query's own block {own}")
    return np.array(sorted(positions), dtype=np.int64)


def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray, positions: np.ndarray, scale: float) -> np.ndarray:
    """Softmax attention of one query head over the given key positions ([basics]).

    ``q``: ``[d]``; ``K``, ``V``: ``[N, d]`` of the query's KV head.
    """
    q = np.asarray(q, dtype=np.float64)
    keys = np.asarray(K[positions], dtype=np.float64)
    vals = np.asarray(V[positions], dtype=np.float64)
    logits = scale * (keys @ q)
    weights = np.exp(logits - logits.max())
    return (weights @ vals) / weights.sum()


def attend_given_selection(q_group, K, V, selection, p, block_size, scale):
    """Outputs ``[G, d]`` of one token's query heads for a given (valid) selection."""
    pos = visible_positions(selection, p, block_size)
    return np.stack([attend(q_group[j], K, V, pos, scale) for j in range(q_group.shape[0])])


def qsa_rows(Q, K, V, block_size, top_k, scale=None, q_pos0=0, rows=None, k_comp=None, keep_tail=False):
    """QSA for every (sequence, query row, KV head) requested.

    ``Q``: ``[b][q_len][Hq][d]``; ``K``, ``V``: ``[b][Hkv][N][d]``; query row
    ``t`` sits at absolute position ``q_pos0 + t``. ``rows`` is an iterable
    of ``(b, t, g)`` (default: all). ``k_comp`` may pass precomputed
    compressed keys ``[b][Hkv][N//Bs][d]``. ``keep_tail`` picks the frame of
    :func:`selection_frame`.

    Returns a dict ``(b, t, g) -> (selection, scores, out[G][d])`` where
    ``scores`` are the float64 candidate scores of that row.
    """
    b_n, q_len, n_q, d = Q.shape
    n_kv = K.shape[1]
    G = n_q // n_kv
    if scale is None or scale == 0:
        scale = default_scale(d)
    if k_comp is None:
        k_comp = compress_keys(K, block_size)
    if rows is None:
        rows = [(b, t, g) for b in range(b_n) for t in range(q_len) for g in range(n_kv)]
    result = {}
    for b, t, g in rows:
        p = q_pos0 + t
        n_cand, forced = selection_frame(p, block_size, keep_tail)
        q_group = Q[b, t, g * G:(g + 1) * G, :].astype(np.float64)
        scores = block_scores(q_group, k_comp[b, g], n_cand, scale)
        sel = select_in_frame(scores, n_cand, forced, top_k)
        out = attend_given_selection(q_group, K[b, g], V[b, g], sel, p, block_size, scale)
        result[(b, t, g)] = (sel, scores, out)
    return result


def qsa_prefill(Q, K, V, block_size, top_k, scale=None, q_pos0=0, keep_tail=False):
    """Causal QSA prefill: returns (out float64 ``[b][q_len][Hq][d]``, sel int32 ``[b][q_len][Hkv][k]``)."""
    b_n, q_len, n_q, d = Q.shape
    n_kv = K.shape[1]
    G = n_q // n_kv
    res = qsa_rows(Q, K, V, block_size, top_k, scale, q_pos0, keep_tail=keep_tail)
    out = np.zeros((b_n, q_len, n_q, d), dtype=np.float64)
    sel = np.zeros((b_n, q_len, n_kv, top_k), dtype=np.int32)
    for (b, t, g), (s, _, o) in res.items():
        sel[b, t, g] = s
        out[b, t, g * G:(g + 1) * G] = o
    return out, sel


def qsa_decode(q, K, V, kv_len, block_size, top_k, scale=None, keep_tail=False):
    """One decode step: ``q`` ``[b][Hq][d]`` at position ``kv_len-1`` over the first ``kv_len`` cached keys.

    Returns (out float64 ``[b][Hq][d]``, sel int32 ``[b][Hkv][k]``).
    """
    out, sel = qsa_prefill(q[:, None], K[:, :, :kv_len], V[:, :, :kv_len], block_size, top_k, scale,
                           q_pos0=kv_len - 1, keep_tail=keep_tail)
    return out[:, 0], sel[:, 0]
