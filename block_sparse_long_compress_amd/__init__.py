"""Qwen Sparse Attention (QSA) for AMD MI355X (gfx950).

Keys are mean-pooled into one compressed key per block, every (token, KV
head) scores the compressed blocks and keeps its top-k (the always-kept block included),
and exact softmax attention runs over the kept blocks only. All steps run in
the hand-written HIP kernels of ``lib/libqsa.so`` behind the C ABI of
``include/qsa.h``; this package is the Python binding (argument marshalling)
plus two convenience pipelines that chain the ABI calls.
"""
from __future__ import annotations

import torch

from .binding import (  # noqa: F401
    EXPORTED,
    LIB,
    LIB_PATH,
    QSA_AGG_MAX,
    QSA_AGG_SOFTMAX,
    QSA_AGG_SUM,
    QSA_BF16,
    QSA_F32,
    QSA_OP_COMPRESS,
    QSA_OP_DECODE,
    QSA_OP_DECODE_STEP,
    QSA_OP_DECODE_STEP_RAGGED,
    QSA_OP_INDEXER_SELECT,
    QSA_OP_PREFILL_Q8,
    QSA_OP_SELECT_RAGGED,
    QSA_OP_PREFILL,
    QSA_OP_SELECT,
    QsaError,
    QsaIndexer,
    QsaShape,
    abi_version,
    make_indexer,
    make_shape,
    qsa_compress_keys,
    qsa_decode_step,
    qsa_decode_step_fused,
    qsa_decode_step_noalloc,
    QSA_NOALLOC_SCRATCH_BYTES,
    qsa_decode_step_ragged,
    qsa_indexer_decode_step,
    qsa_indexer_keys,
    qsa_indexer_select,
    qsa_kv_quantize,
    qsa_sparse_attn_decode_q8,
    qsa_sparse_attn_prefill_q8,
    qsa_decode_step_q8,
    kv_q8_buffers,
    qsa_score_select,
    qsa_score_select_ragged,
    qsa_sparse_attn_decode_ragged,
    qsa_sparse_attn_decode,
    qsa_sparse_attn_prefill,
    qsa_workspace_bytes,
    status_str,
    workspace,
)


def shape_for(q: torch.Tensor, k: torch.Tensor, block_size: int, top_k: int, scale: float = 0.0,
              keep_tail: bool = False) -> QsaShape:
    """ABI shape from Q ``[b][q_len][Hq][d]`` (or ``[b][Hq][d]``) and K ``[b][Hkv][cap][d]``."""
    return make_shape(k.shape[0], q.shape[-2], k.shape[1], k.shape[3], block_size, top_k, q.dtype, scale, keep_tail)


def prefill(q, k, v, block_size, top_k, q_pos0=0, scale=0.0, k_comp=None, with_scores=False, keep_tail=False):
    """Compress, select and attend for ``q_len`` query rows at positions ``q_pos0 ..``.

    Returns ``(out, sel, k_comp[, sel_scores])``; ``k_comp`` is computed for
    every complete block below ``q_pos0 + q_len`` unless given.
    """
    b, q_len, hq, d = q.shape
    hkv, cap = k.shape[1], k.shape[2]
    kv_len = q_pos0 + q_len
    shape = shape_for(q, k, block_size, top_k, scale, keep_tail)
    if k_comp is None:
        k_comp = torch.empty(b, hkv, cap // block_size, d, dtype=torch.float32, device=q.device)
        qsa_compress_keys(shape, k, kv_len, k_comp)
    sel = torch.empty(b, q_len, hkv, top_k, dtype=torch.int32, device=q.device)
    scores = torch.empty(b, q_len, hkv, top_k, dtype=torch.float32, device=q.device) if with_scores else None
    qsa_score_select(shape, q, q_pos0, k_comp, kv_len, cap, sel, scores)
    out = torch.empty_like(q)
    qsa_sparse_attn_prefill(shape, q, k, v, q_pos0, sel, out)
    return (out, sel, k_comp, scores) if with_scores else (out, sel, k_comp)


def decode(q, k, v, kv_len, block_size, top_k, k_comp, scale=0.0, with_scores=False, keep_tail=False):
    """One decode step for ``q`` ``[b][Hq][d]`` at position ``kv_len - 1`` given compressed keys.

    Returns ``(out, sel[, sel_scores])`` with ``sel`` ``[b][Hkv][k]``.
    """
    b, hq, d = q.shape
    hkv, cap = k.shape[1], k.shape[2]
    shape = shape_for(q, k, block_size, top_k, scale, keep_tail)
    sel = torch.empty(b, hkv, top_k, dtype=torch.int32, device=q.device)
    scores = torch.empty(b, hkv, top_k, dtype=torch.float32, device=q.device) if with_scores else None
    qsa_score_select(shape, q.view(b, 1, hq, d), kv_len - 1, k_comp, kv_len, cap, sel, scores)
    out = torch.empty_like(q)
    qsa_sparse_attn_decode(shape, q, k, v, kv_len, sel, out)
    return (out, sel, scores) if with_scores else (out, sel)
