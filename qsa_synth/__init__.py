"""Seeded synthetic inputs for Qwen Sparse Attention (QSA) workloads.

This module is shared by the tests, the benchmark and the oracle checks. It
only draws random tensors and rounds them to the storage type; it performs
none of the attention method's arithmetic (no compression, scoring,
selection or softmax).

Recipe (one independent stream per tensor slice, so any slice can be
regenerated on its own):

* ``numpy.random.Generator(PCG64(SeedSequence([seed, cfg_id, tensor_id, *slice])))``
  with tensor ids Q=0, K=1, V=2, planted-block choice=3; Q slices are per
  sequence ``b``, K and V slices per ``(b, kv_head)``.
* Values are float32 standard normals times ``sigma`` (1.0 or 0.5, both
  exact in binary), rounded once to bfloat16 with round-to-nearest-even for
  the bf16 workloads.
* A ragged decode workload gives sequence ``b`` the length
  ``seq_lengths(w, seed)[b]``: integers drawn uniformly from
  ``[kv_len/8, kv_len]`` (tensor id 4), the last one set to ``kv_len``; the
  inputs are generated for ``kv_len`` positions and a sequence reads only
  its first ``length`` of them.
* A prefill workload with ``q_rows`` set has query rows only for the last
  ``q_rows`` positions (a prefill chunk at the end of a long context); K and
  V still cover every position.
* The planted workload (batched decode) shifts every key of 8 chosen
  complete blocks per ``(b, kv_head)`` by ``2*sigma`` along the unit vector
  of the sum of that KV head's query heads (bf16-rounded), in float32 before
  rounding, so the shifted blocks stand out against the noise keys.

Layouts match the C ABI: Q ``[b][q_len][Hq][d]``, K/V ``[b][Hkv][kv][d]``.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ProcessPoolExecutor

import numpy as np

TENSOR_Q, TENSOR_K, TENSOR_V, TENSOR_PLANT, TENSOR_LEN, TENSOR_WQ, TENSOR_WK = 0, 1, 2, 3, 4, 5, 6


@dataclasses.dataclass(frozen=True)
class Workload:
    """One QSA workload: shapes, dtype and value distribution."""

    name: str
    cfg_id: int
    mode: str  # "prefill" (q_len tokens from position 0) or "decode" (one token at kv_len-1)
    batch: int
    kv_len: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    block_size: int
    top_k: int
    dtype: str  # "f32" or "bf16"
    sigma: float
    planted: int = 0
    keep_tail: bool = False  # selection frame of the released budget (see the oracle)
    ragged: bool = False  # decode: every sequence has its own length (see seq_lengths)
    indexer_dim: int = 0  # learned-indexer selection: indexer dimension (0 = the default selection)
    indexer_agg: int = 0  # its aggregation of a group's head scores: 0 sum, 1 max, 2 softmax
    kv_q8: bool = False   # decode attention over the rotated 8-bit K/V cache
    q_rows: int = 0       # prefill: only the last q_rows positions are query rows (0 = every position)

    @property
    def q_len(self) -> int:
        if self.mode != "prefill":
            return 1
        return self.q_rows if self.q_rows else self.kv_len

    @property
    def q_pos0(self) -> int:
        return self.kv_len - self.q_len

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads: tiny fp32 prefill, bf16 decode at 32K, bf16 prefill at
# 8K, batched bf16 decode at 128K with planted blocks, bf16 decode at 1M; then
# a ragged batched decode and bf16 decode in the released budget regime at 256K.
WORKLOADS = {
    "prefill_512_f32": Workload("prefill_512_f32", 1, "prefill", 1, 512, 2, 1, 64, 32, 4, "f32", 1.0),
    "decode_32k": Workload("decode_32k", 2, "decode", 1, 32768, 16, 2, 128, 64, 16, "bf16", 0.5),
    "prefill_8k": Workload("prefill_8k", 3, "prefill", 1, 8192, 16, 2, 128, 64, 16, "bf16", 0.5),
    "decode_b64_128k": Workload("decode_b64_128k", 4, "decode", 64, 131072, 16, 2, 128, 64, 16, "bf16", 0.5, planted=8),
    "decode_1m": Workload("decode_1m", 5, "decode", 1, 1048576, 16, 2, 128, 64, 32, "bf16", 0.5),
    # the 32K decode with a learned indexer (64 dimensions, max over the heads)
    "decode_32k_indexer": Workload("decode_32k_indexer", 8, "decode", 1, 32768, 16, 2, 128, 64, 16, "bf16", 0.5,
                                   indexer_dim=64, indexer_agg=1),
    # the batched decode with the attention reading a rotated 8-bit K/V cache
    "decode_b64_128k_q8": Workload("decode_b64_128k_q8", 9, "decode", 64, 131072, 16, 2, 128, 64, 16, "bf16", 0.5,
                                   planted=8, kv_q8=True),
    # a ragged batch: 64 sequences of 16K .. 128K tokens
    "decode_b64_ragged": Workload("decode_b64_ragged", 7, "decode", 64, 131072, 16, 2, 128, 64, 16, "bf16", 0.5,
                                  ragged=True),
    # the released budget regime: ratio 4, 2048-token budget (512 blocks + the
    # partial-tail slot), 262144-token context = 65536 compressed blocks
    "decode_256k_r4": Workload("decode_256k_r4", 6, "decode", 1, 262144, 16, 2, 128, 4, 513, "bf16", 0.5,
                               keep_tail=True),
    # the same regime for a prefill chunk: the last 512 query rows of a
    # 262144-token context (every row scores 65536 candidates)
    "prefill_256k_r4_tail": Workload("prefill_256k_r4_tail", 10, "prefill", 1, 262144, 16, 2, 128, 4, 513, "bf16",
                                     0.5, keep_tail=True, q_rows=512),
}


def _rng(seed: int, cfg_id: int, tensor_id: int, *slice_ids: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, cfg_id, tensor_id, *slice_ids])))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even); returns uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _store(x32: np.ndarray, dtype: str) -> np.ndarray:
    """Round to the storage dtype; returns float32 values exactly representable in it."""
    if dtype == "bf16":
        return bf16_bits_to_f32(f32_to_bf16_bits(x32))
    if dtype == "f32":
        return x32
    raise ValueError(dtype)


def gen_q(w: Workload, seed: int, b: int) -> np.ndarray:
    """Queries of sequence b, ``[q_len][Hq][d]`` float32 (values exact in ``w.dtype``)."""
    x = _rng(seed, w.cfg_id, TENSOR_Q, b).standard_normal((w.q_len, w.n_q_heads, w.head_dim), dtype=np.float32)
    return _store(x * np.float32(w.sigma), w.dtype)


def seq_lengths(w: Workload, seed: int) -> list[int]:
    """Per-sequence lengths of a decode workload (all ``kv_len`` unless ``w.ragged``)."""
    if not w.ragged:
        return [w.kv_len] * w.batch
    lo = max(1, w.kv_len // 8)
    n = _rng(seed, w.cfg_id, TENSOR_LEN).integers(lo, w.kv_len + 1, size=w.batch)
    n[-1] = w.kv_len
    return [int(x) for x in n]


def indexer_weights(seed: int, cfg_id: int, d: int, d_idx: int) -> tuple[np.ndarray, np.ndarray]:
    """Synthetic indexer projections ``(W_q, W_k)``, each ``[d][d_idx]`` float32: standard normals
    divided by ``sqrt(d)`` (tensor ids 5 and 6), so projected values keep the inputs' scale."""
    s = np.float32(1.0 / np.sqrt(d))
    w_q = _rng(seed, cfg_id, TENSOR_WQ).standard_normal((d, d_idx), dtype=np.float32) * s
    w_k = _rng(seed, cfg_id, TENSOR_WK).standard_normal((d, d_idx), dtype=np.float32) * s
    return w_q, w_k


def planted_blocks(w: Workload, seed: int, b: int, g: int) -> np.ndarray:
    """The complete blocks whose keys are shifted for ``(b, g)``: distinct, before the query's own block."""
    if not w.planted:
        return np.zeros(0, dtype=np.int64)
    own = (w.kv_len - 1) // w.block_size
    if own < w.planted:
        raise ValueError("not enough complete blocks to plant into")
    return np.sort(_rng(seed, w.cfg_id, TENSOR_PLANT, b, g).choice(own, size=w.planted, replace=False))


def gen_kv(w: Workload, seed: int, tensor_id: int, b: int, g: int, q_b: np.ndarray | None = None) -> np.ndarray:
    """Keys (tensor_id=1) or values (2) of ``(b, g)``: ``[kv_len][d]`` float32 exact in ``w.dtype``.

    For planted workloads the keys need the sequence's queries ``q_b``
    (``[q_len][Hq][d]``, as returned by :func:`gen_q`); the shift direction is
    the normalised sum of KV head ``g``'s query heads at the last query row.
    """
    x = _rng(seed, w.cfg_id, tensor_id, b, g).standard_normal((w.kv_len, w.head_dim), dtype=np.float32)
    x *= np.float32(w.sigma)
    if tensor_id == TENSOR_K and w.planted:
        if q_b is None:
            q_b = gen_q(w, seed, b)
        G = w.group
        direction = q_b[-1, g * G:(g + 1) * G, :].astype(np.float64).sum(axis=0)
        direction /= np.linalg.norm(direction)
        shift = 2.0 * w.sigma * direction
        for c in planted_blocks(w, seed, b, g):
            rows = slice(c * w.block_size, (c + 1) * w.block_size)
            x[rows] = (x[rows].astype(np.float64) + shift).astype(np.float32)
    return _store(x, w.dtype)


def _kv_job(args):
    w, seed, tensor_id, b, g, shm_name, shape = args
    from multiprocessing import shared_memory

    shm = shared_memory.SharedMemory(name=shm_name)
    try:
        out = np.ndarray(shape, dtype=np.uint16 if w.dtype == "bf16" else np.float32, buffer=shm.buf)
        x = gen_kv(w, seed, tensor_id, b, g)
        out[b, g] = f32_to_bf16_bits(x) if w.dtype == "bf16" else x
    finally:
        shm.close()
    return b, g


def gen_all(w: Workload, seed: int = 0, workers: int | None = None):
    """Whole-workload inputs as storage arrays: (Q, K, V).

    bf16 workloads come back as uint16 bit patterns, fp32 ones as float32.
    Large K/V tensors are filled in parallel worker processes (one slice per
    ``(b, g)``); the result does not depend on the worker count.
    """
    store = np.uint16 if w.dtype == "bf16" else np.float32
    Q = np.stack([gen_q(w, seed, b) for b in range(w.batch)])
    Qs = f32_to_bf16_bits(Q) if w.dtype == "bf16" else Q
    shape = (w.batch, w.n_kv_heads, w.kv_len, w.head_dim)
    nbytes = int(np.prod(shape)) * np.dtype(store).itemsize
    jobs = w.batch * w.n_kv_heads
    if workers is None:
        workers = min(16, len(os.sched_getaffinity(0)))
    if nbytes < (64 << 20) or workers <= 1 or jobs == 1:
        K = np.empty(shape, dtype=store)
        V = np.empty(shape, dtype=store)
        for b in range(w.batch):
            for g in range(w.n_kv_heads):
                k = gen_kv(w, seed, TENSOR_K, b, g, Q[b])
                v = gen_kv(w, seed, TENSOR_V, b, g)
                K[b, g] = f32_to_bf16_bits(k) if w.dtype == "bf16" else k
                V[b, g] = f32_to_bf16_bits(v) if w.dtype == "bf16" else v
        return Qs, K, V
    from multiprocessing import shared_memory

    outs = []
    with ProcessPoolExecutor(max_workers=min(workers, jobs)) as ex:
        for tid in (TENSOR_K, TENSOR_V):
            shm = shared_memory.SharedMemory(create=True, size=nbytes)
            try:
                list(ex.map(_kv_job, [(w, seed, tid, b, g, shm.name, shape)
                                      for b in range(w.batch) for g in range(w.n_kv_heads)]))
                arr = np.ndarray(shape, dtype=store, buffer=shm.buf).copy()
            finally:
                shm.close()
                shm.unlink()
            outs.append(arr)
    return Qs, outs[0], outs[1]


def as_f32(x: np.ndarray, dtype: str) -> np.ndarray:
    """Storage array (uint16 bf16 bits or float32) -> float32 values."""
    return bf16_bits_to_f32(x) if dtype == "bf16" else np.asarray(x, dtype=np.float32)
