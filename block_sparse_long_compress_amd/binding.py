"""ctypes binding of the QSA C ABI (``include/qsa.h``).

Argument marshalling only: torch tensors supply device pointers, sizes come
from their shapes, and work is enqueued on torch's current stream of the
tensors' device. Every step of the computation runs in the HIP kernels of
``lib/libqsa.so``; there is no fallback. The library must have been built
(``python -m block_sparse_long_compress_amd.build``); importing this module
without it raises immediately.
"""
from __future__ import annotations

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("QSA_LIB", os.path.join(HERE, "lib", "libqsa.so"))

QSA_F32, QSA_BF16 = 0, 1
QSA_OP_COMPRESS, QSA_OP_SELECT, QSA_OP_DECODE, QSA_OP_PREFILL, QSA_OP_DECODE_STEP = 0, 1, 2, 3, 4
QSA_OP_DECODE_STEP_RAGGED = 5
QSA_OP_INDEXER_SELECT = 6
QSA_OP_PREFILL_Q8 = 7
QSA_OP_SELECT_RAGGED = 8
QSA_AGG_SUM, QSA_AGG_MAX, QSA_AGG_SOFTMAX = 0, 1, 2
STATUS = {0: "QSA_OK", 1: "QSA_ERR_INVALID", 2: "QSA_ERR_UNSUPPORTED", 3: "QSA_ERR_WORKSPACE", 4: "QSA_ERR_HIP"}
EXPORTED = ("qsa_abi_version", "qsa_status_str", "qsa_workspace_bytes", "qsa_compress_keys", "qsa_score_select",
            "qsa_sparse_attn_decode", "qsa_sparse_attn_prefill", "qsa_decode_step", "qsa_decode_step_fused",
            "qsa_decode_step_ragged", "qsa_indexer_keys", "qsa_indexer_select", "qsa_kv_quantize",
            "qsa_sparse_attn_decode_q8", "qsa_sparse_attn_prefill_q8", "qsa_decode_step_q8",
            "qsa_decode_step_noalloc", "qsa_indexer_decode_step", "qsa_score_select_ragged",
            "qsa_sparse_attn_decode_ragged")
QSA_NOALLOC_SCRATCH_BYTES = 8 << 20  # include/qsa.h


class QsaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)}")


class QsaShape(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("n_q_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("top_k", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("keep_tail", ctypes.c_int32),
    ]


class QsaIndexer(ctypes.Structure):
    _fields_ = [("dim", ctypes.c_int32), ("agg", ctypes.c_int32), ("scale", ctypes.c_float)]


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"QSA HIP library not built: {LIB_PATH} is missing "
                          "(run python -m block_sparse_long_compress_amd.build)")
    lib = ctypes.CDLL(LIB_PATH)
    P, I64, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t
    SH = ctypes.POINTER(QsaShape)
    lib.qsa_abi_version.restype = ctypes.c_int
    lib.qsa_abi_version.argtypes = []
    lib.qsa_status_str.restype = ctypes.c_char_p
    lib.qsa_status_str.argtypes = [ctypes.c_int]
    lib.qsa_workspace_bytes.restype = SZ
    lib.qsa_workspace_bytes.argtypes = [SH, ctypes.c_int, I64, I64]
    lib.qsa_compress_keys.restype = ctypes.c_int
    lib.qsa_compress_keys.argtypes = [SH, P, I64, I64, I64, P, P]
    lib.qsa_score_select.restype = ctypes.c_int
    lib.qsa_score_select.argtypes = [SH, P, I64, I64, P, I64, I64, P, P, P, SZ, P]
    lib.qsa_sparse_attn_decode.restype = ctypes.c_int
    lib.qsa_sparse_attn_decode.argtypes = [SH, P, P, P, I64, I64, P, P, P, SZ, P]
    lib.qsa_sparse_attn_prefill.restype = ctypes.c_int
    lib.qsa_sparse_attn_prefill.argtypes = [SH, P, P, P, I64, I64, I64, P, P, P, SZ, P]
    lib.qsa_decode_step.restype = ctypes.c_int
    lib.qsa_decode_step.argtypes = [SH, P, P, P, P, I64, I64, P, P, P, P, SZ, P]
    lib.qsa_decode_step_fused.restype = ctypes.c_int
    lib.qsa_decode_step_fused.argtypes = [SH, I64]
    lib.qsa_decode_step_ragged.restype = ctypes.c_int
    lib.qsa_decode_step_ragged.argtypes = [SH, P, P, P, P, P, I64, I64, P, P, P, P, SZ, P]
    lib.qsa_score_select_ragged.restype = ctypes.c_int
    lib.qsa_score_select_ragged.argtypes = [SH, P, P, P, I64, I64, P, P, P, SZ, P]
    lib.qsa_sparse_attn_decode_ragged.restype = ctypes.c_int
    lib.qsa_sparse_attn_decode_ragged.argtypes = [SH, P, P, P, P, I64, I64, P, P, P, SZ, P]
    IX = ctypes.POINTER(QsaIndexer)
    lib.qsa_indexer_keys.restype = ctypes.c_int
    lib.qsa_indexer_keys.argtypes = [SH, IX, P, P, I64, I64, I64, P, P]
    lib.qsa_indexer_select.restype = ctypes.c_int
    lib.qsa_indexer_select.argtypes = [SH, IX, P, P, I64, I64, P, I64, I64, P, P, P, SZ, P]
    lib.qsa_indexer_decode_step.restype = ctypes.c_int
    lib.qsa_indexer_decode_step.argtypes = [SH, IX, P, P, P, P, P, P, P, I64, I64, P, P, P, P]
    lib.qsa_kv_quantize.restype = ctypes.c_int
    lib.qsa_kv_quantize.argtypes = [SH, P, P, I64, I64, I64, P, P, P, P, P]
    lib.qsa_sparse_attn_decode_q8.restype = ctypes.c_int
    lib.qsa_sparse_attn_decode_q8.argtypes = [SH, P, P, P, P, P, I64, I64, P, P, P, SZ, P]
    lib.qsa_sparse_attn_prefill_q8.restype = ctypes.c_int
    lib.qsa_sparse_attn_prefill_q8.argtypes = [SH, P, P, P, P, P, I64, I64, I64, P, P, P, SZ, P]
    lib.qsa_decode_step_q8.restype = ctypes.c_int
    lib.qsa_decode_step_q8.argtypes = [SH, P, P, P, P, P, P, P, P, I64, I64, P, P, P, P, SZ, P]
    lib.qsa_decode_step_noalloc.restype = ctypes.c_int
    lib.qsa_decode_step_noalloc.argtypes = [SH, P, P, P, P, I64, I64, P, P, P, P]
    return lib


LIB = _load()


def make_shape(batch, n_q_heads, n_kv_heads, head_dim, block_size, top_k, dtype, scale=0.0,
               keep_tail=False) -> QsaShape:
    """Build the ABI shape struct; ``dtype`` is a torch dtype or QSA_F32/QSA_BF16."""
    if isinstance(dtype, torch.dtype):
        dtype = {torch.float32: QSA_F32, torch.bfloat16: QSA_BF16}[dtype]
    return QsaShape(batch, n_q_heads, n_kv_heads, head_dim, block_size, top_k, dtype, float(scale), int(keep_tail))


def abi_version() -> int:
    return LIB.qsa_abi_version()


def status_str(status: int) -> str:
    return LIB.qsa_status_str(status).decode()


def qsa_workspace_bytes(shape: QsaShape, op: int, q_len: int, kv_len: int) -> int:
    n = LIB.qsa_workspace_bytes(ctypes.byref(shape), op, q_len, kv_len)
    if n == ctypes.c_size_t(-1).value:
        raise QsaError(1, "qsa_workspace_bytes")
    return n


def _ptr(t):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError("tensors must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(t, stream):
    if stream is not None:
        return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def workspace(shape: QsaShape, op: int, q_len: int, kv_len: int, device) -> torch.Tensor | None:
    """A zero-filled workspace for these sizes, ready for its first call and reusable afterwards."""
    need = qsa_workspace_bytes(shape, op, q_len, kv_len)
    if need == 0:
        return None
    return torch.zeros(need, dtype=torch.uint8, device=device)


def _workspace(shape, op, q_len, kv_len, ws, device):
    if ws is None:
        ws = workspace(shape, op, q_len, kv_len, device)
    return ws, (ws.numel() * ws.element_size() if ws is not None else 0)


def _check(status: int, where: str):
    if status != 0:
        raise QsaError(status, where)


def qsa_compress_keys(shape: QsaShape, k, kv_len: int, k_comp, block_begin: int = 0, stream=None):
    """Mean-pool complete key blocks ``block_begin .. kv_len//Bs - 1`` into ``k_comp`` (float32)."""
    _check(LIB.qsa_compress_keys(ctypes.byref(shape), _ptr(k), kv_len, k.shape[2], block_begin, _ptr(k_comp),
                                 _stream(k, stream)), "qsa_compress_keys")
    return k_comp


def qsa_score_select(shape: QsaShape, q, q_pos0: int, k_comp, kv_len: int, kv_cap: int, sel, sel_scores=None,
                     ws=None, stream=None):
    """Score compressed blocks and write the kept block ids of every (token, KV head) into ``sel``."""
    q_len = q.shape[1]
    ws, nbytes = _workspace(shape, QSA_OP_SELECT, q_len, kv_len, ws, q.device)
    _check(LIB.qsa_score_select(ctypes.byref(shape), _ptr(q), q_len, q_pos0, _ptr(k_comp), kv_len, kv_cap, _ptr(sel),
                                _ptr(sel_scores), _ptr(ws), nbytes, _stream(q, stream)), "qsa_score_select")
    return sel


def qsa_sparse_attn_decode(shape: QsaShape, q, k, v, kv_len: int, sel, out, ws=None, stream=None):
    """Attention of one token per sequence (``q`` ``[b][Hq][d]``) over its selected blocks."""
    ws, nbytes = _workspace(shape, QSA_OP_DECODE, 1, kv_len, ws, q.device)
    _check(LIB.qsa_sparse_attn_decode(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), kv_len, k.shape[2], _ptr(sel),
                                      _ptr(out), _ptr(ws), nbytes, _stream(q, stream)), "qsa_sparse_attn_decode")
    return out


def qsa_sparse_attn_prefill(shape: QsaShape, q, k, v, q_pos0: int, sel, out, ws=None, stream=None):
    """Causal attention of ``q_len`` tokens (``q`` ``[b][q_len][Hq][d]``) over their selected blocks."""
    q_len = q.shape[1]
    ws, nbytes = _workspace(shape, QSA_OP_PREFILL, q_len, q_pos0 + q_len, ws, q.device)
    _check(LIB.qsa_sparse_attn_prefill(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), q_len, q_pos0, k.shape[2],
                                       _ptr(sel), _ptr(out), _ptr(ws), nbytes, _stream(q, stream)),
           "qsa_sparse_attn_prefill")
    return out


def qsa_decode_step(shape: QsaShape, q, k, v, k_comp, kv_len: int, sel, out, sel_scores=None, ws=None, stream=None):
    """One decode step for ``q`` ``[b][Hq][d]`` at position ``kv_len - 1``: compress the block it completes
    (into ``k_comp``), select (``sel`` ``[b][Hkv][k]``) and attend (``out``)."""
    ws, nbytes = _workspace(shape, QSA_OP_DECODE_STEP, 1, kv_len, ws, q.device)
    _check(LIB.qsa_decode_step(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(k_comp), kv_len, k.shape[2],
                               _ptr(sel), _ptr(sel_scores), _ptr(out), _ptr(ws), nbytes, _stream(q, stream)),
           "qsa_decode_step")
    return out


def qsa_decode_step_noalloc(shape: QsaShape, q, k, v, k_comp, kv_len: int, sel, out, sel_scores=None,
                            stream=None):
    """``qsa_decode_step`` with its workspace in the library's own device memory: nothing is allocated
    (not even here), for callers that cannot allocate. Calls that may overlap on one GPU race."""
    _check(LIB.qsa_decode_step_noalloc(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(k_comp), kv_len,
                                       k.shape[2], _ptr(sel), _ptr(sel_scores), _ptr(out), _stream(q, stream)),
           "qsa_decode_step_noalloc")
    return out


def _check_kv_lens(kv_lens, batch: int, name: str):
    if kv_lens.dtype != torch.int32 or not kv_lens.is_contiguous() or kv_lens.numel() != batch:
        raise QsaError(1, f"{name}: kv_lens must be a contiguous int32 tensor of length batch")


def qsa_score_select_ragged(shape: QsaShape, q, k_comp, kv_lens, max_kv_len: int, kv_cap: int, sel,
                            sel_scores=None, ws=None, stream=None):
    """The selection of a ragged decode batch: sequence ``b``'s token (``q`` ``[b][Hq][d]``) sits at position
    ``kv_lens[b] - 1``; ``sel`` ``[b][Hkv][k]``."""
    _check_kv_lens(kv_lens, q.shape[0], "qsa_score_select_ragged")
    if ws is None and LIB.qsa_workspace_bytes(ctypes.byref(shape), QSA_OP_SELECT_RAGGED, 1,
                                              max_kv_len) == ctypes.c_size_t(-1).value:
        nbytes = 0  # a shape the call does not serve: the call reports why
    else:
        ws, nbytes = _workspace(shape, QSA_OP_SELECT_RAGGED, 1, max_kv_len, ws, q.device)
    _check(LIB.qsa_score_select_ragged(ctypes.byref(shape), _ptr(q), _ptr(k_comp), _ptr(kv_lens), max_kv_len,
                                       kv_cap, _ptr(sel), _ptr(sel_scores), _ptr(ws), nbytes, _stream(q, stream)),
           "qsa_score_select_ragged")
    return sel


def qsa_sparse_attn_decode_ragged(shape: QsaShape, q, k, v, kv_lens, max_kv_len: int, sel, out, ws=None,
                                  stream=None):
    """The attention of a ragged decode batch: sequence ``b``'s token attends at position ``kv_lens[b] - 1``."""
    _check_kv_lens(kv_lens, q.shape[0], "qsa_sparse_attn_decode_ragged")
    ws, nbytes = _workspace(shape, QSA_OP_DECODE, 1, max_kv_len, ws, q.device)
    _check(LIB.qsa_sparse_attn_decode_ragged(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(kv_lens),
                                             max_kv_len, k.shape[2], _ptr(sel), _ptr(out), _ptr(ws), nbytes,
                                             _stream(q, stream)),
           "qsa_sparse_attn_decode_ragged")
    return out


def qsa_decode_step_ragged(shape: QsaShape, q, k, v, k_comp, kv_lens, max_kv_len: int, sel, out, sel_scores=None,
                           ws=None, stream=None):
    """One decode step for a ragged batch: sequence ``b``'s token sits at position ``kv_lens[b] - 1``
    (``kv_lens``: int32 device tensor ``[b]``, each at most ``max_kv_len``)."""
    if kv_lens.dtype != torch.int32 or not kv_lens.is_contiguous() or kv_lens.numel() != k.shape[0]:
        raise QsaError(1, "qsa_decode_step_ragged: kv_lens must be a contiguous int32 tensor of length batch")
    if ws is None and LIB.qsa_workspace_bytes(ctypes.byref(shape), QSA_OP_DECODE_STEP_RAGGED, 1,
                                              max_kv_len) == ctypes.c_size_t(-1).value:
        nbytes = 0  # a shape the ragged step does not serve: the call reports why
    else:
        ws, nbytes = _workspace(shape, QSA_OP_DECODE_STEP_RAGGED, 1, max_kv_len, ws, q.device)
    _check(LIB.qsa_decode_step_ragged(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(k_comp), _ptr(kv_lens),
                                      max_kv_len, k.shape[2], _ptr(sel), _ptr(sel_scores), _ptr(out), _ptr(ws),
                                      nbytes, _stream(q, stream)),
           "qsa_decode_step_ragged")
    return out


def qsa_decode_step_fused(shape: QsaShape, kv_len: int) -> bool:
    """Whether qsa_decode_step runs these sizes as one fused kernel."""
    r = LIB.qsa_decode_step_fused(ctypes.byref(shape), kv_len)
    if r < 0:
        raise QsaError(1, "qsa_decode_step_fused")
    return bool(r)


def make_indexer(dim: int, agg: int, scale: float = 0.0) -> QsaIndexer:
    """Indexer struct: dimension (64 or 128), QSA_AGG_* aggregation, scale (0 = 1/sqrt(dim))."""
    return QsaIndexer(dim, agg, float(scale))


def qsa_indexer_keys(shape: QsaShape, idx: QsaIndexer, w_k, k_comp, kv_len: int, kv_cap: int, k_idx,
                     block_begin: int = 0, stream=None):
    """Indexer keys of complete blocks ``block_begin .. kv_len//Bs - 1`` (``W_k^T`` times the compressed keys)."""
    _check(LIB.qsa_indexer_keys(ctypes.byref(shape), ctypes.byref(idx), _ptr(w_k), _ptr(k_comp), kv_len, kv_cap,
                                block_begin, _ptr(k_idx), _stream(k_comp, stream)),
           "qsa_indexer_keys")
    return k_idx


def qsa_indexer_select(shape: QsaShape, idx: QsaIndexer, w_q, q, q_pos0: int, k_idx, kv_len: int, kv_cap: int, sel,
                       sel_scores=None, ws=None, stream=None):
    """Selection scored in indexer space for ``q`` ``[b][q_len][Hq][d]`` rows at positions ``q_pos0 ..`` (a workspace
    only for top_k > 64)."""
    q_len = q.shape[1]
    ws, nbytes = _workspace(shape, QSA_OP_INDEXER_SELECT, q_len, kv_len, ws, q.device)
    _check(LIB.qsa_indexer_select(ctypes.byref(shape), ctypes.byref(idx), _ptr(w_q), _ptr(q), q_len, q_pos0,
                                  _ptr(k_idx), kv_len, kv_cap, _ptr(sel), _ptr(sel_scores), _ptr(ws), nbytes,
                                  _stream(q, stream)),
           "qsa_indexer_select")
    return sel


def qsa_indexer_decode_step(shape: QsaShape, idx: QsaIndexer, w_q, w_k, q, k, v, k_comp, k_idx, kv_len: int, sel, out,
                            sel_scores=None, stream=None):
    """One decode step with the learned indexer in one kernel: ``q`` ``[b][Hq][d]``, the caches ``[b][Hkv][cap][...]``
    (``k_comp`` and ``k_idx`` gain the block the token at ``kv_len - 1`` closes), ``sel`` ``[b][Hkv][k]``, ``out``
    ``[b][Hq][d]``."""
    _check(LIB.qsa_indexer_decode_step(ctypes.byref(shape), ctypes.byref(idx), _ptr(w_q), _ptr(w_k), _ptr(q), _ptr(k),
                                       _ptr(v), _ptr(k_comp), _ptr(k_idx), kv_len, k.shape[2], _ptr(sel),
                                       _ptr(sel_scores), _ptr(out), _stream(q, stream)),
           "qsa_indexer_decode_step")
    return out


def kv_q8_buffers(k, device=None):
    """Empty 8-bit cache buffers shaped for bf16 ``k`` ``[b][Hkv][cap][d]``: (k_q, v_q, k_scales, v_scales)."""
    b, hkv, cap, d = k.shape
    device = device or k.device
    codes = [torch.empty(b, hkv, cap, d, dtype=torch.int8, device=device) for _ in range(2)]
    scales = [torch.empty(b, hkv, cap, d // 32, dtype=torch.int16, device=device) for _ in range(2)]
    return codes[0], codes[1], scales[0], scales[1]


def qsa_kv_quantize(shape: QsaShape, k, v, kv_len: int, k_q, v_q, k_scales, v_scales, pos_begin: int = 0,
                    stream=None):
    """Rotate and quantize positions ``pos_begin .. kv_len-1`` of K and V into the 8-bit cache."""
    _check(LIB.qsa_kv_quantize(ctypes.byref(shape), _ptr(k), _ptr(v), kv_len, k.shape[2], pos_begin, _ptr(k_q),
                               _ptr(v_q), _ptr(k_scales), _ptr(v_scales), _stream(k, stream)), "qsa_kv_quantize")


def qsa_sparse_attn_decode_q8(shape: QsaShape, q, k_q, v_q, k_scales, v_scales, kv_len: int, sel, out, ws=None,
                              stream=None):
    """Decode attention over the rotated 8-bit cache (``q`` ``[b][Hq][d]``, ``sel`` ``[b][Hkv][k]``)."""
    ws, nbytes = _workspace(shape, QSA_OP_DECODE, 1, kv_len, ws, q.device)
    _check(LIB.qsa_sparse_attn_decode_q8(ctypes.byref(shape), _ptr(q), _ptr(k_q), _ptr(v_q), _ptr(k_scales),
                                         _ptr(v_scales), kv_len, k_q.shape[2], _ptr(sel), _ptr(out), _ptr(ws), nbytes,
                                         _stream(q, stream)), "qsa_sparse_attn_decode_q8")
    return out


def qsa_sparse_attn_prefill_q8(shape: QsaShape, q, k_q, v_q, k_scales, v_scales, q_pos0: int, sel, out, ws=None,
                               stream=None):
    """Prefill attention over the rotated 8-bit cache for ``q`` ``[b][q_len][Hq][d]`` at positions ``q_pos0 ..``
    (``sel`` ``[b][q_len][Hkv][k]``). With its workspace (allocated here when ``ws`` is None) the call takes the
    tiled bf16 kernel over the codes rotated back where that serves the shape; ``ws`` of zero elements forces one
    query row per workgroup over the codes."""
    q_len = q.shape[1]
    ws, nbytes = _workspace(shape, QSA_OP_PREFILL_Q8, q_len, q_pos0 + q_len, ws, q.device)
    _check(LIB.qsa_sparse_attn_prefill_q8(ctypes.byref(shape), _ptr(q), _ptr(k_q), _ptr(v_q), _ptr(k_scales),
                                          _ptr(v_scales), q_len, q_pos0, k_q.shape[2], _ptr(sel), _ptr(out),
                                          _ptr(ws), nbytes, _stream(q, stream)), "qsa_sparse_attn_prefill_q8")
    return out


def qsa_decode_step_q8(shape: QsaShape, q, k, v, k_comp, k_q, v_q, k_scales, v_scales, kv_len: int, sel, out,
                       sel_scores=None, ws=None, stream=None):
    """One decode step over the 8-bit cache: quantize position ``kv_len - 1`` of ``k``/``v`` into it, then compress,
    select and attend over the codes (one kernel on ``qsa_decode_step``'s fused shapes, else the selection call and
    the 8-bit attention)."""
    ws, nbytes = _workspace(shape, QSA_OP_DECODE_STEP, 1, kv_len, ws, q.device)
    _check(LIB.qsa_decode_step_q8(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(k_comp), _ptr(k_q), _ptr(v_q),
                                  _ptr(k_scales), _ptr(v_scales), kv_len, k.shape[2], _ptr(sel), _ptr(sel_scores),
                                  _ptr(out), _ptr(ws), nbytes, _stream(q, stream)), "qsa_decode_step_q8")
    return out
