"""C ABI contract checks that need no GPU.

The library loads, exports every function ``include/qsa.h`` declares, and
rejects invalid arguments on the host with the documented status code
before making any HIP call. Every call here is invalid on purpose, so no
kernel is ever launched (the pointers are never dereferenced).
"""
from __future__ import annotations

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qsa.h")


@pytest.fixture(scope="module")
def qsa():
    import block_sparse_long_compress_amd as m

    return m


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qsa_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_four_steps():
    names = declared_functions()
    for n in ("qsa_compress_keys", "qsa_score_select", "qsa_sparse_attn_decode", "qsa_sparse_attn_prefill"):
        assert n in names


def test_library_exports_every_declared_symbol(qsa):
    lib = ctypes.CDLL(qsa.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert sorted(qsa.EXPORTED) == declared_functions()


def test_version_and_status_strings(qsa):
    assert qsa.abi_version() == 6
    for code, name in [(0, "QSA_OK"), (1, "QSA_ERR_INVALID"), (2, "QSA_ERR_UNSUPPORTED"), (3, "QSA_ERR_WORKSPACE"),
                       (4, "QSA_ERR_HIP")]:
        assert qsa.status_str(code).startswith(name)
    assert qsa.status_str(99) == "QSA_ERR_UNKNOWN"


def good_shape(qsa, **kw):
    args = dict(batch=1, n_q_heads=16, n_kv_heads=2, head_dim=128, block_size=64, top_k=16, dtype=qsa.QSA_BF16)
    args.update(kw)
    return qsa.QsaShape(args["batch"], args["n_q_heads"], args["n_kv_heads"], args["head_dim"], args["block_size"],
                        args["top_k"], args["dtype"], args.get("scale", 0.0), args.get("keep_tail", 0))


def test_workspace_sizes(qsa):
    sh = good_shape(qsa)
    assert qsa.qsa_workspace_bytes(sh, qsa.QSA_OP_COMPRESS, 1, 100) == 0
    # prefill: a V^T staging copy of the cache up to kv_len rounded to blocks
    assert qsa.qsa_workspace_bytes(sh, qsa.QSA_OP_PREFILL, 8192, 8192) == 2 * 8192 * 128 * 2
    assert qsa.qsa_workspace_bytes(sh, qsa.QSA_OP_PREFILL, 100, 100) == 2 * 128 * 128 * 2
    # decode: one partial softmax state per (row, slice) when a row is split
    dec = qsa.qsa_workspace_bytes(sh, qsa.QSA_OP_DECODE, 1, 32768)
    assert (dec - 256) % (2 * (2 * 8 + 8 * 128) * 4) == 0  # arrival counters, then partial states
    # select: arrival counters + chunk lists of the split path (decode), or nothing (tile path)
    assert qsa.qsa_workspace_bytes(sh, qsa.QSA_OP_SELECT, 8192, 8192) == 0
    assert (qsa.qsa_workspace_bytes(sh, qsa.QSA_OP_SELECT, 1, 1 << 20) - 256) % (2 * 15 * 8) == 0
    f32 = good_shape(qsa, dtype=qsa.QSA_F32, head_dim=64, n_q_heads=2, n_kv_heads=1, block_size=32, top_k=4)
    assert qsa.qsa_workspace_bytes(f32, qsa.QSA_OP_PREFILL, 512, 512) == 0
    assert qsa.qsa_workspace_bytes(f32, qsa.QSA_OP_DECODE, 1, 512) == 0
    with pytest.raises(qsa.QsaError):
        qsa.qsa_workspace_bytes(sh, 7, 1, 1)
    with pytest.raises(qsa.QsaError):
        qsa.qsa_workspace_bytes(sh, qsa.QSA_OP_SELECT, 10, 5)


BAD_SHAPES = [
    (dict(batch=0), 1), (dict(n_q_heads=15), 1), (dict(n_kv_heads=0), 1), (dict(top_k=0), 1), (dict(dtype=5), 1),
    (dict(scale=float("nan")), 1), (dict(scale=-1.0), 1), (dict(head_dim=96), 2), (dict(block_size=48), 2),
    (dict(block_size=2), 2), (dict(block_size=256), 2), (dict(top_k=514), 2), (dict(n_q_heads=24, n_kv_heads=2), 2),
    (dict(n_q_heads=64, n_kv_heads=2), 2), (dict(keep_tail=2), 1), (dict(keep_tail=1, top_k=1), 1),
]


@pytest.mark.parametrize("kw,code", BAD_SHAPES)
def test_shape_validation(qsa, kw, code):
    sh = good_shape(qsa, **kw)
    P = ctypes.c_void_p(4096)
    lib = qsa.LIB
    assert lib.qsa_compress_keys(ctypes.byref(sh), P, 64, 64, 0, P, None) == code
    assert lib.qsa_score_select(ctypes.byref(sh), P, 1, 63, P, 64, 64, P, None, P, 1 << 20, None) == code
    assert lib.qsa_sparse_attn_decode(ctypes.byref(sh), P, P, P, 64, 64, P, P, P, 1 << 20, None) == code
    assert lib.qsa_sparse_attn_prefill(ctypes.byref(sh), P, P, P, 64, 0, 64, P, P, P, 1 << 20, None) == code


def test_op_specific_limits(qsa):
    """Shapes every op accepts except the one whose kernels lack the path (checked before any launch)."""
    lib = qsa.LIB
    P = ctypes.c_void_p(4096)
    for kw in (dict(block_size=16), dict(top_k=65), dict(block_size=4, top_k=513, keep_tail=1)):
        sh = ctypes.byref(good_shape(qsa, **kw))
        assert lib.qsa_sparse_attn_prefill(sh, P, P, P, 64, 0, 64, P, P, P, 1 << 30, None) == 2
    # k > 64 selection holds at most 65536 candidates per row
    sh = good_shape(qsa, block_size=4, top_k=513, keep_tail=1)
    n = 4 * 65536
    assert qsa.qsa_workspace_bytes(sh, qsa.QSA_OP_SELECT, 1, n) == 2 * 256 * (256 * 4 + 16 * 8)
    # a too-small workspace is reported only for a supported shape (no launch either way)
    assert lib.qsa_score_select(ctypes.byref(sh), P, 1, n - 1, P, n, n, P, None, P, 8, None) == 3
    assert lib.qsa_score_select(ctypes.byref(sh), P, 1, n + 3, P, n + 4, n + 4, P, None, P, 8, None) == 2


def test_argument_validation(qsa):
    lib = qsa.LIB
    sh = ctypes.byref(good_shape(qsa))
    P, N, MIS = ctypes.c_void_p(4096), None, ctypes.c_void_p(4100)
    big = 1 << 30
    INV, WS = 1, 3
    # compress
    assert lib.qsa_compress_keys(None, P, 64, 64, 0, P, N) == INV
    assert lib.qsa_compress_keys(sh, N, 64, 64, 0, P, N) == INV
    assert lib.qsa_compress_keys(sh, P, 64, 64, 0, N, N) == INV
    assert lib.qsa_compress_keys(sh, MIS, 64, 64, 0, P, N) == INV
    assert lib.qsa_compress_keys(sh, P, 65, 64, 0, P, N) == INV  # kv_len > kv_cap
    assert lib.qsa_compress_keys(sh, P, -1, 64, 0, P, N) == INV
    assert lib.qsa_compress_keys(sh, P, 64, 64, -1, P, N) == INV
    assert lib.qsa_compress_keys(sh, P, 63, 64, 0, P, N) == 0  # no complete block: nothing to do, no launch
    assert lib.qsa_compress_keys(sh, P, 128, 128, 2, P, N) == 0  # range already compressed
    # select
    assert lib.qsa_score_select(sh, P, 1, 63, P, 65, 128, P, N, P, big, N) == INV  # kv_len != q_pos0 + q_len
    assert lib.qsa_score_select(sh, P, 0, 64, P, 64, 128, P, N, P, big, N) == INV
    assert lib.qsa_score_select(sh, P, 1, 64, P, 65, 64, P, N, P, big, N) == INV  # beyond capacity
    assert lib.qsa_score_select(sh, P, 1, -1, P, 0, 64, P, N, P, big, N) == INV
    assert lib.qsa_score_select(sh, N, 1, 63, P, 64, 64, P, N, P, big, N) == INV
    assert lib.qsa_score_select(sh, P, 1, 63, P, 64, 64, MIS, N, P, big, N) == INV
    assert lib.qsa_score_select(sh, P, 1, 63, P, 64, 64, P, MIS, P, big, N) == INV
    assert lib.qsa_score_select(sh, P, 1, (1 << 20) - 1, P, 1 << 20, 1 << 20, P, N, N, 0, N) == WS
    assert lib.qsa_score_select(sh, P, 1, (1 << 20) - 1, P, 1 << 20, 1 << 20, P, N, P, 8, N) == WS
    # decode
    assert lib.qsa_sparse_attn_decode(sh, P, P, P, 0, 64, P, P, P, big, N) == INV
    assert lib.qsa_sparse_attn_decode(sh, P, P, P, 65, 64, P, P, P, big, N) == INV
    assert lib.qsa_sparse_attn_decode(sh, P, N, P, 64, 64, P, P, P, big, N) == INV
    assert lib.qsa_sparse_attn_decode(sh, P, P, P, 64, 64, P, MIS, P, big, N) == INV
    assert lib.qsa_sparse_attn_decode(sh, P, P, P, 32768, 32768, P, P, N, 0, N) == WS
    # prefill
    assert lib.qsa_sparse_attn_prefill(sh, P, P, P, 0, 0, 64, P, P, P, big, N) == INV
    assert lib.qsa_sparse_attn_prefill(sh, P, P, P, 64, 1, 64, P, P, P, big, N) == INV  # beyond capacity
    assert lib.qsa_sparse_attn_prefill(sh, P, P, P, 64, -1, 64, P, P, P, big, N) == INV
    assert lib.qsa_sparse_attn_prefill(sh, P, P, N, 64, 0, 64, P, P, P, big, N) == INV
    assert lib.qsa_sparse_attn_prefill(sh, P, P, P, 64, 0, 64, P, P, N, 0, N) == WS
    assert lib.qsa_sparse_attn_prefill(sh, P, P, P, 64, 0, 64, P, P, P, 16, N) == WS


def test_ragged_decode_step_arguments(qsa):
    """Per-sequence lengths: validated on the host; the ragged step serves only the fused kernel's shapes."""
    lib = qsa.LIB
    sh = good_shape(qsa, batch=4)
    shr = ctypes.byref(sh)
    P, N, MIS4 = ctypes.c_void_p(4096), None, ctypes.c_void_p(4098)
    big = 1 << 30
    INV, UNS, WS = 1, 2, 3
    ws = qsa.qsa_workspace_bytes(sh, qsa.QSA_OP_DECODE_STEP_RAGGED, 1, 131072)
    # same per-row plan; the plain step's workspace also reserves the split
    # selection's counter area (one 4-byte counter per row, 256-byte rounded)
    cnt = (4 * sh.batch * sh.n_kv_heads + 255) // 256 * 256
    assert ws > 0 and qsa.qsa_workspace_bytes(sh, qsa.QSA_OP_DECODE_STEP, 1, 4096) == ws + cnt
    call = lib.qsa_decode_step_ragged
    assert call(shr, P, P, P, P, N, 64, 64, P, N, P, P, big, N) == INV           # no lengths
    assert call(shr, P, P, P, P, MIS4, 64, 64, P, N, P, P, big, N) == INV        # lengths not 4-byte aligned
    assert call(shr, P, P, P, P, P, 65, 64, P, N, P, P, big, N) == INV           # bound beyond capacity
    assert call(shr, P, P, P, P, P, 0, 64, P, N, P, P, big, N) == INV
    assert call(shr, N, P, P, P, P, 64, 64, P, N, P, P, big, N) == INV
    # shapes without the fused kernel: f32, k > 64, Bs < 32
    for kw in (dict(dtype=qsa.QSA_F32), dict(top_k=65), dict(block_size=16)):
        bad = good_shape(qsa, batch=4, **kw)
        assert call(ctypes.byref(bad), P, P, P, P, P, 4096, 4096, P, N, P, P, big, N) == UNS
        with pytest.raises(qsa.QsaError):
            qsa.qsa_workspace_bytes(bad, qsa.QSA_OP_DECODE_STEP_RAGGED, 1, 4096)
    # few long rows: the ragged step still runs fused (the plain step would not)
    one = good_shape(qsa, batch=1)
    assert not qsa.qsa_decode_step_fused(one, 1 << 20)
    assert qsa.qsa_workspace_bytes(one, qsa.QSA_OP_DECODE_STEP_RAGGED, 1, 1 << 20) > 0
    assert call(ctypes.byref(one), P, P, P, P, P, 1 << 20, 1 << 20, P, N, P, P, 8, N) == WS


def test_indexer_arguments(qsa):
    """The indexer calls validate their struct and arguments on the host."""
    lib = qsa.LIB
    sh = ctypes.byref(good_shape(qsa))
    P, N, MIS = ctypes.c_void_p(4096), None, ctypes.c_void_p(4100)
    INV, UNS = 1, 2
    ok = qsa.make_indexer(64, qsa.QSA_AGG_MAX)
    for bad in (qsa.make_indexer(96, 0), qsa.make_indexer(64, 3), qsa.make_indexer(64, -1),
                qsa.make_indexer(64, 0, -1.0), qsa.make_indexer(64, 0, float("inf"))):
        assert lib.qsa_indexer_keys(sh, ctypes.byref(bad), P, P, 128, 128, 0, P, N) == INV
        assert lib.qsa_indexer_select(sh, ctypes.byref(bad), P, P, 1, 127, P, 128, 128, P, N, N) == INV
    ix = ctypes.byref(ok)
    assert lib.qsa_indexer_keys(sh, None, P, P, 128, 128, 0, P, N) == INV
    assert lib.qsa_indexer_keys(sh, ix, N, P, 128, 128, 0, P, N) == INV
    assert lib.qsa_indexer_keys(sh, ix, P, P, 128, 128, 0, MIS, N) == INV
    assert lib.qsa_indexer_keys(sh, ix, P, P, 129, 128, 0, P, N) == INV
    assert lib.qsa_indexer_keys(sh, ix, N, N, 63, 128, 0, N, N) == 0  # no complete block: nothing to do
    assert lib.qsa_indexer_select(sh, ix, P, P, 1, 127, P, 129, 256, P, N, N) == INV  # kv_len != q_pos0 + q_len
    assert lib.qsa_indexer_select(sh, ix, N, P, 1, 127, P, 128, 256, P, N, N) == INV
    assert lib.qsa_indexer_select(sh, ix, P, P, 1, 127, P, 128, 256, MIS, N, N) == INV
    assert lib.qsa_indexer_select(sh, ix, P, P, 1, 127, N, 128, 256, P, N, N) == INV  # candidates, no keys
    big_k = ctypes.byref(good_shape(qsa, top_k=65))
    assert lib.qsa_indexer_select(big_k, ix, P, P, 1, 127, P, 128, 256, P, N, N) == UNS


def test_decode_step_q8_arguments(qsa):
    """The fused step over the 8-bit cache validates its arguments on the host and serves the fused shapes only."""
    lib = qsa.LIB
    sh = good_shape(qsa, batch=4)
    shr = ctypes.byref(sh)
    P, N, MIS = ctypes.c_void_p(4096), None, ctypes.c_void_p(4100)
    big = 1 << 30
    INV, UNS, WS = 1, 2, 3
    call = lib.qsa_decode_step_q8
    #            shape q  k  v  kc kq vq ks vs kv_len kv_cap sel scores out ws  bytes stream
    assert call(shr, P, P, P, P, N, P, P, P, 4096, 4096, P, N, P, P, big, N) == INV      # no key codes
    assert call(shr, P, P, P, P, P, P, MIS, P, 4096, 4096, P, N, P, P, big, N) == INV    # scales misaligned
    assert call(shr, P, P, P, P, P, P, P, P, 4097, 4096, P, N, P, P, big, N) == INV      # beyond capacity
    assert call(shr, P, P, P, P, P, P, P, P, 0, 4096, P, N, P, P, big, N) == INV
    # shapes the fused kernel does not serve: f32, k > 64, Bs < 32, few long rows
    for kw in (dict(dtype=qsa.QSA_F32), dict(top_k=65), dict(block_size=16)):
        bad = ctypes.byref(good_shape(qsa, batch=4, **kw))
        assert call(bad, P, P, P, P, P, P, P, P, 4096, 4096, P, N, P, P, big, N) == UNS
    one = good_shape(qsa, batch=1)
    assert not qsa.qsa_decode_step_fused(one, 1 << 20)
    assert call(ctypes.byref(one), P, P, P, P, P, P, P, P, 1 << 20, 1 << 20, P, N, P, P, big, N) == UNS
    # the workspace of the plain step (same layout)
    need = qsa.qsa_workspace_bytes(sh, qsa.QSA_OP_DECODE_STEP, 1, 4096)
    assert need > 0 and call(shr, P, P, P, P, P, P, P, P, 4096, 4096, P, N, P, P, need - 1, N) == WS
