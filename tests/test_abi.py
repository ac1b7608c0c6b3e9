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
    assert qsa.abi_version() == 12
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
        qsa.qsa_workspace_bytes(sh, 9, 1, 1)  # no such op
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
    # bf16 prefill attention serves every block size and top_k (short blocks and k > 64 one query row per
    # workgroup, without a workspace): no UNSUPPORTED for them, and their workspace is 0 bytes
    for kw in (dict(block_size=16), dict(top_k=65), dict(block_size=4, top_k=513, keep_tail=1)):
        sh = good_shape(qsa, **kw)
        assert qsa.qsa_workspace_bytes(sh, qsa.QSA_OP_PREFILL, 2048, 2048) == 0
        assert lib.qsa_sparse_attn_prefill(ctypes.byref(sh), P, P, P, 0, 0, 64, P, P, P, 0, None) == 1  # invalid
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
    """Per-sequence lengths: validated on the host; the ragged step serves the fused kernel's shapes, and every
    other shape (bf16 with k > 64 or Bs < 32, float32) through the large selection, up to 65536 candidates."""
    lib = qsa.LIB
    sh = good_shape(qsa, batch=4)
    shr = ctypes.byref(sh)
    P, N, MIS4 = ctypes.c_void_p(4096), None, ctypes.c_void_p(4098)
    big = 1 << 30
    INV, UNS, WS = 1, 2, 3
    ws = qsa.qsa_workspace_bytes(sh, qsa.QSA_OP_DECODE_STEP_RAGGED, 1, 131072)
    # same per-row plan and the same layout as the plain step's workspace
    # (two arrival-counter areas, then the slice states)
    assert ws > 0 and qsa.qsa_workspace_bytes(sh, qsa.QSA_OP_DECODE_STEP, 1, 131072) == ws
    call = lib.qsa_decode_step_ragged
    assert call(shr, P, P, P, P, N, 64, 64, P, N, P, P, big, N) == INV           # no lengths
    assert call(shr, P, P, P, P, MIS4, 64, 64, P, N, P, P, big, N) == INV        # lengths not 4-byte aligned
    assert call(shr, P, P, P, P, P, 65, 64, P, N, P, P, big, N) == INV           # bound beyond capacity
    assert call(shr, P, P, P, P, P, 0, 64, P, N, P, P, big, N) == INV
    assert call(shr, N, P, P, P, P, 64, 64, P, N, P, P, big, N) == INV
    # not served: the large selection's candidate limit (unfused shapes, more than 65536 candidates per row)
    for kw, n in ((dict(dtype=qsa.QSA_F32), 64 * 70000), (dict(block_size=16), 16 * 70000),
                  (dict(top_k=513, block_size=4), 4 * 70000)):
        bad = good_shape(qsa, batch=4, **kw)
        assert call(ctypes.byref(bad), P, P, P, P, P, n, n, P, N, P, P, big, N) == UNS
        with pytest.raises(qsa.QsaError):
            qsa.qsa_workspace_bytes(bad, qsa.QSA_OP_DECODE_STEP_RAGGED, 1, n)
    # the large selection's workspace (at least one chunk, even before any candidate exists): k > 64,
    # Bs < 32 with k <= 64, float32 with any k
    for kw, n in ((dict(top_k=65), 4096), (dict(top_k=513, block_size=4), 4 * 20000), (dict(top_k=100, block_size=4), 3),
                  (dict(block_size=16), 4096), (dict(block_size=4, top_k=8), 3), (dict(dtype=qsa.QSA_F32), 4096),
                  (dict(dtype=qsa.QSA_F32, top_k=100, block_size=8), 5000)):
        large = good_shape(qsa, batch=4, **kw)
        need = qsa.qsa_workspace_bytes(large, qsa.QSA_OP_DECODE_STEP_RAGGED, 1, n)
        assert need > 0
        assert call(ctypes.byref(large), P, P, P, P, P, n, n, P, N, P, P, need - 1, N) == WS
    # few long rows: one fused kernel (the rows' scans split over several workgroups), ragged or not
    one = good_shape(qsa, batch=1)
    assert qsa.qsa_decode_step_fused(one, 1 << 20)
    assert qsa.qsa_workspace_bytes(one, qsa.QSA_OP_DECODE_STEP_RAGGED, 1, 1 << 20) > 0
    assert call(ctypes.byref(one), P, P, P, P, P, 1 << 20, 1 << 20, P, N, P, P, 8, N) == WS


def test_ragged_select_and_attention_arguments(qsa):
    """The ragged batch's selection and attention as calls of their own: per-sequence lengths validated on the
    host; the selection takes the large selection's workspace for any top_k (scores and chunk lists of the
    longest row), the attention the decode call's."""
    lib = qsa.LIB
    sh = good_shape(qsa, batch=4)
    shr = ctypes.byref(sh)
    P, N, MIS4 = ctypes.c_void_p(4096), None, ctypes.c_void_p(4098)
    big = 1 << 30
    INV, UNS, WS = 1, 2, 3
    sel = lib.qsa_score_select_ragged
    #           shape q  kc kv_lens max   cap  sel scores ws bytes stream
    assert sel(shr, P, P, N, 4096, 4096, P, N, P, big, N) == INV       # no lengths
    assert sel(shr, P, P, MIS4, 4096, 4096, P, N, P, big, N) == INV    # lengths not 4-byte aligned
    assert sel(shr, P, P, P, 4097, 4096, P, N, P, big, N) == INV       # bound beyond capacity
    assert sel(shr, P, P, P, 0, 4096, P, N, P, big, N) == INV
    assert sel(shr, N, P, P, 4096, 4096, P, N, P, big, N) == INV
    assert sel(shr, P, N, P, 4096, 4096, P, N, P, big, N) == INV       # candidates but no compressed keys
    # every top_k: scores (4 bytes) and chunk lists (16 keys of 8 bytes) of every row's 256-candidate chunks
    rows = 4 * 2
    for kw, n in ((dict(), 4096), (dict(top_k=513, block_size=4, keep_tail=1), 4 * 20000), (dict(top_k=8), 64 * 300)):
        shk = good_shape(qsa, batch=4, **kw)
        need = qsa.qsa_workspace_bytes(shk, qsa.QSA_OP_SELECT_RAGGED, 1, n)
        cand = n // shk.block_size if shk.keep_tail else (n - 1) // shk.block_size
        assert need == rows * ((cand + 255) // 256) * (256 * 4 + 16 * 8)
        assert sel(ctypes.byref(shk), P, P, P, n, n, P, N, P, need - 1, N) == WS
    # no candidate anywhere: no workspace, k_comp not read
    assert qsa.qsa_workspace_bytes(sh, qsa.QSA_OP_SELECT_RAGGED, 1, 64) == 0
    # the large selection's candidate limit
    wide = good_shape(qsa, batch=4, block_size=4, top_k=16)
    with pytest.raises(qsa.QsaError):
        qsa.qsa_workspace_bytes(wide, qsa.QSA_OP_SELECT_RAGGED, 1, 4 * 70000)
    assert sel(ctypes.byref(wide), P, P, P, 4 * 70000, 4 * 70000, P, N, P, big, N) == UNS

    att = lib.qsa_sparse_attn_decode_ragged
    #           shape q  k  v  kv_lens max   cap  sel out ws bytes stream
    assert att(shr, P, P, P, N, 4096, 4096, P, P, P, big, N) == INV    # no lengths
    assert att(shr, P, P, P, MIS4, 4096, 4096, P, P, P, big, N) == INV
    assert att(shr, P, P, P, P, 4097, 4096, P, P, P, big, N) == INV
    assert att(shr, P, P, P, P, 4096, 4096, N, P, P, big, N) == INV    # no selection
    one = good_shape(qsa, batch=1)
    need = qsa.qsa_workspace_bytes(one, qsa.QSA_OP_DECODE, 1, 32768)
    assert need > 0 and att(ctypes.byref(one), P, P, P, P, 32768, 32768, P, P, P, need - 1, N) == WS


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
        assert lib.qsa_indexer_select(sh, ctypes.byref(bad), P, P, 1, 127, P, 128, 128, P, N, N, 0, N) == INV
    ix = ctypes.byref(ok)
    assert lib.qsa_indexer_keys(sh, None, P, P, 128, 128, 0, P, N) == INV
    assert lib.qsa_indexer_keys(sh, ix, N, P, 128, 128, 0, P, N) == INV
    assert lib.qsa_indexer_keys(sh, ix, P, P, 128, 128, 0, MIS, N) == INV
    assert lib.qsa_indexer_keys(sh, ix, P, P, 129, 128, 0, P, N) == INV
    assert lib.qsa_indexer_keys(sh, ix, N, N, 63, 128, 0, N, N) == 0  # no complete block: nothing to do
    sel_ix = lib.qsa_indexer_select
    assert sel_ix(sh, ix, P, P, 1, 127, P, 129, 256, P, N, N, 0, N) == INV  # kv_len != q_pos0 + q_len
    assert sel_ix(sh, ix, N, P, 1, 127, P, 128, 256, P, N, N, 0, N) == INV
    assert sel_ix(sh, ix, P, P, 1, 127, P, 128, 256, MIS, N, N, 0, N) == INV
    assert sel_ix(sh, ix, P, P, 1, 127, N, 128, 256, P, N, N, 0, N) == INV  # candidates, no keys
    # k > 64: the large selection's workspace (none for k <= 64), at most 65536 candidates per row
    big_k = good_shape(qsa, top_k=65, block_size=4)
    need = qsa.qsa_workspace_bytes(big_k, qsa.QSA_OP_INDEXER_SELECT, 1, 4000)
    assert need > 0 and qsa.qsa_workspace_bytes(good_shape(qsa), qsa.QSA_OP_INDEXER_SELECT, 1, 4000) == 0
    assert sel_ix(ctypes.byref(big_k), ix, P, P, 1, 3999, P, 4000, 4096, P, N, N, 0, N) == 3
    assert sel_ix(ctypes.byref(big_k), ix, P, P, 1, 3999, P, 4000, 4096, P, N, P, need - 1, N) == 3
    assert sel_ix(ctypes.byref(big_k), ix, P, P, 1, 4 * 70000 - 1, P, 4 * 70000, 4 * 70000, P, N, P, 1 << 40,
                  N) == UNS
    # the fused indexer decode step: (shape, idx, w_q, w_k, q, k, v, k_comp, k_idx, kv_len, kv_cap, sel,
    # sel_scores, out, stream); bf16 with k <= 64 only
    step = lib.qsa_indexer_decode_step
    for bad in (qsa.make_indexer(96, 0), qsa.make_indexer(64, 3)):
        assert step(sh, ctypes.byref(bad), P, P, P, P, P, P, P, 128, 256, P, N, P, N) == INV
    assert step(sh, None, P, P, P, P, P, P, P, 128, 256, P, N, P, N) == INV
    for i in range(2, 9):  # each required pointer null, then misaligned
        args = [P] * 7
        args[i - 2] = N
        assert step(sh, ix, *args, 128, 256, P, N, P, N) == INV
        args[i - 2] = MIS
        assert step(sh, ix, *args, 128, 256, P, N, P, N) == INV
    assert step(sh, ix, P, P, P, P, P, P, P, 128, 256, N, N, P, N) == INV       # no sel
    assert step(sh, ix, P, P, P, P, P, P, P, 128, 256, P, MIS, P, N) == INV     # misaligned sel_scores
    assert step(sh, ix, P, P, P, P, P, P, P, 128, 256, P, N, N, N) == INV       # no out
    assert step(sh, ix, P, P, P, P, P, P, P, 0, 256, P, N, P, N) == INV         # kv_len < 1
    assert step(sh, ix, P, P, P, P, P, P, P, 257, 256, P, N, P, N) == INV       # kv_len beyond capacity
    assert step(ctypes.byref(big_k), ix, P, P, P, P, P, P, P, 128, 256, P, N, P, N) == UNS
    assert step(ctypes.byref(good_shape(qsa, dtype=qsa.QSA_F32)), ix, P, P, P, P, P, P, P, 128, 256, P, N, P,
                N) == UNS


def test_decode_step_q8_arguments(qsa):
    """The step over the 8-bit cache validates its arguments on the host; bf16 only, any top_k and block size."""
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
    # the 8-bit cache holds bf16 rows
    f32 = ctypes.byref(good_shape(qsa, batch=4, dtype=qsa.QSA_F32))
    assert call(f32, P, P, P, P, P, P, P, P, 4096, 4096, P, N, P, P, big, N) == UNS
    # shapes the fused kernel does not serve (k > 64, Bs < 32) run as the selection and the 8-bit attention, in
    # the workspace of the plain step; k > 64 keeps the large selection's candidate limit
    for kw in (dict(top_k=65), dict(block_size=16), dict(block_size=4, top_k=513)):
        other = good_shape(qsa, batch=4, **kw)
        assert not qsa.qsa_decode_step_fused(other, 4096)
        need = qsa.qsa_workspace_bytes(other, qsa.QSA_OP_DECODE_STEP, 1, 4096)
        assert need > 0
        assert call(ctypes.byref(other), P, P, P, P, P, P, P, P, 4096, 4096, P, N, P, N, need, N) == WS
        assert call(ctypes.byref(other), P, P, P, P, P, P, P, P, 4096, 4096, P, N, P, P, need - 1, N) == WS
    wide = good_shape(qsa, batch=1, block_size=4, top_k=100)  # 262144 candidates per row
    with pytest.raises(qsa.QsaError):
        qsa.qsa_workspace_bytes(wide, qsa.QSA_OP_DECODE_STEP, 1, 1 << 20)
    assert call(ctypes.byref(wide), P, P, P, P, P, P, P, P, 1 << 20, 1 << 20, P, N, P, P, big, N) == UNS
    # few long rows run fused too (scan split over several workgroups): the workspace is checked
    one = good_shape(qsa, batch=1)
    assert qsa.qsa_decode_step_fused(one, 1 << 20)
    assert call(ctypes.byref(one), P, P, P, P, P, P, P, P, 1 << 20, 1 << 20, P, N, P, P, 8, N) == WS
    # the workspace of the plain step (same layout)
    need = qsa.qsa_workspace_bytes(sh, qsa.QSA_OP_DECODE_STEP, 1, 4096)
    assert need > 0 and call(shr, P, P, P, P, P, P, P, P, 4096, 4096, P, N, P, P, need - 1, N) == WS


def test_prefill_q8_arguments(qsa):
    """Prefill over the 8-bit cache validates its arguments on the host: bf16 only, any top_k and block size."""
    lib = qsa.LIB
    sh = good_shape(qsa, batch=2)
    shr = ctypes.byref(sh)
    P, N, MIS = ctypes.c_void_p(4096), None, ctypes.c_void_p(4100)
    INV, UNS = 1, 2
    call = lib.qsa_sparse_attn_prefill_q8
    #            shape q  kq vq ks vs q_len q_pos0 kv_cap sel out ws ws_bytes stream
    assert call(shr, P, N, P, P, P, 64, 0, 4096, P, P, N, 0, N) == INV       # no key codes
    assert call(shr, P, P, P, MIS, P, 64, 0, 4096, P, P, N, 0, N) == INV     # key scales misaligned
    assert call(shr, P, P, P, P, P, 64, 4040, 4096, P, P, N, 0, N) == INV    # rows beyond capacity
    assert call(shr, P, P, P, P, P, 0, 0, 4096, P, P, N, 0, N) == INV        # no rows
    assert call(shr, P, P, P, P, P, 64, -1, 4096, P, P, N, 0, N) == INV
    bad = ctypes.byref(good_shape(qsa, batch=2, dtype=qsa.QSA_F32))
    assert call(bad, P, P, P, P, P, 64, 0, 4096, P, P, N, 0, N) == UNS
    assert call(ctypes.byref(good_shape(qsa, batch=2, head_dim=96)), P, P, P, P, P, 64, 0, 4096, P, P, N, 0, N) == UNS
    # the tiled way's workspace: the 8K prompt from 0 takes it (the rows' selected keys far beyond the
    # positions); a few rows at the end of a long context, blocks shorter than 32 keys and k > 64 do not
    need = qsa.qsa_workspace_bytes(sh, qsa.QSA_OP_PREFILL_Q8, 8192, 8192)
    assert need >= 3 * 2 * 2 * 8192 * 128 * 2
    for kw, q_len, n in ((dict(), 4, 1 << 20), (dict(block_size=16), 8192, 8192), (dict(top_k=65), 8192, 8192)):
        assert qsa.qsa_workspace_bytes(good_shape(qsa, batch=2, **kw), qsa.QSA_OP_PREFILL_Q8, q_len, n) == 0


def test_decode_step_noalloc_arguments(qsa):
    """The allocation-free decode step checks everything on the host first (nothing is launched here) and
    rejects steps whose workspace exceeds the library's scratch array."""
    lib = qsa.LIB
    sh = good_shape(qsa, batch=4)
    shr = ctypes.byref(sh)
    P, N, MIS = ctypes.c_void_p(4096), None, ctypes.c_void_p(4100)
    INV, UNS, WS = 1, 2, 3
    call = lib.qsa_decode_step_noalloc
    #            shape q  k  v  kc  kv_len kv_cap sel scores out stream
    assert call(shr, N, P, P, P, 4096, 4096, P, N, P, N) == INV       # no query
    assert call(shr, P, P, P, MIS, 4096, 4096, P, N, P, N) == INV     # misaligned compressed keys
    assert call(shr, P, P, P, P, 4097, 4096, P, N, P, N) == INV       # beyond capacity
    assert call(shr, P, P, P, P, 0, 4096, P, N, P, N) == INV
    assert call(ctypes.byref(good_shape(qsa, head_dim=96)), P, P, P, P, 4096, 4096, P, N, P, N) == UNS
    # a step whose workspace exceeds the scratch array: the released budget (every candidate's score in
    # the workspace) for 64 sequences of 262,144 positions
    big = good_shape(qsa, batch=64, block_size=4, top_k=513, keep_tail=1)
    need = qsa.qsa_workspace_bytes(big, qsa.QSA_OP_DECODE_STEP, 1, 1 << 18)
    assert need > qsa.QSA_NOALLOC_SCRATCH_BYTES
    assert call(ctypes.byref(big), P, P, P, P, 1 << 18, 1 << 18, P, N, P, N) == WS
    # the header's limit and the binding's agree
    text = open(HEADER).read()
    assert "#define QSA_NOALLOC_SCRATCH_BYTES ((size_t)8 << 20)" in text
    assert qsa.QSA_NOALLOC_SCRATCH_BYTES == 8 << 20
