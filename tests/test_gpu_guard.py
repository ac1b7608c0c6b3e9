"""Guard bands: no kernel writes past the buffers a call is given.

Every output buffer (``out``, ``sel``, ``sel_scores``, ``k_comp``) and the
workspace is carved from a larger allocation whose tail holds a fill
pattern; after the call the tail must still hold it, and the results must be
bitwise those of the same call on plain tensors. ``k_comp`` rows of blocks
the call does not compress are filled with the pattern too and must stay
untouched. The workspace's own bytes follow the documented contract (zeroed
before first use).
"""
from __future__ import annotations

import pytest
import torch

import block_sparse_long_compress_amd as qsa
from gpu_common import Case, log
from test_gpu_parity import W, case_id

pytestmark = pytest.mark.gpu

GUARD = 8192
FILL = 0xA5


class Guarded:
    """A tensor of ``shape``/``dtype`` at the start of a byte buffer whose last GUARD bytes hold FILL."""

    def __init__(self, shape, dtype, fill_body=None):
        n = 1
        for x in shape:
            n *= x
        self.nbytes = n * torch.tensor([], dtype=dtype).element_size()
        self.buf = torch.full((self.nbytes + GUARD,), FILL, dtype=torch.uint8, device="cuda")
        if fill_body is not None:
            self.buf[:self.nbytes].fill_(fill_body)
        self.t = self.buf[:self.nbytes].view(dtype).view(*shape)

    def intact(self) -> bool:
        return bool((self.buf[self.nbytes:] == FILL).all())


def _ws(shape, op, q_len, kv_len):
    n = qsa.qsa_workspace_bytes(shape, op, q_len, kv_len)
    buf = torch.full((max(n, 16) + GUARD,), FILL, dtype=torch.uint8, device="cuda")
    buf[:n].zero_()
    return buf, n


def _same(a: torch.Tensor, b: torch.Tensor) -> bool:
    if a.dtype in (torch.bfloat16, torch.float32):
        a, b = a.view(torch.int16 if a.dtype == torch.bfloat16 else torch.int32), \
            b.view(torch.int16 if b.dtype == torch.bfloat16 else torch.int32)
    return torch.equal(a, b)


STEP_GUARD_CASES = [
    W(mode="decode", batch=3, kv_len=5000, top_k=16),                                   # fused, slices per row
    W(mode="decode", batch=64, kv_len=3008, top_k=16),                                  # fused, one workgroup per row
    W(mode="decode", batch=1, kv_len=200000, top_k=32),                                 # split selection + attention
    W(mode="decode", batch=1, kv_len=4 * 20000, top_k=513, block_size=4, keep_tail=True),  # score + pick/attend
    W(mode="decode", batch=2, kv_len=2240, dtype="f32", sigma=1.0, top_k=5),           # float32 path
]


@pytest.mark.parametrize("w", STEP_GUARD_CASES, ids=case_id)
def test_decode_step_guard_bands(w):
    log(f"guard bands, decode step {case_id(w)}")
    case = Case(w, seed=40, kv_cap=w.kv_len + 3 * w.block_size)  # k_comp rows past the last block must stay
    b, hq, hkv, d, bs, k = w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.block_size, w.top_k
    shape = qsa.shape_for(case.q, case.k, bs, k, keep_tail=w.keep_tail)
    nb_cap = case.kv_cap // bs
    q = case.q.view(b, hq, d)
    # plain tensors: the reference call
    kc_ref = torch.zeros(b, hkv, nb_cap, d, device="cuda")
    qsa.qsa_compress_keys(shape, case.k, w.kv_len - 1, kc_ref)
    sel_ref = torch.empty(b, hkv, k, dtype=torch.int32, device="cuda")
    sc_ref = torch.empty(b, hkv, k, dtype=torch.float32, device="cuda")
    out_ref = torch.empty_like(q)
    qsa.qsa_decode_step(shape, q, case.k, case.v, kc_ref, w.kv_len, sel_ref, out_ref, sel_scores=sc_ref)
    # guarded buffers: k_comp's body holds the pattern except the blocks compressed beforehand
    kc = Guarded((b, hkv, nb_cap, d), torch.float32, fill_body=FILL)
    n_prev = (w.kv_len - 1) // bs
    kc.t[:, :, :n_prev].copy_(kc_ref[:, :, :n_prev])
    sel = Guarded((b, hkv, k), torch.int32)
    sc = Guarded((b, hkv, k), torch.float32)
    out = Guarded(tuple(q.shape), q.dtype)
    ws, n_ws = _ws(shape, qsa.QSA_OP_DECODE_STEP, 1, w.kv_len)
    qsa.qsa_decode_step(shape, q, case.k, case.v, kc.t, w.kv_len, sel.t, out.t, sel_scores=sc.t, ws=ws[:max(n_ws, 16)]
                        if n_ws else None)
    torch.cuda.synchronize()
    for name, g in (("k_comp", kc), ("sel", sel), ("sel_scores", sc), ("out", out)):
        assert g.intact(), f"{name}: bytes past the buffer were written"
    assert bool((ws[max(n_ws, 16):] == FILL).all()), "bytes past the workspace were written"
    nb = w.kv_len // bs
    assert torch.equal(kc.t[:, :, :nb], kc_ref[:, :, :nb])
    assert nb < nb_cap
    if nb < nb_cap:
        assert bool((kc.t[:, :, nb:].contiguous().view(torch.uint8) == FILL).all()), "k_comp rows past the call's blocks"
    assert _same(sel.t, sel_ref) and _same(sc.t, sc_ref) and _same(out.t, out_ref)


PREFILL_GUARD_CASES = [
    W(batch=2, kv_len=1000, top_k=4),
    W(kv_len=3000, top_k=24, block_size=32),
    W(kv_len=700, dtype="f32", sigma=1.0, head_dim=64, n_q_heads=2, n_kv_heads=1, block_size=4, top_k=100,
      keep_tail=True),
]


@pytest.mark.parametrize("w", PREFILL_GUARD_CASES, ids=case_id)
def test_prefill_guard_bands(w):
    """Compress, select and prefill attention calls into guarded buffers."""
    log(f"guard bands, prefill {case_id(w)}")
    case = Case(w, seed=41)
    b, T, hq, hkv, d, bs, k = w.batch, w.kv_len, w.n_q_heads, w.n_kv_heads, w.head_dim, w.block_size, w.top_k
    shape = qsa.shape_for(case.q, case.k, bs, k, keep_tail=w.keep_tail)
    out_ref, sel_ref, kc_ref, sc_ref = qsa.prefill(case.q, case.k, case.v, bs, k, with_scores=True,
                                                   keep_tail=w.keep_tail)
    nb = T // bs
    kc = Guarded((b, hkv, nb, d), torch.float32)
    qsa.qsa_compress_keys(shape, case.k, T, kc.t)
    sel = Guarded((b, T, hkv, k), torch.int32)
    sc = Guarded((b, T, hkv, k), torch.float32)
    ws_s, n_s = _ws(shape, qsa.QSA_OP_SELECT, T, T)
    qsa.qsa_score_select(shape, case.q, 0, kc.t, T, T, sel.t, sc.t, ws=ws_s[:max(n_s, 16)] if n_s else None)
    out = Guarded(tuple(case.q.shape), case.q.dtype)
    ws_p, n_p = _ws(shape, qsa.QSA_OP_PREFILL, T, T)
    qsa.qsa_sparse_attn_prefill(shape, case.q, case.k, case.v, 0, sel.t, out.t, ws=ws_p[:max(n_p, 16)] if n_p else None)
    torch.cuda.synchronize()
    for name, g in (("k_comp", kc), ("sel", sel), ("sel_scores", sc), ("out", out)):
        assert g.intact(), f"{name}: bytes past the buffer were written"
    assert bool((ws_s[max(n_s, 16):] == FILL).all()) and bool((ws_p[max(n_p, 16):] == FILL).all())
    assert torch.equal(kc.t, kc_ref[:, :, :nb])
    assert _same(sel.t, sel_ref) and _same(sc.t, sc_ref) and _same(out.t, out_ref)


def test_separate_decode_guard_bands():
    """The separate decode attention (split rows merged by their last workgroup) into guarded buffers."""
    w = W(mode="decode", batch=2, kv_len=70000, top_k=16)
    case = Case(w, seed=42)
    b, hq, hkv, d, bs, k = w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.block_size, w.top_k
    shape = qsa.shape_for(case.q, case.k, bs, k)
    kc = torch.empty(b, hkv, w.kv_len // bs, d, device="cuda")
    qsa.qsa_compress_keys(shape, case.k, w.kv_len, kc)
    q = case.q.view(b, hq, d)
    out_ref, sel_ref = qsa.decode(q, case.k, case.v, w.kv_len, bs, k, kc)
    out = Guarded(tuple(q.shape), q.dtype)
    ws, n = _ws(shape, qsa.QSA_OP_DECODE, 1, w.kv_len)
    assert n > 0
    qsa.qsa_sparse_attn_decode(shape, q, case.k, case.v, w.kv_len, sel_ref, out.t, ws=ws[:n])
    torch.cuda.synchronize()
    assert out.intact() and bool((ws[n:] == FILL).all())
    assert _same(out.t, out_ref)
