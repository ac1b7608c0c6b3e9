"""qsa_decode_step_noalloc against qsa_decode_step, through the C ABI.

The allocation-free step keeps its workspace in the library's own device
array, shared by every call on the GPU. Each pair below runs two calls in a
row, the second on a smaller input, and compares each with qsa_decode_step
on a fresh zero-filled workspace (the same kernels: selections, scores,
compressed keys and outputs bitwise equal) and with the oracle.
"""
from __future__ import annotations

import pytest
import torch

import block_sparse_long_compress_amd as qsa
from gpu_common import Case, check_rows, from_device, log
from test_gpu_parity import W, case_id

pytestmark = pytest.mark.gpu

PAIRS = [
    # fused kernel: one workgroup per row, then slices of the selection per row
    (W(mode="decode", batch=64, kv_len=3008, top_k=16), W(mode="decode", batch=2, kv_len=1000, top_k=8)),
    # separate calls: split selection (chunk lists) and split attention (slice states)
    (W(mode="decode", batch=1, kv_len=200000, top_k=32), W(mode="decode", batch=1, kv_len=150001, top_k=32)),
    # released budget: score pass (every score in the scratch) and pick + attend
    (W(mode="decode", batch=1, kv_len=4 * 20000, top_k=513, block_size=4, keep_tail=True),
     W(mode="decode", batch=1, kv_len=4 * 15000 + 1, top_k=513, block_size=4, keep_tail=True)),
]


def _run(case: Case, noalloc: bool):
    w = case.w
    b, hq, hkv, d, bs, k = w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.block_size, w.top_k
    shape = qsa.shape_for(case.q, case.k, bs, k, keep_tail=w.keep_tail)
    k_comp = torch.full((b, hkv, case.kv_cap // bs, d), float("nan"), device="cuda")
    qsa.qsa_compress_keys(shape, case.k, w.kv_len - 1, k_comp)
    q = case.q.view(b, hq, d)
    sel = torch.empty(b, hkv, k, dtype=torch.int32, device="cuda")
    scores = torch.empty(b, hkv, k, dtype=torch.float32, device="cuda")
    out = torch.empty_like(q)
    if noalloc:
        qsa.qsa_decode_step_noalloc(shape, q, case.k, case.v, k_comp, w.kv_len, sel, out, sel_scores=scores)
    else:
        ws = qsa.workspace(shape, qsa.QSA_OP_DECODE_STEP, 1, w.kv_len, "cuda")
        qsa.qsa_decode_step(shape, q, case.k, case.v, k_comp, w.kv_len, sel, out, sel_scores=scores, ws=ws)
    return sel, scores, out, k_comp


@pytest.mark.parametrize("pair", PAIRS, ids=lambda p: case_id(p[0]))
def test_noalloc_decode_step_matches_decode_step(pair):
    for w in pair:  # the second call reuses the scratch the first left behind
        log(f"no-alloc decode step {case_id(w)}")
        case = Case(w, seed=50)
        got = _run(case, noalloc=True)
        torch.cuda.synchronize()
        ref = _run(case, noalloc=False)
        torch.cuda.synchronize()
        sel, scores, out, k_comp = got
        assert torch.equal(sel, ref[0]), "selection"
        assert torch.equal(scores.view(torch.int32), ref[1].view(torch.int32)), "selection scores"
        assert torch.equal(out.view(torch.int16), ref[2].view(torch.int16)), "output"
        nb = w.kv_len // w.block_size
        assert torch.equal(k_comp[:, :, :nb], ref[3][:, :, :nb]), "compressed keys"
        rows = [(bb, 0, g) for bb in range(w.batch) for g in range(w.n_kv_heads)]
        st = check_rows(case, sel.cpu().numpy()[:, None], from_device(out)[:, None], rows, w.kv_len - 1,
                        scores_gpu=scores.cpu().numpy()[:, None])
        log(f"  {st}")
