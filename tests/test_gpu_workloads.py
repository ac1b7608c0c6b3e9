"""GPU parity at the full sizes of the bf16 workloads, in the launch
configuration the benchmark times (plans depend only on the shapes).

Selections are checked row by row wherever the oracle can afford it (every
row of the 32K, 8K, 1M and 256K ratio-4 workloads; sampled rows of the 64 x 128K batch,
plus the planted-block property on all of its rows). Outputs are compared on
every row of the decode workloads and on sampled rows of the prefill; the ragged
batch is checked on six sampled sequences at their own lengths.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import block_sparse_long_compress_amd as qsa
import qsa_synth as S
from gpu_common import Case, check_compress, check_rows, from_device, log

pytestmark = pytest.mark.gpu


def decode_full(case: Case):
    w = case.w
    shape = qsa.shape_for(case.q, case.k, w.block_size, w.top_k, keep_tail=w.keep_tail)
    k_comp = torch.empty(w.batch, w.n_kv_heads, case.kv_cap // w.block_size, w.head_dim, device="cuda")
    qsa.qsa_compress_keys(shape, case.k, w.kv_len, k_comp)
    q = case.q.view(w.batch, w.n_q_heads, w.head_dim)
    out, sel, scores = qsa.decode(q, case.k, case.v, w.kv_len, w.block_size, w.top_k, k_comp, with_scores=True,
                                  keep_tail=w.keep_tail)
    torch.cuda.synchronize()
    return sel.cpu().numpy()[:, None], from_device(out)[:, None], scores.cpu().numpy()[:, None], k_comp


@pytest.mark.parametrize("name", ["decode_32k", "decode_1m", "decode_256k_r4"])
def test_decode_workload(name):
    w = S.WORKLOADS[name]
    log(f"workload {name}: generating")
    case = Case(w, seed=0)
    log(f"workload {name}: running")
    sel, out, scores, k_comp = decode_full(case)
    check_compress(case, k_comp)
    rows = [(b, 0, g) for b in range(w.batch) for g in range(w.n_kv_heads)]
    st = check_rows(case, sel, out, rows, w.kv_len - 1, scores_gpu=scores)
    log(f"  {name}: {st}")


def test_prefill_8k_workload():
    w = S.WORKLOADS["prefill_8k"]
    log("workload prefill_8k: generating")
    case = Case(w, seed=0)
    out, sel, k_comp, scores = qsa.prefill(case.q, case.k, case.v, w.block_size, w.top_k, with_scores=True)
    torch.cuda.synchronize()
    sel, out, scores = sel.cpu().numpy(), from_device(out), scores.cpu().numpy()
    check_compress(case, k_comp)
    rows = [(0, t, g) for t in range(w.kv_len) for g in range(w.n_kv_heads)]
    st = check_rows(case, sel, out, rows, 0, check_output=False)
    log(f"  selections: {st}")
    rng = np.random.default_rng(0)
    sample = sorted(set(rng.integers(0, w.kv_len, 200).tolist()) | {0, 1, 63, 64, 1023, 1024, w.kv_len - 1})
    st = check_rows(case, sel, out, [(0, t, g) for t in sample for g in range(2)], 0, scores_gpu=scores)
    log(f"  sampled outputs: {st}")


def test_batched_decode_planted_workload():
    w = S.WORKLOADS["decode_b64_128k"]
    log("workload decode_b64_128k: generating 2 x 4 GiB")
    case = Case(w, seed=0)
    # the oracle compresses only the sampled rows' keys
    log("workload decode_b64_128k: running")
    shape = qsa.shape_for(case.q, case.k, w.block_size, w.top_k)
    k_comp = torch.empty(w.batch, 2, w.kv_len // w.block_size, w.head_dim, device="cuda")
    qsa.qsa_compress_keys(shape, case.k, w.kv_len, k_comp)
    q = case.q.view(w.batch, w.n_q_heads, w.head_dim)
    out, sel, scores = qsa.decode(q, case.k, case.v, w.kv_len, w.block_size, w.top_k, k_comp, with_scores=True)
    torch.cuda.synchronize()
    sel_h = sel.cpu().numpy()
    for b in range(w.batch):
        for g in range(2):
            planted = set(S.planted_blocks(w, 0, b, g).tolist())
            assert planted <= set(sel_h[b, g].tolist()), (b, g)
    sample = [(0, 0), (1, 1), (17, 0), (31, 1), (40, 0), (63, 1)]
    sub_b = sorted({b for b, _ in sample})
    # restrict the oracle's inputs to the sampled sequences
    case.K, case.V, case.Q = case.K[sub_b], case.V[sub_b], case.Q[sub_b]
    idx = {b: i for i, b in enumerate(sub_b)}
    sub = Case.__new__(Case)
    sub.__dict__.update(case.__dict__)
    sub.w = w.replace(batch=len(sub_b))
    sub._kc = None
    sel_s = sel_h[sub_b][:, None]
    out_s = from_device(out)[sub_b][:, None]
    sc_s = scores.cpu().numpy()[sub_b][:, None]
    st = check_rows(sub, sel_s, out_s, [(idx[b], 0, g) for b, g in sample], w.kv_len - 1, scores_gpu=sc_s)
    log(f"  sampled rows: {st}")


def test_ragged_batched_decode_workload():
    """The ragged batch (64 sequences of 16K .. 128K tokens) as the benchmark runs it: one ragged step call."""
    w = S.WORKLOADS["decode_b64_ragged"]
    lens = S.seq_lengths(w, 0)
    log(f"workload decode_b64_ragged: generating 2 x 4 GiB (lengths {min(lens)} .. {max(lens)})")
    case = Case(w, seed=0)
    log("workload decode_b64_ragged: running")
    hq, hkv, d, bs = w.n_q_heads, w.n_kv_heads, w.head_dim, w.block_size
    shape = qsa.shape_for(case.q, case.k, bs, w.top_k)
    one = qsa.make_shape(1, hq, hkv, d, bs, w.top_k, case.q.dtype)
    k_comp = torch.empty(w.batch, hkv, w.kv_len // bs, d, device="cuda")
    for b, n in enumerate(lens):
        qsa.qsa_compress_keys(one, case.k[b:b + 1], n - 1, k_comp[b:b + 1])
    q = case.q.view(w.batch, hq, d)
    kv_lens = torch.tensor(lens, dtype=torch.int32, device="cuda")
    sel = torch.empty(w.batch, hkv, w.top_k, dtype=torch.int32, device="cuda")
    scores = torch.empty(w.batch, hkv, w.top_k, dtype=torch.float32, device="cuda")
    out = torch.empty_like(q)
    qsa.qsa_decode_step_ragged(shape, q, case.k, case.v, k_comp, kv_lens, w.kv_len, sel, out, sel_scores=scores)
    torch.cuda.synchronize()
    sel_h, out_h, sc_h = sel.cpu().numpy(), from_device(out), scores.cpu().numpy()
    # sampled sequences: the shortest, the longest and a spread in between
    order = np.argsort(lens)
    pick = sorted({int(order[0]), int(order[-1]), *[int(order[i]) for i in (10, 25, 40, 55)]})
    case.K, case.V, case.Q = case.K[pick], case.V[pick], case.Q[pick]
    sub = Case.__new__(Case)
    sub.__dict__.update(case.__dict__)
    sub.w = w.replace(batch=len(pick), ragged=False)
    sub._kc = None
    for i, b in enumerate(pick):
        st = check_rows(sub, sel_h[pick][:, None], out_h[pick][:, None], [(i, 0, g) for g in range(hkv)], lens[b] - 1,
                        scores_gpu=sc_h[pick][:, None])
        log(f"  sequence {b} (length {lens[b]}): {st}")


def test_indexer_decode_workload():
    """The 32K decode with a learned indexer (64 dimensions, max over the heads), as the benchmark runs it."""
    from oracle import qsa_indexer as IX
    from oracle import qsa_oracle as O
    from qsa_check import check_selection_frame

    w = S.WORKLOADS["decode_32k_indexer"]
    case = Case(w, seed=0)
    b, hq, hkv, d, bs, k = w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.block_size, w.top_k
    G = hq // hkv
    w_q, w_k = S.indexer_weights(0, w.cfg_id, d, w.indexer_dim)
    shape = qsa.shape_for(case.q, case.k, bs, k)
    ix = qsa.make_indexer(w.indexer_dim, w.indexer_agg)
    k_comp = torch.empty(b, hkv, w.kv_len // bs, d, device="cuda")
    qsa.qsa_compress_keys(shape, case.k, w.kv_len, k_comp)
    k_idx = torch.empty(b, hkv, w.kv_len // bs, w.indexer_dim, device="cuda")
    qsa.qsa_indexer_keys(shape, ix, torch.from_numpy(w_k).cuda(), k_comp, w.kv_len, w.kv_len, k_idx)
    sel = torch.empty(b, 1, hkv, k, dtype=torch.int32, device="cuda")
    qsa.qsa_indexer_select(shape, ix, torch.from_numpy(w_q).cuda(), case.q, w.kv_len - 1, k_idx, w.kv_len, w.kv_len,
                           sel)
    q = case.q.view(b, hq, d)
    out = torch.empty_like(q)
    qsa.qsa_sparse_attn_decode(shape, q, case.k, case.v, w.kv_len, sel.view(b, hkv, k), out)
    torch.cuda.synchronize()
    p = w.kv_len - 1
    n_cand, forced = O.selection_frame(p, bs, False)
    ref_k = IX.indexer_keys(case.K, w_k.astype(np.float64), bs)
    sel_h, out_h = sel.cpu().numpy(), from_device(out)
    for g in range(hkv):
        qg = case.Q[0, 0, g * G:(g + 1) * G].astype(np.float64)
        sc = IX.indexer_scores(qg, w_q.astype(np.float64), ref_k[0, g], n_cand,
                               IX.default_indexer_scale(w.indexer_dim), w.indexer_agg)
        row = [int(x) for x in sel_h[0, 0, g]]
        st = check_selection_frame(row, sc, n_cand, forced, k)
        ref = O.attend_given_selection(qg, case.K[0, g], case.V[0, g], row, p, bs, O.default_scale(d))
        err = float(np.abs(out_h[0, g * G:(g + 1) * G] - ref).max())
        assert err <= 2e-2
        log(f"  KV head {g}: selection {st}, output error {err:.2e}")


def test_batched_decode_q8_workload():
    """The 64 x 128K batch with the attention reading the rotated 8-bit cache (sampled rows)."""
    from oracle import qsa_kv_q8 as Q
    from oracle import qsa_oracle as O

    w = S.WORKLOADS["decode_b64_128k_q8"]
    log("workload decode_b64_128k_q8: generating 2 x 4 GiB")
    case = Case(w, seed=0)
    hq, hkv, d, bs, k = w.n_q_heads, w.n_kv_heads, w.head_dim, w.block_size, w.top_k
    G = hq // hkv
    shape = qsa.shape_for(case.q, case.k, bs, k)
    kq, vq, ks, vs = qsa.kv_q8_buffers(case.k)
    qsa.qsa_kv_quantize(shape, case.k, case.v, w.kv_len, kq, vq, ks, vs)
    k_comp = torch.empty(w.batch, hkv, w.kv_len // bs, d, device="cuda")
    qsa.qsa_compress_keys(shape, case.k, w.kv_len, k_comp)
    sel = torch.empty(w.batch, 1, hkv, k, dtype=torch.int32, device="cuda")
    qsa.qsa_score_select(shape, case.q, w.kv_len - 1, k_comp, w.kv_len, w.kv_len, sel)
    q = case.q.view(w.batch, hq, d)
    out = torch.empty_like(q)
    qsa.qsa_sparse_attn_decode_q8(shape, q, kq, vq, ks, vs, w.kv_len, sel.view(w.batch, hkv, k), out)
    torch.cuda.synchronize()
    sel_h, out_h = sel.cpu().numpy(), from_device(out)
    for b in range(w.batch):  # planted blocks are found from the unrotated compressed keys
        for g in range(hkv):
            assert set(S.planted_blocks(w, 0, b, g).tolist()) <= set(sel_h[b, 0, g].tolist())
    p = w.kv_len - 1
    for b, g in [(0, 0), (17, 1), (63, 0)]:
        kq_o, ks_o = Q.quantize_cache(case.K[b, g])
        vq_o, vs_o = Q.quantize_cache(case.V[b, g])
        assert np.array_equal(kq[b, g].cpu().numpy(), kq_o), "codes"
        qg = case.Q[b, 0, g * G:(g + 1) * G].astype(np.float64)
        ref = Q.attend_q8(qg, kq_o, ks_o, vq_o, vs_o, [int(x) for x in sel_h[b, 0, g]], p, bs, O.default_scale(d))
        err = float(np.abs(out_h[b, g * G:(g + 1) * G] - ref).max())
        assert err <= 2e-2
        log(f"  row {(b, g)}: output error {err:.2e}")
