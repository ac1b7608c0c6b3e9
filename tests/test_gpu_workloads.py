"""GPU parity at the full sizes of the bf16 workloads.

The decode tests run the call the benchmark times on that workload
(``qsa_decode_step``, ``qsa_decode_step_q8`` or ``qsa_decode_step_ragged``, with
the compressed keys holding the blocks closed before the new token, exactly
as the benchmark sets them up, so the kernels and launch plans are the
benchmark's) and, on the same inputs, the separate select + attend calls.
Selections are checked on every row of every decode workload (the oracle
streams the 64 x 128K batch row by row) and of the 8K prefill; outputs on
every decode row (sampled rows of the 8-bit cache batch, whose oracle
rebuilds a row's whole 8-bit cache) and on sampled prefill rows. Every
output check applies the 2e-2 acceptance bound and the per-row companion
bound of ``qsa_check``.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import block_sparse_long_compress_amd as qsa
import qsa_synth as S
from gpu_common import Case, check_compress, check_rows, from_device, log

pytestmark = pytest.mark.gpu


def bench_decode_step(case: Case):
    """``qsa_decode_step`` as the benchmark runs it: k_comp holds every block closed before the new token,
    the step compresses the one it closes, selects and attends. Returns host (sel, out, scores) with a
    query-row axis, and the device k_comp."""
    w = case.w
    b, hq, hkv, d, bs, k = w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.block_size, w.top_k
    shape = qsa.shape_for(case.q, case.k, bs, k, keep_tail=w.keep_tail)
    k_comp = torch.full((b, hkv, case.kv_cap // bs, d), float("nan"), device="cuda")
    qsa.qsa_compress_keys(shape, case.k, w.kv_len - 1, k_comp)
    q = case.q.view(b, hq, d)
    sel = torch.empty(b, hkv, k, dtype=torch.int32, device="cuda")
    scores = torch.empty(b, hkv, k, dtype=torch.float32, device="cuda")
    out = torch.empty_like(q)
    ws = qsa.workspace(shape, qsa.QSA_OP_DECODE_STEP, 1, w.kv_len, "cuda")
    qsa.qsa_decode_step(shape, q, case.k, case.v, k_comp, w.kv_len, sel, out, sel_scores=scores, ws=ws)
    torch.cuda.synchronize()
    return sel.cpu().numpy()[:, None], from_device(out)[:, None], scores.cpu().numpy()[:, None], k_comp


def separate_decode(case: Case, k_comp):
    """The separate select + decode attention calls on compressed keys of every complete block."""
    w = case.w
    q = case.q.view(w.batch, w.n_q_heads, w.head_dim)
    out, sel, scores = qsa.decode(q, case.k, case.v, w.kv_len, w.block_size, w.top_k, k_comp, with_scores=True,
                                  keep_tail=w.keep_tail)
    torch.cuda.synchronize()
    return sel.cpu().numpy()[:, None], from_device(out)[:, None], scores.cpu().numpy()[:, None]


@pytest.mark.parametrize("name", ["decode_32k", "decode_1m", "decode_256k_r4"])
def test_decode_workload(name):
    """The step the benchmark times, then the separate calls, against the oracle on every row."""
    w = S.WORKLOADS[name]
    log(f"workload {name}: generating")
    case = Case(w, seed=0)
    shape = qsa.shape_for(case.q, case.k, w.block_size, w.top_k, keep_tail=w.keep_tail)
    log(f"workload {name}: decode step (fused kernel: {qsa.qsa_decode_step_fused(shape, w.kv_len)})")
    sel, out, scores, k_comp = bench_decode_step(case)
    check_compress(case, k_comp)
    rows = [(b, 0, g) for b in range(w.batch) for g in range(w.n_kv_heads)]
    st = check_rows(case, sel, out, rows, w.kv_len - 1, scores_gpu=scores)
    log(f"  decode step: {st}")
    log(f"workload {name}: separate calls")
    sel2, out2, scores2 = separate_decode(case, k_comp)
    st = check_rows(case, sel2, out2, rows, w.kv_len - 1, scores_gpu=scores2)
    log(f"  separate calls: {st}")
    if not (w.keep_tail and w.kv_len % w.block_size == 0):
        assert np.array_equal(sel, sel2), "the step and the separate calls select differently"


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
    sample = sorted(set(rng.integers(0, w.kv_len, 400).tolist()) | {0, 1, 63, 64, 1023, 1024, w.kv_len - 1})
    st = check_rows(case, sel, out, [(0, t, g) for t in sample for g in range(2)], 0, scores_gpu=scores)
    log(f"  sampled outputs: {st}")


def test_prefill_256k_r4_tail_workload():
    """The released budget at full context: the last 512 query rows of a 262144-token prefill (ratio 4,
    top-513 with the partial-tail slot). Every row scores 65536 candidates, so the selection takes the
    tiled large-k score pass with per-chunk lists, and the bf16 attention one query row per workgroup.
    Every row's selection and sampled rows' outputs against the oracle."""
    w = S.WORKLOADS["prefill_256k_r4_tail"]
    log("workload prefill_256k_r4_tail: generating")
    case = Case(w, seed=0)
    out, sel, k_comp, scores = qsa.prefill(case.q, case.k, case.v, w.block_size, w.top_k, q_pos0=w.q_pos0,
                                           with_scores=True, keep_tail=True)
    torch.cuda.synchronize()
    sel, out, scores = sel.cpu().numpy(), from_device(out), scores.cpu().numpy()
    check_compress(case, k_comp)
    rows = [(0, t, g) for t in range(w.q_len) for g in range(w.n_kv_heads)]
    st = check_rows(case, sel, out, rows, w.q_pos0, scores_gpu=scores, check_output=False)
    log(f"  selections of all {len(rows)} rows: {st}")
    rng = np.random.default_rng(0)
    sample = sorted(set(rng.integers(0, w.q_len, 24).tolist()) | {0, 15, 16, w.q_len - 1})
    st = check_rows(case, sel, out, [(0, t, g) for t in sample for g in range(2)], w.q_pos0)
    log(f"  sampled outputs: {st}")


@pytest.fixture(scope="module")
def batch_128k():
    w = S.WORKLOADS["decode_b64_128k"]
    log("workload decode_b64_128k: generating 2 x 4 GiB")
    return Case(w, seed=0)


def test_batched_decode_planted_workload(batch_128k):
    """The 64 x 128K batch through the benchmark's step: every planted block kept, and every one of the
    128 rows' selections and outputs against the oracle."""
    case = batch_128k
    w = case.w
    log("workload decode_b64_128k: decode step")
    sel, out, scores, k_comp = bench_decode_step(case)
    for b in range(w.batch):
        for g in range(2):
            planted = set(S.planted_blocks(w, 0, b, g).tolist())
            assert planted <= set(sel[b, 0, g].tolist()), (b, g)
    check_compress(case, k_comp)
    rows = [(b, 0, g) for b in range(w.batch) for g in range(w.n_kv_heads)]
    st = check_rows(case, sel, out, rows, w.kv_len - 1, scores_gpu=scores)
    log(f"  decode step, all {len(rows)} rows: {st}")


def test_batched_decode_separate_calls(batch_128k):
    """The same batch through the separate select + decode attention calls (sampled output rows)."""
    case = batch_128k
    w = case.w
    shape = qsa.shape_for(case.q, case.k, w.block_size, w.top_k)
    k_comp = torch.empty(w.batch, 2, w.kv_len // w.block_size, w.head_dim, device="cuda")
    qsa.qsa_compress_keys(shape, case.k, w.kv_len, k_comp)
    sel, out, scores = separate_decode(case, k_comp)
    rows = [(b, 0, g) for b in range(w.batch) for g in range(w.n_kv_heads)]
    st = check_rows(case, sel, out, rows, w.kv_len - 1, scores_gpu=scores, check_output=False)
    log(f"  separate calls, selections of all rows: {st}")
    sample = [(0, 0, 0), (1, 0, 1), (17, 0, 0), (31, 0, 1), (40, 0, 0), (63, 0, 1)]
    st = check_rows(case, sel, out, sample, w.kv_len - 1)
    log(f"  separate calls, sampled outputs: {st}")


def test_ragged_batched_decode_workload():
    """The ragged batch (64 sequences of 16K .. 128K tokens) as the benchmark runs it: one ragged step call;
    every sequence's selections and outputs at its own length."""
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
    sel_h, out_h, sc_h = sel.cpu().numpy()[:, None], from_device(out)[:, None], scores.cpu().numpy()[:, None]
    worst = 0.0
    for b, n in enumerate(lens):
        st = check_rows(case, sel_h, out_h, [(b, 0, g) for g in range(hkv)], n - 1, scores_gpu=sc_h)
        worst = max(worst, st["max_err_over_row_bound"])
        if b % 16 == 0:
            log(f"  sequence {b} (length {n}): {st}")
    log(f"  all {w.batch} sequences checked; largest error over the row bound {worst:.3f}")


def test_indexer_decode_workload():
    """The 32K decode with a learned indexer (64 dimensions, max over the heads), as the benchmark runs it: one
    fused indexer decode step."""
    from oracle import qsa_indexer as IX
    from oracle import qsa_oracle as O
    from qsa_check import check_output_row, check_selection_frame

    w = S.WORKLOADS["decode_32k_indexer"]
    case = Case(w, seed=0)
    b, hq, hkv, d, bs, k = w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.block_size, w.top_k
    G = hq // hkv
    w_q, w_k = S.indexer_weights(0, w.cfg_id, d, w.indexer_dim)
    shape = qsa.shape_for(case.q, case.k, bs, k)
    ix = qsa.make_indexer(w.indexer_dim, w.indexer_agg)
    # the caches hold the blocks closed before the new token; the step (one qsa_indexer_decode_step call, as the
    # benchmark times it) adds the block the token closes, selects and attends
    wk_d = torch.from_numpy(w_k).cuda()
    k_comp = torch.full((b, hkv, w.kv_len // bs, d), float("nan"), device="cuda")
    qsa.qsa_compress_keys(shape, case.k, w.kv_len - 1, k_comp)
    k_idx = torch.full((b, hkv, w.kv_len // bs, w.indexer_dim), float("nan"), device="cuda")
    qsa.qsa_indexer_keys(shape, ix, wk_d, k_comp, w.kv_len - 1, w.kv_len, k_idx)
    q = case.q.view(b, hq, d)
    sel = torch.empty(b, 1, hkv, k, dtype=torch.int32, device="cuda")
    out = torch.empty_like(q)
    qsa.qsa_indexer_decode_step(shape, ix, torch.from_numpy(w_q).cuda(), wk_d, q, case.k, case.v, k_comp, k_idx,
                                w.kv_len, sel.view(b, hkv, k), out)
    torch.cuda.synchronize()
    assert not torch.isnan(k_comp).any() and not torch.isnan(k_idx).any(), "every block's keys written"
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
        ratio = check_output_row(out_h[0, g * G:(g + 1) * G], ref, "bf16", where=f"KV head {g}:")
        log(f"  KV head {g}: selection {st}, output error over the row bound {ratio:.3f}")


def test_batched_decode_q8_workload():
    """The 64 x 128K batch with the attention reading the rotated 8-bit cache, through the benchmark's call
    (``qsa_decode_step_q8``: quantize the new position, compress, select and attend in one kernel): codes of
    the new position as the quantize call writes them, every row's selection against the oracle, outputs of
    sampled rows against the 8-bit oracle; then the separate 8-bit attention call."""
    from oracle import qsa_kv_q8 as Q
    from oracle import qsa_oracle as O
    from qsa_check import check_output_row

    w = S.WORKLOADS["decode_b64_128k_q8"]
    log("workload decode_b64_128k_q8: generating 2 x 4 GiB")
    case = Case(w, seed=0)
    b_n, hq, hkv, d, bs, k = w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.block_size, w.top_k
    G, n = hq // hkv, w.kv_len
    shape = qsa.shape_for(case.q, case.k, bs, k)
    assert qsa.qsa_decode_step_fused(shape, n)
    kq, vq, ks, vs = qsa.kv_q8_buffers(case.k)
    qsa.qsa_kv_quantize(shape, case.k, case.v, n - 1, kq, vq, ks, vs)  # the step quantizes position n - 1
    k_comp = torch.full((b_n, hkv, n // bs, d), float("nan"), device="cuda")
    qsa.qsa_compress_keys(shape, case.k, n - 1, k_comp)
    q = case.q.view(b_n, hq, d)
    sel = torch.empty(b_n, hkv, k, dtype=torch.int32, device="cuda")
    scores = torch.empty(b_n, hkv, k, dtype=torch.float32, device="cuda")
    out = torch.empty_like(q)
    ws = qsa.workspace(shape, qsa.QSA_OP_DECODE_STEP, 1, n, "cuda")
    qsa.qsa_decode_step_q8(shape, q, case.k, case.v, k_comp, kq, vq, ks, vs, n, sel, out, sel_scores=scores, ws=ws)
    out_sep = torch.empty_like(q)
    qsa.qsa_sparse_attn_decode_q8(shape, q, kq, vq, ks, vs, n, sel, out_sep)
    torch.cuda.synchronize()
    sel_h, out_h, sep_h, sc_h = sel.cpu().numpy(), from_device(out), from_device(out_sep), scores.cpu().numpy()
    check_compress(case, k_comp)
    for b in range(b_n):  # planted blocks are found from the unrotated compressed keys
        for g in range(hkv):
            assert set(S.planted_blocks(w, 0, b, g).tolist()) <= set(sel_h[b, g].tolist())
    rows = [(b, 0, g) for b in range(b_n) for g in range(hkv)]
    st = check_rows(case, sel_h[:, None], out_h[:, None], rows, n - 1, scores_gpu=sc_h[:, None], check_output=False)
    log(f"  selections of all {len(rows)} rows: {st}")
    p = n - 1
    worst = 0.0
    for b, g in [(0, 0), (17, 1), (40, 0), (63, 1)]:
        kq_o, ks_o = Q.quantize_cache(case.K[b, g])
        vq_o, vs_o = Q.quantize_cache(case.V[b, g])
        assert np.array_equal(kq[b, g].cpu().numpy(), kq_o), "codes"
        assert np.array_equal(vq[b, g].cpu().numpy(), vq_o), "codes"
        qg = case.Q[b, 0, g * G:(g + 1) * G].astype(np.float64)
        ref = Q.attend_q8(qg, kq_o, ks_o, vq_o, vs_o, [int(x) for x in sel_h[b, g]], p, bs, O.default_scale(d))
        for got, what in ((out_h, "step"), (sep_h, "separate call")):
            r = check_output_row(got[b, g * G:(g + 1) * G], ref, "bf16", rel=Q8_ROW_REL_TOL, where=f"{what} {(b, g)}:")
            worst = max(worst, r)
    log(f"  sampled outputs (step and separate call): largest error over the row bound {worst:.3f}")


# The 8-bit attention rounds the rotated query heads to bf16 and widens the codes with their float16 scales
# before the products; its outputs match the 8-bit oracle within the bf16 companion bound's terms plus the
# rotation back of an output whose rotated form carries the bf16 rounding of the weights. A factor of four
# over the bf16 bound covers it.
Q8_ROW_REL_TOL = 2.0 ** -5
