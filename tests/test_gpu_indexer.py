"""GPU parity of the learned-indexer selection against the fp64 indexer oracle.

Indexer keys are compared element by element within the float32 bound of a
block mean followed by a d-term projection; selections follow the acceptance
rule of ``qsa_check`` applied to the oracle's aggregated scores (exact kept
set wherever the cutoff gap exceeds 1e-3 relative); the kept candidates'
reported scores are compared within a float32 bound; the attention over the
indexer's selection is compared with the oracle's attention over the same
selection.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import block_sparse_long_compress_amd as qsa
import qsa_synth as S
from gpu_common import Case, from_device, log
from oracle import qsa_indexer as I
from oracle import qsa_oracle as O
from qsa_check import BF16_ABS_TOL, F32_REL_TOL, check_selection_frame

pytestmark = pytest.mark.gpu


def W(**kw) -> S.Workload:
    base = dict(name="idx", cfg_id=91, mode="decode", batch=2, kv_len=9000, n_q_heads=16, n_kv_heads=2,
                head_dim=128, block_size=64, top_k=16, dtype="bf16", sigma=0.5)
    base.update(kw)
    return S.Workload(**base)


CASES = [
    (W(), 64, I.AGG_SUM),
    (W(), 64, I.AGG_MAX),
    (W(), 64, I.AGG_SOFTMAX),
    (W(), 128, I.AGG_MAX),
    (W(kv_len=64 * 150, keep_tail=True, top_k=8), 64, I.AGG_SOFTMAX),                  # closes a block
    (W(dtype="f32", sigma=1.0, head_dim=64, block_size=32, top_k=12, kv_len=3001), 128, I.AGG_SUM),
    (W(n_q_heads=16, n_kv_heads=1, batch=3, kv_len=5000), 64, I.AGG_SOFTMAX),          # G = 16
    (W(mode="prefill", batch=1, kv_len=1000, block_size=32, top_k=8), 64, I.AGG_MAX),
    (W(mode="prefill", batch=1, kv_len=777, block_size=32, top_k=6), 128, I.AGG_SOFTMAX),
    (W(mode="decode", batch=1, kv_len=40, top_k=4), 64, I.AGG_SUM),                     # no candidate yet
    # k > 64: every score to the workspace, then the large selection's pick (the pool of all scores up to
    # 12288 candidates, the per-chunk lists beyond)
    (W(block_size=4, top_k=100, kv_len=4 * 2000 + 3), 64, I.AGG_SUM),
    (W(batch=1, block_size=4, top_k=513, kv_len=4 * 20000, keep_tail=True), 64, I.AGG_MAX),
    (W(batch=1, block_size=8, top_k=129, kv_len=8 * 14000 + 5), 128, I.AGG_SOFTMAX),
    (W(mode="prefill", batch=1, kv_len=700, block_size=4, top_k=100, head_dim=64), 64, I.AGG_SUM),
    (W(mode="decode", batch=1, kv_len=3, block_size=4, top_k=100), 64, I.AGG_SUM),      # no candidate yet
]


def case_id(c):
    w, dim, agg = c
    return f"{w.mode}-{w.dtype}-b{w.batch}-n{w.kv_len}-h{w.n_q_heads}x{w.n_kv_heads}-d{w.head_dim}-bs{w.block_size}" \
           f"-k{w.top_k}{'-tail' if w.keep_tail else ''}-i{dim}-{I.AGG_NAMES[agg]}"


@pytest.mark.parametrize("c", CASES, ids=[case_id(c) for c in CASES])
def test_indexer_selection_parity(c):
    w, dim, agg = c
    log(f"indexer {case_id(c)}")
    case = Case(w, seed=21, kv_cap=w.kv_len + 64)
    b, hq, hkv, d, bs, k = w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.block_size, w.top_k
    G = hq // hkv
    w_q, w_k = S.indexer_weights(21, w.cfg_id, d, dim)
    wq_d, wk_d = torch.from_numpy(w_q).cuda(), torch.from_numpy(w_k).cuda()
    shape = qsa.shape_for(case.q, case.k, bs, k, keep_tail=w.keep_tail)
    ix = qsa.make_indexer(dim, agg)
    nb_cap = case.kv_cap // bs
    k_comp = torch.full((b, hkv, nb_cap, d), float("nan"), device="cuda")
    qsa.qsa_compress_keys(shape, case.k, w.kv_len, k_comp)
    k_idx = torch.full((b, hkv, nb_cap, dim), float("nan"), device="cuda")
    qsa.qsa_indexer_keys(shape, ix, wk_d, k_comp, w.kv_len, case.kv_cap, k_idx)
    q_len, q_pos0 = w.q_len, w.q_pos0
    sel = torch.empty(b, q_len, hkv, k, dtype=torch.int32, device="cuda")
    scores = torch.empty(b, q_len, hkv, k, dtype=torch.float32, device="cuda")
    qsa.qsa_indexer_select(shape, ix, wq_d, case.q, q_pos0, k_idx, w.kv_len, case.kv_cap, sel, scores)
    torch.cuda.synchronize()

    # indexer keys: mean of Bs keys then a d-term projection, in float32
    nb = w.kv_len // bs
    ref_k = I.indexer_keys(case.K[:, :, :w.kv_len], w_k.astype(np.float64), bs)
    got_k = k_idx[:, :, :nb].cpu().numpy().astype(np.float64)
    Kb = np.abs(case.K[:, :, :nb * bs].astype(np.float64)).reshape(b, hkv, nb, bs, d).mean(axis=3)
    mag = Kb @ np.abs(w_k.astype(np.float64))
    assert np.all(np.abs(got_k - ref_k) <= (bs + d) * 2.0 ** -24 * mag + 1e-30), "indexer keys"

    sel_h, sc_h = sel.cpu().numpy(), scores.cpu().numpy()
    scale = I.default_indexer_scale(dim)
    stats = {"clear": 0, "ambiguous": 0}
    for bb in range(b):
        for t in range(q_len):
            p = q_pos0 + t
            n_cand, forced = O.selection_frame(p, bs, w.keep_tail)
            for g in range(hkv):
                qg = case.Q[bb, t, g * G:(g + 1) * G].astype(np.float64)
                per_head = I.head_scores(qg, w_q.astype(np.float64), ref_k[bb, g], n_cand, scale)
                agg_sc = I.aggregate(per_head, agg)
                row = [int(x) for x in sel_h[bb, t, g]]
                stats[check_selection_frame(row, agg_sc, n_cand, forced, k)] += 1
                kept = [x for x in row if 0 <= x < n_cand]
                got = sc_h[bb, t, g, :len(kept)].astype(np.float64)
                if agg == I.AGG_SOFTMAX:
                    tol = 1e-5 * G  # probabilities: float32 sums and exponentials
                else:
                    qi = np.abs(qg @ w_q.astype(np.float64)) * scale
                    tol = (d + dim + G + bs) * 2.0 ** -23 * (qi @ np.abs(ref_k[bb, g, kept]).T).max(axis=0) + 1e-30
                assert np.all(np.abs(got - agg_sc[kept]) <= tol), f"scores of row {(bb, t, g)}"
    log(f"  selections: {stats}")


def test_indexer_selection_drives_attention():
    """Decode attention over the indexer's selection matches the oracle's attention over the same blocks."""
    w = W(batch=2, kv_len=12000, top_k=16)
    case = Case(w, seed=22)
    b, hq, hkv, d, bs, k = w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.block_size, w.top_k
    G = hq // hkv
    w_q, w_k = S.indexer_weights(22, w.cfg_id, d, 64)
    shape = qsa.shape_for(case.q, case.k, bs, k)
    ix = qsa.make_indexer(64, I.AGG_MAX)
    k_comp = torch.empty(b, hkv, w.kv_len // bs, d, device="cuda")
    qsa.qsa_compress_keys(shape, case.k, w.kv_len, k_comp)
    k_idx = torch.empty(b, hkv, w.kv_len // bs, 64, device="cuda")
    qsa.qsa_indexer_keys(shape, ix, torch.from_numpy(w_k).cuda(), k_comp, w.kv_len, w.kv_len, k_idx)
    sel = torch.empty(b, 1, hkv, k, dtype=torch.int32, device="cuda")
    qsa.qsa_indexer_select(shape, ix, torch.from_numpy(w_q).cuda(), case.q, w.kv_len - 1, k_idx, w.kv_len, w.kv_len,
                           sel)
    q = case.q.view(b, hq, d)
    out = torch.empty_like(q)
    qsa.qsa_sparse_attn_decode(shape, q, case.k, case.v, w.kv_len, sel.view(b, hkv, k), out)
    torch.cuda.synchronize()
    out_h, sel_h = from_device(out), sel.cpu().numpy()
    worst = 0.0
    for bb in range(b):
        for g in range(hkv):
            qg = case.Q[bb, 0, g * G:(g + 1) * G].astype(np.float64)
            ref = O.attend_given_selection(qg, case.K[bb, g], case.V[bb, g], [int(x) for x in sel_h[bb, 0, g]],
                                           w.kv_len - 1, bs, O.default_scale(d))
            err = np.abs(out_h[bb, g * G:(g + 1) * G] - ref).max()
            worst = max(worst, float(err))
            assert err <= BF16_ABS_TOL
    log(f"  attention over the indexer's selection: max error {worst:.2e} (tolerance {BF16_ABS_TOL}; f32 rel {F32_REL_TOL})")


STEP_CASES = [
    (W(kv_len=9000, top_k=16), 64, I.AGG_SUM),                                          # no block closed
    (W(kv_len=64 * 150, top_k=16), 64, I.AGG_MAX),                                      # closes its own block
    (W(kv_len=64 * 150, keep_tail=True, top_k=8), 64, I.AGG_SOFTMAX),                   # closes a candidate
    (W(kv_len=64 * 150 + 1, keep_tail=True, top_k=8), 128, I.AGG_MAX),
    (W(n_q_heads=16, n_kv_heads=1, batch=3, kv_len=5000), 64, I.AGG_SOFTMAX),          # G = 16
    (W(head_dim=64, n_q_heads=8, block_size=16, top_k=24, kv_len=16 * 400), 128, I.AGG_SUM),  # gathered blocks
    (W(kv_len=64, top_k=4), 64, I.AGG_SUM),                                             # block 0 closed, no candidate
    (W(kv_len=1, top_k=1), 64, I.AGG_MAX),                                              # the first token
    (W(batch=130, kv_len=2000, top_k=16), 64, I.AGG_MAX),                               # 260 rows: 4-wave workgroups
]


@pytest.mark.parametrize("c", STEP_CASES, ids=[case_id(c) for c in STEP_CASES])
def test_indexer_decode_step(c):
    """The fused indexer decode step: caches and selections bit for bit those of the separate calls, selections
    and outputs against the oracle."""
    from qsa_check import check_output_row
    w, dim, agg = c
    log(f"indexer step {case_id(c)}")
    case = Case(w, seed=31, kv_cap=w.kv_len + 64)
    b, hq, hkv, d, bs, k = w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.block_size, w.top_k
    G, n, cap = hq // hkv, w.kv_len, case.kv_cap
    w_q, w_k = S.indexer_weights(31, w.cfg_id, d, dim)
    wq_d, wk_d = torch.from_numpy(w_q).cuda(), torch.from_numpy(w_k).cuda()
    shape = qsa.shape_for(case.q, case.k, bs, k, keep_tail=w.keep_tail)
    ix = qsa.make_indexer(dim, agg)
    # the caches as they stand before the new token
    k_comp = torch.full((b, hkv, cap // bs, d), float("nan"), device="cuda")
    k_idx = torch.full((b, hkv, cap // bs, dim), float("nan"), device="cuda")
    qsa.qsa_compress_keys(shape, case.k, n - 1, k_comp)
    qsa.qsa_indexer_keys(shape, ix, wk_d, k_comp, n - 1, cap, k_idx)
    # the separate calls
    k_comp2, k_idx2 = k_comp.clone(), k_idx.clone()
    blk = (n - 1) // bs
    qsa.qsa_compress_keys(shape, case.k, n, k_comp2, block_begin=blk)
    qsa.qsa_indexer_keys(shape, ix, wk_d, k_comp2, n, cap, k_idx2, block_begin=blk)
    q = case.q.view(b, 1, hq, d)
    sel2 = torch.empty(b, 1, hkv, k, dtype=torch.int32, device="cuda")
    sc2 = torch.empty(b, 1, hkv, k, dtype=torch.float32, device="cuda")
    qsa.qsa_indexer_select(shape, ix, wq_d, q, n - 1, k_idx2, n, cap, sel2, sc2)
    out2 = torch.empty(b, hq, d, dtype=case.q.dtype, device="cuda")
    qsa.qsa_sparse_attn_decode(shape, q.view(b, hq, d), case.k, case.v, n, sel2.view(b, hkv, k), out2)
    # the fused step
    sel = torch.empty(b, hkv, k, dtype=torch.int32, device="cuda")
    sc = torch.empty(b, hkv, k, dtype=torch.float32, device="cuda")
    out = torch.empty(b, hq, d, dtype=case.q.dtype, device="cuda")
    qsa.qsa_indexer_decode_step(shape, ix, wq_d, wk_d, q.view(b, hq, d), case.k, case.v, k_comp, k_idx, n, sel, out,
                                sel_scores=sc)
    torch.cuda.synchronize()
    nb = n // bs
    assert torch.equal(k_comp[:, :, :nb], k_comp2[:, :, :nb]), "compressed keys differ from the separate calls"
    assert torch.equal(k_idx[:, :, :nb], k_idx2[:, :, :nb]), "indexer keys differ from the separate calls"
    assert torch.equal(sel, sel2.view(b, hkv, k)), "selection differs from the separate calls"
    assert torch.equal(sc, sc2.view(b, hkv, k)), "selection scores differ from the separate calls"
    diff = (out.float() - out2.float()).abs().max().item()
    assert diff <= BF16_ABS_TOL, f"output differs from the separate calls by {diff}"
    # against the oracle
    p = n - 1
    n_cand, forced = O.selection_frame(p, bs, w.keep_tail)
    ref_k = I.indexer_keys(case.K[:, :, :n], w_k.astype(np.float64), bs)
    sel_h, out_h = sel.cpu().numpy(), from_device(out)
    scale = I.default_indexer_scale(dim)
    stats, worst = {"clear": 0, "ambiguous": 0}, 0.0
    for bb in range(b):
        for g in range(hkv):
            qg = case.Q[bb, 0, g * G:(g + 1) * G].astype(np.float64)
            agg_sc = I.aggregate(I.head_scores(qg, w_q.astype(np.float64), ref_k[bb, g], n_cand, scale), agg)
            row = [int(x) for x in sel_h[bb, g]]
            stats[check_selection_frame(row, agg_sc, n_cand, forced, k)] += 1
            ref = O.attend_given_selection(qg, case.K[bb, g], case.V[bb, g], row, p, bs, O.default_scale(d))
            worst = max(worst, check_output_row(out_h[bb, g * G:(g + 1) * G], ref, "bf16", where=f"row {(bb, g)}:"))
    log(f"  selections {stats}, output error over the row bound {worst:.3f}, against the separate calls {diff:.2e}")
