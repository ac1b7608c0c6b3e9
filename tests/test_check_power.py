"""Power of the output checks used by the GPU parity tests (CPU only).

The acceptance bound for bf16 outputs is 2e-2 absolute. On the sigma-0.5
workloads an output row averages about a thousand value rows and its
elements are only ~0.05 in size, so a kernel that gathers one wrong block
(or drops one) moves the output by ~1e-2: often inside 2e-2. The companion
row bound of ``qsa_check.check_output_row`` must reject every such mistake
while accepting what bf16 arithmetic legitimately does to a correct output
("Qwen4 in llama.cpp: Dissecting PR #27742", section "The PR's Numerical
Evidence Is Layered Correctly": compare the outputs and, separately, the
selected address set).

Every expected value here comes from the oracle: the correct output is the
oracle's attention over the oracle's selection, the mistaken outputs are
the oracle's attention over a selection with one block replaced or removed.
"""
from __future__ import annotations

import numpy as np
import pytest

import qsa_synth as S
from oracle import qsa_oracle as O
from qsa_check import BF16_ABS_TOL, OutputMismatch, check_output_row


def _bf16(x: np.ndarray) -> np.ndarray:
    return S.bf16_bits_to_f32(S.f32_to_bf16_bits(np.asarray(x, dtype=np.float32))).astype(np.float64)


def _attend_bf16_weights(q_group, K, V, sel, p, bs, scale):
    """Attention with every softmax weight rounded to bf16 before the weighted sums (numerator and
    denominator from the same rounded weights), the output rounded to bf16: the rounding steps of the
    bf16 attention kernels, applied to the oracle's float64 arithmetic."""
    pos = O.visible_positions(sel, p, bs)
    keys = K[pos].astype(np.float64)
    vals = V[pos].astype(np.float64)
    out = []
    for j in range(q_group.shape[0]):
        z = scale * (keys @ q_group[j])
        w = _bf16(np.exp(z - z.max()))
        out.append(_bf16((w @ vals) / w.sum()))
    return np.stack(out)


def _decode_row(w: S.Workload, g: int):
    q = S.gen_q(w, 0, 0)
    K = S.gen_kv(w, 0, S.TENSOR_K, 0, g, q)
    V = S.gen_kv(w, 0, S.TENSOR_V, 0, g)
    G, p = w.group, w.kv_len - 1
    qg = q[0, g * G:(g + 1) * G].astype(np.float64)
    scale = O.default_scale(w.head_dim)
    kc = O.compress_keys(K, w.block_size)
    n_cand, forced = O.selection_frame(p, w.block_size)
    scores = O.block_scores(qg, kc, n_cand, scale)
    sel = O.select_in_frame(scores, n_cand, forced, w.top_k)
    return qg, K, V, sel, scores, p, scale


def _mistakes(sel, scores, own):
    """Selections with one kept candidate block replaced (by each neighbour that is not kept, and by the
    best dropped block) or removed."""
    kept = [c for c in sel if 0 <= c < own]
    out = []
    dropped = [c for c in range(own) if c not in kept]
    best_dropped = max(dropped, key=lambda c: scores[c]) if dropped else -1
    for c in kept[:6]:
        for r in sorted({c - 1, c + 1, best_dropped}):
            if 0 <= r < own and r not in kept:
                s = sorted([x for x in kept if x != c] + [r, own])
                out.append(("replace", c, r, s + [-1] * (len(sel) - len(s))))
        s = sorted([x for x in kept if x != c] + [own])
        out.append(("drop", c, None, s + [-1] * (len(sel) - len(s))))
    return out


@pytest.mark.parametrize("g", [0, 1])
def test_row_bound_rejects_one_block_gather_errors_at_32k(g):
    """32K decode rows: every one-block mistake fails the companion bound; many pass the 2e-2 bound alone."""
    w = S.WORKLOADS["decode_32k"]
    qg, K, V, sel, scores, p, scale = _decode_row(w, g)
    ref = O.attend_given_selection(qg, K, V, sel, p, w.block_size, scale)
    # what bf16 arithmetic does to the correct output passes
    legit = _attend_bf16_weights(qg, K, V, sel, p, w.block_size, scale)
    assert check_output_row(legit, ref, "bf16") <= 0.5
    own = p // w.block_size
    mistakes = _mistakes(sel, scores, own)
    assert len(mistakes) >= 12
    inside_abs = 0
    for kind, c, r, bad_sel in mistakes:
        bad = O.attend_given_selection(qg, K, V, bad_sel, p, w.block_size, scale)
        inside_abs += int(np.abs(bad - ref).max() <= BF16_ABS_TOL)
        with pytest.raises(OutputMismatch):
            check_output_row(bad, ref, "bf16", where=f"{kind} {c}->{r}")
    # the reason the companion bound exists: the absolute bound alone misses some of these
    assert inside_abs > 0


def test_row_bound_rejects_gather_errors_in_prefill_rows():
    """Sampled rows of the 8K prefill (dense-regime and sparse rows): one-block mistakes fail the companion
    bound; bf16 rounding of the correct output passes it."""
    w = S.WORKLOADS["prefill_8k"]
    Qs, Ks, Vs = S.gen_all(w, 0, workers=1)
    Q, K, V = (S.as_f32(x, "bf16") for x in (Qs, Ks, Vs))
    G, bs, k = w.group, w.block_size, w.top_k
    scale = O.default_scale(w.head_dim)
    kc = O.compress_keys(K[0], bs)
    worst_legit = 0.0
    for t in (200, 1500, 4095, 8191):
        for g in range(2):
            qg = Q[0, t, g * G:(g + 1) * G].astype(np.float64)
            n_cand, forced = O.selection_frame(t, bs)
            sc = O.block_scores(qg, kc[g], n_cand, scale)
            sel = O.select_in_frame(sc, n_cand, forced, k)
            ref = O.attend_given_selection(qg, K[0, g], V[0, g], sel, t, bs, scale)
            worst_legit = max(worst_legit, check_output_row(
                _attend_bf16_weights(qg, K[0, g], V[0, g], sel, t, bs, scale), ref, "bf16"))
            if n_cand == 0:
                continue
            for kind, c, r, bad_sel in _mistakes(sel, sc, n_cand)[:4]:
                bad = O.attend_given_selection(qg, K[0, g], V[0, g], bad_sel, t, bs, scale)
                with pytest.raises(OutputMismatch):
                    check_output_row(bad, ref, "bf16", where=f"t={t} {kind} {c}->{r}")
    assert worst_legit <= 0.5


def test_row_bound_rejects_gather_errors_on_planted_rows():
    """A 64 x 128K-shaped row with planted blocks: dropping or replacing a planted block fails the bound."""
    w = S.WORKLOADS["decode_b64_128k"].replace(batch=1)
    q = S.gen_q(w, 0, 0)
    g = 1
    K = S.gen_kv(w, 0, S.TENSOR_K, 0, g, q)
    V = S.gen_kv(w, 0, S.TENSOR_V, 0, g)
    G, p, bs = w.group, w.kv_len - 1, w.block_size
    qg = q[0, g * G:(g + 1) * G].astype(np.float64)
    scale = O.default_scale(w.head_dim)
    own = p // bs
    sc = O.block_scores(qg, O.compress_keys(K, bs), own, scale)
    sel = O.select_in_frame(sc, own, own, w.top_k)
    planted = set(S.planted_blocks(w, 0, 0, g).tolist())
    assert planted <= set(sel)
    ref = O.attend_given_selection(qg, K, V, sel, p, bs, scale)
    assert check_output_row(_attend_bf16_weights(qg, K, V, sel, p, bs, scale), ref, "bf16") <= 0.5
    for kind, c, r, bad_sel in _mistakes(sel, sc, own):
        bad = O.attend_given_selection(qg, K, V, bad_sel, p, bs, scale)
        with pytest.raises(OutputMismatch):
            check_output_row(bad, ref, "bf16", where=f"{kind} {c}->{r}")


def test_fp32_row_bound_rejects_one_block_errors():
    """The 512-token fp32 workload: replacing one block fails the 1e-5 relative row bound."""
    w = S.WORKLOADS["prefill_512_f32"]
    Qs, Ks, Vs = S.gen_all(w, 0, workers=1)
    bs, k = w.block_size, w.top_k
    scale = O.default_scale(w.head_dim)
    kc = O.compress_keys(Ks[0], bs)
    for t in (300, 511):
        qg = Qs[0, t].astype(np.float64)
        n_cand, forced = O.selection_frame(t, bs)
        sc = O.block_scores(qg, kc[0], n_cand, scale)
        sel = O.select_in_frame(sc, n_cand, forced, k)
        ref = O.attend_given_selection(qg, Ks[0, 0], Vs[0, 0], sel, t, bs, scale)
        assert check_output_row(ref.astype(np.float32), ref, "f32") <= 0.1
        for kind, c, r, bad_sel in _mistakes(sel, sc, n_cand)[:3]:
            bad = O.attend_given_selection(qg, Ks[0, 0], Vs[0, 0], bad_sel, t, bs, scale)
            with pytest.raises(OutputMismatch):
                check_output_row(bad, ref, "f32")
