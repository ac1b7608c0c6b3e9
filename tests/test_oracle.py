"""Pins of the fp64 oracle against things other than itself.

Each test fixes one part of the oracle with an independent formulation:
brute force on tiny inputs, dense causal attention from a library routine,
closed forms, the pages' printed regime, Hadamard invariance, block size 1,
planted blocks. A mistake anywhere in compress / score / select / attend
(a dropped term, a wrong sign or index, a transposed operand, a wrong tie
order, an off-by-one in the own block) fails at least one of them.
"""
from __future__ import annotations

import itertools
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import qsa_oracle as O
import qsa_synth as S
from qsa_check import SelectionMismatch, check_selection, jaccard

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- brute force

def brute_compress(K, Bs):
    b_n, g_n, N, d = K.shape
    out = np.zeros((b_n, g_n, N // Bs, d))
    for b in range(b_n):
        for g in range(g_n):
            for c in range(N // Bs):
                for e in range(d):
                    acc = 0.0
                    for u in range(Bs):
                        acc += float(K[b, g, c * Bs + u, e])
                    out[b, g, c, e] = acc / Bs
    return out


def brute_scores(qg, kc, n_cand, scale):
    out = []
    for c in range(n_cand):
        acc = 0.0
        for j in range(qg.shape[0]):
            for e in range(qg.shape[1]):
                acc += float(qg[j, e]) * float(kc[c, e])
        out.append(scale * acc)
    return out


def brute_select(scores, own, top_k):
    """The unique subset whose every member beats every non-member (score, then smaller id)."""
    slots = min(top_k - 1, own)

    def beats(x, y):
        return scores[x] > scores[y] or (scores[x] == scores[y] and x < y)

    valid = []
    for subset in itertools.combinations(range(own), slots):
        rest = [y for y in range(own) if y not in subset]
        if all(beats(x, y) for x in subset for y in rest):
            valid.append(subset)
    assert len(valid) == 1
    kept = sorted(list(valid[0]) + [own])
    return kept + [-1] * (top_k - len(kept))


def brute_attend(q, K, V, sel, p, Bs, scale):
    """Masked dense attention: all N logits, -inf outside the visible set."""
    own = p // Bs
    N = K.shape[0]
    logits = np.full(N, -np.inf)
    for t in range(N):
        blk = t // Bs
        visible = (blk in sel and blk < own) or (own * Bs <= t <= p)
        if visible:
            logits[t] = scale * sum(float(q[e]) * float(K[t, e]) for e in range(K.shape[1]))
    w = np.exp(logits - logits.max())
    return (w[:, None] * V.astype(np.float64)).sum(0) / w.sum()


def _tiny_inputs(rng, b, N, hq, hkv, d, integer):
    if integer:  # small integers make scores exact and ties frequent
        Q = rng.integers(-2, 3, size=(b, N, hq, d)).astype(np.float64)
        K = rng.integers(-2, 3, size=(b, hkv, N, d)).astype(np.float64)
    else:
        Q = rng.standard_normal((b, N, hq, d))
        K = rng.standard_normal((b, hkv, N, d))
    V = rng.standard_normal((b, hkv, N, d))
    return Q, K, V


TINY = [(N, Bs, k) for N in (7, 16, 40) for Bs in (1, 2, 4) for k in (1, 2, 3, 64)
        if not (N == 40 and Bs == 1 and k in (3,))]


@pytest.mark.parametrize("N,Bs,k", TINY)
def test_brute_force_tiny(N, Bs, k):
    """Every oracle step equals an independently written brute force, over many seeds, with ties."""
    b, hq, hkv, d = 2, 4, 2, 4
    G = hq // hkv
    seeds = range(6) if N == 40 else range(12)
    for seed in seeds:
        rng = np.random.default_rng([seed, N, Bs, k])
        Q, K, V = _tiny_inputs(rng, b, N, hq, hkv, d, integer=(seed % 2 == 0))
        scale = 0.5 if seed % 3 == 0 else O.default_scale(d)
        kc = O.compress_keys(K, Bs)
        np.testing.assert_allclose(kc, brute_compress(K, Bs), rtol=0, atol=1e-13)
        out, sel = O.qsa_prefill(Q, K, V, Bs, k, scale=scale)
        for bb in range(b):
            for t in range(N):
                own = t // Bs
                for g in range(hkv):
                    qg = Q[bb, t, g * G:(g + 1) * G]
                    sc = brute_scores(qg, kc[bb, g], own, scale)
                    np.testing.assert_allclose(O.block_scores(qg, kc[bb, g], own, scale), sc, rtol=1e-13, atol=1e-13)
                    if math.comb(own, min(k - 1, own)) <= 5000:
                        assert list(sel[bb, t, g]) == brute_select(sc, own, k)
                    for j in range(G):
                        ref = brute_attend(qg[j], K[bb, g], V[bb, g], list(sel[bb, t, g]), t, Bs, scale)
                        np.testing.assert_allclose(out[bb, t, g * G + j], ref, rtol=1e-12, atol=1e-13)


# ------------------------------------------- the keep_tail frame, by brute force

def brute_select_tail(scores, p, Bs, top_k):
    """Released-budget frame from first principles: blocks whose last position is at most p compete."""
    complete = [c for c in range(p // Bs + 1) if (c + 1) * Bs - 1 <= p]
    slots = min(top_k - 1, len(complete))

    def beats(x, y):
        return scores[x] > scores[y] or (scores[x] == scores[y] and x < y)

    valid = [sub for sub in itertools.combinations(complete, slots)
             if all(beats(x, y) for x in sub for y in complete if y not in sub)]
    assert len(valid) == 1
    kept = list(valid[0])
    if (p + 1) % Bs:  # positions past the last complete block: their block is always kept
        kept.append(p // Bs)
    kept = sorted(kept)
    return kept + [-1] * (top_k - len(kept))


def brute_attend_tail(q, K, V, sel, p, Bs, scale):
    """Logits of every position <= p that lies in a selected block or past the last complete block."""
    last_complete_end = (p + 1) // Bs * Bs
    logits = np.full(K.shape[0], -np.inf)
    for t in range(p + 1):
        if t // Bs in sel or t >= last_complete_end:
            logits[t] = scale * sum(float(q[e]) * float(K[t, e]) for e in range(K.shape[1]))
    w = np.exp(logits - logits.max())
    return (w[:, None] * V.astype(np.float64)).sum(0) / w.sum()


def test_keep_tail_needs_two_slots():
    """With top_k = 1 the keep_tail frame would leave a complete-block row with nothing to attend."""
    with pytest.raises(ValueError):
        O.select_in_frame(np.zeros(4), 4, None, 1)


@pytest.mark.parametrize("N,Bs,k", [(N, Bs, k) for N in (9, 24) for Bs in (1, 2, 4) for k in (2, 3, 5)])
def test_brute_force_tiny_keep_tail(N, Bs, k):
    """The keep_tail frame equals a brute force written from its definition, ties included."""
    b, hq, hkv, d = 1, 4, 2, 4
    G = hq // hkv
    for seed in range(8):
        rng = np.random.default_rng([seed, N, Bs, k, 7])
        Q, K, V = _tiny_inputs(rng, b, N, hq, hkv, d, integer=(seed % 2 == 0))
        scale = O.default_scale(d)
        kc = O.compress_keys(K, Bs)
        out, sel = O.qsa_prefill(Q, K, V, Bs, k, keep_tail=True)
        for t in range(N):
            n_complete = (t + 1) // Bs
            for g in range(hkv):
                qg = Q[0, t, g * G:(g + 1) * G]
                sc = brute_scores(qg, kc[0, g], n_complete, scale)
                if math.comb(n_complete, min(k - 1, n_complete)) <= 5000:
                    assert list(sel[0, t, g]) == brute_select_tail(sc, t, Bs, k)
                for j in range(G):
                    ref = brute_attend_tail(qg[j], K[0, g], V[0, g], list(sel[0, t, g]), t, Bs, scale)
                    np.testing.assert_allclose(out[0, t, g * G + j], ref, rtol=1e-12, atol=1e-13)


def test_keep_tail_matches_default_while_own_block_fills():
    """The two frames differ only for rows whose own block is complete ((p + 1) % Bs == 0)."""
    rng = np.random.default_rng(11)
    N, Bs, k = 120, 4, 6
    Q = rng.standard_normal((1, N, 4, 8))
    K = rng.standard_normal((1, 2, N, 8))
    V = rng.standard_normal((1, 2, N, 8))
    out_d, sel_d = O.qsa_prefill(Q, K, V, Bs, k)
    out_t, sel_t = O.qsa_prefill(Q, K, V, Bs, k, keep_tail=True)
    filling = np.array([(t + 1) % Bs != 0 for t in range(N)])
    np.testing.assert_array_equal(sel_d[0, filling], sel_t[0, filling])
    np.testing.assert_array_equal(out_d[0, filling], out_t[0, filling])
    assert (sel_d[0, ~filling] != sel_t[0, ~filling]).any()


def test_keep_tail_drops_a_complete_own_block():
    """A complete own block that scores lowest is not visible, not even to its last query (SDPA mask)."""
    d, Bs = 4, 2
    Q = np.zeros((1, 4, 1, d))
    Q[0, :, 0, 0] = 1.0
    K = np.zeros((1, 1, 4, d))
    K[0, 0, :2, 0] = 2.0    # block 0 points along the query
    K[0, 0, 2:, 0] = -2.0   # block 1 points away from it
    K[0, 0, :, 1] = [0.3, -0.1, 0.7, 0.2]
    V = np.arange(16, dtype=np.float64).reshape(1, 1, 4, d)
    out, sel = O.qsa_prefill(Q, K, V, Bs, 2, keep_tail=True)
    assert list(sel[0, 3, 0]) == [0, -1]
    mask = np.array([[True, True, False, False]])
    ref = _sdpa(Q[:, 3:4], K, V, O.default_scale(d), mask=mask)
    np.testing.assert_allclose(out[0, 3], ref[0, 0], rtol=0, atol=1e-12)
    _, sel_default = O.qsa_prefill(Q, K, V, Bs, 2)
    assert list(sel_default[0, 3, 0]) == [0, 1]  # the default frame keeps it


def test_tie_break_smaller_index():
    scores = np.array([1.0, 3.0, 3.0, 2.0, 3.0])
    assert O.select_blocks(scores, 5, 3) == [1, 2, 5]
    assert O.select_blocks(scores, 5, 4) == [1, 2, 4, 5]
    assert O.select_blocks(scores, 5, 1) == [5]
    assert O.select_blocks(scores, 5, 9) == [0, 1, 2, 3, 4, 5, -1, -1, -1]


# ------------------------------------------------- library routine: dense SDPA

def _sdpa(Q, K, V, scale, mask=None, causal=False):
    G = Q.shape[2] // K.shape[1]
    q = torch.from_numpy(np.ascontiguousarray(Q.transpose(0, 2, 1, 3)))
    k = torch.from_numpy(K).repeat_interleave(G, dim=1)
    v = torch.from_numpy(V).repeat_interleave(G, dim=1)
    o = F.scaled_dot_product_attention(q, k, v, attn_mask=None if mask is None else torch.from_numpy(mask),
                                       is_causal=causal, scale=scale)
    return o.numpy().transpose(0, 2, 1, 3)


@pytest.mark.parametrize("N,Bs,k,G", [(512, 32, 16, 2), (96, 8, 12, 4), (64, 4, 17, 1), (200, 16, 13, 8)])
def test_dense_equivalence_below_budget(N, Bs, k, G):
    """When top_k covers every causal block the result is dense causal attention.

    "Qwen4 in llama.cpp: Dissecting PR #27742", section "QSA Is an
    Address-Selection Problem...": below the budget nothing can be discarded
    and sparse must equal dense.
    """
    assert k >= (N - 1) // Bs + 1
    rng = np.random.default_rng(N + k)
    hkv = 2 if G < 8 else 1
    Q = rng.standard_normal((1, N, hkv * G, 64 if N == 512 else 16))
    K = rng.standard_normal((1, hkv, N, Q.shape[-1]))
    V = rng.standard_normal((1, hkv, N, Q.shape[-1]))
    scale = O.default_scale(Q.shape[-1])
    out, sel = O.qsa_prefill(Q, K, V, Bs, k)
    ref = _sdpa(Q, K, V, scale, causal=True)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)
    for t in range(N):
        own = t // Bs
        assert list(sel[0, t, 0][: own + 1]) == list(range(own + 1))


@pytest.mark.parametrize("d", [16, 64, 128])
def test_default_scale_is_the_library_default(d):
    """The oracle's default scale (scale=None) is the one scaled dot-product attention uses by default:
    torch's SDPA with ``scale=None`` takes 1/sqrt(head_dim) itself, so nothing of the oracle's is
    passed to the reference ("Qwen Model Architecture: From Transformer to MoE...", section "Attention:
    what the model is 'looking at'": dot-product relevance, then a weighted sum of V)."""
    rng = np.random.default_rng(d)
    N, Bs = 96, 8
    k = N // Bs + 1  # dense regime: every causal block kept
    Q = rng.standard_normal((1, N, 4, d))
    K = rng.standard_normal((1, 2, N, d))
    V = rng.standard_normal((1, 2, N, d))
    out, _ = O.qsa_prefill(Q, K, V, Bs, k, scale=None)
    G = 2
    q = torch.from_numpy(np.ascontiguousarray(Q.transpose(0, 2, 1, 3)))
    kk = torch.from_numpy(K).repeat_interleave(G, dim=1)
    vv = torch.from_numpy(V).repeat_interleave(G, dim=1)
    ref = F.scaled_dot_product_attention(q, kk, vv, is_causal=True).numpy().transpose(0, 2, 1, 3)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)
    # a decode row too: the last row's output with the default scale
    o_dec, _ = O.qsa_decode(Q[:, -1], K, V, N, Bs, k, scale=None)
    np.testing.assert_allclose(o_dec, ref[:, -1], rtol=0, atol=1e-12)
    # and the value itself, worked by hand for d = 64: 1/sqrt(64) = 1/8
    assert O.default_scale(64) == 0.125


def test_default_scale_changes_the_output():
    """The pin above has power: a scale of 1/d or sqrt(d) instead of 1/sqrt(d) moves the output."""
    rng = np.random.default_rng(5)
    N, Bs, d = 64, 8, 64
    Q = rng.standard_normal((1, N, 2, d))
    K = rng.standard_normal((1, 1, N, d))
    V = rng.standard_normal((1, 1, N, d))
    ref, _ = O.qsa_prefill(Q, K, V, Bs, N // Bs + 1, scale=None)
    for wrong in (1.0 / d, math.sqrt(d), 1.0):
        bad, _ = O.qsa_prefill(Q, K, V, Bs, N // Bs + 1, scale=wrong)
        assert np.abs(bad - ref).max() > 1e-2


@pytest.mark.parametrize("N,Bs,k", [(64, 4, 17), (99, 8, 13), (50, 1, 51)])
def test_dense_equivalence_keep_tail(N, Bs, k):
    """keep_tail: with top_k - 1 slots for every complete block, sparse equals dense causal attention."""
    assert k - 1 >= N // Bs
    rng = np.random.default_rng(N * k)
    Q = rng.standard_normal((1, N, 4, 16))
    K = rng.standard_normal((1, 2, N, 16))
    V = rng.standard_normal((1, 2, N, 16))
    out, _ = O.qsa_prefill(Q, K, V, Bs, k, keep_tail=True)
    np.testing.assert_allclose(out, _sdpa(Q, K, V, O.default_scale(16), causal=True), rtol=0, atol=1e-12)


def test_dense_rows_of_sparse_config():
    """Rows whose own block index is below top_k are dense even when later rows are sparse."""
    rng = np.random.default_rng(3)
    N, Bs, k, d = 256, 16, 4, 16
    Q = rng.standard_normal((1, N, 4, d))
    K = rng.standard_normal((1, 2, N, d))
    V = rng.standard_normal((1, 2, N, d))
    out, _ = O.qsa_prefill(Q, K, V, Bs, k)
    ref = _sdpa(Q, K, V, O.default_scale(d), causal=True)
    dense_rows = k * Bs
    np.testing.assert_allclose(out[:, :dense_rows], ref[:, :dense_rows], rtol=0, atol=1e-12)
    assert np.abs(out[:, dense_rows:] - ref[:, dense_rows:]).max() > 1e-3


def test_top1_is_block_local_causal():
    """top_k = 1 keeps only the own block: SDPA with a block-diagonal causal mask."""
    rng = np.random.default_rng(7)
    N, Bs, d = 100, 8, 16
    Q = rng.standard_normal((2, N, 4, d))
    K = rng.standard_normal((2, 2, N, d))
    V = rng.standard_normal((2, 2, N, d))
    out, sel = O.qsa_prefill(Q, K, V, Bs, 1)
    t = np.arange(N)
    mask = (t[:, None] // Bs == t[None, :] // Bs) & (t[None, :] <= t[:, None])
    ref = _sdpa(Q, K, V, O.default_scale(d), mask=mask)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)
    assert (sel[..., 0] == (t // Bs)[None, :, None]).all()


def test_first_row_returns_first_value():
    rng = np.random.default_rng(11)
    Q = rng.standard_normal((1, 5, 4, 8))
    K = rng.standard_normal((1, 2, 5, 8))
    V = rng.standard_normal((1, 2, 5, 8))
    out, _ = O.qsa_prefill(Q, K, V, 2, 2)
    np.testing.assert_array_equal(out[0, 0, :2], np.repeat(V[0, 0, :1], 2, axis=0))
    np.testing.assert_array_equal(out[0, 0, 2:], np.repeat(V[0, 1, :1], 2, axis=0))


# ------------------------------------------------------------- closed forms

@pytest.mark.parametrize("Bs,k", [(4, 3), (8, 5), (16, 16), (32, 4)])
def test_visible_width_closed_form(Bs, k):
    """|V(p)| = min(p+1, (k-1)*Bs + (p mod Bs) + 1), candidates = p // Bs, for every row."""
    rng = np.random.default_rng(Bs * 100 + k)
    N = 12 * Bs + 5
    Q = rng.standard_normal((1, N, 2, 8))
    K = rng.standard_normal((1, 1, N, 8))
    res = O.qsa_rows(Q, K, K, Bs, k)
    for (b, t, g), (sel, scores, _) in res.items():
        assert len(scores) == t // Bs
        width = len(O.visible_positions(sel, t, Bs))
        assert width == min(t + 1, (k - 1) * Bs + (t % Bs) + 1)


def test_pages_released_regime():
    """The regime the pages print: budget 2048 tokens, ratio 4, bound 2051, 65536 blocks at 262144."""
    with open(os.path.join(GOLDEN, "pages_regime.json")) as f:
        gold = json.load(f)
    Bs = gold["compression_ratio"]
    k = gold["indexer_budget_tokens"] // Bs + 1  # scored slots + the own block
    bound = gold["visible_width_bound"]
    n_ctx = gold["context_tokens"]
    assert O.compress_keys(np.zeros((n_ctx, 1), dtype=np.float32), Bs).shape[0] == gold["compressed_blocks"]
    rng = np.random.default_rng(0)
    widths = {}
    for p in list(range(0, 2100)) + list(range(4090, 4110)) + list(range(n_ctx - 8, n_ctx)):
        own = p // Bs
        sel = O.select_blocks(rng.standard_normal(own), own, k)
        widths[p] = len(O.visible_positions(sel, p, Bs))
        if p + 1 <= bound:
            assert widths[p] == p + 1  # dense regime: nothing can be discarded
        if p % Bs <= Bs - 2:  # own block still filling: the pages' bound holds exactly
            assert widths[p] <= min(p + 1, bound)
        else:  # own block complete: it stays the forced block (one more token than the bound)
            assert widths[p] == min(p + 1, bound + 1)
    assert max(w for p, w in widths.items() if p % Bs <= Bs - 2) == bound
    assert len(O.block_scores(np.zeros((1, 1)), np.zeros((gold["compressed_blocks"], 1)),
                              (n_ctx - 1) // Bs, 1.0)) == gold["compressed_blocks"] - 1


def test_pages_released_regime_keep_tail():
    """keep_tail reproduces the printed bound exactly: width <= min(n_kv, 2051) at every position,
    dense up to 2051 cached positions, 2051 reached, and all 65536 blocks compete at 262144."""
    with open(os.path.join(GOLDEN, "pages_regime.json")) as f:
        gold = json.load(f)
    Bs = gold["compression_ratio"]
    k = gold["indexer_budget_tokens"] // Bs + 1  # budget blocks + the slot of the partial tail
    bound = gold["visible_width_bound"]
    n_ctx = gold["context_tokens"]
    rng = np.random.default_rng(1)
    widest = 0
    for p in list(range(0, 2100)) + list(range(4090, 4110)) + list(range(n_ctx - 8, n_ctx)):
        n_kv = p + 1
        n_cand, forced = O.selection_frame(p, Bs, keep_tail=True)
        sel = O.select_in_frame(rng.standard_normal(n_cand), n_cand, forced, k)
        width = len(O.visible_positions(sel, p, Bs))
        assert width <= min(n_kv, bound)
        if n_kv <= bound:
            assert width == n_kv  # below the budget nothing can be discarded
        widest = max(widest, width)
    assert widest == bound
    assert O.selection_frame(n_ctx - 1, Bs, keep_tail=True) == (gold["compressed_blocks"], None)


# ------------------------------------------------------------ invariances

def test_score_identity_group_sum():
    """Sum of per-head scores equals the score of the summed query (two code paths, one value)."""
    rng = np.random.default_rng(5)
    qg = rng.standard_normal((8, 128))
    kc = rng.standard_normal((300, 128)) * 0.06
    a = O.block_scores(qg, kc, 300, 0.125)
    b = 0.125 * (kc @ qg.sum(0))
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-14)


def test_block_size_one_is_token_topk():
    """Block size 1: compressed keys are the keys, selection is a per-token top-(k-1) (numpy lexsort)."""
    rng = np.random.default_rng(9)
    N, d, k = 60, 8, 7
    Q = rng.standard_normal((1, N, 2, d))
    K = rng.standard_normal((1, 1, N, d))
    V = rng.standard_normal((1, 1, N, d))
    np.testing.assert_array_equal(O.compress_keys(K, 1), K)
    out, sel = O.qsa_prefill(Q, K, V, 1, k)
    scale = O.default_scale(d)
    for t in range(N):
        s = scale * (K[0, 0, :t] @ Q[0, t].sum(0))
        top = np.lexsort((np.arange(t), -s))[: min(k - 1, t)]
        expect = sorted(list(top) + [t])
        assert list(sel[0, t, 0][: len(expect)]) == expect


@pytest.mark.parametrize("d", json.load(open(os.path.join(GOLDEN, "hadamard_identity.json")))["orders"])
def test_hadamard_rotation_invariance(d):
    """Q' = QH, K' = KH, V' = VH (H orthonormal Hadamard): same selection, O' = O H."""
    from scipy.linalg import hadamard

    H = hadamard(d).astype(np.float64) / math.sqrt(d)
    np.testing.assert_allclose(H @ H, np.eye(d), atol=1e-14)  # its own inverse
    rng = np.random.default_rng(d)
    N, Bs, k = 96, 8, 4
    Q = rng.standard_normal((1, N, 4, d))
    K = rng.standard_normal((1, 2, N, d))
    V = rng.standard_normal((1, 2, N, d))
    out, sel = O.qsa_prefill(Q, K, V, Bs, k)
    out_r, sel_r = O.qsa_prefill(Q @ H, K @ H, V @ H, Bs, k)
    np.testing.assert_array_equal(sel, sel_r)
    np.testing.assert_allclose(out_r, out @ H, rtol=0, atol=1e-12)
    np.testing.assert_allclose(out_r @ H, out, rtol=0, atol=1e-12)


def test_decode_equals_last_prefill_row():
    rng = np.random.default_rng(13)
    N, Bs, k = 77, 8, 3
    Q = rng.standard_normal((2, N, 4, 8))
    K = rng.standard_normal((2, 2, N + 9, 8))  # cache capacity beyond kv_len is ignored
    V = rng.standard_normal((2, 2, N + 9, 8))
    out_p, sel_p = O.qsa_prefill(Q, K[:, :, :N], V[:, :, :N], Bs, k)
    out_d, sel_d = O.qsa_decode(Q[:, -1], K, V, N, Bs, k)
    np.testing.assert_array_equal(sel_d, sel_p[:, -1])
    np.testing.assert_array_equal(out_d, out_p[:, -1])


# --------------------------------------------------------- planted workload

@pytest.mark.parametrize("b,g", [(0, 0), (63, 1)])
def test_planted_blocks_are_selected(b, g):
    """Batched-decode workload: all 8 planted blocks of a row are kept (margin ~16 noise sigmas)."""
    w = S.WORKLOADS["decode_b64_128k"]
    q = S.gen_q(w, 0, b)
    K = S.gen_kv(w, 0, S.TENSOR_K, b, g, q)
    kc = O.compress_keys(K, w.block_size)
    own = (w.kv_len - 1) // w.block_size
    G = w.group
    scores = O.block_scores(q[0, g * G:(g + 1) * G], kc, own, O.default_scale(w.head_dim))
    sel = O.select_blocks(scores, own, w.top_k)
    planted = S.planted_blocks(w, 0, b, g)
    assert len(planted) == 8 and planted.max() < own
    assert set(planted.tolist()) <= set(sel)
    assert sel[-1] == own


# --------------------------------------------------- generator and checker

def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal(100000) * 10 ** rng.uniform(-6, 6, 100000)).astype(np.float32)
    x[:4] = [1.00390625, 1.01171875, -1.00390625, 3.0e38]  # exact ties and a large value
    ours = S.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)


def test_generator_slices_are_independent_and_deterministic():
    w = S.WORKLOADS["decode_32k"].replace(kv_len=4096)
    Q, K, V = S.gen_all(w, seed=3)
    Q2, K2, V2 = S.gen_all(w, seed=3, workers=1)
    np.testing.assert_array_equal(K, K2)
    np.testing.assert_array_equal(V, V2)
    np.testing.assert_array_equal(S.f32_to_bf16_bits(S.gen_kv(w, 3, S.TENSOR_V, 0, 1)), V[0, 1])
    assert not np.array_equal(K[0, 0], K[0, 1])
    assert Q.dtype == np.uint16 and Q.shape == (1, 1, 16, 128)


def test_selection_checker_rejects_planted_mistakes():
    """Mistakes planted in the oracle's selection must be caught by the acceptance rule."""
    rng = np.random.default_rng(21)
    scores = rng.standard_normal(50)
    own, k = 50, 6
    good = O.select_blocks(scores, own, k)
    assert check_selection(good, scores, own, k) == "clear"
    order = np.argsort(-scores)
    swapped = sorted([int(c) for c in order[: k - 2]] + [int(order[k - 1]), own])
    with pytest.raises(SelectionMismatch):
        check_selection(swapped, scores, own, k)
    with pytest.raises(SelectionMismatch):
        check_selection(sorted(good[:-1]) + [own - 1], scores, own, k)  # own block dropped
    with pytest.raises(SelectionMismatch):
        check_selection(list(reversed(good)), scores, own, k)
    near = scores.copy()
    near[order[k - 1]] = near[order[k - 2]] * (1 - 1e-5)  # boundary within the gap: both answers valid
    alt = sorted([int(c) for c in order[: k - 2]] + [int(order[k - 1]), own])
    assert check_selection(alt, near, own, k) == "ambiguous"
    assert jaccard([1, 2, 3, -1], [2, 3, 4]) == 0.5
