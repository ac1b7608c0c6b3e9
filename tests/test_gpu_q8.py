"""GPU parity of the rotated 8-bit K/V cache path.

Codes and float16 scales are integers decided in float32: they must equal
the oracle's bit for bit. The decode and prefill attention over the cache
are compared with the oracle's float64 attention over the same dequantized
cache and the same selection (bf16 output tolerance; the prefill rows also
against the per-row companion bound), and the decode reported against plain
bf16 attention for scale.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import block_sparse_long_compress_amd as qsa
import qsa_synth as S
from gpu_common import Case, from_device, log
from oracle import qsa_kv_q8 as Q
from oracle import qsa_oracle as O
from qsa_check import BF16_ABS_TOL, check_output_row

pytestmark = pytest.mark.gpu


def W(**kw) -> S.Workload:
    base = dict(name="q8", cfg_id=92, mode="decode", batch=2, kv_len=9000, n_q_heads=16, n_kv_heads=2,
                head_dim=128, block_size=64, top_k=16, dtype="bf16", sigma=0.5)
    base.update(kw)
    return S.Workload(**base)


CASES = [
    W(),                                                                  # several slices per row
    W(batch=3, kv_len=5000, top_k=64, block_size=32, head_dim=64),
    W(batch=1, kv_len=40000, top_k=16, n_q_heads=16, n_kv_heads=1),      # G = 16
    W(batch=40, kv_len=2000, top_k=8, block_size=128, n_q_heads=8),       # 80 rows
    W(batch=1, kv_len=50, top_k=4),                                       # own block only
    W(batch=64, kv_len=3000, top_k=16),                                   # 128 rows: 8-wave workgroups
    # blocks shorter than a 32-key unit: each unit gathers its rows from several entries
    W(batch=3, kv_len=3000, top_k=16, block_size=16),
    W(batch=1, kv_len=8 * 700 + 5, top_k=24, block_size=8, head_dim=64),
    W(batch=2, kv_len=4 * 2000 + 3, top_k=100, block_size=4),             # k > 64: several slices
]


def case_id(w):
    return f"b{w.batch}-n{w.kv_len}-h{w.n_q_heads}x{w.n_kv_heads}-d{w.head_dim}-bs{w.block_size}-k{w.top_k}"


def quantized(case):
    w = case.w
    shape = qsa.shape_for(case.q, case.k, w.block_size, w.top_k)
    kq, vq, ks, vs = qsa.kv_q8_buffers(case.k)
    qsa.qsa_kv_quantize(shape, case.k, case.v, w.kv_len, kq, vq, ks, vs)
    return shape, kq, vq, ks, vs


@pytest.mark.parametrize("w", CASES, ids=case_id)
def test_q8_codes_bit_exact(w):
    log(f"q8 codes {case_id(w)}")
    case = Case(w, seed=31)
    _, kq, vq, ks, vs = quantized(case)
    torch.cuda.synchronize()
    n = w.kv_len
    rng = np.random.default_rng(0)
    rows = [(b, g) for b in range(w.batch) for g in range(w.n_kv_heads)]
    if len(rows) > 8:
        rows = [rows[i] for i in sorted(rng.choice(len(rows), 8, replace=False))]
    for b, g in rows:
        for X, codes, sc in ((case.K, kq, ks), (case.V, vq, vs)):
            want_c, want_s = Q.quantize_cache(X[b, g, :n])
            got_c = codes[b, g, :n].cpu().numpy()
            got_s = sc[b, g, :n].cpu().numpy().view(np.uint16)
            assert np.array_equal(got_c, want_c), f"codes of {(b, g)}"
            assert np.array_equal(got_s, want_s.view(np.uint16)), f"scales of {(b, g)}"


def test_q8_incremental_quantization():
    """Quantizing positions in two calls (pos_begin) writes the same cache as one call."""
    w = W(batch=2, kv_len=3000)
    case = Case(w, seed=32)
    shape, kq, vq, ks, vs = quantized(case)
    kq2, vq2, ks2, vs2 = qsa.kv_q8_buffers(case.k)
    qsa.qsa_kv_quantize(shape, case.k, case.v, 1777, kq2, vq2, ks2, vs2)
    qsa.qsa_kv_quantize(shape, case.k, case.v, w.kv_len, kq2, vq2, ks2, vs2, pos_begin=1777)
    torch.cuda.synchronize()
    n = w.kv_len
    for a, c in ((kq, kq2), (vq, vq2), (ks, ks2), (vs, vs2)):
        assert torch.equal(a[:, :, :n], c[:, :, :n])


@pytest.mark.parametrize("w", CASES, ids=case_id)
def test_q8_decode_parity(w):
    log(f"q8 decode {case_id(w)}")
    case = Case(w, seed=33)
    b, hq, hkv, d, bs, k = w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.block_size, w.top_k
    G = hq // hkv
    shape, kq, vq, ks, vs = quantized(case)
    # the selection reads the unrotated compressed keys, as without the 8-bit cache
    k_comp = torch.empty(b, hkv, max(1, w.kv_len // bs), d, device="cuda")
    qsa.qsa_compress_keys(shape, case.k, w.kv_len, k_comp)
    q = case.q.view(b, hq, d)
    sel = torch.empty(b, 1, hkv, k, dtype=torch.int32, device="cuda")
    qsa.qsa_score_select(shape, case.q, w.kv_len - 1, k_comp, w.kv_len, w.kv_len, sel)
    out = torch.empty_like(q)
    qsa.qsa_sparse_attn_decode_q8(shape, q, kq, vq, ks, vs, w.kv_len, sel.view(b, hkv, k), out)
    out_bf = torch.empty_like(q)
    qsa.qsa_sparse_attn_decode(shape, q, case.k, case.v, w.kv_len, sel.view(b, hkv, k), out_bf)
    torch.cuda.synchronize()
    out_h, sel_h, bf_h = from_device(out), sel.cpu().numpy(), from_device(out_bf)
    rng = np.random.default_rng(1)
    rows = [(bb, g) for bb in range(b) for g in range(hkv)]
    if len(rows) > 12:
        rows = [rows[i] for i in sorted(rng.choice(len(rows), 12, replace=False))]
    worst, vs_plain = 0.0, 0.0
    p = w.kv_len - 1
    for bb, g in rows:
        qg = case.Q[bb, 0, g * G:(g + 1) * G].astype(np.float64)
        selr = [int(x) for x in sel_h[bb, 0, g]]
        kq_o, ks_o = Q.quantize_cache(case.K[bb, g, :w.kv_len])  # the oracle's own cache
        vq_o, vs_o = Q.quantize_cache(case.V[bb, g, :w.kv_len])
        ref = Q.attend_q8(qg, kq_o, ks_o, vq_o, vs_o, selr, p, bs, O.default_scale(d))
        got = out_h[bb, g * G:(g + 1) * G]
        err = float(np.abs(got - ref).max())
        assert err <= BF16_ABS_TOL, f"row {(bb, g)}: error {err:.3e}"
        worst = max(worst, err)
        vs_plain = max(vs_plain, float(np.abs(got - bf_h[bb, g * G:(g + 1) * G]).max()))
    log(f"  max error against the 8-bit oracle {worst:.2e}; largest difference from bf16 attention {vs_plain:.2e}")


PREFILL_CASES = [
    # (workload, first query row): prefill rows over the 8-bit cache, one workgroup per row
    (W(mode="prefill", batch=1, kv_len=700, top_k=6), 0),                                  # every row from 0
    (W(mode="prefill", batch=2, kv_len=1500, top_k=80, block_size=32, head_dim=64), 1100),  # k > 64: two chunks
    (W(mode="prefill", batch=1, kv_len=64 * 40 + 7, top_k=8, keep_tail=True), 64 * 40 - 60),  # keep-tail frame
    (W(mode="prefill", batch=1, kv_len=600, top_k=4, block_size=128, n_q_heads=16, n_kv_heads=1), 0),  # G = 16
    # gathered units: the released budget's blocks of 4 keys past a prefix, and blocks of 16 from row 0
    (W(mode="prefill", batch=1, kv_len=4 * 300 + 2, top_k=100, block_size=4), 4 * 300 - 40),
    (W(mode="prefill", batch=1, kv_len=16 * 60 + 3, top_k=8, block_size=16, head_dim=64), 0),
]


@pytest.mark.parametrize("c", PREFILL_CASES, ids=lambda c: f"{case_id(c[0])}-from{c[1]}")
def test_q8_prefill_parity(c):
    """Prefill rows over the 8-bit cache against the oracle's attention over its own dequantized cache and the
    GPU's selection (the bf16 selection path, checked elsewhere), on sampled rows of every (sequence, KV head):
    the 2e-2 acceptance bound and the per-row companion bound."""
    w, q_pos0 = c
    log(f"q8 prefill {case_id(w)} from {q_pos0}")
    case = Case(w, seed=34)
    b, hq, hkv, d, bs, k = w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.block_size, w.top_k
    G = hq // hkv
    shape, kq, vq, ks, vs = quantized(case)
    k_comp = torch.empty(b, hkv, max(1, w.kv_len // bs), d, device="cuda")
    qsa.qsa_compress_keys(shape, case.k, w.kv_len, k_comp)
    q_rows = case.q[:, q_pos0:].contiguous()
    n = w.kv_len - q_pos0
    sel = torch.empty(b, n, hkv, k, dtype=torch.int32, device="cuda")
    qsa.qsa_score_select(shape, q_rows, q_pos0, k_comp, w.kv_len, w.kv_len, sel)
    out = torch.empty_like(q_rows)
    qsa.qsa_sparse_attn_prefill_q8(shape, q_rows, kq, vq, ks, vs, q_pos0, sel, out)
    torch.cuda.synchronize()
    out_h, sel_h = from_device(out), sel.cpu().numpy()
    rng = np.random.default_rng(2)
    ts = sorted(set(rng.integers(0, n, 10).tolist()) | {0, n - 1})
    worst = 0.0
    for bb in range(b):
        for g in range(hkv):
            kq_o, ks_o = Q.quantize_cache(case.K[bb, g, :w.kv_len])  # the oracle's own cache
            vq_o, vs_o = Q.quantize_cache(case.V[bb, g, :w.kv_len])
            for t in ts:
                p = q_pos0 + t
                qg = case.Q[bb, p, g * G:(g + 1) * G].astype(np.float64)
                selr = [int(x) for x in sel_h[bb, t, g]]
                ref = Q.attend_q8(qg, kq_o, ks_o, vq_o, vs_o, selr, p, bs, O.default_scale(d))
                worst = max(worst, check_output_row(out_h[bb, t, g * G:(g + 1) * G], ref, "bf16",
                                                    where=f"row {(bb, p, g)}:"))
    log(f"  largest error over its row bound {worst:.3f}")


STEP_CASES = [
    W(),                                                                  # slices of the selection per row
    W(batch=64, kv_len=3000, top_k=16),                                   # 128 rows: one workgroup per row
    W(batch=2, kv_len=64 * 40, top_k=8, keep_tail=True),                  # the closed block competes
    W(batch=2, kv_len=64 * 40 + 1, top_k=8),                              # the new token opens a block
    W(batch=3, kv_len=5000, top_k=64, block_size=32, head_dim=64),
    W(batch=1, kv_len=40000, top_k=16, n_q_heads=16, n_kv_heads=1),      # G = 16
    W(batch=1, kv_len=50, top_k=4),                                       # own block only
    W(batch=1, kv_len=64 * 5000 + 3, top_k=16),                           # long rows: the scan split over workgroups
    # shapes without the fused kernel: the selection call, then the 8-bit decode attention
    W(batch=2, kv_len=4000, top_k=16, block_size=16),
    W(batch=2, kv_len=8 * 600, top_k=8, block_size=8, keep_tail=True),   # Bs 8, the closed block competes
    W(batch=1, kv_len=4 * 3000 + 1, top_k=64, block_size=4),
    W(batch=2, kv_len=20000, top_k=100),                                  # k > 64: the large selection
    W(batch=1, kv_len=4 * 30000, top_k=513, block_size=4, keep_tail=True),
]


@pytest.mark.parametrize("w", STEP_CASES, ids=lambda w: case_id(w) + ("-tail" if w.keep_tail else ""))
def test_q8_decode_step_parity(w):
    """The decode step over the 8-bit cache (fused where the kernel serves the shape, else the selection call and
    the 8-bit attention): the new position's codes and the closed block's compressed key as the separate calls
    write them, the bf16 step's selection, and the 8-bit oracle's attention over it."""
    log(f"q8 decode step {case_id(w)}")
    case = Case(w, seed=34, kv_cap=w.kv_len + 70)
    b, hq, hkv, d, bs, k = w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.block_size, w.top_k
    G, n = hq // hkv, w.kv_len
    shape = qsa.shape_for(case.q, case.k, bs, k, keep_tail=w.keep_tail)
    assert qsa.qsa_decode_step_fused(shape, n) == (bs >= 32 and k <= 64)
    kq, vq, ks, vs = qsa.kv_q8_buffers(case.k)
    qsa.qsa_kv_quantize(shape, case.k, case.v, n - 1, kq, vq, ks, vs)  # the step quantizes position n - 1
    nb_cap = case.kv_cap // bs
    k_comp = torch.full((b, hkv, nb_cap, d), float("nan"), device="cuda")
    qsa.qsa_compress_keys(shape, case.k, n - 1, k_comp)
    k_comp_bf = k_comp.clone()
    q = case.q.view(b, hq, d)
    sel = torch.empty(b, hkv, k, dtype=torch.int32, device="cuda")
    scores = torch.empty(b, hkv, k, dtype=torch.float32, device="cuda")
    out = torch.empty_like(q)
    qsa.qsa_decode_step_q8(shape, q, case.k, case.v, k_comp, kq, vq, ks, vs, n, sel, out, sel_scores=scores)
    # The fused kernel writes position n - 1 into the cache and its attention reads it back: a second step over
    # the cache as the first left it (the position already written) must give the same output bit for bit, which
    # fails if the first step's attention read the position before its codes were written.
    out_again = torch.empty_like(q)
    qsa.qsa_decode_step_q8(shape, q, case.k, case.v, k_comp.clone(), kq, vq, ks, vs, n, torch.empty_like(sel),
                           out_again)
    # references from the separate calls and the bf16 fused step
    kq2, vq2, ks2, vs2 = qsa.kv_q8_buffers(case.k)
    qsa.qsa_kv_quantize(shape, case.k, case.v, n, kq2, vq2, ks2, vs2)
    k_comp_ref = torch.full_like(k_comp, float("nan"))
    qsa.qsa_compress_keys(shape, case.k, n, k_comp_ref)
    sel_bf = torch.empty_like(sel)
    out_bf = torch.empty_like(q)
    qsa.qsa_decode_step(shape, q, case.k, case.v, k_comp_bf, n, sel_bf, out_bf)
    out_sep = torch.empty_like(q)
    qsa.qsa_sparse_attn_decode_q8(shape, q, kq2, vq2, ks2, vs2, n, sel, out_sep)
    torch.cuda.synchronize()
    for a, c in ((kq, kq2), (vq, vq2), (ks, ks2), (vs, vs2)):
        assert torch.equal(a[:, :, :n], c[:, :, :n]), "8-bit cache differs from the quantize call"
    assert torch.equal(out, out_again), "the step's output depends on whether the new position was in the cache"
    nb = n // bs
    assert torch.equal(k_comp[:, :, :nb], k_comp_ref[:, :, :nb]), "compressed keys differ from the compress call"
    if not (w.keep_tail and n % bs == 0):  # else the new block's score may round differently
        assert torch.equal(sel, sel_bf), "selection differs from the bf16 fused step"
    out_h, sel_h, sep_h = from_device(out), sel.cpu().numpy(), from_device(out_sep)
    assert np.abs(out_h - sep_h).max() <= BF16_ABS_TOL, "output differs from the separate 8-bit call"
    rng = np.random.default_rng(2)
    rows = [(bb, g) for bb in range(b) for g in range(hkv)]
    if len(rows) > 10:
        rows = [rows[i] for i in sorted(rng.choice(len(rows), 10, replace=False))]
    worst = 0.0
    for bb, g in rows:
        qg = case.Q[bb, 0, g * G:(g + 1) * G].astype(np.float64)
        kq_o, ks_o = Q.quantize_cache(case.K[bb, g, :n])  # the oracle's own cache
        vq_o, vs_o = Q.quantize_cache(case.V[bb, g, :n])
        ref = Q.attend_q8(qg, kq_o, ks_o, vq_o, vs_o, [int(x) for x in sel_h[bb, g]], n - 1, bs, O.default_scale(d))
        err = float(np.abs(out_h[bb, g * G:(g + 1) * G] - ref).max())
        assert err <= BF16_ABS_TOL, f"row {(bb, g)}: error {err:.3e}"
        worst = max(worst, err)
    log(f"  max error against the 8-bit oracle {worst:.2e}")


@pytest.mark.parametrize("c", [(W(mode="prefill", batch=2, kv_len=1500, top_k=8), 0),
                               (W(mode="prefill", batch=1, kv_len=64 * 40 + 7, top_k=16, keep_tail=True), 64 * 20),
                               (W(mode="prefill", batch=1, kv_len=800, top_k=6, head_dim=64, block_size=32), 0)],
                         ids=lambda c: f"{case_id(c[0])}-from{c[1]}")
def test_q8_prefill_tiled_and_rows(c):
    """Prefill over the 8-bit cache both ways: the tiled way (the codes rotated back into bf16 rows in the
    workspace, then the tiled bf16 kernel) and one row per workgroup over the codes (a workspace of zero bytes),
    each against the 8-bit oracle with the acceptance and companion bounds on sampled rows."""
    w, q_pos0 = c
    log(f"q8 prefill both ways {case_id(w)} from {q_pos0}")
    case = Case(w, seed=35)
    b, hq, hkv, d, bs, k = w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.block_size, w.top_k
    G = hq // hkv
    shape, kq, vq, ks, vs = quantized(case)
    n = w.kv_len - q_pos0
    assert qsa.qsa_workspace_bytes(shape, qsa.QSA_OP_PREFILL_Q8, n, w.kv_len) > 0, "the tiled way serves this shape"
    k_comp = torch.empty(b, hkv, max(1, w.kv_len // bs), d, device="cuda")
    qsa.qsa_compress_keys(shape, case.k, w.kv_len, k_comp)
    q_rows = case.q[:, q_pos0:].contiguous()
    sel = torch.empty(b, n, hkv, k, dtype=torch.int32, device="cuda")
    qsa.qsa_score_select(shape, q_rows, q_pos0, k_comp, w.kv_len, w.kv_len, sel)
    out_t, out_r = torch.empty_like(q_rows), torch.empty_like(q_rows)
    qsa.qsa_sparse_attn_prefill_q8(shape, q_rows, kq, vq, ks, vs, q_pos0, sel, out_t)
    qsa.qsa_sparse_attn_prefill_q8(shape, q_rows, kq, vq, ks, vs, q_pos0, sel, out_r,
                                   ws=torch.empty(0, dtype=torch.uint8, device="cuda"))
    torch.cuda.synchronize()
    sel_h = sel.cpu().numpy()
    rng = np.random.default_rng(3)
    ts = sorted(set(rng.integers(0, n, 8).tolist()) | {0, n - 1})
    worst = {"tiled": 0.0, "rows": 0.0}
    for name, out in (("tiled", out_t), ("rows", out_r)):
        out_h = from_device(out)
        for bb in range(b):
            for g in range(hkv):
                kq_o, ks_o = Q.quantize_cache(case.K[bb, g, :w.kv_len])
                vq_o, vs_o = Q.quantize_cache(case.V[bb, g, :w.kv_len])
                for t in ts:
                    p = q_pos0 + t
                    qg = case.Q[bb, p, g * G:(g + 1) * G].astype(np.float64)
                    ref = Q.attend_q8(qg, kq_o, ks_o, vq_o, vs_o, [int(x) for x in sel_h[bb, t, g]], p, bs,
                                      O.default_scale(d))
                    worst[name] = max(worst[name], check_output_row(out_h[bb, t, g * G:(g + 1) * G], ref, "bf16",
                                                                    where=f"{name} row {(bb, p, g)}:"))
    diff = (out_t.float() - out_r.float()).abs().max().item()
    assert diff <= BF16_ABS_TOL, f"the two ways differ by {diff}"
    log(f"  largest error over its row bound: tiled {worst['tiled']:.3f}, rows {worst['rows']:.3f}; "
        f"the two ways differ by at most {diff:.2e}")
