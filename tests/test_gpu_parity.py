"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Selections must satisfy the acceptance rule of ``qsa_check`` (bit-exact on
clear rows), compressed keys must stay within the float32 summation bound,
outputs within 2e-2 absolute (bf16) or 1e-5 relative per row (fp32) of the
oracle's attention over the GPU's own (validated) selection.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import block_sparse_long_compress_amd as qsa
import qsa_synth as S
from oracle import qsa_oracle as O
from gpu_common import Case, check_compress, check_rows, from_device, log

pytestmark = pytest.mark.gpu


def W(**kw) -> S.Workload:
    base = dict(name="case", cfg_id=90, mode="prefill", batch=1, kv_len=512, n_q_heads=16, n_kv_heads=2,
                head_dim=128, block_size=64, top_k=4, dtype="bf16", sigma=0.5)
    base.update(kw)
    return S.Workload(**base)


def run_prefill(case: Case, q_pos0: int = 0, q_rows=None):
    """Full prefill path on rows [q_pos0, kv_len); returns host (sel, out, scores, k_comp)."""
    w = case.w
    q = case.q if q_rows is None else case.q[:, q_rows].contiguous()
    out, sel, k_comp, scores = qsa.prefill(q, case.k, case.v, w.block_size, w.top_k, q_pos0=q_pos0, with_scores=True,
                                           keep_tail=w.keep_tail)
    torch.cuda.synchronize()
    return sel.cpu().numpy(), from_device(out), scores.cpu().numpy(), k_comp


def all_rows(w: S.Workload, q_len: int):
    return [(b, t, g) for b in range(w.batch) for t in range(q_len) for g in range(w.n_kv_heads)]


PREFILL_CASES = [
    # tiny fp32 prefill (the 512-token workload), sparse and dense top-k
    S.WORKLOADS["prefill_512_f32"],
    S.WORKLOADS["prefill_512_f32"].replace(top_k=16),
    # bf16, several query tiles, ragged last block and last tile, batch 2
    W(batch=2, kv_len=1000, top_k=4),
    W(kv_len=777, top_k=8, head_dim=64, block_size=32),
    W(kv_len=600, top_k=3, block_size=128),
    W(kv_len=700, top_k=1),                                   # own block only
    W(kv_len=700, top_k=64, block_size=32),                    # k beyond the candidates: dense
    W(kv_len=3000, top_k=24, block_size=32),                   # top_k > 16: threshold-select tile path
    W(kv_len=530, n_q_heads=4, n_kv_heads=4, top_k=5),         # G = 1
    W(kv_len=530, n_q_heads=8, n_kv_heads=4, top_k=5),         # G = 2
    W(kv_len=530, n_q_heads=8, n_kv_heads=2, top_k=5),         # G = 4
    W(kv_len=530, n_q_heads=16, n_kv_heads=1, top_k=5),        # G = 16
    # d = 64 with every kernel variant (G decides waves and CGs per wave)
    W(kv_len=900, head_dim=64, n_q_heads=8, n_kv_heads=2, top_k=6),                   # G = 4
    W(kv_len=650, head_dim=64, n_q_heads=4, n_kv_heads=2, top_k=5, block_size=128),   # G = 2
    W(kv_len=530, head_dim=64, n_q_heads=2, n_kv_heads=2, top_k=4),                   # G = 1
    W(kv_len=530, head_dim=64, n_q_heads=16, n_kv_heads=1, top_k=4, block_size=64),   # G = 16
    W(kv_len=300, dtype="f32", sigma=1.0, top_k=3, head_dim=128),
    W(kv_len=15, top_k=2),                                     # shorter than one block
    # keep_tail frame: a complete own block competes (tile select, MFMA attention)
    W(kv_len=777, top_k=6, keep_tail=True),
    W(batch=2, kv_len=640, top_k=3, head_dim=64, block_size=32, keep_tail=True),
    # blocks shorter than 32 keys and k > 64 (float32 attention, large-k selection)
    W(kv_len=300, dtype="f32", sigma=1.0, head_dim=64, n_q_heads=4, n_kv_heads=2, block_size=8, top_k=5),
    W(kv_len=700, dtype="f32", sigma=1.0, head_dim=64, n_q_heads=2, n_kv_heads=1, block_size=4, top_k=100,
      keep_tail=True),
    # bf16, one query row per workgroup: blocks shorter than 32 keys (gathered units), k > 64
    W(kv_len=300, head_dim=64, n_q_heads=4, n_kv_heads=2, block_size=8, top_k=5),
    W(kv_len=1500, block_size=16, top_k=20),
    W(kv_len=700, head_dim=64, n_q_heads=2, n_kv_heads=1, block_size=4, top_k=100, keep_tail=True),
    W(kv_len=3000, block_size=64, top_k=80),                                    # k > 64, whole-block units
    # the released budget (512 blocks of 4 keys plus the tail, keep-tail frame): dense up to 2051 cached
    # positions, the first discard at 2052 (rows 2050 and 2051), sparse rows after
    W(kv_len=2600, block_size=4, top_k=513, keep_tail=True),
]


def case_id(w: S.Workload) -> str:
    return (f"{w.dtype}-b{w.batch}-n{w.kv_len}-h{w.n_q_heads}x{w.n_kv_heads}-d{w.head_dim}-bs{w.block_size}"
            f"-k{w.top_k}" + ("-tail" if w.keep_tail else ""))


@pytest.mark.parametrize("w", PREFILL_CASES, ids=case_id)
def test_prefill_parity(w):
    log(f"prefill parity {w}")
    case = Case(w, seed=1, kv_cap=w.kv_len + 40)
    sel, out, scores, k_comp = run_prefill(case)
    check_compress(case, k_comp)
    st = check_rows(case, sel, out, all_rows(w, w.kv_len), 0, scores_gpu=scores)
    log(f"  {st}")


CHUNKED_CASES = [
    (W(batch=2, kv_len=900, top_k=6), 333),
    # long prefixes: several 128-candidate rounds of the row selection path
    (W(batch=1, kv_len=64 * 300 + 5, top_k=16), 64 * 300 - 100),
    (W(batch=2, kv_len=32 * 400 + 31, top_k=9, head_dim=64, block_size=32, keep_tail=True), 32 * 400 - 70),
    (W(batch=1, kv_len=64 * 260, top_k=12, dtype="f32", sigma=1.0), 64 * 260 - 129),
    # the released budget, rows past a long prefix (one query row per workgroup)
    (W(batch=1, kv_len=4 * 5000 + 2, top_k=513, block_size=4, keep_tail=True), 4 * 5000 - 300),
    # k > 64 past the pick pool (12288 candidates): the tiled score pass writes per-chunk lists
    # (3 tiles of 16 rows, the last ragged)
    (W(batch=1, kv_len=4 * 20000 + 2, top_k=513, block_size=4, keep_tail=True), 4 * 20000 - 40),
    (W(batch=2, kv_len=4 * 14000 + 1, top_k=129, block_size=4, head_dim=64), 4 * 14000 - 19),
]


@pytest.mark.parametrize("c", CHUNKED_CASES, ids=lambda c: f"{case_id(c[0])}-from{c[1]}")
def test_chunked_prefill_parity(c):
    """Query rows [q_pos0, kv_len) over a cache that already holds the earlier keys."""
    w, q_pos0 = c
    case = Case(w, seed=2)
    sel, out, scores, _ = run_prefill(case, q_pos0=q_pos0, q_rows=slice(q_pos0, w.kv_len))
    # oracle rows are indexed by absolute position: shift the query view
    case.Q = case.Q[:, q_pos0:]
    st = check_rows(case, sel, out, all_rows(w, w.kv_len - q_pos0), q_pos0, scores_gpu=scores)
    log(f"chunked prefill {st}")


DECODE_CASES = [
    W(mode="decode", batch=3, kv_len=1000, top_k=8),
    W(mode="decode", batch=2, kv_len=64 * 16, top_k=16),        # exactly dense
    W(mode="decode", batch=2, kv_len=50, top_k=4),              # only the own block
    W(mode="decode", batch=2, kv_len=5000, top_k=1),
    W(mode="decode", batch=1, kv_len=9000, top_k=64, block_size=32),
    W(mode="decode", batch=5, kv_len=4099, top_k=12, head_dim=64, block_size=128),
    W(mode="decode", batch=2, kv_len=3000, n_q_heads=16, n_kv_heads=1, top_k=7),
    W(mode="decode", batch=2, kv_len=3000, n_q_heads=2, n_kv_heads=2, top_k=7),
    W(mode="decode", batch=2, kv_len=2222, dtype="f32", sigma=1.0, top_k=5),
    # 128 rows: one 8-wave workgroup per row over the whole selection
    W(mode="decode", batch=64, kv_len=3000, top_k=16),
    W(mode="decode", batch=64, kv_len=1001, top_k=9, block_size=4, head_dim=64),     # gathered units
    # keep_tail: own block complete (it competes) and still filling
    W(mode="decode", batch=2, kv_len=64 * 40, top_k=8, keep_tail=True),
    W(mode="decode", batch=2, kv_len=64 * 40 + 17, top_k=8, keep_tail=True),
    # blocks of 4, 8, 16 keys: several blocks per 32-key MFMA step
    W(mode="decode", batch=2, kv_len=3001, top_k=9, block_size=4),
    W(mode="decode", batch=2, kv_len=2050, top_k=17, block_size=8, head_dim=64),
    W(mode="decode", batch=1, kv_len=5003, top_k=12, block_size=16, keep_tail=True),
    # k > 64: every score to the workspace, radix-selected cutoff
    W(mode="decode", batch=2, kv_len=4 * 4096 + 3, top_k=129, block_size=4),             # pool of all scores
    W(mode="decode", batch=1, kv_len=60001, top_k=513, block_size=4, keep_tail=True),     # pool of chunk lists
    W(mode="decode", batch=1, kv_len=4 * 30000, top_k=513, block_size=4, keep_tail=True, n_kv_heads=1,
      n_q_heads=8),
    W(mode="decode", batch=1, kv_len=2051, top_k=513, block_size=4, keep_tail=True),      # dense: 2051 positions
    W(mode="decode", batch=1, kv_len=2052, top_k=513, block_size=4, keep_tail=True),      # first discard
    W(mode="decode", batch=1, kv_len=64 * 3000 + 10, top_k=200, block_size=64),
    W(mode="decode", batch=1, kv_len=9000, top_k=100, block_size=8, dtype="f32", sigma=1.0, keep_tail=True),
]


def run_decode(case: Case):
    w = case.w
    b, hq, d = w.batch, w.n_q_heads, w.head_dim
    shape = qsa.shape_for(case.q, case.k, w.block_size, w.top_k, keep_tail=w.keep_tail)
    k_comp = torch.full((b, w.n_kv_heads, case.kv_cap // w.block_size, d), float("nan"), device="cuda")
    qsa.qsa_compress_keys(shape, case.k, w.kv_len, k_comp)
    q = case.q.view(b, hq, d)
    out, sel, scores = qsa.decode(q, case.k, case.v, w.kv_len, w.block_size, w.top_k, k_comp, with_scores=True,
                                  keep_tail=w.keep_tail)
    torch.cuda.synchronize()
    return sel.cpu().numpy()[:, None], from_device(out)[:, None], scores.cpu().numpy()[:, None], k_comp


@pytest.mark.parametrize("w", DECODE_CASES, ids=case_id)
def test_decode_parity(w):
    log(f"decode parity {w}")
    case = Case(w, seed=3, kv_cap=w.kv_len + 100)
    sel, out, scores, k_comp = run_decode(case)
    check_compress(case, k_comp)
    rows = [(b, 0, g) for b in range(w.batch) for g in range(w.n_kv_heads)]
    st = check_rows(case, sel, out, rows, w.kv_len - 1, scores_gpu=scores)
    log(f"  {st}")


def test_decode_matches_last_prefill_row():
    w = W(batch=2, kv_len=1500, top_k=6)
    case = Case(w, seed=4)
    sel_p, out_p, _, k_comp = run_prefill(case)
    q = case.q[:, -1].contiguous()
    out_d, sel_d = qsa.decode(q, case.k, case.v, w.kv_len, w.block_size, w.top_k, k_comp)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(sel_d.cpu().numpy(), sel_p[:, -1])
    np.testing.assert_allclose(from_device(out_d), out_p[:, -1], rtol=0, atol=2e-2)


def test_bitwise_determinism():
    w = W(batch=2, kv_len=2100, top_k=6)
    case = Case(w, seed=5)
    a = run_prefill(case)
    b = run_prefill(case)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])
    np.testing.assert_array_equal(a[2], b[2])
    d = W(mode="decode", batch=4, kv_len=70000, top_k=16)
    dc = Case(d, seed=6)
    x, y = run_decode(dc), run_decode(dc)
    np.testing.assert_array_equal(x[0], y[0])
    np.testing.assert_array_equal(x[1], y[1])


STEP_DETERMINISM = [
    W(mode="decode", batch=1, kv_len=300000, top_k=16),                                   # 64 scan parts per row
    W(mode="decode", batch=64, kv_len=20000, top_k=16),                                   # 2 scan parts per row
    W(mode="decode", batch=1, kv_len=9000, top_k=16),                                     # slices per row
    W(mode="decode", batch=1, kv_len=4 * 20000 + 2, top_k=513, block_size=4, keep_tail=True),  # score + pick-attend
]


@pytest.mark.parametrize("w", STEP_DETERMINISM, ids=case_id)
def test_step_bitwise_determinism(w):
    """The decode step twice on the same inputs: selections, scores, outputs and compressed keys bit for bit
    (the cross-workgroup list exchange and the slice merges fold in a fixed order)."""
    case = Case(w, seed=8)
    b, hq, hkv, d = w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim
    shape = qsa.shape_for(case.q, case.k, w.block_size, w.top_k, keep_tail=w.keep_tail)
    q = case.q.view(b, hq, d)
    ws = qsa.workspace(shape, qsa.QSA_OP_DECODE_STEP, 1, w.kv_len, "cuda")
    runs = []
    for _ in range(2):
        k_comp = torch.zeros(b, hkv, case.kv_cap // w.block_size, d, device="cuda")
        qsa.qsa_compress_keys(shape, case.k, w.kv_len - 1, k_comp)
        sel = torch.empty(b, hkv, w.top_k, dtype=torch.int32, device="cuda")
        sc = torch.empty(b, hkv, w.top_k, dtype=torch.float32, device="cuda")
        out = torch.empty_like(q)
        qsa.qsa_decode_step(shape, q, case.k, case.v, k_comp, w.kv_len, sel, out, sel_scores=sc, ws=ws)
        torch.cuda.synchronize()
        runs.append((sel.clone(), sc.clone(), out.clone(), k_comp.clone()))
    for x, y, name in zip(runs[0], runs[1], ("selections", "scores", "outputs", "compressed keys")):
        assert torch.equal(x.view(torch.uint8) if x.dtype == torch.bfloat16 else x,
                           y.view(torch.uint8) if y.dtype == torch.bfloat16 else y), f"{name} differ between runs"
    log(f"  step determinism {case_id(w)}: fused {qsa.qsa_decode_step_fused(shape, w.kv_len)}")


@pytest.mark.parametrize("bs,d", [(64, 128), (4, 128), (4, 64), (8, 64), (16, 128)])
def test_incremental_compress_matches_full(bs, d):
    """Compressing block by block (a decode loop) gives the same compressed keys as one call."""
    w = W(batch=2, kv_len=1100, block_size=bs, head_dim=d)
    case = Case(w, seed=7)
    shape = qsa.shape_for(case.q, case.k, w.block_size, w.top_k)
    nb = w.kv_len // w.block_size
    full = torch.zeros(2, 2, nb, d, device="cuda")
    inc = torch.zeros(2, 2, nb, d, device="cuda")
    qsa.qsa_compress_keys(shape, case.k, w.kv_len, full)
    for n in range(1, w.kv_len + 1):
        if n % w.block_size == 0:
            qsa.qsa_compress_keys(shape, case.k, n, inc, block_begin=n // w.block_size - 1)
    torch.cuda.synchronize()
    assert torch.equal(full, inc)


REUSE_CASES = [
    (W(mode="decode", batch=4, kv_len=40033, block_size=32, top_k=16), [40000, 40031, 40032, 40033, 39000]),
    (W(mode="decode", batch=1, kv_len=4 * 20000 + 3, block_size=4, top_k=513, keep_tail=True),
     [80003, 80000, 79999, 60001, 40000, 50000]),
]


@pytest.mark.parametrize("w,steps", REUSE_CASES, ids=lambda x: case_id(x) if isinstance(x, S.Workload) else "")
def test_workspace_reuse_across_decode_steps(w, steps):
    """One select and one decode workspace, filled with garbage once (the
    decode counters zeroed), serve a run of decode steps (split selection and
    split attention): every step equals a call with fresh workspaces, so every
    call leaves the counters at zero."""
    case = Case(w, seed=8)
    b, hq, d = w.batch, w.n_q_heads, w.head_dim
    shape = qsa.shape_for(case.q, case.k, w.block_size, w.top_k, keep_tail=w.keep_tail)
    k_comp = torch.zeros(b, w.n_kv_heads, w.kv_len // w.block_size, d, device="cuda")
    qsa.qsa_compress_keys(shape, case.k, w.kv_len, k_comp)
    q_sel = case.q.view(b, 1, hq, d)
    q_dec = case.q.view(b, hq, d)
    n_sel = max(qsa.qsa_workspace_bytes(shape, qsa.QSA_OP_SELECT, 1, n) for n in steps)
    n_dec = max(qsa.qsa_workspace_bytes(shape, qsa.QSA_OP_DECODE, 1, n) for n in steps)
    assert n_sel > 0 and n_dec > 0, "both calls must take their split paths"
    # arrival counters zero-filled once (the documented precondition), garbage
    # in the scratch part of both workspaces
    n_cnt = (4 * b * w.n_kv_heads + 255) // 256 * 256
    ws_sel = torch.full((n_sel,), 0xA5, dtype=torch.uint8, device="cuda")
    ws_dec = torch.full((n_dec,), 0x5A, dtype=torch.uint8, device="cuda")
    ws_dec[:n_cnt].zero_()
    split_select = w.top_k <= 64  # the split selection path keeps counters too
    if split_select:
        ws_sel[:n_cnt].zero_()
    for n in steps:
        log(f"workspace reuse step kv_len={n}")
        outs = []
        for wss, wsd in ((ws_sel, ws_dec), (None, None)):
            sel = torch.empty(b, 1, w.n_kv_heads, w.top_k, dtype=torch.int32, device="cuda")
            out = torch.empty(b, hq, d, dtype=case.q.dtype, device="cuda")
            qsa.qsa_score_select(shape, q_sel, n - 1, k_comp, n, w.kv_len, sel, ws=wss)
            qsa.qsa_sparse_attn_decode(shape, q_dec, case.k, case.v, n, sel.view(b, w.n_kv_heads, w.top_k), out,
                                       ws=wsd)
            outs.append((sel, out))
        torch.cuda.synchronize()
        assert torch.equal(outs[0][0], outs[1][0])
        assert torch.equal(outs[0][1].view(torch.int16), outs[1][1].view(torch.int16))
        assert int(ws_dec[:n_cnt].count_nonzero()) == 0, "decode arrival counters not left at zero"
        if split_select:
            assert int(ws_sel[:n_cnt].count_nonzero()) == 0, "selection arrival counters not left at zero"
    # the last step against the oracle (rows at position n - 1 read only
    # blocks and keys below n)
    rows = [(bb, 0, g) for bb in range(b) for g in range(w.n_kv_heads)]
    st = check_rows(case, outs[0][0].cpu().numpy(), from_device(outs[0][1])[:, None], rows, steps[-1] - 1)
    log(f"  {st}")


def test_decode_step_workspace_reuse():
    """A decode loop on one zero-initialised workspace whose steps switch
    between the fused kernel's plans (short rows: slices of the selection
    with arrival counters; long rows: the scan split over several
    workgroups, with a ticket word and slice counters): every step equals a
    call with a fresh workspace, so the counter areas sit where every plan
    expects them and every call leaves them at zero."""
    w = W(mode="decode", batch=1, kv_len=32 * 5000 + 9, top_k=32, block_size=32, head_dim=64, n_q_heads=8,
          n_kv_heads=1)
    case = Case(w, seed=9)
    b, hq, d, bs = w.batch, w.n_q_heads, w.head_dim, w.block_size
    shape = qsa.shape_for(case.q, case.k, bs, w.top_k)
    steps = [40000, 160009, 160000, 50001, 159999, 120001, 140000, 30000, 160009]
    # compressed keys of 256 bytes: rows up to 2,048 candidates (65,536 positions) are short, the rest long
    assert any(n // 32 * 256 <= 512 << 10 for n in steps) and any(n // 32 * 256 > 512 << 10 for n in steps)
    n_ws = max(qsa.qsa_workspace_bytes(shape, qsa.QSA_OP_DECODE_STEP, 1, n) for n in steps)
    ws = torch.zeros(n_ws, dtype=torch.uint8, device="cuda")
    q = case.q.view(b, hq, d)
    for n in steps:
        log(f"decode step workspace reuse kv_len={n}")
        outs = []
        for wsx in (ws, None):
            k_comp = torch.zeros(b, w.n_kv_heads, w.kv_len // bs, d, device="cuda")
            qsa.qsa_compress_keys(shape, case.k, n - 1, k_comp)
            sel = torch.empty(b, w.n_kv_heads, w.top_k, dtype=torch.int32, device="cuda")
            out = torch.empty_like(q)
            qsa.qsa_decode_step(shape, q, case.k, case.v, k_comp, n, sel, out, ws=wsx)
            outs.append((sel, out))
        torch.cuda.synchronize()
        assert torch.equal(outs[0][0], outs[1][0])
        assert torch.equal(outs[0][1].view(torch.int16), outs[1][1].view(torch.int16))
    rows = [(bb, 0, g) for bb in range(b) for g in range(w.n_kv_heads)]
    st = check_rows(case, outs[0][0].cpu().numpy()[:, None], from_device(outs[0][1])[:, None], rows, steps[-1] - 1)
    log(f"  {st}")


def _restore_keys(case: Case, K32: np.ndarray) -> None:
    """Replace the case's keys by ``K32`` rounded to its storage type (host view and device copy)."""
    w = case.w
    if w.dtype == "bf16":
        bits = S.f32_to_bf16_bits(K32.astype(np.float32))
        case.K = S.bf16_bits_to_f32(bits)
        case.k = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()
    else:
        case.K = K32.astype(np.float32)
        case.k = torch.from_numpy(case.K).cuda()
    case._kc = None


def test_large_k_equal_scores_keep_smallest_ids():
    """Zero queries give every candidate the same score: the smallest ids win. The list pool's cutoff
    is reached by the lists of the first 32 chunks, so all 32 are re-expanded from the stored scores
    (the most the pool allows at k = 513)."""
    w = W(mode="decode", batch=1, kv_len=4 * 20000, top_k=513, block_size=4)
    case = Case(w, seed=6)
    case.Q = np.zeros_like(case.Q)
    case.q = torch.zeros_like(case.q)
    sel, out, scores, _ = run_decode(case)
    own = (w.kv_len - 1) // 4
    for g in range(w.n_kv_heads):
        assert sel[0, 0, g].tolist() == list(range(512)) + [own]
    st = check_rows(case, sel, out, [(0, 0, g) for g in range(2)], w.kv_len - 1, scores_gpu=scores)
    log(f"equal scores: {st}")


def test_large_k_clustered_winners():
    """Keys of 600 consecutive blocks shifted toward the query (about four noise deviations of the
    score): most kept blocks sit in three chunks of 256 candidates, whose lists saturate and are
    re-expanded."""
    w = W(mode="decode", batch=1, kv_len=4 * 40000 + 2, top_k=513, block_size=4, keep_tail=True)
    case = Case(w, seed=7)
    K32 = case.K.astype(np.float64)
    G = w.group
    for g in range(w.n_kv_heads):
        u = case.Q[0, -1, g * G:(g + 1) * G].astype(np.float64).sum(0)
        u /= np.linalg.norm(u)
        K32[0, g, 4 * 10000:4 * 10600] += 2.0 * w.sigma * u
    _restore_keys(case, K32)
    sel, out, scores, _ = run_decode(case)
    for g in range(w.n_kv_heads):
        inside = sum(1 for c in sel[0, 0, g] if 10000 <= c < 10600)
        assert inside > 300, inside
    st = check_rows(case, sel, out, [(0, 0, g) for g in range(2)], w.kv_len - 1, scores_gpu=scores)
    log(f"clustered winners: {st}")


STEP_CASES = [
    W(mode="decode", batch=3, kv_len=1000, top_k=8),
    W(mode="decode", batch=2, kv_len=64 * 40, top_k=8),                     # the new token closes a block
    W(mode="decode", batch=2, kv_len=64 * 40, top_k=8, keep_tail=True),     # ... which then competes
    W(mode="decode", batch=1, kv_len=64, top_k=4, keep_tail=True),          # its only candidate is the new block
    W(mode="decode", batch=2, kv_len=50, top_k=4),                          # own block only
    W(mode="decode", batch=1, kv_len=9000, top_k=64, block_size=32),
    W(mode="decode", batch=5, kv_len=4096, top_k=12, head_dim=64, block_size=128),
    W(mode="decode", batch=2, kv_len=3000, n_q_heads=16, n_kv_heads=1, top_k=7),
    W(mode="decode", batch=2, kv_len=3000, n_q_heads=2, n_kv_heads=2, top_k=7),
    W(mode="decode", batch=40, kv_len=5000, top_k=16, n_q_heads=8, n_kv_heads=2),  # 80 rows: fused though long
    # long rows, few of them: the scan split over many workgroups per row
    W(mode="decode", batch=1, kv_len=200000, top_k=16),
    W(mode="decode", batch=3, kv_len=64 * 9000 + 7, top_k=32, keep_tail=True),
    W(mode="decode", batch=1, kv_len=64 * 9000, top_k=64, n_q_heads=16, n_kv_heads=1),   # closes a block
    # long rows, k <= 64: chunk lists merged in every attention slice
    W(mode="decode", batch=1, kv_len=32 * 5000 + 9, top_k=32, block_size=32, head_dim=64, n_q_heads=8,
      n_kv_heads=1),                                                         # 20 lists of 31
    W(mode="decode", batch=2, kv_len=64 * 3200, top_k=16),                  # closes a block
    W(mode="decode", batch=1, kv_len=32 * 5000, top_k=32, block_size=32, head_dim=64, n_q_heads=8, n_kv_heads=1,
      keep_tail=True),                                                       # the closed block competes
    W(mode="decode", batch=1, kv_len=4 * 20000, top_k=513, block_size=4, keep_tail=True),
    W(mode="decode", batch=2, kv_len=2222, dtype="f32", sigma=1.0, top_k=5),
    W(mode="decode", batch=2, kv_len=2240, dtype="f32", sigma=1.0, top_k=5, keep_tail=True),   # closes a block
    W(mode="decode", batch=1, kv_len=8 * 3000, top_k=100, block_size=8),                    # large-k, closes
    W(mode="decode", batch=2, kv_len=32 * 700 + 5, top_k=129, block_size=32, head_dim=64),  # large-k, whole units
    W(mode="decode", batch=2, kv_len=16 * 3000, n_q_heads=16, n_kv_heads=1, top_k=200, block_size=16),  # G = 16
    W(mode="decode", batch=1, kv_len=3, top_k=513, block_size=4, keep_tail=True),           # no candidate yet
    # k > 64, default frame, the new token closes block 0: no candidate to score, the block is still compressed
    W(mode="decode", batch=1, kv_len=4, top_k=100, block_size=4),
    W(mode="decode", batch=2, kv_len=64, top_k=129, block_size=64),
    W(mode="decode", batch=2, kv_len=32, top_k=70, block_size=32, dtype="f32", sigma=1.0),
    W(mode="decode", batch=3, kv_len=4 * 700, top_k=513, block_size=4, keep_tail=True),     # fewer than k blocks
]


@pytest.mark.parametrize("w", STEP_CASES, ids=case_id)
def test_decode_step_parity(w):
    """qsa_decode_step = compress of the closed block + selection + decode attention, fused or not."""
    log(f"decode step parity {w}")
    case = Case(w, seed=11, kv_cap=w.kv_len + 100)
    b, hq, d, bs = w.batch, w.n_q_heads, w.head_dim, w.block_size
    shape = qsa.shape_for(case.q, case.k, bs, w.top_k, keep_tail=w.keep_tail)
    nb = w.kv_len // bs
    # k_comp holds the blocks closed before the new token; the step adds the one it closes
    k_comp = torch.full((b, w.n_kv_heads, case.kv_cap // bs, d), float("nan"), device="cuda")
    qsa.qsa_compress_keys(shape, case.k, w.kv_len - 1, k_comp)
    k_comp_ref = k_comp.clone()
    qsa.qsa_compress_keys(shape, case.k, w.kv_len, k_comp_ref)
    q = case.q.view(b, hq, d)
    sel = torch.empty(b, w.n_kv_heads, w.top_k, dtype=torch.int32, device="cuda")
    scores = torch.empty(b, w.n_kv_heads, w.top_k, dtype=torch.float32, device="cuda")
    out = torch.empty_like(q)
    qsa.qsa_decode_step(shape, q, case.k, case.v, k_comp, w.kv_len, sel, out, sel_scores=scores)
    out2, sel2 = qsa.decode(q, case.k, case.v, w.kv_len, bs, w.top_k, k_comp_ref, keep_tail=w.keep_tail)
    torch.cuda.synchronize()
    assert torch.equal(k_comp[:, :, :nb], k_comp_ref[:, :, :nb]), "compressed keys differ from the compress call"
    if not (w.keep_tail and w.kv_len % bs == 0):  # else the new block's score may round differently
        assert torch.equal(sel, sel2), "selection differs from the separate calls"
    rows = [(bb, 0, g) for bb in range(b) for g in range(w.n_kv_heads)]
    st = check_rows(case, sel.cpu().numpy()[:, None], from_device(out)[:, None], rows, w.kv_len - 1,
                    scores_gpu=scores.cpu().numpy()[:, None])
    log(f"  {st}")


def _lengths(batch: int, max_len: int, seed: int) -> list[int]:
    rng = np.random.default_rng(seed)
    n = [int(x) for x in rng.integers(1, max_len + 1, size=batch)]
    n[-1] = max_len
    return n


RAGGED_CASES = [
    # single token, one short of a block, closing the first block, mid, closing block 65, the longest
    (W(mode="decode", batch=6, kv_len=9000, top_k=16), [1, 63, 64, 1000, 4160, 9000]),
    (W(mode="decode", batch=5, kv_len=5000, top_k=8, block_size=32, keep_tail=True), [32, 33, 2048, 4999, 5000]),
    (W(mode="decode", batch=70, kv_len=3000, top_k=16, n_q_heads=8, n_kv_heads=2, head_dim=64, block_size=128),
     _lengths(70, 3000, 5)),   # 140 rows: one workgroup per row
    (W(mode="decode", batch=3, kv_len=40000, top_k=64, n_q_heads=16, n_kv_heads=1), [17, 20000, 40000]),  # G = 16
    # k > 64: the large selection's score pass and the pick-and-attend kernel read the lengths. The
    # released budget (one token, no complete block, the first block closed, the first discard, past the
    # pick pool), a default frame with gathered 8-key blocks, and a batch with no candidate anywhere
    (W(mode="decode", batch=5, kv_len=4 * 20000 + 2, top_k=513, block_size=4, keep_tail=True),
     [1, 3, 4, 2052, 4 * 20000 + 2]),
    (W(mode="decode", batch=4, kv_len=8 * 3000, top_k=129, block_size=8), [8, 9, 1000, 8 * 3000]),
    (W(mode="decode", batch=3, kv_len=4, top_k=100, block_size=4), [1, 2, 4]),
    # the other shapes without the fused kernel go through the same large selection: bf16 blocks shorter
    # than 32 keys with k <= 64 (pick-and-attend; past the pick pool; no candidate anywhere), and float32
    # (per-row pick, then the float32 attention) with k <= 64 and k > 64
    (W(mode="decode", batch=5, kv_len=16 * 500, top_k=16, block_size=16), [1, 16, 17, 4000, 16 * 500]),
    (W(mode="decode", batch=3, kv_len=4 * 13000 + 1, top_k=64, block_size=4, keep_tail=True), [4, 2000, 4 * 13000 + 1]),
    (W(mode="decode", batch=3, kv_len=8, top_k=8, block_size=8), [1, 7, 8]),
    (W(mode="decode", batch=4, kv_len=3000, top_k=16, dtype="f32", sigma=1.0), [1, 64, 1500, 3000]),
    (W(mode="decode", batch=3, kv_len=8 * 1200, top_k=100, block_size=8, dtype="f32", sigma=1.0, keep_tail=True),
     [8, 801, 8 * 1200]),
]


@pytest.mark.parametrize("w,lens", RAGGED_CASES, ids=lambda x: case_id(x) if isinstance(x, S.Workload) else None)
def test_decode_step_ragged(w, lens):
    """A ragged batch: every sequence matches the oracle at its own length, and the per-sequence step."""
    log(f"ragged decode step {w} lens={lens[:8]}")
    case = Case(w, seed=13, kv_cap=w.kv_len + 100)
    b, hq, hkv, d, bs = w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.block_size
    shape = qsa.shape_for(case.q, case.k, bs, w.top_k, keep_tail=w.keep_tail)
    one = qsa.make_shape(1, hq, hkv, d, bs, w.top_k, case.q.dtype, keep_tail=w.keep_tail)
    nbc = case.kv_cap // bs
    k_comp = torch.full((b, hkv, nbc, d), float("nan"), device="cuda")
    k_ref = torch.full((b, hkv, nbc, d), float("nan"), device="cuda")
    for bb, n in enumerate(lens):  # the blocks closed before each sequence's new token
        qsa.qsa_compress_keys(one, case.k[bb:bb + 1], n - 1, k_comp[bb:bb + 1])
        qsa.qsa_compress_keys(one, case.k[bb:bb + 1], n, k_ref[bb:bb + 1])
    q = case.q.view(b, hq, d)
    kv_lens = torch.tensor(lens, dtype=torch.int32, device="cuda")
    sel = torch.empty(b, hkv, w.top_k, dtype=torch.int32, device="cuda")
    scores = torch.empty(b, hkv, w.top_k, dtype=torch.float32, device="cuda")
    out = torch.empty_like(q)
    qsa.qsa_decode_step_ragged(shape, q, case.k, case.v, k_comp, kv_lens, w.kv_len, sel, out, sel_scores=scores)
    torch.cuda.synchronize()
    sel_h, out_h, sc_h = sel.cpu().numpy(), from_device(out), scores.cpu().numpy()
    for bb, n in enumerate(lens):
        nb = n // bs
        assert torch.equal(k_comp[bb, :, :nb], k_ref[bb, :, :nb]), f"sequence {bb}: compressed keys"
        rows = [(bb, 0, g) for g in range(hkv)]
        st = check_rows(case, sel_h[:, None], out_h[:, None], rows, n - 1, scores_gpu=sc_h[:, None])
        if bb < 8 or bb == b - 1:
            log(f"  seq {bb} len {n}: {st}")
    # the same sequences one at a time through the plain step
    k_one = k_ref.clone()
    for bb, n in list(enumerate(lens))[:: max(1, len(lens) // 6)]:
        k_one[bb:bb + 1].copy_(k_comp[bb:bb + 1])
        s1 = torch.empty(1, hkv, w.top_k, dtype=torch.int32, device="cuda")
        o1 = torch.empty(1, hq, d, dtype=q.dtype, device="cuda")
        qsa.qsa_decode_step(one, q[bb:bb + 1], case.k[bb:bb + 1], case.v[bb:bb + 1], k_one[bb:bb + 1], n, s1, o1)
        torch.cuda.synchronize()
        if not (w.keep_tail and n % bs == 0):
            assert torch.equal(s1[0], sel[bb]), f"sequence {bb}: selection differs from the single-sequence step"
        err = (o1[0].float() - out[bb].float()).abs().max().item()
        assert err <= 2e-2, f"sequence {bb}: output differs from the single-sequence step by {err}"



@pytest.mark.parametrize("w,lens", RAGGED_CASES, ids=lambda x: case_id(x) if isinstance(x, S.Workload) else None)
def test_ragged_select_and_attention_calls(w, lens):
    """A ragged batch through the separate calls (qsa_score_select_ragged, then qsa_sparse_attn_decode_ragged
    on its selection): every sequence matches the oracle at its own length; for k > 64 the selection equals the
    per-sequence qsa_score_select bit for bit, and every output matches the per-sequence decode call on the same
    selection."""
    log(f"ragged separate calls {w} lens={lens[:8]}")
    case = Case(w, seed=17, kv_cap=w.kv_len + 100)
    b, hq, hkv, d, bs = w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.block_size
    shape = qsa.shape_for(case.q, case.k, bs, w.top_k, keep_tail=w.keep_tail)
    one = qsa.make_shape(1, hq, hkv, d, bs, w.top_k, case.q.dtype, keep_tail=w.keep_tail)
    nbc = case.kv_cap // bs
    k_comp = torch.full((b, hkv, nbc, d), float("nan"), device="cuda")
    for bb, n in enumerate(lens):  # every block complete at each sequence's token
        qsa.qsa_compress_keys(one, case.k[bb:bb + 1], n, k_comp[bb:bb + 1])
    q = case.q.view(b, hq, d)
    kv_lens = torch.tensor(lens, dtype=torch.int32, device="cuda")
    sel = torch.empty(b, hkv, w.top_k, dtype=torch.int32, device="cuda")
    scores = torch.empty(b, hkv, w.top_k, dtype=torch.float32, device="cuda")
    out = torch.empty_like(q)
    qsa.qsa_score_select_ragged(shape, q, k_comp, kv_lens, w.kv_len, case.kv_cap, sel, sel_scores=scores)
    qsa.qsa_sparse_attn_decode_ragged(shape, q, case.k, case.v, kv_lens, w.kv_len, sel, out)
    torch.cuda.synchronize()
    sel_h, out_h, sc_h = sel.cpu().numpy(), from_device(out), scores.cpu().numpy()
    for bb, n in enumerate(lens):
        rows = [(bb, 0, g) for g in range(hkv)]
        st = check_rows(case, sel_h[:, None], out_h[:, None], rows, n - 1, scores_gpu=sc_h[:, None])
        if bb < 8 or bb == b - 1:
            log(f"  seq {bb} len {n}: {st}")
    for bb, n in list(enumerate(lens))[:: max(1, len(lens) // 6)]:
        if w.top_k > 64:
            s1 = torch.empty(1, hkv, w.top_k, dtype=torch.int32, device="cuda")
            sc1 = torch.empty(1, hkv, w.top_k, dtype=torch.float32, device="cuda")
            qsa.qsa_score_select(one, q[bb:bb + 1].view(1, 1, hq, d), n - 1, k_comp[bb:bb + 1], n, case.kv_cap, s1, sc1)
            torch.cuda.synchronize()
            assert torch.equal(s1[0], sel[bb]), f"sequence {bb}: selection differs from the single-sequence call"
            assert torch.equal(sc1[0], scores[bb]), f"sequence {bb}: scores differ from the single-sequence call"
        o1 = torch.empty(1, hq, d, dtype=q.dtype, device="cuda")
        qsa.qsa_sparse_attn_decode(one, q[bb:bb + 1], case.k[bb:bb + 1], case.v[bb:bb + 1], n, sel[bb:bb + 1].clone(),
                                   o1)
        torch.cuda.synchronize()
        err = (o1[0].float() - out[bb].float()).abs().max().item()
        assert err <= 2e-2, f"sequence {bb}: output differs from the single-sequence decode call by {err}"


TIE_CASES = [
    W(kv_len=3000, top_k=16, block_size=32),                      # prefill row path
    W(kv_len=3000, top_k=24, block_size=32),                      # prefill threshold-select tile path
    W(kv_len=2000, top_k=12, block_size=32, keep_tail=True),      # row path, keep-tail frame
    W(mode="decode", batch=2, kv_len=64 * 3000, top_k=16),        # split decode path (chunk lists)
]


@pytest.mark.parametrize("w", TIE_CASES, ids=lambda w: case_id(w) + "-" + w.mode)
def test_equal_scores_keep_smallest_ids(w):
    """Zero queries give every candidate the same score: each row keeps its smallest candidate ids (and its
    forced block), on every selection path; the outputs match the oracle over that selection."""
    case = Case(w, seed=7)
    case.Q = np.zeros_like(case.Q)
    case.q = torch.zeros_like(case.q)
    bs, k = w.block_size, w.top_k
    if w.mode == "prefill":
        sel, out, scores, _ = run_prefill(case)
        q_len, pos0 = w.kv_len, 0
    else:
        sel, out, scores, _ = run_decode(case)
        q_len, pos0 = 1, w.kv_len - 1
    for bb in range(w.batch):
        for t in range(q_len):
            n_cand, forced = O.selection_frame(pos0 + t, bs, w.keep_tail)
            kept = list(range(min(n_cand, k - 1))) + ([forced] if forced is not None else [])
            want = sorted(kept) + [-1] * (k - len(kept))
            for g in range(w.n_kv_heads):
                assert sel[bb, t, g].tolist() == want, f"row {(bb, t, g)}"
    rows = all_rows(w, q_len)
    if len(rows) > 600:
        rng = np.random.default_rng(3)
        rows = [rows[i] for i in sorted(rng.choice(len(rows), 600, replace=False))]
    st = check_rows(case, sel, out, rows, pos0, scores_gpu=scores)
    log(f"equal scores ({w.mode}, k={k}): {st}")


SCAN_FALLBACK_CASES = [
    W(mode="decode", batch=64, kv_len=64 * 1100 + 5, top_k=16),                          # 128 rows: 2 scan parts
    W(mode="decode", batch=40, kv_len=64 * 2000, top_k=16, n_q_heads=8, n_kv_heads=2),  # 80 rows: 3 parts, closes a block
    W(mode="decode", batch=64, kv_len=64 * 1040, top_k=8, keep_tail=True),              # the closed block competes
    W(mode="decode", batch=1, kv_len=64 * 20000, top_k=32),                             # 2 long rows: 32 parts each
]


@pytest.mark.parametrize("w", SCAN_FALLBACK_CASES, ids=case_id)
def test_decode_step_scan_wait_fallback(w, monkeypatch):
    """Rows whose candidate scan is split over several workgroups exchange their top lists through the
    workspace; a part that finds a list missing when its bounded wait ends scores the other parts'
    candidates itself. With the wait cut to nothing from the host (QSA_SCAN_WAIT_POLLS=0), the first part
    of every row to post takes that path: the step's results must equal the normal step's bitwise, and
    the oracle's."""
    case = Case(w, seed=21, kv_cap=w.kv_len + 64)
    b, hq, d, bs, k = w.batch, w.n_q_heads, w.head_dim, w.block_size, w.top_k
    shape = qsa.shape_for(case.q, case.k, bs, k, keep_tail=w.keep_tail)
    assert qsa.qsa_decode_step_fused(shape, w.kv_len)
    q = case.q.view(b, hq, d)
    results = []
    for polls in (None, "0"):
        if polls is None:
            monkeypatch.delenv("QSA_SCAN_WAIT_POLLS", raising=False)
        else:
            monkeypatch.setenv("QSA_SCAN_WAIT_POLLS", polls)
        k_comp = torch.full((b, w.n_kv_heads, case.kv_cap // bs, d), float("nan"), device="cuda")
        qsa.qsa_compress_keys(shape, case.k, w.kv_len - 1, k_comp)
        sel = torch.empty(b, w.n_kv_heads, k, dtype=torch.int32, device="cuda")
        scores = torch.empty(b, w.n_kv_heads, k, dtype=torch.float32, device="cuda")
        out = torch.empty_like(q)
        qsa.qsa_decode_step(shape, q, case.k, case.v, k_comp, w.kv_len, sel, out, sel_scores=scores)
        torch.cuda.synchronize()
        results.append((sel, scores, out, k_comp))
    monkeypatch.delenv("QSA_SCAN_WAIT_POLLS", raising=False)
    (s0, c0, o0, k0), (s1, c1, o1, k1) = results
    nb = w.kv_len // bs
    assert torch.equal(s0, s1), "selection"
    assert torch.equal(c0.view(torch.int32), c1.view(torch.int32)), "selection scores"
    assert torch.equal(o0.view(torch.int16), o1.view(torch.int16)), "output"
    assert torch.equal(k0[:, :, :nb], k1[:, :, :nb]), "compressed keys"
    rows = [(bb, 0, g) for bb in range(b) for g in range(w.n_kv_heads)]
    st = check_rows(case, s1.cpu().numpy()[:, None], from_device(o1)[:, None], rows, w.kv_len - 1,
                    scores_gpu=c1.cpu().numpy()[:, None])
    log(f"scan wait fallback {case_id(w)}: {st}")
