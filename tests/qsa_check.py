"""Acceptance rules used by the parity tests.

Selection: the top-k boundary is discontinuous, so a selection is compared
with the oracle's scores, not only with the oracle's own choice. For a row
with ``m`` scored slots let ``s_m`` be the m-th best oracle score and
``s_m1`` the best dropped one. If their relative gap
``(s_m - s_m1) / max(|s_m|, |s_m1|)`` exceeds ``REL_GAP`` the kept set must
equal the oracle's exactly; otherwise every kept candidate must score at
least ``s_m - tol`` and every dropped one at most ``s_m1 + tol`` with
``tol = REL_GAP * max(|s_m|, |s_m1|)``.

Outputs: bf16 results must lie within ``BF16_ABS_TOL`` absolute of the
oracle (the acceptance bound), and, per (row, head), within
``BF16_ROW_REL_TOL * max|o_ref| + BF16_ROW_ABS_FLOOR`` (the companion bound
of :func:`check_output_row`), which a one-block gather error cannot pass.
fp32 results must lie within ``F32_REL_TOL`` of the row's largest output.

Overlap between two selections is reported as the Jaccard index
``|A ∩ B| / |A ∪ B|`` ("Qwen4 in llama.cpp: Dissecting PR #27742", section
"QSA Is an Address-Selection Problem, Not a New Attention Equation").
"""
from __future__ import annotations

import numpy as np

REL_GAP = 1e-3
BF16_ABS_TOL = 2e-2
F32_REL_TOL = 1e-5
# Companion bound of a bf16 output row (one query head's d outputs), derived
# from the arithmetic the attention kernels do in bf16:
#  * the output is rounded once to bf16: at most 2^-9 of |o| per element;
#  * each softmax weight is rounded to bf16 (relative error <= 2^-9) before
#    the PV product, and numerator and denominator use the same rounded
#    weights, so the output stays an exact weighted average whose weights are
#    perturbed by independent errors of at most 2^-9: the error of an element
#    behaves like a sum of n random terms of size 2^-9 * w_t * |v_t - o|,
#    about 0.6 * 2^-9 * sigma / sqrt(n) per element and below 2 * 2^-9 * the
#    row's largest |o| (itself about 2.5 * sigma / sqrt(n)) at the tail of
#    the rows checked;
#  * scores and accumulators are float32 (relative 2^-24 per operation),
#    negligible next to the two terms above.
# 2^-7 = 4 * 2^-9 covers their sum with room to spare; the absolute floor
# covers rows whose outputs are all near zero. Swapping one kept block for
# another moves an output row by far more (about a quarter of its largest
# element on the sigma-0.5 workloads), which the absolute bound of 2e-2 does
# not see when outputs are ~0.05.
BF16_ROW_REL_TOL = 2.0 ** -7
BF16_ROW_ABS_FLOOR = 1e-4


class SelectionMismatch(AssertionError):
    pass


class OutputMismatch(AssertionError):
    pass


def output_row_bound(ref, rel: float = BF16_ROW_REL_TOL, floor: float = BF16_ROW_ABS_FLOOR) -> np.ndarray:
    """Companion bound of every output row: ``rel * max_e |ref| + floor`` over the last axis (kept)."""
    ref = np.asarray(ref, dtype=np.float64)
    return rel * np.abs(ref).max(axis=-1, keepdims=True) + floor


def check_output_row(got, ref, dtype: str, rel: float = BF16_ROW_REL_TOL, floor: float = BF16_ROW_ABS_FLOOR,
                     where: str = "") -> float:
    """Check GPU outputs ``got`` against oracle outputs ``ref`` (rows on the last axis).

    bf16: every element within ``BF16_ABS_TOL`` (the acceptance bound) and
    every row within :func:`output_row_bound` (the companion bound). fp32:
    every row within ``F32_REL_TOL`` of its largest reference output.
    Returns the largest ratio of error to the row bound (<= 1 when it passes);
    raises :class:`OutputMismatch` otherwise.
    """
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = np.abs(got - ref)
    if dtype == "bf16":
        if not err.max() <= BF16_ABS_TOL:
            raise OutputMismatch(f"{where} bf16 error {err.max():.3e} above {BF16_ABS_TOL}")
        lim = output_row_bound(ref, rel, floor)
    else:
        lim = F32_REL_TOL * np.abs(ref).max(axis=-1, keepdims=True) + 1e-30
    ratio = float((err / lim).max()) if err.size else 0.0
    if not ratio <= 1.0:
        raise OutputMismatch(f"{where} {dtype} output error {ratio:.3f} x its row bound (max abs {err.max():.3e})")
    return ratio


def jaccard(a, b) -> float:
    a = {int(x) for x in a if x >= 0}
    b = {int(x) for x in b if x >= 0}
    if not a and not b:
        return 1.0
    return len(a & b) / len(a | b)


def check_selection(sel_row, scores, own_block: int, top_k: int, rel_gap: float = REL_GAP) -> str:
    """Validate one row's selection (default frame: own block forced, candidates below it)."""
    return check_selection_frame(sel_row, scores, own_block, own_block, top_k, rel_gap)


def check_selection_frame(sel_row, scores, n_cand: int, forced, top_k: int, rel_gap: float = REL_GAP) -> str:
    """Validate one row's selection against the oracle's float64 candidate scores.

    ``n_cand`` candidates ``0 .. n_cand-1`` compete for ``min(top_k-1, n_cand)``
    slots; ``forced`` (a block id, or None) must be kept, as the last entry.
    Returns ``"clear"`` (exact match required and found) or ``"ambiguous"``
    (boundary within the gap, selection valid); raises
    :class:`SelectionMismatch` otherwise.
    """
    sel = [int(x) for x in sel_row]
    kept = [x for x in sel if x >= 0]
    pad = sel[len(kept):]
    if any(x >= 0 for x in pad) or len(sel) != top_k:
        raise SelectionMismatch(f"padding not at the tail: {sel}")
    if kept != sorted(set(kept)):
        raise SelectionMismatch(f"ids not strictly ascending: {sel}")
    if forced is not None:
        if forced not in kept or kept[-1] != forced:
            raise SelectionMismatch(f"forced block {forced} missing or not last: {sel}")
        scored = kept[:-1]
    else:
        scored = kept
    slots = min(top_k - 1, n_cand)
    if len(scored) != slots:
        raise SelectionMismatch(f"expected {slots} scored blocks, got {len(scored)}: {sel}")
    if any(c < 0 or c >= n_cand for c in scored):
        raise SelectionMismatch(f"scored id out of range: {sel}")
    if slots == n_cand or slots == 0:
        return "clear"  # every candidate (or none) is kept: one valid answer
    scores = np.asarray(scores, dtype=np.float64)
    order = sorted(range(n_cand), key=lambda c: (-scores[c], c))
    expect = sorted(order[:slots])
    s_m, s_m1 = scores[order[slots - 1]], scores[order[slots]]
    denom = max(abs(s_m), abs(s_m1))
    gap = (s_m - s_m1) / denom if denom > 0 else 0.0
    if gap > rel_gap:
        if scored != expect:
            raise SelectionMismatch(
                f"clear row (gap {gap:.3e}) differs: got {scored}, expected {expect}")
        return "clear"
    tol = rel_gap * denom
    chosen = set(scored)
    for c in range(n_cand):
        if c in chosen and scores[c] < s_m - tol:
            raise SelectionMismatch(f"kept block {c} scores {scores[c]} below cutoff {s_m}")
        if c not in chosen and scores[c] > s_m1 + tol:
            raise SelectionMismatch(f"dropped block {c} scores {scores[c]} above cutoff {s_m1}")
    return "ambiguous"
