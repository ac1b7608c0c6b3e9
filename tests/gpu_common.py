"""Shared helpers of the GPU parity tests: device inputs, oracle comparison."""
from __future__ import annotations

import sys

import numpy as np
import torch

import qsa_synth as S
from oracle import qsa_oracle as O
from qsa_check import check_output_row, check_selection_frame, jaccard


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def to_device(arr: np.ndarray, dtype: str) -> torch.Tensor:
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32))
    return t.cuda()


def from_device(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return S.bf16_bits_to_f32(t.view(torch.int16).cpu().numpy().view(np.uint16))
    return t.cpu().numpy()


class Case:
    """Storage-exact inputs of one workload (host float32 views + device tensors)."""

    def __init__(self, w: S.Workload, seed: int = 0, kv_cap: int | None = None):
        self.w = w
        Qs, Ks, Vs = S.gen_all(w, seed)
        cap = kv_cap or w.kv_len
        if cap > w.kv_len:  # spare capacity filled with garbage that must never be read
            pad = ((0, 0), (0, 0), (0, cap - w.kv_len), (0, 0))
            fill = 0x7FC0 if w.dtype == "bf16" else np.float32(np.nan)  # NaN
            Ks = np.pad(Ks, pad, constant_values=fill)
            Vs = np.pad(Vs, pad, constant_values=fill)
        self.Q = S.as_f32(Qs, w.dtype)
        self.K = S.as_f32(Ks, w.dtype)
        self.V = S.as_f32(Vs, w.dtype)
        self.q = to_device(Qs, w.dtype)
        self.k = to_device(Ks, w.dtype)
        self.v = to_device(Vs, w.dtype)
        self.kv_cap = cap
        self.scale = O.default_scale(w.head_dim)
        self._kc = None

    def k_comp64(self):
        if self._kc is None:
            self._kc = O.compress_keys(self.K[:, :, : self.w.kv_len], self.w.block_size)
        return self._kc


def check_compress(case: Case, k_comp_dev: torch.Tensor) -> None:
    """GPU compressed keys vs the oracle within the float32 summation bound."""
    w = case.w
    nb = w.kv_len // w.block_size
    got = k_comp_dev[:, :, :nb].cpu().numpy().astype(np.float64)
    ref = case.k_comp64()
    Kb = np.abs(case.K[:, :, : nb * w.block_size].astype(np.float64)).reshape(
        w.batch, w.n_kv_heads, nb, w.block_size, w.head_dim)
    bound = (w.block_size - 1) * 2.0 ** -24 * Kb.sum(axis=3) / w.block_size + 1e-30
    err = np.abs(got - ref)
    assert (err <= bound).all(), f"compress error {err.max():.3e} above bound"


def check_rows(case: Case, sel: np.ndarray, out: np.ndarray, rows, q_pos0: int, scores_gpu: np.ndarray | None = None,
               check_output=True) -> dict:
    """Selection (acceptance rule) and output parity for the given (b, t, g) rows.

    Outputs are compared with the oracle's attention over the GPU's own
    (validated) selection by :func:`qsa_check.check_output_row`: bf16 within
    the 2e-2 acceptance bound and the per-row companion bound, fp32 within
    1e-5 of each row's largest output.

    ``sel`` is ``[b][q_len][Hkv][k]``, ``out`` ``[b][q_len][Hq][d]`` (GPU, as float32).
    """
    w = case.w
    G, Bs, k = w.group, w.block_size, w.top_k
    kc = case.k_comp64()
    stats = {"clear": 0, "ambiguous": 0, "jaccard": []}
    max_err = max_ratio = 0.0
    for b, t, g in rows:
        p = q_pos0 + t
        n_cand, forced = O.selection_frame(p, Bs, w.keep_tail)
        qg = case.Q[b, t, g * G:(g + 1) * G].astype(np.float64)
        sc = O.block_scores(qg, kc[b, g], n_cand, case.scale)
        row_sel = [int(x) for x in sel[b, t, g]]
        stats[check_selection_frame(row_sel, sc, n_cand, forced, k)] += 1
        stats["jaccard"].append(jaccard(row_sel, O.select_in_frame(sc, n_cand, forced, k)))
        if scores_gpu is not None:
            kept = [c for c in row_sel if 0 <= c < n_cand]
            got = scores_gpu[b, t, g, : len(kept)]
            ref = sc[kept]
            mag = case.scale * (np.abs(qg).sum(0)[None, :] * np.abs(kc[b, g, kept])).sum(1)
            assert (np.abs(got - ref) <= (w.head_dim + G + Bs + 8) * 2.0 ** -24 * mag + 1e-30).all()
            rest = scores_gpu[b, t, g, len(kept):]
            if forced is not None:
                assert rest[0] == np.inf
                rest = rest[1:]
            assert (rest == -np.inf).all()
        if check_output:
            ref = O.attend_given_selection(qg, case.K[b, g], case.V[b, g], row_sel, p, Bs, case.scale)
            got = out[b, t, g * G:(g + 1) * G].astype(np.float64)
            ratio = check_output_row(got, ref, w.dtype, where=f"row {(b, t, g)}:")
            max_ratio = max(max_ratio, ratio)
            max_err = max(max_err, float(np.abs(got - ref).max()))
    stats["max_err"] = max_err
    stats["max_err_over_row_bound"] = round(max_ratio, 4)
    stats["mean_jaccard"] = float(np.mean(stats["jaccard"])) if stats["jaccard"] else 1.0
    del stats["jaccard"]
    return stats
