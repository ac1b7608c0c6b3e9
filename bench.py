"""QSA benchmark on one MI355X.

``python bench.py [--workload NAME] [--prefill-workload NAME|none] [--steps K] [--warmup W] [--gpus 1]``

A step is one pass of the whole QSA hot path over one batch of synthetic
input, with every input already resident in HBM:

* decode workloads: compress the key block completed by the new token (when
  its position closes a block), score + select, sparse decode attention
  (on the 64 x 128K batch: the one qsa_decode_step call, a single fused
  kernel); throughput is tokens (= sequences) per second;
* prefill workloads: compress every block, score + select for every token,
  sparse prefill attention; throughput is prompt tokens per second.

The line's workload is the 64-sequence 131,072-token batched decode (the
largest decode configuration, where the HBM bound is meaningful); the 8,192-
token prefill (the MFMA-bound configuration) is reported as its second
record under "prefill", with the same fields.

Timed region: exactly ``steps`` steps, each preceded by a 1 GiB read that
evicts L2 and the 256 MiB MALL, with HIP events on the launch stream around
every ABI call of the step (the flush lies outside them); ``value`` and
``ms_per_step`` are the mean of those cold steps. A second figure ("hot")
replays the step back to back from HIP graphs with warm caches. The roofline
entry is the call with the largest mean duration, priced against the bound of
its kernels (HBM bytes or bf16 MFMA flops, algorithmic counts only).

The CPU baseline is the fp64 oracle, unmodified, timed on a bounded sample of
the same workload by a pool of single-threaded worker processes (one per host
core this process may use, at most 16), scaled to the same unit.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "QSA decode tokens/s + achieved HBM GB/s (% peak); prefill MFMA TFLOP/s (% peak)"
HBM_PEAK_GBS = 8000.0             # MI355X HBM3E, 8 TB/s
BF16_PEAK_TFLOPS = 2516.6         # 256 CU x 2.4 GHz x 4096 dense bf16 flop/clk
DEFAULT_WORKLOAD = "decode_b64_128k"  # the largest decode configuration: the HBM bound is meaningful there
PREFILL_WORKLOAD = "prefill_8k"       # the MFMA-bound prefill configuration, the line's second record


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD, help="the line's workload (its figures are the line's)")
    ap.add_argument("--prefill-workload", default=PREFILL_WORKLOAD,
                    help="prefill workload reported as the line's second record ('none' to skip)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="budget of each oracle baseline worker")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph-steps", type=int, default=8,
                    help="steps per graph of the hot (back-to-back) replay")
    ap.add_argument("--flush-mib", type=int, default=1024, help="memory read before every timed step")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="also run a plain device copy of this many MiB (reference for memory counters)")
    return ap.parse_args()


# ------------------------------------------------------------- algorithmic work

def frame(p: int, bs: int, keep_tail: bool):
    """(candidate blocks, always-kept block or None) of a query at position p."""
    if not keep_tail:
        return p // bs, p // bs
    n = (p + 1) // bs
    return n, (n if (p + 1) % bs else None)


def visible_keys(p: int, bs: int, k: int, keep_tail: bool = False) -> int:
    """Keys a query at position p attends to under the selection rule."""
    n_cand, forced = frame(p, bs, keep_tail)
    return min(k - 1, n_cand) * bs + (0 if forced is None else p - forced * bs + 1)


def work_model(w, n_new_blocks: int, lens=None):
    """Algorithmic bytes / flops per ABI call of one step (nothing QSA skips is counted).

    ``lens``: per-sequence lengths of a ragged decode batch (the sum of every
    sequence's own model, each closing a block when its length is a multiple
    of the block size)."""
    if lens is not None and w.ragged:
        total = {}
        for n in lens:
            one = work_model(w.replace(batch=1, kv_len=n, ragged=False), 1 if n % w.block_size == 0 else 0)
            for key, val in one.items():
                acc = total.setdefault(key, {"bytes": 0, "flops": 0})
                acc["bytes"] += val["bytes"]
                acc["flops"] += val["flops"]
        return total
    b, hq, hkv, d, bs, k = w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.block_size, w.top_k
    el = 2 if w.dtype == "bf16" else 4
    m = {}
    if w.mode == "decode":
        p = w.kv_len - 1
        cand = frame(p, bs, w.keep_tail)[0]
        rows = b * hkv
        m["compress"] = {"bytes": rows * n_new_blocks * (bs * d * el + d * 4), "flops": 0}
        if w.indexer_dim:
            di, G = w.indexer_dim, hq // hkv
            m["index_keys"] = {"bytes": rows * n_new_blocks * (d + di) * 4 + d * di * 4,
                               "flops": 2 * d * di * rows * n_new_blocks}
            m["select"] = {"bytes": rows * cand * di * 4 + b * hq * d * el + d * di * 4 + rows * k * 4,
                           "flops": rows * (2 * G * d * di + 2 * G * di * cand)}
        else:
            m["select"] = {"bytes": rows * cand * d * 4 + b * hq * d * el + rows * k * 4,
                           "flops": 2 * d * rows * cand}
        vis = visible_keys(p, bs, k, w.keep_tail)
        if w.kv_q8:
            # 8-bit codes plus a float16 scale per 32 values, for K and V
            m["quantize"] = {"bytes": rows * 2 * (d * el + d + d // 32 * 2), "flops": 0}
            m["attend"] = {"bytes": rows * vis * (d + d // 32 * 2) * 2 + 2 * b * hq * d * el + rows * k * 4,
                           "flops": 4 * d * hq * b * vis}
        else:
            m["attend"] = {"bytes": rows * vis * d * el * 2 + 2 * b * hq * d * el + rows * k * 4,
                           "flops": 4 * d * hq * b * vis}
    else:
        # query rows [q_pos0, kv_len) over every key below kv_len; the blocks
        # completed before q_pos0 are already compressed
        T, t0 = w.kv_len, w.q_pos0
        qn = T - t0
        nb = T // bs
        rows = b * hkv
        m["compress"] = {"bytes": rows * n_new_blocks * (bs * d * el + d * 4), "flops": 0}
        cand_sum = sum(frame(t, bs, w.keep_tail)[0] for t in range(t0, T))
        m["select"] = {"bytes": rows * nb * d * 4 + b * qn * hq * d * el + b * qn * hkv * k * 4,
                       "flops": 2 * d * rows * cand_sum}
        vis_sum = sum(visible_keys(t, bs, k, w.keep_tail) for t in range(t0, T))
        m["attend"] = {"bytes": 2 * b * qn * hq * d * el + rows * T * d * el * 2 + b * qn * hkv * k * 4,
                       "flops": 4 * d * hq * b * vis_sum}
    return m


# ------------------------------------------------------------- GPU step

class Step:
    """The ABI calls of one step on resident device buffers."""

    def __init__(self, w, seed, inputs):
        import torch
        import qsa_synth as S
        import block_sparse_long_compress_amd as qsa

        self.w, self.qsa, self.torch = w, qsa, torch
        Qs, Ks, Vs = inputs

        def dev(x):
            t = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16) if w.dtype == "bf16" else torch.from_numpy(x)
            return t.cuda()

        self.q, self.k, self.v = dev(Qs), dev(Ks), dev(Vs)
        del Qs, Ks, Vs
        b, hq, hkv, d, bs, k = w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.block_size, w.top_k
        cap = w.kv_len
        self.shape = qsa.make_shape(b, hq, hkv, d, bs, k, self.q.dtype, keep_tail=w.keep_tail)
        self.k_comp = torch.empty(b, hkv, cap // bs, d, dtype=torch.float32, device="cuda")
        q_len, q_pos0 = w.q_len, w.q_pos0
        self.sel = torch.empty(b, q_len, hkv, k, dtype=torch.int32, device="cuda")
        self.out = torch.empty_like(self.q)
        self.ws_sel = self._ws(qsa.QSA_OP_SELECT, q_len, w.kv_len)
        self.fused = False
        if w.mode == "decode":
            self.q_dec = self.q.view(b, hq, d)
            self.out_dec = self.out.view(b, hq, d)
            self.sel_dec = self.sel.view(b, hkv, k)
            self.ws_att = self._ws(qsa.QSA_OP_DECODE, 1, w.kv_len)
            self.lens = S.seq_lengths(w, seed)
            if w.ragged:
                # every sequence at its own length: one ragged step call
                self.ws_step = self._ws(qsa.QSA_OP_DECODE_STEP_RAGGED, 1, w.kv_len)
                self.fused = True
                self.kv_lens = torch.tensor(self.lens, dtype=torch.int32, device="cuda")
                one = qsa.make_shape(1, hq, hkv, d, bs, k, self.q.dtype, keep_tail=w.keep_tail)
                for bb, n in enumerate(self.lens):
                    qsa.qsa_compress_keys(one, self.k[bb:bb + 1], n - 1, self.k_comp[bb:bb + 1])
                self.blk_begin = 0
                self.n_new_blocks = sum(1 for n in self.lens if n % bs == 0)
            elif w.kv_q8:
                # the attention reads the rotated 8-bit cache: one qsa_decode_step_q8 call (quantize the
                # new position, compress, select and attend in one kernel) where the fused kernel serves
                # the shape, else the separate calls
                self.fused = qsa.qsa_decode_step_fused(self.shape, w.kv_len)
                self.ws_step = self._ws(qsa.QSA_OP_DECODE_STEP, 1, w.kv_len) if self.fused else None
                self.kq, self.vq, self.ks, self.vs = qsa.kv_q8_buffers(self.k)
                qsa.qsa_kv_quantize(self.shape, self.k, self.v, w.kv_len - 1, self.kq, self.vq, self.ks, self.vs)
                qsa.qsa_compress_keys(self.shape, self.k, w.kv_len - 1, self.k_comp)
                self.blk_begin = (w.kv_len - 1) // bs
                self.n_new_blocks = w.kv_len // bs - self.blk_begin
            elif w.indexer_dim:
                # learned-indexer selection: one qsa_indexer_decode_step call where it serves the shape
                # (bf16, k <= 64), else the separate calls (compress and project the closed block, indexer
                # select, decode attention)
                self.ws_step = None
                self.fused = w.dtype == "bf16" and w.top_k <= 64
                w_q, w_k = S.indexer_weights(seed, w.cfg_id, d, w.indexer_dim)
                self.w_q, self.w_k = torch.from_numpy(w_q).cuda(), torch.from_numpy(w_k).cuda()
                self.ix = qsa.make_indexer(w.indexer_dim, w.indexer_agg)
                self.k_idx = torch.empty(b, hkv, cap // bs, w.indexer_dim, dtype=torch.float32, device="cuda")
                qsa.qsa_compress_keys(self.shape, self.k, w.kv_len - 1, self.k_comp)
                qsa.qsa_indexer_keys(self.shape, self.ix, self.w_k, self.k_comp, w.kv_len - 1, cap, self.k_idx)
                self.blk_begin = (w.kv_len - 1) // bs
                self.n_new_blocks = w.kv_len // bs - self.blk_begin
            else:
                self.ws_step = self._ws(qsa.QSA_OP_DECODE_STEP, 1, w.kv_len)
                self.fused = qsa.qsa_decode_step_fused(self.shape, w.kv_len)
                # everything before the new token is already compressed
                qsa.qsa_compress_keys(self.shape, self.k, w.kv_len - 1, self.k_comp)
                self.blk_begin = (w.kv_len - 1) // bs
                self.n_new_blocks = w.kv_len // bs - self.blk_begin
        else:
            self.ws_att = self._ws(qsa.QSA_OP_PREFILL, q_len, w.kv_len)
            # a prefill chunk at q_pos0: the blocks completed before it are already compressed
            self.blk_begin = q_pos0 // bs
            if self.blk_begin > 0:
                qsa.qsa_compress_keys(self.shape, self.k, q_pos0, self.k_comp)
            self.n_new_blocks = w.kv_len // bs - self.blk_begin
        torch.cuda.synchronize()
        # `calls`: the ABI calls of a step, each timed on its own; `step_calls`:
        # what one step enqueues (a decode step is the one qsa_decode_step call,
        # which runs the separate calls itself when it is not fused)
        self.calls = [("select", self.select), ("attend", self.attend)]
        if self.n_new_blocks > 0:
            self.calls.insert(0, ("compress", self.compress))
        if self.n_new_blocks > 0 and w.indexer_dim:
            self.calls.insert(1, ("index_keys", self.index_keys))
        if w.kv_q8:
            self.calls.insert(len(self.calls) - 2, ("quantize", self.quantize))
        separate = (w.indexer_dim or w.kv_q8) and not self.fused
        self.step_calls = [("step", self.decode_step)] if w.mode == "decode" and not separate else self.calls
        # a decode step is timed as the one step call wherever it is one (also where the step runs more than
        # one kernel, as for k > 64)
        if self.fused or (w.mode == "decode" and not separate):
            self.calls = self.step_calls

    def _ws(self, op, q_len, kv_len):
        ws = self.qsa.workspace(self.shape, op, q_len, kv_len, "cuda")
        return ws if ws is not None else self.torch.empty(16, dtype=self.torch.uint8, device="cuda")

    def decode_step(self):
        w = self.w
        if w.indexer_dim:
            self.qsa.qsa_indexer_decode_step(self.shape, self.ix, self.w_q, self.w_k, self.q_dec, self.k, self.v,
                                             self.k_comp, self.k_idx, w.kv_len, self.sel_dec, self.out_dec)
            return
        if w.kv_q8:
            self.qsa.qsa_decode_step_q8(self.shape, self.q_dec, self.k, self.v, self.k_comp, self.kq, self.vq,
                                        self.ks, self.vs, w.kv_len, self.sel_dec, self.out_dec, ws=self.ws_step)
            return
        if w.ragged:
            self.qsa.qsa_decode_step_ragged(self.shape, self.q_dec, self.k, self.v, self.k_comp, self.kv_lens,
                                            w.kv_len, self.sel_dec, self.out_dec, ws=self.ws_step)
            return
        self.qsa.qsa_decode_step(self.shape, self.q_dec, self.k, self.v, self.k_comp, w.kv_len, self.sel_dec,
                                 self.out_dec, ws=self.ws_step)

    def compress(self):
        self.qsa.qsa_compress_keys(self.shape, self.k, self.w.kv_len, self.k_comp, block_begin=self.blk_begin)

    def quantize(self):
        w = self.w
        self.qsa.qsa_kv_quantize(self.shape, self.k, self.v, w.kv_len, self.kq, self.vq, self.ks, self.vs,
                                 pos_begin=w.kv_len - 1)

    def index_keys(self):
        w = self.w
        self.qsa.qsa_indexer_keys(self.shape, self.ix, self.w_k, self.k_comp, w.kv_len, w.kv_len, self.k_idx,
                                  block_begin=self.blk_begin)

    def select(self):
        w = self.w
        if w.indexer_dim:
            self.qsa.qsa_indexer_select(self.shape, self.ix, self.w_q, self.q, w.q_pos0, self.k_idx, w.kv_len,
                                        w.kv_len, self.sel)
            return
        self.qsa.qsa_score_select(self.shape, self.q, w.q_pos0, self.k_comp, w.kv_len, w.kv_len, self.sel,
                                  ws=self.ws_sel)

    def attend(self):
        w = self.w
        if w.mode == "decode" and w.kv_q8:
            self.qsa.qsa_sparse_attn_decode_q8(self.shape, self.q_dec, self.kq, self.vq, self.ks, self.vs, w.kv_len,
                                               self.sel_dec, self.out_dec, ws=self.ws_att)
        elif w.mode == "decode":
            self.qsa.qsa_sparse_attn_decode(self.shape, self.q_dec, self.k, self.v, w.kv_len, self.sel,
                                            self.out_dec, ws=self.ws_att)
        else:
            self.qsa.qsa_sparse_attn_prefill(self.shape, self.q, self.k, self.v, w.q_pos0, self.sel, self.out,
                                             ws=self.ws_att)




# ------------------------------------------------------------- GPU timing

def _event(torch):
    return torch.cuda.Event(enable_timing=True)


def run_gpu(w, inputs, steps, warmup, seed, graph_steps=8, flush_mib=1024):
    """Time one workload on the GPU.

    Timed region (the reported rate): exactly ``steps`` whole steps, each
    preceded by a read of ``flush_mib`` MiB of other memory that evicts L2 and
    the 256 MiB MALL, so every step starts from HBM. HIP events recorded on the
    launch stream bracket each ABI call of the step; the flush lies outside
    them. The whole region is bracketed by ``torch.cuda.synchronize()``.

    Secondary (hot): ``steps`` steps replayed back to back from HIP graphs of
    ``graph_steps`` steps each (caches warm: a 64 x 128K step's 202 MB fits the
    MALL), wall clock between two synchronisations.
    """
    import torch

    st = Step(w, seed, inputs)
    stream = torch.cuda.Stream()
    flush = torch.ones(max(1, flush_mib) << 18, dtype=torch.int32, device="cuda")
    with torch.cuda.stream(stream):
        for _, fn in st.step_calls + st.calls:
            fn()  # eager warm-up before capture
        torch.cuda.synchronize()
        step_graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(step_graph, stream=stream):
            for _, fn in st.step_calls:
                fn()
        group = max(1, graph_steps)
        group_graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(group_graph, stream=stream):
            for _ in range(group):
                for _, fn in st.step_calls:
                    fn()
        torch.cuda.synchronize()
        for _ in range(warmup):
            flush.amax()
            for _, fn in st.calls:
                fn()
            step_graph.replay()
        torch.cuda.synchronize()

        # timed region: cold steps, events around every call of each step
        n_calls = len(st.calls)
        ev = [[_event(torch) for _ in range(n_calls + 1)] for _ in range(steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for r in range(steps):
            flush.amax()
            ev[r][0].record(stream)
            for i, (_, fn) in enumerate(st.calls):
                fn()
                ev[r][i + 1].record(stream)
        torch.cuda.synchronize()
        wall_cold = time.perf_counter() - t0

        # hot: back-to-back graph replays
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        for _ in range(steps // group):
            group_graph.replay()
        for _ in range(steps % group):
            step_graph.replay()
        torch.cuda.synchronize()
        wall_hot = time.perf_counter() - t1
    del flush
    per_call = {name: [1e-3 * ev[r][i].elapsed_time(ev[r][i + 1]) for r in range(steps)]
                for i, (name, _) in enumerate(st.calls)}
    step_s = [1e-3 * ev[r][0].elapsed_time(ev[r][n_calls]) for r in range(steps)]
    return st, {"step_s": step_s, "per_call_s": per_call, "wall_cold_s": wall_cold, "wall_hot_s": wall_hot}


# ------------------------------------------------------------- CPU baseline (the oracle, unmodified)

def _cpu_workers() -> int:
    """Host cores the baseline's process pool uses: this process's CPU affinity, at most 16 (one GPU's
    share of the host)."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def _cpu_decode_worker(job):
    """One worker: decode steps of one sequence with the fp64 oracle, single BLAS thread, for ``budget_s``
    seconds. The compressed keys of the blocks closed before the new token are built beforehand (outside
    the timed loop), as the GPU step has them; every step compresses the block the token closes."""
    w, seed, b, budget_s = job
    from threadpoolctl import threadpool_limits

    import qsa_synth as S
    from oracle import qsa_oracle as O

    with threadpool_limits(limits=1):
        G, bs, k = w.group, w.block_size, w.top_k
        scale = O.default_scale(w.head_dim)
        q = S.gen_q(w, seed, b)
        K = np.stack([S.gen_kv(w, seed, S.TENSOR_K, b, g, q) for g in range(w.n_kv_heads)])
        V = np.stack([S.gen_kv(w, seed, S.TENSOR_V, b, g) for g in range(w.n_kv_heads)])
        n0 = S.seq_lengths(w, seed)[b]
        p = n0 - 1
        n_prev = p // bs
        kc = np.zeros((w.n_kv_heads, w.kv_len // bs, w.indexer_dim or w.head_dim))
        if w.indexer_dim:
            from oracle import qsa_indexer as IX
            w_q, w_k = (x.astype(np.float64) for x in S.indexer_weights(seed, w.cfg_id, w.head_dim, w.indexer_dim))
            iscale = IX.default_indexer_scale(w.indexer_dim)
            kc[:, :n_prev] = IX.indexer_keys(K[:, : n_prev * bs], w_k, bs)
        else:
            kc[:, :n_prev] = O.compress_keys(K[:, : n_prev * bs], bs)
        n_cand, forced = O.selection_frame(p, bs, w.keep_tail)
        n_steps, t0 = 0, time.perf_counter()
        while True:
            if (p + 1) % bs == 0:  # the new token completes its block
                blk = K[:, n_prev * bs:(n_prev + 1) * bs]
                kc[:, n_prev:n_prev + 1] = IX.indexer_keys(blk, w_k, bs) if w.indexer_dim else O.compress_keys(blk, bs)
            for g in range(w.n_kv_heads):
                qg = q[0, g * G:(g + 1) * G].astype(np.float64)
                if w.indexer_dim:
                    sc = IX.indexer_scores(qg, w_q, kc[g], n_cand, iscale, w.indexer_agg)
                else:
                    sc = O.block_scores(qg, kc[g], n_cand, scale)
                sel = O.select_in_frame(sc, n_cand, forced, k)
                O.attend_given_selection(qg, K[g], V[g], sel, p, bs, scale)
            n_steps += 1
            el = time.perf_counter() - t0
            if el >= budget_s:
                break
    return n_steps, el, n0, n_cand


def _cpu_prefill_worker(job):
    """One worker: the prompt's compression (timed), then the given query rows (both KV heads) for at most
    ``budget_s`` seconds."""
    w, seed, rows, budget_s = job
    from threadpoolctl import threadpool_limits

    import qsa_synth as S
    from oracle import qsa_oracle as O

    with threadpool_limits(limits=1):
        G, bs, k = w.group, w.block_size, w.top_k
        scale = O.default_scale(w.head_dim)
        Qs, Ks, Vs = S.gen_all(w, seed, workers=1)
        Q, K, V = (S.as_f32(x, w.dtype) for x in (Qs, Ks, Vs))
        # blocks completed before the chunk's first row are already compressed (untimed)
        blk0, nb = w.q_pos0 // bs, w.kv_len // bs
        kc_old = O.compress_keys(K[:, :, : blk0 * bs], bs) if blk0 else None
        t0 = time.perf_counter()
        kc = O.compress_keys(K[:, :, blk0 * bs: nb * bs], bs)
        t_comp = time.perf_counter() - t0
        if kc_old is not None:
            kc = np.concatenate([kc_old, kc], axis=2)
        done, t1 = 0, time.perf_counter()
        for t in rows:
            n_cand, forced = O.selection_frame(int(t), bs, w.keep_tail)
            for g in range(w.n_kv_heads):
                qg = Q[0, t - w.q_pos0, g * G:(g + 1) * G].astype(np.float64)
                sc = O.block_scores(qg, kc[0, g], n_cand, scale)
                sel = O.select_in_frame(sc, n_cand, forced, k)
                O.attend_given_selection(qg, K[0, g], V[0, g], sel, int(t), bs, scale)
            done += 1
            if time.perf_counter() - t1 >= budget_s:
                break
    return done, time.perf_counter() - t1, t_comp


def cpu_baseline(w, seed, budget_s):
    """The fp64 oracle, unchanged, on a bounded sample of the same workload, run by a pool of single-threaded
    worker processes (one per host core this process may use, at most 16), each on independent work.

    decode: worker i runs decode steps of sequence i (both KV heads); the rate is the sum of the workers'
    rates (tokens/s), i.e. the whole pool's decode throughput.
    prefill: the workers split a random order of the prompt's query rows; the prompt time is one
    compression plus all rows at the pool's measured row rate.
    Worker processes are forked before this process touches the GPU (they never use it)."""
    import multiprocessing as mp

    n = _cpu_workers()
    ctx = mp.get_context("fork")
    if w.mode == "decode":
        jobs = [(w, seed, i % w.batch, budget_s) for i in range(n)]
        with ctx.Pool(n) as pool:
            res = pool.map(_cpu_decode_worker, jobs)
        rate = sum(steps / el for steps, el, _, _ in res)
        total = sum(steps for steps, _, _, _ in res)
        _, el0, n0, n_cand = res[0]
        return {"value": rate, "unit": "tokens/s", "cores": n, "kind": "oracle",
                "sample": f"{n} single-threaded worker processes, each {budget_s:.0f} s of decode steps of one "
                          f"sequence ({total} steps in all; sequence of {n0} tokens, both KV heads: compress of "
                          f"the completed block, scores over {n_cand} candidates, top-{w.top_k} selection, "
                          f"attention); rate = sum of the workers' rates"}
    order = w.q_pos0 + np.random.default_rng(seed).permutation(w.q_len)
    jobs = [(w, seed, order[i::n], budget_s) for i in range(n)]
    with ctx.Pool(n) as pool:
        res = pool.map(_cpu_prefill_worker, jobs)
    row_rate = sum(done / el for done, el, _ in res)
    done = sum(d for d, _, _ in res)
    t_comp = float(np.median([tc for _, _, tc in res]))
    est = t_comp + w.q_len / row_rate
    n_new = w.kv_len // w.block_size - w.q_pos0 // w.block_size
    return {"value": w.batch * w.q_len / est, "unit": "tokens/s", "cores": n, "kind": "oracle",
            "sample": f"{n} single-threaded worker processes, each {budget_s:.0f} s: compression of the "
                      f"{n_new} blocks the prompt completes ({t_comp:.3f} s) + {done} of its {w.q_len} query "
                      f"rows (both KV heads) in all, drawn in random order; the prompt time is one compression "
                      f"plus every row at the pool's row rate ({row_rate:.1f} rows/s)"}


# ------------------------------------------------------------- measured traffic

def source_sha256():
    """SHA-256 over the kernel sources (name, then bytes, in name order)."""
    import hashlib

    h = hashlib.sha256()
    d = os.path.join(ROOT, "block_sparse_long_compress_amd", "csrc")
    for n in sorted(os.listdir(d)):
        if n.endswith((".hip", ".h", ".cpp")):
            h.update(n.encode())
            with open(os.path.join(d, n), "rb") as f:
                h.update(f.read())
    return h.hexdigest()


def measured_traffic(workload, call):
    """HBM bytes (read + written) per launch of `call` from the committed memory-counter
    table, or None when it is missing or the kernels changed since it was taken."""
    path = os.path.join(ROOT, "profiles", "traffic.md")
    try:
        text = open(path).read()
        table = json.loads(text.split("```json", 1)[1].split("```", 1)[0])
    except (OSError, IndexError, ValueError):
        return None
    if table.get("source_sha256") != source_sha256():
        return None
    entry = table.get("workloads", {}).get(workload, {}).get(call)
    return None if entry is None else entry["read_bytes"] + entry["write_bytes"]


# ------------------------------------------------------------- report

KERNELS = {
    "step": "decode_step_kernel (compress of the closed block, selection and attention in one kernel)",
    "step_q8": "decode_step_kernel over the 8-bit cache (quantize of the new position, compress, selection and attention in one kernel)",
    "step_indexer": "indexer_select_kernel as the indexer decode step (compress and indexer key of the closed "
                    "block, indexer selection and attention in one kernel)",
    "step_large": "select_large_score_kernel (scores, with the closed block's compression) + pick_attend_kernel "
                  "(per-row pick and attention): the decode step for k > 64",
    "attend_prefill": "vt_pack_kernel + prefill_attn_kernel",
}


def record(w, st, timing, steps, seed, graph_steps):
    """The workload's figures: rate from the timed (cold) steps, roofline of its dominant call."""
    model = work_model(w, st.n_new_blocks, getattr(st, "lens", None))
    model["step"] = {"bytes": sum(m["bytes"] for m in model.values()), "flops": sum(m["flops"] for m in model.values())}
    tokens = w.batch if w.mode == "decode" else w.batch * w.q_len
    step_s = float(np.mean(timing["step_s"]))
    per_call = {n: float(np.mean(v)) for n, v in timing["per_call_s"].items()}
    dominant = max(per_call, key=lambda n: per_call[n])
    dur = per_call[dominant]
    if w.mode == "prefill" and dominant == "attend":
        achieved, peak, unit, bound = model[dominant]["flops"] / dur / 1e12, BF16_PEAK_TFLOPS, "TFLOP/s", "mfma"
        kernel = KERNELS["attend_prefill"]
    else:
        achieved, peak, unit, bound = model[dominant]["bytes"] / dur / 1e9, HBM_PEAK_GBS, "GB/s", "hbm"
        step_kernel = (KERNELS["step_q8"] if w.kv_q8 else KERNELS["step_indexer"] if w.indexer_dim
                       else KERNELS["step"] if st.fused else KERNELS["step_large"])
        kernel = step_kernel if dominant == "step" else f"{dominant} call"
    calls = {}
    for n, t in per_call.items():
        entry = {"us": round(t * 1e6, 3), "p10_us": round(1e6 * float(np.percentile(timing["per_call_s"][n], 10)), 3),
                 "p90_us": round(1e6 * float(np.percentile(timing["per_call_s"][n], 90)), 3),
                 "bytes": model[n]["bytes"], "GB/s": round(model[n]["bytes"] / t / 1e9, 1)}
        if model[n]["flops"]:
            entry["flops"] = model[n]["flops"]
            entry["TFLOP/s"] = round(model[n]["flops"] / t / 1e12, 2)
        calls[n] = entry
    hot_s = timing["wall_hot_s"] / steps
    cfg = {"workload": w.name, "mode": w.mode, "batch": w.batch, "kv_len": w.kv_len,
           "q_heads": w.n_q_heads, "kv_heads": w.n_kv_heads, "head_dim": w.head_dim,
           "block_size": w.block_size, "top_k": w.top_k, "keep_tail": w.keep_tail, "seed": seed,
           "fused_decode_step": bool(st.fused), "ragged": w.ragged}
    if w.kv_q8:
        cfg["kv_cache"] = "rotated 8-bit (codes + float16 scale per 32)"
    if w.indexer_dim:
        cfg.update({"indexer_dim": w.indexer_dim, "indexer_agg": ["sum", "max", "softmax"][w.indexer_agg]})
    if w.ragged:
        cfg.update({"mean_kv_len": round(float(np.mean(st.lens)), 1), "min_kv_len": int(min(st.lens))})
    if w.mode == "prefill" and w.q_pos0:
        cfg.update({"q_rows": w.q_len, "q_pos0": w.q_pos0})
    return {
        "value": round(tokens / step_s, 2),
        "ms_per_step": round(1e3 * step_s, 5),
        "config": cfg,
        "roofline": {"bound": bound, "kernel": kernel, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
                     "frac": round(achieved / peak, 4), "traffic": measured_traffic(w.name, dominant),
                     "timing": f"mean of {steps} cold steps, HIP events on the launch stream around the call"},
        "calls": calls,
        "timed_region": {"steps": steps, "wall_s": round(timing["wall_cold_s"], 4),
                         "note": "each step preceded by a 1 GiB read (outside the events) that evicts L2 and MALL"},
        "hot": {"ms_per_step": round(1e3 * hot_s, 5), "value": round(tokens / hot_s, 2),
                "note": f"steps replayed back to back from HIP graphs of {graph_steps} steps, caches warm"},
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU: --gpus must be 1 (no multi-GPU path; the design "
                                   "notes describe how the work would shard)"}), flush=True)
        sys.exit(2)
    import qsa_synth as S

    w = S.WORKLOADS[args.workload]
    wp = None if args.prefill_workload == "none" or args.prefill_workload == args.workload \
        else S.WORKLOADS[args.prefill_workload]
    # host work first, before anything touches the GPU: the oracle baselines (a forked process pool) and
    # the inputs (generated by forked workers too)
    cpu = {}
    if not args.no_cpu_baseline:
        for x in (w, wp):
            if x is not None:
                cpu[x.name] = cpu_baseline(x, args.seed, args.cpu_seconds)
                cpu[x.name]["value"] = round(cpu[x.name]["value"], 3)
    inputs = S.gen_all(w, args.seed)
    inputs_p = S.gen_all(wp, args.seed) if wp is not None else None

    st, timing = run_gpu(w, inputs, args.steps, args.warmup, args.seed, args.graph_steps, args.flush_mib)
    del inputs
    main_rec = record(w, st, timing, args.steps, args.seed, args.graph_steps)
    del st
    line = {
        "metric": METRIC,
        "value": main_rec["value"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": main_rec["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": main_rec["config"],
        "roofline": main_rec["roofline"],
        "calls": main_rec["calls"],
        "timed_region": main_rec["timed_region"],
        "hot": main_rec["hot"],
    }
    if w.name in cpu:
        line["cpu_baseline"] = cpu[w.name]
    if wp is not None:
        import torch

        torch.cuda.empty_cache()
        stp, tp = run_gpu(wp, inputs_p, args.steps, args.warmup, args.seed, args.graph_steps, args.flush_mib)
        rec = record(wp, stp, tp, args.steps, args.seed, args.graph_steps)
        rec["unit"] = "tokens/s"
        rec["dtype"] = wp.dtype
        if wp.name in cpu:
            rec["cpu_baseline"] = cpu[wp.name]
        line["prefill"] = rec
    if args.copy_calibration_mib > 0:
        import torch

        n = args.copy_calibration_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        line["copy_calibration_bytes"] = n
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
