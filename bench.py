"""QSA benchmark on one MI355X.

``python bench.py [--workload NAME] [--steps K] [--warmup W] [--gpus 1]``

A step is one pass of the whole QSA hot path over one batch of synthetic
input, with every input already resident in HBM:

* decode workloads: compress the key block completed by the new token (when
  its position closes a block), score + select, sparse decode attention;
  throughput is tokens (= sequences) per second;
* prefill workloads: compress every block, score + select for every token,
  sparse prefill attention; throughput is prompt tokens per second.

The step is captured in HIP graphs, `--graph-steps` whole steps back to back
per graph (8 by default, so the host's graph-launch cost, tens of
microseconds, does not starve the GPU between short steps), and the timed
region runs exactly `steps` steps (wall clock, synchronised on both sides). A
decode step is the one qsa_decode_step call. A second timed region launches
each ABI call eagerly with HIP events recorded between the calls on the
launch stream, giving per-call durations. The roofline entry is
the call with the largest average duration, against the bound of its kernels
(HBM bytes or bf16 MFMA flops, algorithmic counts only).

The CPU baseline is the fp64 oracle, unmodified, timed on a bounded sample of
the same workload on the host (single thread), scaled to the same unit.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "QSA decode tokens/s + achieved HBM GB/s (% peak); prefill MFMA TFLOP/s (% peak)"
HBM_PEAK_GBS = 8000.0             # MI355X HBM3E, 8 TB/s
BF16_PEAK_TFLOPS = 2516.6         # 256 CU x 2.4 GHz x 4096 dense bf16 flop/clk
DEFAULT_WORKLOAD = "decode_32k"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="budget of the oracle baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="launch the calls eagerly instead of replaying graphs")
    ap.add_argument("--graph-steps", type=int, default=8,
                    help="whole steps captured back to back in one graph (amortises the host's graph launch)")
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
        T = w.kv_len
        nb = T // bs
        rows = b * hkv
        m["compress"] = {"bytes": rows * nb * (bs * d * el + d * 4), "flops": 0}
        cand_sum = sum(frame(t, bs, w.keep_tail)[0] for t in range(T))
        m["select"] = {"bytes": rows * nb * d * 4 + b * T * hq * d * el + b * T * hkv * k * 4,
                       "flops": 2 * d * rows * cand_sum}
        vis_sum = sum(visible_keys(t, bs, k, w.keep_tail) for t in range(T))
        m["attend"] = {"bytes": 2 * b * T * hq * d * el + rows * T * d * el * 2 + b * T * hkv * k * 4,
                       "flops": 4 * d * hq * b * vis_sum}
    return m


# ------------------------------------------------------------- GPU step

class Step:
    """The ABI calls of one step on resident device buffers."""

    def __init__(self, w, seed):
        import torch
        import qsa_synth as S
        import block_sparse_long_compress_amd as qsa

        self.w, self.qsa, self.torch = w, qsa, torch
        Qs, Ks, Vs = S.gen_all(w, seed)

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
                # new position, then compress, select and attend in one kernel) where the fused kernel
                # serves the shape, else the separate calls
                self.fused = qsa.qsa_decode_step_fused(self.shape, w.kv_len)
                self.ws_step = self._ws(qsa.QSA_OP_DECODE_STEP, 1, w.kv_len) if self.fused else None
                self.kq, self.vq, self.ks, self.vs = qsa.kv_q8_buffers(self.k)
                qsa.qsa_kv_quantize(self.shape, self.k, self.v, w.kv_len - 1, self.kq, self.vq, self.ks, self.vs)
                qsa.qsa_compress_keys(self.shape, self.k, w.kv_len - 1, self.k_comp)
                self.blk_begin = (w.kv_len - 1) // bs
                self.n_new_blocks = w.kv_len // bs - self.blk_begin
            elif w.indexer_dim:
                # learned-indexer selection: the separate calls (compress and project the closed block,
                # indexer select, decode attention)
                self.ws_step = None
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
            self.blk_begin = 0
            self.n_new_blocks = w.kv_len // bs
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
        separate = w.indexer_dim or (w.kv_q8 and not self.fused)
        self.step_calls = [("step", self.decode_step)] if w.mode == "decode" and not separate else self.calls
        if self.fused:
            self.calls = self.step_calls

    def _ws(self, op, q_len, kv_len):
        ws = self.qsa.workspace(self.shape, op, q_len, kv_len, "cuda")
        return ws if ws is not None else self.torch.empty(16, dtype=self.torch.uint8, device="cuda")

    def decode_step(self):
        w = self.w
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
            self.qsa.qsa_sparse_attn_prefill(self.shape, self.q, self.k, self.v, 0, self.sel, self.out,
                                             ws=self.ws_att)


def capture_step(torch, st, stream):
    """Enqueue one step: the ABI calls in order on the launch stream. (A decode
    step's compression could run beside select + attend, since the block it
    closes is the token's own block and never one of its candidates; a
    forked graph branch costs more than the few microseconds it would hide.)"""
    for _, fn in st.step_calls:
        fn()


def run_gpu(w, steps, warmup, seed, use_graph, graph_steps=8):
    """Timed region: exactly `steps` whole steps, replayed from graphs that hold
    `graph_steps` consecutive steps each (plus a one-step graph for the
    remainder), wall clock, synchronised on both sides. Every step recomputes
    everything from the resident inputs; the grouping only spreads the host's
    graph-launch cost (tens of microseconds) over several steps.

    Per-call durations: the calls are launched eagerly, HIP events recorded
    between them on the launch stream, all queued behind a GPU sleep so that
    the events bracket GPU work only (no host submission gaps, no graph launch
    cost). Cold steps: the step graph replayed after a 1 GiB device read that
    evicts L2 and the 256 MiB MALL, timed by events around the replay."""
    import torch

    st = Step(w, seed)
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        for _, fn in st.step_calls + st.calls:
            fn()  # eager warm-up before capture
        torch.cuda.synchronize()
        group = max(1, graph_steps) if use_graph else 1
        if use_graph:
            step_graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(step_graph, stream=stream):
                capture_step(torch, st, stream)
            run_step = step_graph.replay
            group_graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(group_graph, stream=stream):
                for _ in range(group):
                    capture_step(torch, st, stream)
            run_group = group_graph.replay
        else:
            def run_step():
                capture_step(torch, st, stream)
            run_group = run_step
        torch.cuda.synchronize()
        for _ in range(warmup):
            run_step()
        for _ in range(max(1, warmup // group)):
            run_group()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps // group):
            run_group()
        for _ in range(steps % group):
            run_step()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0

        # per-call durations (HIP events on the launch stream, eager launches)
        n_calls = len(st.calls)
        reps = max(10, min(steps, 50))
        events = [[torch.cuda.Event(enable_timing=True) for _ in range(n_calls + 1)] for _ in range(reps)]
        for _, fn in st.calls:
            fn()
        torch.cuda.synchronize()
        s0 = torch.cuda.Event(enable_timing=True)
        s0.record(stream)
        torch.cuda._sleep(int(1e8))  # GPU busy while the host queues every launch below
        h0 = time.perf_counter()
        for r in range(reps):
            ev = events[r]
            ev[0].record(stream)
            for i, (_, fn) in enumerate(st.calls):
                fn()
                ev[i + 1].record(stream)
        enqueue_s = time.perf_counter() - h0
        torch.cuda.synchronize()
        # the host must finish queueing before the sleep ends, or gaps enter the events
        sleep_s = 1e-3 * s0.elapsed_time(events[0][0])

        # cold steps: evict L2 and MALL before each replay by reading 1 GiB
        # (a read leaves clean lines: nothing is written back during the step)
        flush = torch.ones(1 << 28, dtype=torch.int32, device="cuda")
        cold_reps = 10
        cold = []
        for _ in range(cold_reps):
            flush.amax()
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            run_step()
            b.record(stream)
            cold.append((a, b))
        torch.cuda.synchronize()
        del flush
    per_call = {}
    for i, (name, _) in enumerate(st.calls):
        per_call[name] = 1e-3 * float(np.mean([events[r][i].elapsed_time(events[r][i + 1]) for r in range(reps)]))
    cold_s = 1e-3 * float(np.mean([a.elapsed_time(b) for a, b in cold]))
    return st, wall, per_call, cold_s, {"host_enqueue_ms": round(1e3 * enqueue_s, 2),
                                        "gpu_sleep_ms": round(1e3 * sleep_s, 2), "reps": reps}


# ------------------------------------------------------------- CPU baseline

def cpu_baseline(w, seed, budget_s):
    """fp64 oracle on a bounded sample of the same workload, single thread."""
    from threadpoolctl import threadpool_limits

    import qsa_synth as S
    from oracle import qsa_oracle as O

    with threadpool_limits(limits=1):
        G, bs, k = w.group, w.block_size, w.top_k
        scale = O.default_scale(w.head_dim)
        if w.mode == "decode":
            # one sequence: its keys compressed once beforehand (as on the GPU), then repeated steps
            q = S.gen_q(w, seed, 0)
            K = np.stack([S.gen_kv(w, seed, S.TENSOR_K, 0, g, q) for g in range(w.n_kv_heads)])
            V = np.stack([S.gen_kv(w, seed, S.TENSOR_V, 0, g) for g in range(w.n_kv_heads)])
            n0 = S.seq_lengths(w, seed)[0]  # sequence 0's length (all kv_len unless ragged)
            p = n0 - 1
            n_prev = p // bs  # blocks complete before the new token
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
                if el >= budget_s or n_steps >= 100000:
                    break
            return {"value": n_steps / el, "unit": "tokens/s", "cores": 1, "kind": "oracle",
                    "sample": f"{n_steps} decode steps of one sequence of {n0} tokens (both KV heads: compress of "
                              f"the completed "
                              f"block, scores over {n_cand} candidates, top-{k} selection, attention) in {el:.1f} s"
                              + (" (sequence 0 of the ragged batch; its steps stand for the batch's)" if w.ragged
                                 else "")}
        # prefill: compress everything, then a uniform sample of query rows, scaled to the full prompt
        Qs, Ks, Vs = S.gen_all(w, seed)
        Q, K, V = (S.as_f32(x, w.dtype) for x in (Qs, Ks, Vs))
        t0 = time.perf_counter()
        kc = O.compress_keys(K, bs)
        t_comp = time.perf_counter() - t0
        rng = np.random.default_rng(seed)
        order = rng.permutation(w.kv_len)
        done, t1 = 0, time.perf_counter()
        for t in order:
            n_cand, forced = O.selection_frame(int(t), bs, w.keep_tail)
            for g in range(w.n_kv_heads):
                qg = Q[0, t, g * G:(g + 1) * G].astype(np.float64)
                sc = O.block_scores(qg, kc[0, g], n_cand, scale)
                sel = O.select_in_frame(sc, n_cand, forced, k)
                O.attend_given_selection(qg, K[0, g], V[0, g], sel, t, bs, scale)
            done += 1
            if time.perf_counter() - t1 >= budget_s:
                break
        t_rows = time.perf_counter() - t1
        est = t_comp + t_rows * w.kv_len / done
        return {"value": w.batch * w.kv_len / est, "unit": "tokens/s", "cores": 1, "kind": "oracle",
                "sample": f"compress of all {w.kv_len // bs} blocks ({t_comp:.2f} s) + {done} uniformly sampled "
                          f"query tokens of {w.kv_len} ({t_rows:.1f} s), scaled to the whole prompt"}


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


# ------------------------------------------------------------- main

def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1"}))
        sys.exit(2)
    import qsa_synth as S

    w = S.WORKLOADS[args.workload]
    st, wall, per_call, cold_s, call_timing = run_gpu(w, args.steps, args.warmup, args.seed, not args.no_graph,
                                                      args.graph_steps)
    model = work_model(w, st.n_new_blocks, getattr(st, "lens", None))
    model["step"] = {"bytes": sum(m["bytes"] for m in model.values()), "flops": sum(m["flops"] for m in model.values())}
    ms_per_step = 1e3 * wall / args.steps
    tokens = w.batch if w.mode == "decode" else w.batch * w.kv_len
    value = tokens * args.steps / wall

    dominant = max(per_call, key=lambda n: per_call[n])
    dur = per_call[dominant]
    if w.mode == "prefill" and dominant == "attend":
        achieved, peak, unit, bound = model[dominant]["flops"] / dur / 1e12, BF16_PEAK_TFLOPS, "TFLOP/s", "mfma"
    else:
        achieved, peak, unit, bound = model[dominant]["bytes"] / dur / 1e9, HBM_PEAK_GBS, "GB/s", "hbm"
    calls = {}
    for n, t in per_call.items():
        entry = {"us": round(t * 1e6, 3), "bytes": model[n]["bytes"], "GB/s": round(model[n]["bytes"] / t / 1e9, 1)}
        if model[n]["flops"]:
            entry["TFLOP/s"] = round(model[n]["flops"] / t / 1e12, 2)
        calls[n] = entry
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "mode": w.mode, "batch": w.batch, "kv_len": w.kv_len,
                   "q_heads": w.n_q_heads, "kv_heads": w.n_kv_heads, "head_dim": w.head_dim,
                   "block_size": w.block_size, "top_k": w.top_k, "keep_tail": w.keep_tail, "seed": args.seed,
                   "graphs": not args.no_graph, "graph_steps": 1 if args.no_graph else max(1, args.graph_steps),
                   "fused_decode_step": st.fused, "ragged": w.ragged,
                   **({"kv_cache": "rotated 8-bit (codes + float16 scale per 32)"} if w.kv_q8 else {}),
                   **({"indexer_dim": w.indexer_dim, "indexer_agg": ["sum", "max", "softmax"][w.indexer_agg]}
                      if w.indexer_dim else {}),
                   **({"mean_kv_len": round(float(np.mean(st.lens)), 1), "min_kv_len": int(min(st.lens))}
                      if w.ragged else {})},
        "roofline": {"bound": bound,
                     "kernel": (("kv_quantize_kernel + decode_step_kernel over the 8-bit cache (the whole step)"
                                 if w.kv_q8 else "decode_step_kernel (the whole step)")
                                if dominant == "step" else f"{dominant} call"),
                     "achieved": round(achieved, 2), "peak": peak,
                     "unit": unit, "frac": round(achieved / peak, 4),
                     "traffic": measured_traffic(w.name, dominant)},
        "calls": calls,
        "call_timing": call_timing,
        "cold": {"ms_per_step": round(1e3 * cold_s, 5), "value": round(tokens / cold_s, 2),
                 "note": "step replayed after reading 1 GiB, which evicts L2 and MALL"},
    }
    if args.copy_calibration_mib > 0:
        import torch

        n = args.copy_calibration_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        line["copy_calibration_bytes"] = n
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, args.seed, args.cpu_seconds)
        line["cpu_baseline"]["value"] = round(line["cpu_baseline"]["value"], 3)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
