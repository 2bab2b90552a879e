#!/usr/bin/env python3
"""Benchmark of the paged-KV attention hot path on one MI355X.

One step = one pass of the whole path over one batch of each workload below,
inputs resident in HBM. A decode workload is: pack metadata (host, one pinned
buffer, one copy) -> store_kvcache of each sequence's new token -> paged decode
attention with the split over all waves and its combine. A prefill workload
is: pack -> store_kvcache of every new token -> varlen causal prefill
attention. The default step holds, in this order:

  decode  Qwen3-8B-shaped long-context decode: 32 q / 8 kv heads, head_dim
          128, block size 256, 512 sequences, context log-uniform in
          [256, 32768]                                      (the `value`)
  prefill prefix-cache hits: 32 prompts of 2048 tokens, the even ones sharing
          a cached 1024-token prefix read through the block tables, 16 q /
          8 kv heads, head_dim 128                          (secondary)
  decode  Qwen3-0.6B-shaped decode: 16 q / 8 kv heads, 64 sequences,
          context U{512..4096}                              (extra part)
  prefill varlen: 16 prompts U{128..2048} under a 16384-token budget
                                                            (extra part)

`value` is the long-context decode attention's algorithmic HBM throughput
(GB/s); the prefix-hit prefill attention's TFLOP/s and fraction of the bf16
MFMA peak sit beside it. Each call is timed with HIP events on the stream it
runs on, after untimed calls of the same kind have taken the card's clock to
the state it holds under continuous work (EVENT_SETTLE_S). Several copies of
the inputs are used in rotation so that no step
finds its data in the 256 MB last-level cache. A read-only streaming kernel
(libpkv_probe) is timed on a 2 GiB buffer in the same run, as an achievable
reference beside the published HBM peak, and at each part's own byte counts
a decode-shaped read (decode calls under 2 GiB) and a device copy (stores), so
that short calls have a reference that pays the same launch ramp and drain.

`--workload` selects other combinations (see WORKLOADS).
"""
from __future__ import annotations

import argparse
import gc
import hashlib
import json
import math
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np
import torch

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
METRIC = "paged decode attn HBM GB/s (% peak) + varlen prefill attn TFLOP/s (% MFMA peak)"

WORKLOADS = {
    "default": [("decode", 5), ("prefill", 4), ("decode", 2), ("prefill", 3)],
    "small": [("decode", 2), ("prefill", 3)],
    "decode": [("decode", 2)],
    "prefill": [("prefill", 3)],
    "decode-long": [("decode", 5)],
    "prefill-prefix": [("prefill", 4)],
    # the two parts the headline figures come from
    "headline": [("decode", 5), ("prefill", 4)],
    # decode rows through the varlen prefill call, beside the decode kernel on
    # the same batch; and a mixed step (decode rows + two prompt chunks)
    "decode-in-varlen": [("decode", 2), ("prefill", 6)],
    "mixed": [("prefill", 7), ("prefill+split", 7)],
    # preset 3's step with the rotary embedding fused into the store
    "rope-store": [("prefill+rope", 3)],
    # store and attention as two calls, then as one fused call: preset 3
    # (keys are the call's rows), preset 4 (prefix hits through the pool)
    "fused-store": [("prefill", 3), ("prefill+fused", 3)],
    "fused-store-prefix": [("prefill", 4), ("prefill+fused", 4)],
    # preset 2's decode, plus 28-layer decode steps eager vs replayed hipGraphs
    "decode-graph": [("decode", 2)],
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ----------------------------------------------------------------- work counts

def decode_bytes(w) -> float:
    """Algorithmic bytes of one decode attention call: every context token's K
    and V row of every kv head, q and out, the block-table entries in use and
    the context lengths."""
    es = 2 if w.dtype == torch.bfloat16 else 4
    ctx = np.asarray(w.seq_lens, dtype=np.int64)
    kv = int(ctx.sum()) * 2 * w.num_kv_heads * w.head_dim * es
    qo = 2 * len(ctx) * w.num_q_heads * w.head_dim * es
    meta = int(np.sum(-(-ctx // w.block_size))) * 4 + len(ctx) * 4
    return float(kv + qo + meta)


ROPE_BASE, ROPE_MAX_POS = 1e6, 40960


def rope_store_bytes(w) -> float:
    """Fused rotary embedding + store, per token: q read and written, k read
    and written to the cache (and back in place when the step's prefill reads
    k directly), v read and written, the slot and the position, and one
    position's cos/sin row (head_dim floats)."""
    es = 2 if w.dtype == torch.bfloat16 else 4
    q = 2 * w.num_q_heads * w.head_dim * es
    kv = w.num_kv_heads * w.head_dim * es
    k = kv * (3 if not w.use_block_tables else 2)
    return float(w.total_q * (q + k + 2 * kv + 8 + 4 * w.head_dim))


def prefill_bytes(w) -> float:
    """Algorithmic bytes of one prefill attention call: every key position's K
    and V row of every kv head read once, q read and out written once, plus
    the cu_seqlens and (paged) the block-table entries in use."""
    es = 2 if w.dtype == torch.bfloat16 else 4
    lk = np.asarray(w.seq_lens, dtype=np.int64)
    kv = int(lk.sum()) * 2 * w.num_kv_heads * w.head_dim * es
    qo = 2 * w.total_q * w.num_q_heads * w.head_dim * es
    meta = 2 * (len(lk) + 1) * 4 + int(np.sum(-(-lk // w.block_size))) * 4
    return float(kv + qo + meta)


def store_bytes(w) -> float:
    """Read the new K and V rows, write them, read the slot: per token
    2 * (2 * Hkv * d * es) + 4 bytes."""
    es = 2 if w.dtype == torch.bfloat16 else 4
    return float(w.total_q * (2 * (2 * w.num_kv_heads * w.head_dim * es) + 4))


def prefill_flops(w) -> float:
    """4 * d * Hq per visible (query, key) pair, the diagonal included."""
    pairs = 0
    for n, c in zip(w.seq_lens, w.num_cached):
        lq = n - c
        pairs += lq * c + lq * (lq + 1) // 2
    return float(4 * w.head_dim * w.num_q_heads * pairs)


# ----------------------------------------------------------------- GPU side

def _pinned(nbytes: int) -> torch.Tensor:
    """A pinned staging buffer, written once here: the first write to each
    page of a new pinned allocation faults it in (about 1 us a page), a cost
    a serving loop that reuses its staging buffers pays only once."""
    return torch.empty(nbytes, dtype=torch.uint8, pin_memory=True).zero_()


class Part:
    """One workload of the step, with `ncopies` resident copies of its inputs."""

    def __init__(self, phase, preset, ncopies):
        import paged_kv_cache_125_amd as pkv
        from paged_kv_cache_125_amd.step import alloc_pool, step_inputs_of, write_ranges
        from workloads import make_workload
        self.pkv = pkv
        # "prefill+rope": the store is the fused rotary embedding + store;
        # "prefill+split": a mixed step's decode rows (first) go through the
        # decode kernel, the rest through the varlen call;
        self.rope = phase.endswith("+rope")
        self.split = phase.endswith("+split")
        # "prefill+fused": store and attention in one call
        # (prefill_store_attention_varlen); the store interval is then empty
        self.fused = phase.endswith("+fused")
        phase = phase.split("+")[0]
        self.phase, self.preset = phase, preset
        self.copies = []
        w = None
        for c in range(ncopies):
            w = make_workload(preset, device="cuda")
            kc, vc = alloc_pool(w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim, w.dtype, "cuda")
            write_ranges(w.hist, w.block_tables, w.block_size, w.k_hist, w.v_hist, kc, vc)
            w.k_hist = w.v_hist = None      # only the pool holds the history now
            out = torch.empty_like(w.q)
            self.copies.append((w, kc, vc, out))
        self.w = w
        self.s = step_inputs_of(w)
        if self.split:
            from paged_kv_cache_125_amd.step import StepInputs, decode_rows_first
            nd = self.nd = decode_rows_first(self.s)
            self.sd = StepInputs("decode", self.s.seq_lens[:nd], self.s.num_cached[:nd],
                                 self.s.block_tables[:nd], w.block_size, w.scale)
            self.sp = StepInputs("prefill", self.s.seq_lens[nd:], self.s.num_cached[nd:],
                                 self.s.block_tables[nd:], w.block_size, w.scale)
            need = pkv.decode_workspace_bytes(nd, max(self.sd.seq_lens), w.num_q_heads,
                                              w.num_kv_heads, w.head_dim, w.block_size, w.dtype)
            self.ws = torch.empty(max(need, 256), dtype=torch.uint8, device="cuda")
        if phase == "decode":
            need = pkv.decode_workspace_bytes(len(w.seq_lens), max(w.seq_lens), w.num_q_heads,
                                              w.num_kv_heads, w.head_dim, w.block_size, w.dtype)
            self.ws = torch.empty(max(need, 256), dtype=torch.uint8, device="cuda")
            self.partition = pkv.decode_partition_size(len(w.seq_lens), max(w.seq_lens),
                                                       w.num_q_heads, w.num_kv_heads, w.head_dim,
                                                       w.block_size, w.dtype)
        if self.rope:
            # Qwen3's rotary embedding: the whole head rotated, base 1e6,
            # "rotate half" pairing, positions up to 40960
            self.cos_sin = pkv.rope_cos_sin_table(ROPE_MAX_POS, w.head_dim, ROPE_BASE, device="cuda")
        self.names = ["pack", "store", "attention"]
        self.times = {n: [] for n in self.names}
        self.ring = []
        torch.cuda.synchronize()

    def prepare(self, n):
        """n (pinned host, device) metadata buffers, one per pass, so that the
        passes allocate nothing (a new pinned allocation can stall the host)."""
        pkv, s = self.pkv, self.s
        if self.split:
            md = pkv.pack_decode(self.sd.seq_lens, self.sd.block_tables, s.block_size, device="cpu")
            mp = pkv.pack_prefill(self.sp.seq_lens, self.sp.num_cached, self.sp.block_tables,
                                  s.block_size, device="cpu")
            nd, npf = int(md["layout"].total_bytes), int(mp["layout"].total_bytes)
            self.ring = [((_pinned(nd), torch.empty(nd, dtype=torch.uint8, device="cuda")),
                          (_pinned(npf), torch.empty(npf, dtype=torch.uint8, device="cuda")))
                         for _ in range(n)]
            return
        if self.phase == "decode":
            meta = pkv.pack_decode(s.seq_lens, s.block_tables, s.block_size, device="cpu")
        else:
            meta = pkv.pack_prefill(s.seq_lens, s.num_cached, s.block_tables, s.block_size, device="cpu")
        nbytes = int(meta["layout"].total_bytes)
        self.ring = [(_pinned(nbytes), torch.empty(nbytes, dtype=torch.uint8, device="cuda"))
                     for _ in range(n)]

    def run(self, i, events):
        """Pass i (each pass has its own metadata buffers); events is a list of
        4 torch.cuda.Event or None."""
        pkv, s = self.pkv, self.s
        w, kc, vc, out = self.copies[i % len(self.copies)]
        rec = (lambda j: events[j].record()) if events else (lambda j: None)
        if self.split:
            (hd, dd), (hp, dp) = self.ring[i]
            nd = self.nd
            rec(0)
            md = pkv.pack_decode(self.sd.seq_lens, self.sd.block_tables, s.block_size,
                                 host_buffer=hd, dev_buffer=dd)
            mp = pkv.pack_prefill(self.sp.seq_lens, self.sp.num_cached, self.sp.block_tables,
                                  s.block_size, host_buffer=hp, dev_buffer=dp)
            rec(1)
            pkv.store_kvcache(w.k_new[:nd], w.v_new[:nd], kc, vc, md["slot_mapping"])
            pkv.store_kvcache(w.k_new[nd:], w.v_new[nd:], kc, vc, mp["slot_mapping"])
            rec(2)
            pkv.decode_attention_paged(w.q[:nd], kc, vc, md["block_tables"], md["context_lens"],
                                       md["max_seqlen_k"], s.scale, out=out[:nd], workspace=self.ws)
            pkv.prefill_attention_varlen(w.q[nd:], mp["cu_seqlens_q"], mp["cu_seqlens_k"],
                                         mp["max_seqlen_q"], mp["max_seqlen_k"], s.scale,
                                         k_cache=kc, v_cache=vc, block_tables=mp["block_tables"],
                                         out=out[nd:])
            rec(3)
            return (md, mp)
        hb, db = self.ring[i]
        rec(0)
        if self.phase == "decode":
            meta = pkv.pack_decode(s.seq_lens, s.block_tables, s.block_size, host_buffer=hb, dev_buffer=db)
            rec(1)
            pkv.store_kvcache(w.k_new, w.v_new, kc, vc, meta["slot_mapping"])
            rec(2)
            pkv.decode_attention_paged(w.q, kc, vc, meta["block_tables"], meta["context_lens"],
                                       meta["max_seqlen_k"], s.scale, out=out, workspace=self.ws)
            rec(3)
        else:
            meta = pkv.pack_prefill(s.seq_lens, s.num_cached, s.block_tables, s.block_size,
                                    host_buffer=hb, dev_buffer=db)
            rec(1)
            if self.fused:
                rec(2)
                pkv.prefill_store_attention_varlen(w.q, w.k_new, w.v_new, kc, vc, meta["slot_mapping"],
                                                   meta["cu_seqlens_q"], meta["cu_seqlens_k"],
                                                   meta["max_seqlen_q"], meta["max_seqlen_k"], s.scale,
                                                   block_tables=meta["block_tables"], out=out)
                rec(3)
                return meta
            if self.rope:
                pkv.rope_store_kvcache(w.q, w.k_new, w.v_new, kc, vc, meta["slot_mapping"],
                                       meta["positions"], self.cos_sin,
                                       write_k=meta["block_tables"] is None)
            else:
                pkv.store_kvcache(w.k_new, w.v_new, kc, vc, meta["slot_mapping"])
            rec(2)
            if meta["block_tables"] is not None:
                pkv.prefill_attention_varlen(w.q, meta["cu_seqlens_q"], meta["cu_seqlens_k"],
                                             meta["max_seqlen_q"], meta["max_seqlen_k"], s.scale,
                                             k_cache=kc, v_cache=vc,
                                             block_tables=meta["block_tables"], out=out)
            else:
                pkv.prefill_attention_varlen(w.q, meta["cu_seqlens_q"], meta["cu_seqlens_k"],
                                             meta["max_seqlen_q"], meta["max_seqlen_k"], s.scale,
                                             k=w.k_new, v=w.v_new, out=out)
            rec(3)
        return meta   # keeps the packed buffers alive until the stream has run

    def collect(self, events_per_step):
        for evs in events_per_step:
            for j, n in enumerate(self.names):
                self.times[n].append(evs[j].elapsed_time(evs[j + 1]) * 1e-3)

    def summary(self):
        w = self.w
        t_attn = float(np.mean(self.times["attention"]))
        t_store = float(np.mean(self.times["store"]))
        t_pack = float(np.mean(self.times["pack"]))
        sb = rope_store_bytes(w) if self.rope else store_bytes(w)
        d = {"workload": w.name + ("+rope" if self.rope else "") + ("+split" if self.split else "")
             + ("+fused" if self.fused else ""),
             "preset": self.preset, "phase": self.phase,
             "store": ("rope_store_kvcache" if self.rope else
                       "in the attention call (prefill_store_attention_varlen)" if self.fused else
                       "store_kvcache"),
             "num_seqs": len(w.seq_lens), "tokens_q": w.total_q,
             "context_tokens": int(sum(w.seq_lens)),
             "pack_us": t_pack * 1e6, "store_us": t_store * 1e6, "attention_us": t_attn * 1e6,
             "attention_us_p10": float(np.percentile(self.times["attention"], 10)) * 1e6,
             "attention_us_p90": float(np.percentile(self.times["attention"], 90)) * 1e6,
             "store_GBps": None, "store_frac_hbm": None}
        if self.fused:
            # one interval holds both: its rate counts the attention's work only
            d.update({"store_us": 0.0, "store_and_attention_us": t_attn * 1e6})
        else:
            d.update({"store_GBps": sb / t_store / 1e9, "store_frac_hbm": sb / t_store / 1e9 / HBM_PEAK_GBS})
        if self.phase == "decode":
            b = decode_bytes(w)
            d.update({"attention_bytes": b, "attention_GBps": b / t_attn / 1e9,
                      "attention_frac_hbm": b / t_attn / 1e9 / HBM_PEAK_GBS,
                      "partition_size": self.partition})
        else:
            f = prefill_flops(w)
            b = prefill_bytes(w)
            d.update({"attention_flops": f, "attention_TFLOPs": f / t_attn / 1e12,
                      "attention_frac_mfma": f / t_attn / 1e12 / MFMA_BF16_PEAK_TFLOPS,
                      "attention_bytes": b, "attention_GBps": b / t_attn / 1e9,
                      "attention_frac_hbm": b / t_attn / 1e9 / HBM_PEAK_GBS})
        return d


# ----------------------------------------------------------------- host side

def block_manager_host(reps: int = 20) -> dict:
    """Host cost of the block manager on the prefix-hit step's structure
    (32 prompts of 2048 tokens, the even ones sharing a 1024-token prefix,
    block size 256), each repetition on a fresh manager: allocate every prompt
    (chained hashing of all 65536 tokens; the first sharer registers the
    prefix, the other 15 find its 4 blocks), gather the tables and pack the
    step's metadata into a host buffer, then release everything."""
    import paged_kv_cache_125_amd as pkv
    rng = np.random.default_rng(1004)
    prefix = rng.integers(0, 151936, 1024, dtype=np.int64)
    prompts = [np.concatenate([prefix if s % 2 == 0 else rng.integers(0, 151936, 1024, dtype=np.int64),
                               rng.integers(0, 151936, 1024, dtype=np.int64)]) for s in range(32)]
    t_alloc, t_pack, t_free, cached = [], [], [], 0
    for _ in range(reps):
        m = pkv.BlockManager(2048, 256)
        t0 = time.perf_counter()
        cached = sum(m.allocate(s, p) for s, p in enumerate(prompts))
        t1 = time.perf_counter()
        lens, nc, tables = m.gather(range(32))
        pkv.pack_prefill(lens, nc, tables, 256, device="cpu")
        t2 = time.perf_counter()
        for s in range(32):
            m.deallocate(s)
        t3 = time.perf_counter()
        t_alloc.append(t1 - t0)
        t_pack.append(t2 - t1)
        t_free.append(t3 - t2)
    med = lambda v: float(np.median(v)) * 1e6
    return {"allocate_us": med(t_alloc), "gather_pack_us": med(t_pack), "deallocate_us": med(t_free),
            "tokens_hashed": 32 * 2048, "cached_tokens_per_step": int(cached),
            "note": "host only, median of fresh managers; 32 x 2048-token prompts (int64 ids), "
                    "16 sharing a 1024-token prefix, bs 256; times include the Python binding's calls"}


def decode_graph_compare(num_layers: int = 28, batches=(1, 8, 64), steps: int = 30) -> dict:
    """Decode steps of `num_layers` layers (store + attention per layer, each
    layer with its own pool) run eagerly -- one C-ABI call per kernel -- and as
    a replayed hipGraph of the batch's bucket, on preset 2's first B
    sequences. Both include the step's metadata packing and upload; the
    layers' q, k, v stay resident (in a model, earlier kernels of the step
    produce them). Wall time per step, synchronized at both ends."""
    import paged_kv_cache_125_amd as pkv
    from paged_kv_cache_125_amd.graphs import DecodeGraphs, bucket_for
    from paged_kv_cache_125_amd.step import alloc_pool, write_ranges
    from workloads import make_workload, restrict
    full = make_workload(2, device="cuda")
    res = {}
    for B in batches:
        w = restrict(full, list(range(B)), device="cuda")
        layers = []
        for _ in range(num_layers):
            kc, vc = alloc_pool(w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim, w.dtype, "cuda")
            write_ranges(w.hist, w.block_tables, w.block_size, w.k_hist, w.v_hist, kc, vc)
            layers.append((kc, vc))
        maxb = max(len(t) for t in w.block_tables)
        g = DecodeGraphs(layers, w.num_q_heads, max_context_len=4096, max_blocks_per_seq=maxb,
                         scale=w.scale, buckets=[bucket_for(B)])
        # the same graphs with the store as a call of its own in every layer
        g2 = DecodeGraphs(layers, w.num_q_heads, max_context_len=4096, max_blocks_per_seq=maxb,
                          scale=w.scale, buckets=[bucket_for(B)], fuse_store=False)
        qs, ks, vs = [w.q] * num_layers, [w.k_new] * num_layers, [w.v_new] * num_layers
        meta = pkv.pack_decode(w.seq_lens, w.block_tables, w.block_size, device="cuda")
        g.prepare(qs, ks, vs, meta["slot_mapping"], meta["context_lens"], meta["block_tables"])
        g2.prepare(qs, ks, vs, meta["slot_mapping"], meta["context_lens"], meta["block_tables"])

        def eager():
            m = pkv.pack_decode(w.seq_lens, w.block_tables, w.block_size, device="cuda")
            g.run_eager(qs, ks, vs, m["slot_mapping"], m["context_lens"], m["block_tables"],
                        m["max_seqlen_k"])

        def graph():
            m = pkv.pack_decode(w.seq_lens, w.block_tables, w.block_size, device="cuda")
            g.replay(g.prepare_meta(m["slot_mapping"], m["context_lens"], m["block_tables"]))

        def graph_two_calls():
            m = pkv.pack_decode(w.seq_lens, w.block_tables, w.block_size, device="cuda")
            g2.replay(g2.prepare_meta(m["slot_mapping"], m["context_lens"], m["block_tables"]))

        times = {}
        for name, fn in (("eager", eager), ("graph", graph), ("graph_two_calls", graph_two_calls),
                         ("eager", eager), ("graph", graph), ("graph_two_calls", graph_two_calls)):
            for _ in range(3):
                fn()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(steps):
                fn()
            torch.cuda.synchronize()
            times[name] = (time.perf_counter() - t0) / steps * 1e3   # the second round counts
        res[f"B{B}"] = {"eager_ms_per_step": times["eager"], "graph_ms_per_step": times["graph"],
                        "graph_two_calls_ms_per_step": times["graph_two_calls"],
                        "speedup": times["eager"] / times["graph"], "bucket": bucket_for(B),
                        "context_tokens": int(sum(w.seq_lens))}
        del layers, g, g2
        torch.cuda.empty_cache()
    return {"layers": num_layers, "per_batch": res,
            "note": "decode attention side of one step (store + attention per layer) for the first B "
                    "sequences of preset 2; wall clock per step incl. metadata pack+upload; eager and "
                    "graph use the fused store + decode call per layer, graph_two_calls a store call "
                    "and a decode call"}


# ----------------------------------------------------------------- oracle side

def cpu_baseline(phase, preset, budget_s):
    """The oracle, as it stands, on the host cores, over a bounded sample of
    the preset: whole sequences from the front of the batch, each run through
    the oracle's store and attention exactly as the GPU step runs them
    (prefix-hit sequences read their keys through the block tables), repeated
    until the time budget is spent. Returns the rate in the unit of the GPU
    figure (GB/s for decode, TFLOP/s for prefill)."""
    import oracle
    from workloads import make_workload, restrict
    shape = make_workload(preset, values=False)
    threads = oracle.max_threads()
    cpu = platform.processor() or platform.machine()
    if phase == "decode":
        # whole sequences from the front of the batch, up to ~200K context tokens
        take, tot = [], 0
        for s, n in enumerate(shape.seq_lens):
            if take and tot + n > 200_000:
                break
            take.append(s)
            tot += n
        w = restrict(shape, take)
        kp, vp, slots = oracle.pools_after_store(w)     # setup: history + first write
        reps, t = 0, 0.0
        while t < budget_s:
            t0 = time.perf_counter()
            oracle.store(w.k_new, kp, slots)
            oracle.store(w.v_new, vp, slots)
            oracle.attention(w.q, w.q_lens, w.seq_lens, w.num_kv_heads, w.scale,
                             k_cache=kp, v_cache=vp, tables=w.block_tables, block_size=w.block_size)
            t += time.perf_counter() - t0
            reps += 1
        rate = decode_bytes(w) * reps / t / 1e9
        return {"value": rate, "unit": "GB/s", "cores": threads, "kind": "oracle",
                "sample": f"{len(take)} of {len(shape.seq_lens)} sequences ({tot} context tokens): "
                          f"oracle store + decode attention, {reps} repetition(s), {t:.1f} s",
                "cpu": cpu}
    # prefill: one sequence per oracle call, cycling over the front of the batch
    # (rate in GB/s for a batch below the ridge point, as for the GPU figure)
    byte_bound = prefill_flops(shape) / prefill_bytes(shape) < MFMA_BF16_PEAK_TFLOPS * 1e3 / HBM_PEAK_GBS
    t, flops, nbytes, calls, seen = 0.0, 0.0, 0.0, 0, set()
    s = 0
    while t < budget_s:
        w = restrict(shape, [s])
        kp = vp = None
        if w.use_block_tables:
            kp, vp, slots = oracle.pools_after_store(w)
        t0 = time.perf_counter()
        if w.use_block_tables:
            oracle.store(w.k_new, kp, slots)
            oracle.store(w.v_new, vp, slots)
            oracle.attention(w.q, w.q_lens, w.seq_lens, w.num_kv_heads, w.scale,
                             k_cache=kp, v_cache=vp, tables=w.block_tables, block_size=w.block_size)
        else:
            oracle.attention(w.q, w.q_lens, w.seq_lens, w.num_kv_heads, w.scale,
                             k=w.k_new, v=w.v_new)
        t += time.perf_counter() - t0
        flops += prefill_flops(w)
        nbytes += prefill_bytes(w)
        calls += 1
        seen.add(s)
        s = (s + 1) % len(shape.seq_lens)
    value, unit = (nbytes / t / 1e9, "GB/s") if byte_bound else (flops / t / 1e12, "TFLOP/s")
    return {"value": value, "unit": unit, "cores": threads, "kind": "oracle",
            "sample": f"{calls} oracle prefill calls, one sequence each, over {len(seen)} of the "
                      f"preset's {len(shape.seq_lens)} sequences (store + attention through the "
                      f"block tables where the preset reads the cache), {t:.1f} s",
            "cpu": cpu}


# ----------------------------------------------------------------- traffic

COUNTERS_JSON = os.path.join(ROOT, "profiles", "counters.json")
CALIBRATION_BYTES = 1 << 30     # the plain device copy timed under the counters


def device_copy_rate(reps: int = 5) -> float:
    """GB/s (bytes read + bytes written) of a 1 GiB device-to-device copy,
    the runtime's own copy kernel, timed with events: a measured ceiling for
    streaming kernels on this GPU, reported beside the published HBM peak."""
    src = torch.empty(CALIBRATION_BYTES, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    sec = e0.elapsed_time(e1) * 1e-3 / reps
    del src, dst
    torch.cuda.empty_cache()
    return 2 * CALIBRATION_BYTES / sec / 1e9


STREAM_BYTES = 2 << 30          # buffer of the read-only streaming reference


def stream_read_rates(reps: int = 5) -> dict:
    """GB/s of libpkv_probe's read-only streaming kernels over a 2 GiB buffer
    of random words (8x the last-level cache, so every pass comes from HBM),
    timed with events on the current stream: the plain grid-stride form, the
    decode-shaped form (2 KB rows of eight 256-byte heads, one head per wave)
    and one contiguous span per wave, each at 1, 2, 3, 4, 6, 8 and 16
    workgroups per CU (the rate is not monotonic in the count: the grid-stride
    form reads addresses a grid apart, and some grid sizes land them on few
    channels), the best of each kept. An achievable streaming-read reference
    beside the published 8 TB/s."""
    import ctypes
    from paged_kv_cache_125_amd.build import PROBE_LIB
    L = ctypes.CDLL(PROBE_LIB)
    L.pkv_probe_stream_read.restype = ctypes.c_int
    L.pkv_probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_int32,
                                        ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    gen = torch.Generator(device="cuda")
    gen.manual_seed(77)
    buf = torch.randint(-2 ** 31, 2 ** 31 - 1, (STREAM_BYTES // 4,), dtype=torch.int32, device="cuda",
                        generator=gen)
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    out = {}
    for mode, name in ((0, "plain"), (1, "decode_shaped"), (2, "span")):
        best = None
        for per_cu in (1, 2, 3, 4, 6, 8, 16):
            blocks = cus * per_cu
            args = (ctypes.c_void_p(buf.data_ptr()), STREAM_BYTES, mode, 2048, blocks,
                    ctypes.c_void_p(sink.data_ptr()), stream)
            if L.pkv_probe_stream_read(*args) != 0:
                raise RuntimeError("pkv_probe_stream_read failed")
            e0.record()
            for _ in range(reps):
                L.pkv_probe_stream_read(*args)
            e1.record()
            torch.cuda.synchronize()
            gbps = STREAM_BYTES * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
            if best is None or gbps > best["GBps"]:
                best = {"GBps": gbps, "frac_of_peak": gbps / HBM_PEAK_GBS, "workgroups_per_cu": per_cu}
        out[name] = best
    del buf
    torch.cuda.empty_cache()
    out["best"] = max((out[n] for n in ("plain", "decode_shaped", "span")), key=lambda r: r["GBps"])
    out["bytes_read"] = STREAM_BYTES
    return out


ISSUE_MODES = {   # mode: (what one pass issues, instructions the rate is per)
    0: ("16 ds_read_b128, K-operand addresses", 16), 1: ("32 ds_read_b64_tr_b16, V^T addresses", 32),
    2: ("16 v_mfma_f32_32x32x16_bf16", 16), 3: ("32 v_exp_f32", 32), 4: ("32 v_fma_f32", 32),
    5: ("16 x (MFMA + 1 K read), per MFMA", 16), 6: ("16 x (MFMA + 2 V^T reads), per MFMA", 16),
    7: ("16 MFMA + 24 reads (tile mix), per MFMA", 16),
    11: ("16 x (MFMA + 4 fma, one wave), per MFMA", 16), 12: ("16 x (MFMA + 2 exp + 2 fma, one wave), per MFMA", 16),
    13: ("16 x (MFMA + 8 fma, one wave), per MFMA", 16),
    14: ("16 x (MFMA + 1.5 reads + 4 fma, one wave), per MFMA", 16),
    15: ("16 x (MFMA + 1.5 reads + 2 exp + 2 fma, one wave), per MFMA", 16),
    16: ("mode 14 with AGPR accumulators, per MFMA", 16), 17: ("mode 15 with AGPR accumulators, per MFMA", 16)}


def issue_rates() -> str:
    """libpkv_probe's issue-rate probes (pkv_probe_issue) as markdown: cycles
    per instruction per SIMD (the slowest wave of each CU's workgroup, over
    all the instructions its SIMD's waves issued) and per wave, at 1, 2 and 4
    waves per SIMD; then one MFMA wave and one VALU wave per SIMD, alone and
    together."""
    import ctypes
    from paged_kv_cache_125_amd.build import PROBE_LIB
    L = ctypes.CDLL(PROBE_LIB)
    L.pkv_probe_issue.restype = ctypes.c_int
    L.pkv_probe_issue.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                  ctypes.c_void_p, ctypes.c_void_p]
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    cyc = torch.zeros(cus * 16, dtype=torch.int64, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    passes = 64

    def run(mode, wps):
        for _ in range(2):   # the first launch loads the code
            if L.pkv_probe_issue(mode, wps, cus, ctypes.c_void_p(cyc.data_ptr()),
                                 ctypes.c_void_p(sink.data_ptr()), stream) != 0:
                raise RuntimeError(f"pkv_probe_issue mode {mode} failed")
        torch.cuda.synchronize()
        return cyc.view(cus, 16).cpu().numpy().astype(np.float64)

    out = ["| Block | waves per SIMD | cycles per instruction per SIMD | per wave |", "|---|---|---|---|"]
    for mode, (name, n) in ISSUE_MODES.items():
        # (at 4 waves per SIMD modes 5, 6 and 11-17 exceed their 128 registers and spill)
        for wps in ((1, 2) if mode in (5, 6, 11, 12, 13, 14, 15, 16, 17) else (1, 2, 4)):
            c = run(mode, wps)[:, :4 * wps]
            per_simd = c.max(axis=1).mean() / (passes * n * wps)
            out.append(f"| {name} | {wps} | {per_simd:.1f} | {c.mean() / (passes * n):.1f} |")
    out += ["", "| One MFMA wave and one VALU wave per SIMD | MFMA wave: cycles per pass (16 MFMAs) | "
            "VALU wave: cycles per pass (32 exp + 32 fma) |", "|---|---|---|"]
    for mode, name in ((9, "MFMA waves alone"), (10, "VALU waves alone"), (8, "both")):
        c = run(mode, 2)
        a = c[:, :4].max(axis=1).mean() / passes if mode != 10 else float("nan")
        b = c[:, 4:8].max(axis=1).mean() / passes if mode != 9 else float("nan")
        out.append(f"| {name} | {a:.0f} | {b:.0f} |")
    return "\n".join(out)


def size_matched_rates(parts, summaries, per_cu: int, cycles: int, reps: int = 20) -> dict:
    """Plain data movement of each part's own byte counts, every launch alone
    between two events behind a spin kernel (as the timed pass times the
    attention and store calls), over as many rotating buffers as the part
    keeps input copies: a decode-shaped read-only stream of a decode call's
    bytes (parts under 2 GiB), and a device-to-device copy of a store's bytes.
    What streaming itself reaches at that size, launch ramp and drain
    included. Returns {workload: {...}}."""
    import ctypes
    from paged_kv_cache_125_amd.build import PROBE_LIB
    L = ctypes.CDLL(PROBE_LIB)
    L.pkv_probe_stream_read.restype = ctypes.c_int
    L.pkv_probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_int32,
                                        ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]

    def timed(launch):
        launch(0)                       # warm
        torch.cuda.synchronize()
        torch.cuda._sleep(cycles)
        for i, (a, b) in enumerate(ev):
            a.record()
            launch(i)
            b.record()
        torch.cuda.synchronize()
        return float(np.mean([a.elapsed_time(b) * 1e-3 for a, b in ev]))

    out = {}
    for p, sm in zip(parts, summaries):
        rec = {}
        n = len(p.copies)
        if p.phase == "decode" and sm["attention_bytes"] < STREAM_BYTES:
            nb = int(-(-sm["attention_bytes"] // 2048) * 2048)
            bufs = [torch.empty(nb, dtype=torch.uint8, device="cuda").fill_(0x5A + i) for i in range(n)]
            t = timed(lambda i: L.pkv_probe_stream_read(ctypes.c_void_p(bufs[i % n].data_ptr()), nb, 1, 2048,
                                                        cus * per_cu, ctypes.c_void_p(sink.data_ptr()), stream))
            rec["stream_read"] = {"bytes": nb, "us": t * 1e6, "GBps": nb / t / 1e9,
                                  "attention_over_stream": sm["attention_GBps"] / (nb / t / 1e9)}
            del bufs
        sb = rope_store_bytes(p.w) if p.rope else store_bytes(p.w)
        half = int(sb // 2)
        # sources and destinations both rotate, as the store's inputs and
        # pools do, so the copy finds no more of its data in the MALL than
        # the store does
        srcs = [torch.empty(half, dtype=torch.uint8, device="cuda").fill_(0x33 + i) for i in range(n)]
        dsts = [torch.empty(half, dtype=torch.uint8, device="cuda") for _ in range(n)]
        t = timed(lambda i: dsts[i % n].copy_(srcs[i % n]))
        rec["device_copy"] = {"bytes": 2 * half, "us": t * 1e6, "GBps": 2 * half / t / 1e9,
                              "store_over_copy": (None if sm["store_GBps"] is None else
                                                  sm["store_GBps"] / (2 * half / t / 1e9))}
        del srcs, dsts
        torch.cuda.empty_cache()
        out[sm["workload"]] = rec
    return out


def _source_sha(kernel_file: str) -> str:
    src = os.path.join(ROOT, "paged_kv_cache_125_amd", "csrc", kernel_file)
    return hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]


def counters_traffic(kernel_file: str, key: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, or None if
    the kernel source changed since they were taken."""
    try:
        ent = json.load(open(COUNTERS_JSON))[key]
        if ent.get("source_sha") != _source_sha(kernel_file):
            return None
        return ent["hbm_bytes_per_launch"]
    except (OSError, KeyError, ValueError):
        return None


def _read_counter_csvs(d):
    """{kernel name: {counter: [value per dispatch]}} from a rocprofv3 --pmc run."""
    import csv
    import glob
    out = {}
    for path in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(path)):
            out.setdefault(r["Kernel_Name"], {}).setdefault(r["Counter_Name"], []).append(
                float(r["Counter_Value"]))
    return out


def summarize_counters(fetch_dir, write_dir, workload):
    """Scale FETCH_SIZE / WRITE_SIZE (KiB per dispatch) by what they read for
    the calibration copy of CALIBRATION_BYTES, and store HBM bytes per launch
    of the hot kernels in profiles/counters.json."""
    f, w = _read_counter_csvs(fetch_dir), _read_counter_csvs(write_dir)

    def avg(tab, needle, counter):
        vals = [v for k, c in tab.items() if needle in k for v in c.get(counter, [])]
        return sum(vals) / len(vals) if vals else None

    kib = CALIBRATION_BYTES / 1024

    def calib(tab, counter):
        # the 1 GiB copies, not the small metadata uploads that share the blit kernel
        vals = [v for k, c in tab.items() if "copy" in k.lower() for v in c.get(counter, []) if v > kib / 4]
        return sum(vals) / len(vals) if vals else None

    copy_f, copy_w = calib(f, "FETCH_SIZE"), calib(w, "WRITE_SIZE")
    if copy_f is None or copy_w is None:
        raise SystemExit("no calibration copy kernel in the counter runs")
    ff, fw = copy_f / kib, copy_w / kib
    data = json.load(open(COUNTERS_JSON)) if os.path.exists(COUNTERS_JSON) else {}
    groups = {
        "decode": (["decode_sk_kernel", "decode_sk_reduce_kernel", "decode_blk_kernel",
                    "decode_mfma_kernel", "decode_generic_kernel", "decode_reduce_kernel"], "decode.hip"),
        "prefill": (["prefill_mfma_kernel"], "prefill.hip"),
    }
    parts = WORKLOADS[workload]
    for name, (kernels, src) in groups.items():
        # kernel names match by substring; a longer name listed later must not
        # be counted twice under a shorter one
        tabs = {}
        for tab, counter in ((f, "FETCH_SIZE"), (w, "WRITE_SIZE")):
            tot = 0.0
            for k in kernels:
                vals = [v for kn, c in tab.items() if k in kn and not any(
                    o != k and k in o and o in kn for o in kernels) for v in c.get(counter, [])]
                tot += sum(vals) / len(vals) if vals else 0.0
            tabs[counter] = tot
        fetch, write = tabs["FETCH_SIZE"], tabs["WRITE_SIZE"]
        if fetch == 0 and write == 0:
            continue
        keys = [p for ph, p in parts if ph == name]
        for p in keys:
            data[f"{name}-preset{p}"] = {
                "kernels": kernels, "source_sha": _source_sha(src),
                "fetch_kib_raw": fetch, "write_kib_raw": write,
                "copy_calibration": {"bytes": CALIBRATION_BYTES, "fetch_factor": ff, "write_factor": fw},
                "hbm_bytes_per_launch": (fetch / ff + write / fw) * 1024,
                "note": "mean over the dispatches of the counter run"}
    os.makedirs(os.path.dirname(COUNTERS_JSON), exist_ok=True)
    json.dump(data, open(COUNTERS_JSON, "w"), indent=1, sort_keys=True)
    print(json.dumps({k: data[k]["hbm_bytes_per_launch"] for k in sorted(data)}, indent=1))


def summarize_pmc(pmc_dir, command):
    """Mean per dispatch of every counter of a rocprofv3 --pmc run, by
    kernel, as markdown. With SQ_VALU_MFMA_BUSY_CYCLES and GRBM_GUI_ACTIVE in
    the run, also the matrix cores' busy share: busy cycles summed over the
    SIMDs / (SIMDs x active cycles per XCD; GRBM_GUI_ACTIVE sums the 8 XCDs)."""
    tab = _read_counter_csvs(pmc_dir)
    if not tab:
        raise SystemExit(f"no counter_collection.csv under {pmc_dir}")
    counters = sorted({c for v in tab.values() for c in v})
    simds = 4 * torch.cuda.get_device_properties(0).multi_processor_count if torch.cuda.is_available() else 1024
    out = [f"Command: `{command}`", "",
           "| Kernel | Dispatches | " + " | ".join(counters) + " | MFMA busy |",
           "|---|---|" + "---|" * len(counters) + "---|"]
    for k in sorted(tab, key=lambda n: -sum(sum(v) for v in tab[n].values())):
        short = k.split("(")[0].replace("void ", "")
        if not any(t in short for t in ("pkv::", "copyBuffer")):
            continue
        c = tab[k]
        n = max(len(v) for v in c.values())
        means = [float(np.mean(c[x])) if c.get(x) else float("nan") for x in counters]
        busy = ""
        if c.get("SQ_VALU_MFMA_BUSY_CYCLES") and c.get("GRBM_GUI_ACTIVE"):
            busy = f"{np.mean(c['SQ_VALU_MFMA_BUSY_CYCLES']) / (simds * np.mean(c['GRBM_GUI_ACTIVE']) / 8):.3f}"
        out.append(f"| `{short}` | {n} | " + " | ".join(f"{m:.4g}" for m in means) + f" | {busy} |")
    print("\n".join(out))


# ----------------------------------------------------------------- kernel trace

# Attention kernels each part's call dispatches once per step, by phase.
TRACE_KERNELS = {"decode": ["decode_sk_kernel", "decode_sk_reduce_kernel"],
                 "prefill": ["prefill_mfma_kernel"]}


def summarize_trace(trace_dir, workload, steps, warmup, command, settle=None):
    """Per-workload kernel durations from a `rocprofv3 --kernel-trace` run of
    `bench.py --workload W --steps K --warmup W'`. The bench runs every pass
    (warmup, wall-clock, event-timed) part by part, so the n-th dispatch of an
    attention kernel belongs to a known part; that order is rebuilt here and
    checked against the dispatch count. Durations of the two timed passes only
    (warmup and the event pass's settle steps excluded); `settle` is the run's
    settle steps per chunk, by part, as its bench line reports them. Prints a
    markdown summary."""
    import csv
    import glob
    rows = []
    for path in glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True):
        rows += list(csv.DictReader(open(path)))
    if not rows:
        raise SystemExit(f"no kernel_trace.csv under {trace_dir}")
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    parts = WORKLOADS[workload]
    names = {2: "decode 0.6B b64", 3: "prefill varlen 16x", 4: "prefill prefix-hit 32x2048",
             5: "decode 8B b512 long"}
    out = [f"Command: `{command}`", "",
           "| Kernel | Workload | Dispatches (timed) | Mean us | Median us | Min us | Max us |",
           "|---|---|---|---|---|---|---|"]
    first = []   # (start, part, pass) of each step's first attention dispatch
    for phase, kernels in TRACE_KERNELS.items():
        mine = [p for p in parts if p[0] == phase]
        if not mine:
            continue
        settle_of = dict(zip(parts, settle or [0] * len(parts)))
        # the warmup pass ends with the three steps that time a part's step
        n_warm = warmup + min(3, warmup + steps)
        order = [(p, pas) for pas, n in (("warmup", n_warm), ("timed", steps)) for p in mine for _ in range(n)]
        for p in mine:
            for c0 in range(0, steps, EVENT_CHUNK_STEPS):
                order += [(p, "settle")] * settle_of[p]
                order += [(p, "events")] * (min(c0 + EVENT_CHUNK_STEPS, steps) - c0)
        for k in kernels:
            durs = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-3
                    for r in rows if r["Kernel_Name"].split("(")[0].split("<")[0].endswith(k)]
            if not durs:
                continue
            if len(durs) != len(order):
                raise SystemExit(f"{k}: {len(durs)} dispatches, expected {len(order)}")
            for p in mine:
                d = [t for t, (pp, pas) in zip(durs, order) if pp == p and pas in ("timed", "events")]
                out.append(f"| {k} | {names.get(p[1], p[1])} (preset {p[1]}) | {len(d)} | "
                           f"{np.mean(d):.1f} | {np.median(d):.1f} | {min(d):.1f} | {max(d):.1f} |")
            if k == kernels[0]:
                first += [(int(r["Start_Timestamp"]), p, pas) for r, (p, pas) in
                          zip([r for r in rows if r["Kernel_Name"].split("(")[0].split("<")[0].endswith(k)],
                              order)]
    # the store of a step is the last store dispatch before that step's attention
    stores = [r for r in rows if "store_kvcache_kernel" in r["Kernel_Name"]
              and "rope" not in r["Kernel_Name"]]
    starts = [int(r["Start_Timestamp"]) for r in stores]
    per = {}
    for t0, p, pas in sorted(first, key=lambda x: x[0]):
        i = int(np.searchsorted(starts, t0)) - 1
        if i >= 0 and pas in ("timed", "events"):
            r = stores[i]
            per.setdefault(p, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-3)
    for p in parts:
        d = per.get(p)
        if d:
            out.append(f"| store_kvcache_kernel | {names.get(p[1], p[1])} (preset {p[1]}) | {len(d)} | "
                       f"{np.mean(d):.1f} | {np.median(d):.1f} | {min(d):.1f} | {max(d):.1f} |")
    print("\n".join(out))


# ----------------------------------------------------------------- main

# Steps per chunk of the event-timed pass (see the comment there).
EVENT_CHUNK_STEPS = 10
# Untimed steps of the same part that run between each chunk's pre-roll and
# its timed steps: about this much GPU time (from three steps timed after the
# warmup), at least 2 and at most 80 steps.
# After the idle pre-roll the card's clock goes through a transient under a
# sudden MFMA load (a prefix-hit prefill call goes ~540 -> ~720 -> ~505 us
# over its first ~30 ms of back-to-back calls); the settle steps let it pass,
# so the timed calls see the clock of continuous work.
EVENT_SETTLE_S = 0.06
EVENT_SETTLE_MAX = 80


def preroll_cycles(seconds: float) -> int:
    """Argument of torch.cuda._sleep that keeps the GPU busy for about
    `seconds` (calibrated once with events), capped at 0.5 s."""
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(1000)          # first launch loads the kernel
    n = 20_000_000
    a.record()
    torch.cuda._sleep(n)
    b.record()
    b.synchronize()
    per_cycle = max(a.elapsed_time(b) * 1e-3 / n, 1e-12)
    return int(min(max(seconds, 1e-3), 0.5) / per_cycle)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="default", choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=10.0, help="seconds of oracle work per part")
    ap.add_argument("--copies", type=int, default=0, help="resident input copies (0 = auto)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run a plain 1 GiB device copy (scales the HBM byte counters)")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="turn two rocprofv3 --pmc runs into profiles/counters.json and exit")
    ap.add_argument("--issue-rates", action="store_true",
                    help="print the issue-rate probes (libpkv_probe) as markdown and exit")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("PMC_DIR", "COMMAND"),
                    help="per-kernel means of a rocprofv3 --pmc run, then exit")
    ap.add_argument("--trace-settle", default="",
                    help="with --summarize-trace: the traced run's settle steps per chunk, by part "
                         "(event_timing.settle_steps_per_chunk of its bench line), comma-separated")
    ap.add_argument("--summarize-trace", nargs=2, metavar=("TRACE_DIR", "COMMAND"),
                    help="per-workload kernel durations of a rocprofv3 --kernel-trace run of "
                         "the bench with the same --workload/--steps/--warmup, then exit")
    args = ap.parse_args()
    if args.summarize_counters:
        if len({ph for ph, _ in WORKLOADS[args.workload]}) != len(WORKLOADS[args.workload]):
            raise SystemExit("counter runs need a workload with one part per phase "
                             "(the counters are averaged per kernel name)")
        summarize_counters(*args.summarize_counters, args.workload)
        return
    if args.summarize_pmc:
        summarize_pmc(*args.summarize_pmc)
        return
    if args.summarize_trace:
        summarize_trace(args.summarize_trace[0], args.workload, args.steps, args.warmup,
                        args.summarize_trace[1],
                        [int(x) for x in args.trace_settle.split(",")] if args.trace_settle else None)
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(no sharding, no collectives). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    if args.issue_rates:
        print(issue_rates(), flush=True)
        return
    import paged_kv_cache_125_amd as pkv
    pkv.lib()

    parts = []
    for phase, preset in WORKLOADS[args.workload]:
        nc = args.copies or (2 if (phase == "decode" and preset == 5) else 3)
        log(f"[bench] setting up {phase} preset {preset} ({nc} copies)")
        parts.append(Part(phase, preset, nc))

    copy_gbps = device_copy_rate()
    log(f"[bench] 1 GiB device copy: {copy_gbps:.0f} GB/s (read + write)")
    stream_read = stream_read_rates()
    log(f"[bench] 2 GiB read-only stream: plain {stream_read['plain']['GBps']:.0f} GB/s, "
        f"decode-shaped {stream_read['decode_shaped']['GBps']:.0f} GB/s, "
        f"span {stream_read['span']['GBps']:.0f} GB/s")
    if args.copy_calibration:
        src = torch.empty(CALIBRATION_BYTES, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    for p in parts:
        p.prepare(args.warmup + args.steps)
    # With two workloads, each pass runs one workload's steps back to back,
    # then the other's: every kernel is timed after calls of its own kind
    # (right after a prefill call the decode kernel runs about 15% slower,
    # which would hide its own speed). A step is one step of each workload.
    order = lambda base: [(base + i, p) for p in parts for i in range(args.steps)]
    log("[bench] warmup")
    step_s = []   # a part's step on the GPU after its warmup (sets its settle count)
    for p in parts:
        metas = [p.run(i, None) for i in range(args.warmup)]
        torch.cuda.synchronize()
        t_w = time.perf_counter()
        n_cal = min(3, args.warmup + args.steps)   # metadata buffers the warmup has finished with
        metas += [p.run(i, None) for i in range(n_cal)]
        torch.cuda.synchronize()
        step_s.append((time.perf_counter() - t_w) / n_cal)
        del metas

    # Whole steps, wall clock: host packing, uploads and every kernel, with a
    # synchronize on both sides. The objects made during set-up (torch's own
    # included, ~170k) are collected and frozen first, so that the garbage
    # collector does not traverse them all inside the timed pass (a full
    # collection there stalls the host for ~37 ms, longer than the 50 steps).
    gc.collect()
    gc.freeze()
    log(f"[bench] timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    keep = [p.run(i, None) for (i, p) in order(args.warmup)]
    t_host = time.perf_counter() - t0
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    del keep

    # The same steps again, each call bracketed by HIP events on its stream.
    # The host enqueues them while a short spin kernel holds the GPU, so the
    # kernels run back to back and no interval contains host launch latency.
    # The pass goes in chunks of a few steps, each behind its own spin and
    # followed by a synchronize: with hundreds of commands outstanding the
    # runtime makes the host wait for queue space, and the GPU would then
    # idle inside the timed intervals. Between the spin and the timed steps
    # of a chunk, untimed steps of the same part (EVENT_SETTLE_S of GPU time)
    # take the card from the idle spin to the clock it holds under
    # continuous work.
    chunk = EVENT_CHUNK_STEPS
    settle = [int(min(EVENT_SETTLE_MAX, max(2, math.ceil(EVENT_SETTLE_S / max(t, 1e-6))))) for t in step_s]
    for p, n_settle in zip(parts, settle):
        p.prepare(args.steps + n_settle)   # the settle steps use their own metadata buffers
    events = [[[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in parts]
              for _ in range(args.steps)]
    # torch creates the HIP event on its first record: do that outside the
    # timed pass, so that recording costs the host only microseconds there.
    for ev_step in events:
        for evs in ev_step:
            for e in evs:
                e.record()
    torch.cuda.synchronize()
    t_enq_max, late = 0.0, 0
    for p, n_settle in zip(parts, settle):
        preroll_s = 4 * t_host * (chunk + n_settle) / args.steps + 5e-3
        cycles = preroll_cycles(preroll_s)
        for c0 in range(0, args.steps, chunk):
            torch.cuda._sleep(cycles)
            t_enq = time.perf_counter()
            keep = [p.run(args.steps + j, None) for j in range(n_settle)]
            keep += [p.run(i, events[i][parts.index(p)]) for i in range(c0, min(c0 + chunk, args.steps))]
            t_enq = time.perf_counter() - t_enq
            torch.cuda.synchronize()
            del keep
            t_enq_max = max(t_enq_max, t_enq)
            late += t_enq > preroll_s
    if late:
        log(f"[bench] WARNING: in {late} chunk(s) the host enqueue outlasted the pre-roll; "
            "those intervals may hold host gaps")
    log(f"[bench] wall {wall * 1e3:.2f} ms for {args.steps} steps (host {t_host * 1e3:.1f} ms); "
        f"event pass in chunks of {chunk} steps: longest host enqueue {t_enq_max * 1e3:.2f} ms "
        f"behind a {preroll_s * 1e3:.1f} ms pre-roll; settle steps per chunk {settle}")
    for j, p in enumerate(parts):
        p.collect([events[i][j] for i in range(args.steps)])
    summaries = [p.summary() for p in parts]
    log("[bench] " + json.dumps(summaries))
    log("[bench] size-matched streaming references")
    size_matched = size_matched_rates(parts, summaries, stream_read["decode_shaped"]["workgroups_per_cu"],
                                      preroll_cycles(5e-3))

    cpu = {}
    if not args.no_cpu_baseline:
        for p in parts:
            log(f"[bench] oracle cpu baseline: {p.phase} preset {p.preset}")
            if p.phase not in cpu:
                cpu[p.phase] = cpu_baseline(p.phase, p.preset, args.cpu_budget)

    dec = next((s for s in summaries if s["phase"] == "decode"), None)
    pre = next((s for s in summaries if s["phase"] == "prefill"), None)
    if dec is not None:
        value, unit = dec["attention_GBps"], "GB/s"
        per_launch = dec["attention_bytes"]
        roof = {"bound": "hbm", "achieved": value, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": value / HBM_PEAK_GBS,
                "traffic": counters_traffic("decode.hip", f"decode-preset{dec['preset']}"),
                "kernel": ("decode_sk_kernel + decode_sk_reduce_kernel" if dec["partition_size"] == 0
                           else "fixed-partition decode kernel + decode_reduce_kernel")
                          + " (one decode_attention_paged call)",
                "algorithmic_bytes_per_launch": per_launch, "avg_launch_us": dec["attention_us"]}
        cpu_main = cpu.get("decode")
    elif pre["attention_flops"] / pre["attention_bytes"] >= MFMA_BF16_PEAK_TFLOPS * 1e3 / HBM_PEAK_GBS:
        value, unit = pre["attention_TFLOPs"], "TFLOP/s"
        roof = {"bound": "mfma", "achieved": value, "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": value / MFMA_BF16_PEAK_TFLOPS,
                "traffic": counters_traffic("prefill.hip", f"prefill-preset{pre['preset']}"),
                "kernel": "prefill_mfma_kernel", "algorithmic_flops_per_launch": pre["attention_flops"],
                "avg_launch_us": pre["attention_us"]}
        cpu_main = cpu.get("prefill")
    else:
        # a prefill call below the ridge point (decode rows, short chunks over
        # long cached contexts) is bound by its K/V bytes
        value, unit = pre["attention_GBps"], "GB/s"
        roof = {"bound": "hbm", "achieved": value, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": value / HBM_PEAK_GBS,
                "traffic": counters_traffic("prefill.hip", f"prefill-preset{pre['preset']}"),
                "kernel": "prefill_mfma_kernel", "algorithmic_bytes_per_launch": pre["attention_bytes"],
                "avg_launch_us": pre["attention_us"]}
        cpu_main = cpu.get("prefill")
    names = {2: "decode-qwen3-0.6b-b64-ctx512-4096", 3: "prefill-varlen-16x-u128-2048-budget16384",
             4: "prefill-prefix-hit-32x2048", 5: "decode-qwen3-8b-b512-ctx256-32768",
             6: "decode-in-varlen-qwen3-0.6b-b64", 7: "mixed-b64-decode+2x512-chunks"}
    config = {"workload": " + ".join(names[p.preset] for p in parts),
              "parts": [{"phase": p.phase, **p.w.describe()} for p in parts],
              "copies_in_rotation": [len(p.copies) for p in parts]}
    line = {
        "metric": METRIC, "value": value, "unit": unit, "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": wall / args.steps * 1e3, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": config, "roofline": roof, "cpu_baseline": cpu_main,
        "secondary": {}, "parts": summaries, "cpu_baselines": cpu,
        "event_timing": {"chunk_steps": EVENT_CHUNK_STEPS, "chunks_with_host_gaps": late,
                         "settle_steps_per_chunk": settle, "settle_target_s": EVENT_SETTLE_S},
    }
    if any(p.preset == 4 for p in parts):
        line["block_manager_host"] = block_manager_host()
    if args.workload == "decode-graph":
        log("[bench] 28-layer decode steps: eager vs hipGraph")
        line["decode_graph"] = decode_graph_compare()
    sec = line["secondary"]
    if pre is not None:
        sec["prefill_attention_TFLOPs"] = pre["attention_TFLOPs"]
        sec["prefill_frac_of_mfma_peak"] = pre["attention_frac_mfma"]
        sec["prefill_workload"] = names[pre["preset"]]
        if dec is not None:
            # the MFMA side of the step, in the same form as `roofline`
            sec["prefill_roofline"] = {
                "bound": "mfma", "achieved": pre["attention_TFLOPs"], "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": pre["attention_frac_mfma"],
                "traffic": counters_traffic("prefill.hip", f"prefill-preset{pre['preset']}"),
                "kernel": "prefill_mfma_kernel", "algorithmic_flops_per_launch": pre["attention_flops"],
                "avg_launch_us": pre["attention_us"]}
    if dec is not None:
        sec["decode_frac_of_hbm_peak"] = dec["attention_frac_hbm"]
        # the same call against the best read-only stream this GPU reached in this run
        sec["decode_over_best_stream_read"] = dec["attention_GBps"] / stream_read["best"]["GBps"]
    # every part's attention figure, by workload
    for sm in summaries:
        k = names[sm["preset"]] + ("+fused-store" if sm["workload"].endswith("+fused") else "")
        if sm["phase"] == "decode":
            sec.setdefault("per_workload", {})[k] = {
                "GBps": sm["attention_GBps"], "frac_of_hbm_peak": sm["attention_frac_hbm"],
                "attention_us": sm["attention_us"]}
        else:
            sec.setdefault("per_workload", {})[k] = {
                "TFLOPs": sm["attention_TFLOPs"], "frac_of_mfma_peak": sm["attention_frac_mfma"],
                "attention_us": sm["attention_us"]}
    # what plain streaming kernels reach on this GPU, beside the published peak
    sec["device_copy_GBps"] = copy_gbps
    sec["stream_read"] = stream_read
    sec["size_matched"] = size_matched
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
