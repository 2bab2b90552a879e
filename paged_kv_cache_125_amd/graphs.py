"""Decode steps captured as HIP graphs, one per batch-size bucket.

"Nano vLLM 解读（5）：解析 ModelRunner", "run_model" and "capture_cudagraph":
decode batches of at most 512 sequences replay a graph captured for the
smallest bucket (1, 2, 4, 8, then multiples of 16 up to 512) that holds them,
after copying the step's inputs into static buffers; rows past the batch are
padding -- their slot is -1 (the store skips them) and their context length
is 0 (the attention writes zeros) -- and graphs are captured largest first.
Here a graph holds, for every layer given, store_kvcache of the new token's
K/V followed by decode_attention_paged: the attention-side kernels of one
decode step, with no host work between them. On ROCm, torch.cuda.CUDAGraph is
a hipGraph; every kernel in it is one of libpkv's, launched through the C ABI
on the capturing stream. Nothing in a captured step clears memory with a
memset: padding rows are fixed in the static buffers before each replay.
"""
from __future__ import annotations

from typing import List, Optional, Sequence, Tuple

import torch

from . import (decode_attention_paged, decode_store_attention_paged, decode_workspace_bytes,
               store_kvcache)

BUCKETS: List[int] = [1, 2, 4, 8] + list(range(16, 513, 16))


def bucket_for(batch: int, buckets: Sequence[int] = BUCKETS) -> int:
    """The smallest bucket holding ``batch`` sequences."""
    for b in buckets:
        if b >= batch:
            return b
    raise ValueError(f"batch {batch} exceeds the largest bucket {buckets[-1]}")


class DecodeGraphs:
    """Captured decode steps over ``layers`` (a list of (k_cache, v_cache),
    each [num_blocks, block_size, Hkv, d]) for every bucket in ``buckets``.

    ``run`` takes one step's inputs -- per layer q [B, Hq, d] and the new
    token's k, v [B, Hkv, d], plus the shared slot_mapping [B], context_lens
    [B] and block_tables [B, w] (int32, device) -- and returns the per-layer
    outputs (views of static buffers, valid until the next run).

    With ``fuse_store`` (the default) each layer is one
    decode_store_attention_paged call, which on the fixed-partition path of
    small batches runs the store inside the attention launch; without it, a
    store_kvcache call and a decode_attention_paged call."""

    def __init__(self, layers: Sequence[Tuple[torch.Tensor, torch.Tensor]], num_q_heads: int,
                 max_context_len: int, max_blocks_per_seq: int, scale: float,
                 buckets: Sequence[int] = BUCKETS, fuse_store: bool = True):
        self.layers = list(layers)
        self.fuse_store = bool(fuse_store)
        kc = self.layers[0][0]
        _, bs, hkv, d = kc.shape
        self.dtype, self.device = kc.dtype, kc.device
        self.hq, self.hkv, self.d, self.bs = num_q_heads, hkv, d, bs
        self.max_ctx, self.maxb, self.scale = int(max_context_len), int(max_blocks_per_seq), float(scale)
        self.buckets = sorted(int(b) for b in buckets)
        B = self.buckets[-1]
        L = len(self.layers)
        dev, dt = self.device, self.dtype
        # static buffers, sized for the largest bucket; bucket b uses rows [:b]
        self.q = torch.zeros(L, B, self.hq, d, dtype=dt, device=dev)
        self.k = torch.zeros(L, B, hkv, d, dtype=dt, device=dev)
        self.v = torch.zeros(L, B, hkv, d, dtype=dt, device=dev)
        self.out = torch.zeros(L, B, self.hq, d, dtype=dt, device=dev)
        self.slots = torch.full((B,), -1, dtype=torch.int32, device=dev)
        self.ctx = torch.zeros(B, dtype=torch.int32, device=dev)
        self.tables = torch.full((B, self.maxb), -1, dtype=torch.int32, device=dev)
        need = max(decode_workspace_bytes(b, self.max_ctx, self.hq, hkv, d, bs, dt) for b in self.buckets)
        self.workspace = torch.zeros(max(need, 256), dtype=torch.uint8, device=dev)
        self.graphs = {}
        self._capture()

    def _step(self, b: int) -> None:
        for l, (kc, vc) in enumerate(self.layers):
            if self.fuse_store:
                decode_store_attention_paged(self.q[l, :b], self.k[l, :b], self.v[l, :b], kc, vc,
                                             self.slots[:b], self.tables[:b], self.ctx[:b],
                                             self.max_ctx, self.scale, out=self.out[l, :b],
                                             workspace=self.workspace)
                continue
            store_kvcache(self.k[l, :b], self.v[l, :b], kc, vc, self.slots[:b])
            decode_attention_paged(self.q[l, :b], kc, vc, self.tables[:b], self.ctx[:b],
                                   self.max_ctx, self.scale, out=self.out[l, :b],
                                   workspace=self.workspace)

    def _capture(self) -> None:
        # the static rows are all padding while capturing: slots -1, contexts 0
        stream = torch.cuda.Stream()
        stream.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(stream):
            for b in self.buckets:          # eager warm-up: kernels loaded, plans cached
                self._step(b)
        torch.cuda.current_stream().wait_stream(stream)
        torch.cuda.synchronize()
        pool = None
        for b in reversed(self.buckets):    # largest first, one shared memory pool
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, pool=pool):
                self._step(b)
            if pool is None:
                pool = g.pool()
            self.graphs[b] = g
        torch.cuda.synchronize()

    def prepare(self, q: Sequence[torch.Tensor], k: Sequence[torch.Tensor], v: Sequence[torch.Tensor],
                slot_mapping: torch.Tensor, context_lens: torch.Tensor,
                block_tables: torch.Tensor) -> int:
        """Copy one step's inputs into the static buffers (padding rows: slot
        -1, context 0); returns the bucket to replay."""
        B = int(slot_mapping.numel())
        for l in range(len(self.layers)):
            self.q[l, :B].copy_(q[l])
            self.k[l, :B].copy_(k[l])
            self.v[l, :B].copy_(v[l])
        return self.prepare_meta(slot_mapping, context_lens, block_tables)

    def prepare_meta(self, slot_mapping: torch.Tensor, context_lens: torch.Tensor,
                     block_tables: torch.Tensor) -> int:
        """Copy only the step's metadata (the layers' q, k, v already sit in
        the static buffers, as when earlier kernels of the same graph produce
        them); returns the bucket to replay."""
        B = int(slot_mapping.numel())
        b = bucket_for(B, self.buckets)
        w = int(block_tables.shape[1])
        if w > self.maxb:
            raise ValueError("block tables wider than the captured maximum")
        self.slots[:B].copy_(slot_mapping)
        self.slots[B:b].fill_(-1)
        self.ctx[:B].copy_(context_lens)
        self.ctx[B:b].fill_(0)
        self.tables[:B, :w].copy_(block_tables)
        return b

    def replay(self, b: int) -> None:
        self.graphs[b].replay()

    def run(self, q, k, v, slot_mapping, context_lens, block_tables) -> List[torch.Tensor]:
        B = int(slot_mapping.numel())
        b = self.prepare(q, k, v, slot_mapping, context_lens, block_tables)
        self.replay(b)
        return [self.out[l, :B] for l in range(len(self.layers))]

    def run_eager(self, q, k, v, slot_mapping, context_lens, block_tables,
                  max_context_len: Optional[int] = None) -> List[torch.Tensor]:
        """The same step without graphs (for comparison)."""
        outs = []
        mc = self.max_ctx if max_context_len is None else int(max_context_len)
        for l, (kc, vc) in enumerate(self.layers):
            if self.fuse_store:
                outs.append(decode_store_attention_paged(q[l], k[l], v[l], kc, vc, slot_mapping,
                                                         block_tables, context_lens, mc, self.scale,
                                                         workspace=self.workspace))
                continue
            store_kvcache(k[l], v[l], kc, vc, slot_mapping)
            outs.append(decode_attention_paged(q[l], kc, vc, block_tables, context_lens, mc,
                                               self.scale, workspace=self.workspace))
        return outs
