"""One pass of the hot path over a batch: pack the step's metadata on the host
(one pinned buffer, one copy), store this step's K/V into the pool, then run
prefill or decode attention. All compute is in libpkv's kernels.

The batch is described the way the pages' ModelRunner sees it: per sequence,
its length, how many leading tokens are already cached, and its block table.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List, Optional, Sequence, Tuple

import torch

from . import (decode_attention_paged, decode_store_attention_paged, decode_workspace_bytes,
               pack_decode, pack_prefill, prefill_attention_varlen, prefill_store_attention_varlen,
               store_kvcache)


def alloc_pool(num_blocks: int, block_size: int, num_kv_heads: int, head_dim: int,
               dtype: torch.dtype, device, fill: float = float("nan")) -> Tuple[torch.Tensor, torch.Tensor]:
    """K and V caches [num_blocks, bs, Hkv, d], every element ``fill`` (NaN by
    default, so a read of an unwritten slot shows in the output)."""
    shape = (num_blocks, block_size, num_kv_heads, head_dim)
    k = torch.full(shape, fill, dtype=dtype, device=device)
    v = torch.full(shape, fill, dtype=dtype, device=device)
    return k, v


def write_ranges(ranges: Sequence[Tuple[int, int, int]], block_tables: Sequence[Sequence[int]],
                 block_size: int, k_rows: torch.Tensor, v_rows: torch.Tensor,
                 k_cache: torch.Tensor, v_cache: torch.Tensor, stream=None) -> None:
    """Store K/V rows for positions [b, e) of sequences s, for each (s, b, e),
    rows in list order -- e.g. a cached prefix written before the step."""
    if not ranges:
        return
    meta = pack_prefill([e for _, _, e in ranges], [b for _, b, _ in ranges],
                        [block_tables[s] for s, _, _ in ranges], block_size,
                        device=k_cache.device, stream=stream)
    store_kvcache(k_rows, v_rows, k_cache, v_cache, meta["slot_mapping"], stream=stream)


@dataclass
class StepInputs:
    phase: str
    seq_lens: List[int]
    num_cached: List[int]
    block_tables: List[List[int]]
    block_size: int
    scale: float
    use_block_tables: bool = True
    partition_size: int = 0
    fuse_store: bool = False


def run_step(s: StepInputs, q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
             k_cache: torch.Tensor, v_cache: torch.Tensor, out: Optional[torch.Tensor] = None,
             workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Pack + store + attention for one step. Decode: one new token per
    sequence (num_cached = len - 1). Prefill: keys read from the pool through
    the block tables when the batch has a cached prefix (or when
    ``use_block_tables``), else from this step's contiguous k/v. With
    ``fuse_store`` the store and the attention are one call."""
    dev = k_cache.device
    if s.phase == "decode":
        meta = pack_decode(s.seq_lens, s.block_tables, s.block_size, device=dev, stream=stream)
        if s.fuse_store:
            return decode_store_attention_paged(q, k_new, v_new, k_cache, v_cache, meta["slot_mapping"],
                                                meta["block_tables"], meta["context_lens"],
                                                meta["max_seqlen_k"], s.scale, out=out,
                                                partition_size=s.partition_size, workspace=workspace,
                                                stream=stream)
        store_kvcache(k_new, v_new, k_cache, v_cache, meta["slot_mapping"], stream=stream)
        return decode_attention_paged(q, k_cache, v_cache, meta["block_tables"],
                                      meta["context_lens"], meta["max_seqlen_k"], s.scale,
                                      out=out, partition_size=s.partition_size,
                                      workspace=workspace, stream=stream)
    meta = pack_prefill(s.seq_lens, s.num_cached, s.block_tables, s.block_size, device=dev,
                        stream=stream)
    bt = meta["block_tables"]
    if bt is None and s.use_block_tables:
        # a batch without a cached prefix may still read its keys from the pool
        meta_bt = pack_decode(s.seq_lens, s.block_tables, s.block_size, device=dev, stream=stream)
        bt = meta_bt["block_tables"]
    if s.fuse_store:
        return prefill_store_attention_varlen(q, k_new, v_new, k_cache, v_cache, meta["slot_mapping"],
                                              meta["cu_seqlens_q"], meta["cu_seqlens_k"],
                                              meta["max_seqlen_q"], meta["max_seqlen_k"], s.scale,
                                              block_tables=bt, out=out, stream=stream)
    store_kvcache(k_new, v_new, k_cache, v_cache, meta["slot_mapping"], stream=stream)
    if bt is not None:
        return prefill_attention_varlen(q, meta["cu_seqlens_q"], meta["cu_seqlens_k"],
                                        meta["max_seqlen_q"], meta["max_seqlen_k"], s.scale,
                                        k_cache=k_cache, v_cache=v_cache, block_tables=bt,
                                        out=out, stream=stream)
    return prefill_attention_varlen(q, meta["cu_seqlens_q"], meta["cu_seqlens_k"],
                                    meta["max_seqlen_q"], meta["max_seqlen_k"], s.scale,
                                    k=k_new, v=v_new, out=out, stream=stream)


def decode_rows_first(s: StepInputs) -> int:
    """Number of leading sequences of a prefill step that are decode rows
    (exactly one new token on top of a cached context)."""
    n = 0
    for L, c in zip(s.seq_lens, s.num_cached):
        if L - c != 1 or c < 1:
            break
        n += 1
    return n


def run_mixed_step(s: StepInputs, q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                   k_cache: torch.Tensor, v_cache: torch.Tensor, out: Optional[torch.Tensor] = None,
                   workspace: Optional[torch.Tensor] = None, stream=None,
                   side_stream=None) -> torch.Tensor:
    """A mixed (chunked-prefill) step whose decode rows come first: those go
    through the decode kernel -- the K/V of a kv head streamed once for its
    whole query-head group and split over every SIMD -- and the prompts and
    prompt chunks that follow through the varlen call. Same results as
    ``run_step`` on the whole batch.

    With ``side_stream`` (a default-priority stream) the prompt part runs
    there, ordered after the work already queued on ``stream``, and
    ``stream`` waits for it before returning: the two parts write disjoint
    rows and cache slots, so the chunks can start on CUs whose decode waves
    have finished."""
    nd = decode_rows_first(s)
    if nd == 0 or nd == len(s.seq_lens):
        return run_step(s if nd == 0 else StepInputs("decode", s.seq_lens, s.num_cached,
                                                        s.block_tables, s.block_size, s.scale),
                        q, k_new, v_new, k_cache, v_cache, out=out, workspace=workspace, stream=stream)
    if out is None:
        out = torch.empty_like(q)
    dec = StepInputs("decode", s.seq_lens[:nd], s.num_cached[:nd], s.block_tables[:nd],
                     s.block_size, s.scale)
    pre = StepInputs("prefill", s.seq_lens[nd:], s.num_cached[nd:], s.block_tables[nd:],
                     s.block_size, s.scale, s.use_block_tables)
    main = stream if stream is not None else torch.cuda.current_stream()
    if side_stream is not None:
        side_stream.wait_stream(main)
    run_step(dec, q[:nd], k_new[:nd], v_new[:nd], k_cache, v_cache, out=out[:nd],
             workspace=workspace, stream=main)
    run_step(pre, q[nd:], k_new[nd:], v_new[nd:], k_cache, v_cache, out=out[nd:],
             stream=side_stream if side_stream is not None else main)
    if side_stream is not None:
        main.wait_stream(side_stream)
    return out


def step_inputs_of(w, partition_size: int = 0, fuse_store: bool = False) -> StepInputs:
    """StepInputs from any object with the batch fields (e.g. a seeded workload)."""
    return StepInputs(phase=w.phase, seq_lens=list(w.seq_lens), num_cached=list(w.num_cached),
                      block_tables=[list(t) for t in w.block_tables], block_size=w.block_size,
                      scale=w.scale, use_block_tables=w.use_block_tables,
                      partition_size=partition_size, fuse_store=fuse_store)
