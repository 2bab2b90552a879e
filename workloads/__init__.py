"""Seeded synthetic inputs for the paged-KV attention hot path.

This module is shared by the oracle's tests and the HIP path's tests and bench. It
holds no arithmetic of the method itself: no slot computation, no gather, no
softmax. It only draws

* the shape of a batch: per-sequence total length (``seq_lens``), how many leading
  tokens already have K/V in the cache (``num_cached``), and each sequence's
  block table (a list of physical block ids, drawn as a random permutation of the
  pool, as the pages' paging model allows any physical placement);
* the values: q for the tokens processed by this call, K/V for those tokens, and
  K/V for the already-cached ("history") tokens, all N(0, 1) drawn in float32 and
  rounded to the workload dtype (bf16 rounding is torch's round-to-nearest-even).

The five presets follow the workload descriptions (tiny fp32 paged attention;
Qwen3-0.6B-shaped decode; varlen prefill under a 16384-token batch budget;
prefill with prefix-cache hits; Qwen3-8B-shaped long-context decode). Seeds are
``1000 + preset number``.

Ordering conventions (the pages' prepare_prefill / prepare_decode walk the batch
sequence by sequence, tokens in position order):

* rows of ``q``, ``k_new``, ``v_new`` are sequence-major, positions ascending,
  covering positions ``[num_cached[s], seq_lens[s])`` of each sequence;
* ``hist`` lists (seq, begin, end) position ranges whose K/V must be written into
  the pool before the call; rows of ``k_hist`` / ``v_hist`` follow that list. A
  shared prefix is listed once (under its first owner); the other sequences point
  their block tables at the same physical blocks.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional, Tuple

import numpy as np
import torch

__all__ = ["Workload", "make_workload", "PRESETS", "custom_workload"]


@dataclasses.dataclass
class Workload:
    name: str
    phase: str                      # "prefill" or "decode"
    dtype: torch.dtype              # torch.float32 or torch.bfloat16
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    scale: float
    seq_lens: List[int]             # len(seq) after this call's tokens are appended
    num_cached: List[int]           # leading tokens whose K/V is already in the pool
    block_tables: List[List[int]]   # physical block ids per sequence, logical order
    hist: List[Tuple[int, int, int]]  # (seq, begin, end) ranges pre-written into the pool
    use_block_tables: bool          # prefill: read keys through the pool (prefix hits)
    q: Optional[torch.Tensor] = None      # [Tq, Hq, d]
    k_new: Optional[torch.Tensor] = None  # [Tq, Hkv, d]
    v_new: Optional[torch.Tensor] = None  # [Tq, Hkv, d]
    k_hist: Optional[torch.Tensor] = None  # [Th, Hkv, d]
    v_hist: Optional[torch.Tensor] = None  # [Th, Hkv, d]
    seed: int = 0

    @property
    def num_seqs(self) -> int:
        return len(self.seq_lens)

    @property
    def q_lens(self) -> List[int]:
        return [n - c for n, c in zip(self.seq_lens, self.num_cached)]

    @property
    def total_q(self) -> int:
        return sum(self.q_lens)

    @property
    def total_hist(self) -> int:
        return sum(e - b for _, b, e in self.hist)

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    def describe(self) -> dict:
        return {
            "workload": self.name, "phase": self.phase,
            "dtype": "bf16" if self.dtype == torch.bfloat16 else "f32",
            "num_seqs": self.num_seqs, "num_q_heads": self.num_q_heads,
            "num_kv_heads": self.num_kv_heads, "head_dim": self.head_dim,
            "block_size": self.block_size, "num_blocks": self.num_blocks,
            "total_q_tokens": self.total_q, "total_context_tokens": int(sum(self.seq_lens)),
            "seed": self.seed,
        }


def _blocks_for(n: int, bs: int) -> int:
    # number of pool blocks a sequence of n tokens occupies (page count)
    return -(-n // bs)


def _draw(gen: torch.Generator, rows: int, heads: int, d: int, dtype: torch.dtype,
          device: str, chunk_rows: int = 1 << 16) -> torch.Tensor:
    """N(0,1) in float32, rounded to ``dtype``; drawn in row chunks to bound the
    float32 temporary."""
    out = torch.empty((rows, heads, d), dtype=dtype, device=device)
    for r0 in range(0, rows, chunk_rows):
        r1 = min(rows, r0 + chunk_rows)
        t = torch.randn((r1 - r0, heads, d), generator=gen, dtype=torch.float32, device=device)
        out[r0:r1].copy_(t)
    return out


def _fill_values(w: Workload, device: str) -> Workload:
    gen = torch.Generator(device=device)
    gen.manual_seed(w.seed)
    Hq, Hkv, d = w.num_q_heads, w.num_kv_heads, w.head_dim
    w.q = _draw(gen, w.total_q, Hq, d, w.dtype, device)
    w.k_new = _draw(gen, w.total_q, Hkv, d, w.dtype, device)
    w.v_new = _draw(gen, w.total_q, Hkv, d, w.dtype, device)
    w.k_hist = _draw(gen, w.total_hist, Hkv, d, w.dtype, device)
    w.v_hist = _draw(gen, w.total_hist, Hkv, d, w.dtype, device)
    return w


def _tables_from_perm(perm: np.ndarray, counts: List[int]) -> List[List[int]]:
    tables, at = [], 0
    for c in counts:
        tables.append([int(x) for x in perm[at:at + c]])
        at += c
    return tables


def _preset1(rng: np.random.Generator, phase: str) -> dict:
    # tiny fp32 paged attention: prompts 37 and 100, bs 16, 32-block pool,
    # seq0 takes perm[0:3], seq1 perm[3:10]; then one decode token each.
    perm = rng.permutation(32)
    tables = [[int(x) for x in perm[0:3]], [int(x) for x in perm[3:10]]]
    prompts = [37, 100]
    base = dict(dtype=torch.float32, num_q_heads=4, num_kv_heads=2, head_dim=64,
                block_size=16, num_blocks=32, block_tables=tables)
    if phase == "prefill":
        return dict(base, phase="prefill", seq_lens=prompts, num_cached=[0, 0],
                    hist=[], use_block_tables=False)
    lens = [p + 1 for p in prompts]
    return dict(base, phase="decode", seq_lens=lens, num_cached=[n - 1 for n in lens],
                hist=[(s, 0, n - 1) for s, n in enumerate(lens)], use_block_tables=True)


def _decode_batch(rng, B, lo, hi, log_uniform, bs, Hq, Hkv, pool=None) -> dict:
    if log_uniform:
        ctx = np.floor(np.exp(rng.uniform(math.log(lo), math.log(hi), size=B))).astype(np.int64)
        ctx = np.clip(ctx, lo, hi)
    else:
        ctx = rng.integers(lo, hi + 1, size=B)
    counts = [_blocks_for(int(n), bs) for n in ctx]
    if pool is None:
        pool = sum(counts)
    perm = rng.permutation(pool)
    tables = _tables_from_perm(perm, counts)
    lens = [int(n) for n in ctx]
    return dict(phase="decode", dtype=torch.bfloat16, num_q_heads=Hq, num_kv_heads=Hkv,
                head_dim=128, block_size=bs, num_blocks=pool, block_tables=tables,
                seq_lens=lens, num_cached=[n - 1 for n in lens],
                hist=[(s, 0, n - 1) for s, n in enumerate(lens)], use_block_tables=True)


def _preset2(rng, phase):
    # Qwen3-0.6B-shaped decode: 16 q / 8 kv heads, d 128, bs 256, 64 seqs,
    # context U{512..4096}, block tables from a permutation of a 2048-block pool.
    return _decode_batch(rng, 64, 512, 4096, False, 256, 16, 8, pool=2048)


def _preset3(rng, phase):
    # varlen causal prefill: 16 prompts U{128..2048}, redrawn until the batch fits
    # the 16384-token budget; all tokens stored into a 256-token-block pool.
    while True:
        lens = rng.integers(128, 2049, size=16)
        if int(lens.sum()) <= 16384:
            break
    counts = [_blocks_for(int(n), 256) for n in lens]
    perm = rng.permutation(2048)
    return dict(phase="prefill", dtype=torch.bfloat16, num_q_heads=16, num_kv_heads=8,
                head_dim=128, block_size=256, num_blocks=2048,
                block_tables=_tables_from_perm(perm, counts),
                seq_lens=[int(n) for n in lens], num_cached=[0] * 16, hist=[],
                use_block_tables=False)


def _preset4(rng, phase):
    # prefix-cache hits: 32 seqs of 2048 tokens; the even-indexed ones share one
    # cached 1024-token prefix held in the same 4 physical blocks.
    bs, n, pre = 256, 2048, 1024
    perm = rng.permutation(2048)
    shared = [int(x) for x in perm[0:pre // bs]]
    at = pre // bs
    tables, cached, hist = [], [], []
    for s in range(32):
        if s % 2 == 0:
            own = [int(x) for x in perm[at:at + (n - pre) // bs]]
            at += (n - pre) // bs
            tables.append(shared + own)
            cached.append(pre)
            if s == 0:
                hist.append((0, 0, pre))
        else:
            tables.append([int(x) for x in perm[at:at + n // bs]])
            at += n // bs
            cached.append(0)
    return dict(phase="prefill", dtype=torch.bfloat16, num_q_heads=16, num_kv_heads=8,
                head_dim=128, block_size=bs, num_blocks=2048, block_tables=tables,
                seq_lens=[n] * 32, num_cached=cached, hist=hist, use_block_tables=True)


def _preset5(rng, phase):
    # Qwen3-8B-shaped long-context decode: 32 q / 8 kv heads, 512 seqs,
    # context log-uniform in [256, 32768], pool sized to fit exactly.
    return _decode_batch(rng, 512, 256, 32768, True, 256, 32, 8, pool=None)


def _preset6(rng, phase):
    # Decode through the varlen prefill call: preset 2's batch (the same context
    # lengths and block tables, drawn from preset 2's seed) as one prefill step
    # whose every sequence has all but its newest token cached (Lq = 1).
    spec = _decode_batch(np.random.default_rng(1002), 64, 512, 4096, False, 256, 16, 8, pool=2048)
    return dict(spec, phase="prefill")


def _preset7(rng, phase):
    # A mixed (chunked-prefill) step: preset 2's kind of decode batch -- 64
    # sequences, context U{512..4096}, Lq = 1 -- plus two prompts of 2048 tokens
    # whose first 1536 are cached, each contributing a 512-token chunk, in one
    # varlen call. The chunks' blocks follow the decode pool.
    spec = _decode_batch(rng, 64, 512, 4096, False, 256, 16, 8, pool=2048)
    bs, n, c = 256, 2048, 1536
    pool = spec["num_blocks"]
    for i in range(2):
        s = len(spec["seq_lens"])
        spec["block_tables"].append(list(range(pool + i * (n // bs), pool + (i + 1) * (n // bs))))
        spec["seq_lens"].append(n)
        spec["num_cached"].append(c)
        spec["hist"].append((s, 0, c))
    spec["num_blocks"] = pool + 2 * (n // bs)
    return dict(spec, phase="prefill")


PRESETS = {
    1: ("tiny-fp32-paged", _preset1),
    2: ("decode-qwen3-0.6b-b64", _preset2),
    3: ("prefill-varlen-16x-u128-2048", _preset3),
    4: ("prefill-prefix-hit-32x2048", _preset4),
    5: ("decode-qwen3-8b-b512-long", _preset5),
    6: ("decode-in-varlen-qwen3-0.6b-b64", _preset6),
    7: ("mixed-b64-decode+2x512-chunks", _preset7),
}


def make_workload(preset: int, phase: Optional[str] = None, device: str = "cpu",
                  values: bool = True) -> Workload:
    """Build preset ``preset`` (1..7). Preset 1 has both phases: ``phase`` picks
    "prefill" (default) or "decode". ``values=False`` skips drawing tensors."""
    name, fn = PRESETS[preset]
    seed = 1000 + preset
    rng = np.random.default_rng(seed)
    spec = fn(rng, phase or "prefill")
    d = spec["head_dim"]
    w = Workload(name=name + ("-" + spec["phase"] if preset == 1 else ""),
                 scale=1.0 / math.sqrt(d), seed=seed, **spec)
    return _fill_values(w, device) if values else w


def custom_workload(*, phase: str, seq_lens: List[int], num_cached: List[int],
                    num_q_heads: int, num_kv_heads: int, head_dim: int, block_size: int,
                    dtype: torch.dtype = torch.bfloat16, seed: int = 7,
                    extra_blocks: int = 3, use_block_tables: Optional[bool] = None,
                    shared_prefix: bool = False, device: str = "cpu",
                    scale: Optional[float] = None) -> Workload:
    """A small seeded workload of arbitrary shape, for edge cases.

    ``num_cached[s]`` leading tokens of sequence s are history (pre-written);
    the rest are processed by the call. With ``shared_prefix`` every sequence
    whose ``num_cached`` equals the first one's shares the first one's prefix
    blocks (the prefix must be whole blocks)."""
    rng = np.random.default_rng(seed)
    counts = [_blocks_for(n, block_size) for n in seq_lens]
    pool = sum(counts) + extra_blocks
    perm = [int(x) for x in rng.permutation(pool)]
    tables, hist, at = [], [], 0
    first_pre = num_cached[0] if seq_lens else 0
    shared_blocks = None
    for s, (n, c) in enumerate(zip(seq_lens, num_cached)):
        nb = counts[s]
        if shared_prefix and c == first_pre and c > 0 and c % block_size == 0:
            npre = c // block_size
            if shared_blocks is None:
                shared_blocks = perm[at:at + npre]
                at += npre
                hist.append((s, 0, c))
            own = perm[at:at + nb - npre]
            at += nb - npre
            tables.append(list(shared_blocks) + own)
        else:
            tables.append(perm[at:at + nb])
            at += nb
            if c > 0:
                hist.append((s, 0, c))
    if use_block_tables is None:
        use_block_tables = phase == "decode" or sum(num_cached) > 0
    w = Workload(name="custom", phase=phase, dtype=dtype, num_q_heads=num_q_heads,
                 num_kv_heads=num_kv_heads, head_dim=head_dim, block_size=block_size,
                 num_blocks=pool, scale=scale if scale is not None else 1.0 / math.sqrt(head_dim),
                 seq_lens=list(seq_lens), num_cached=list(num_cached), block_tables=tables,
                 hist=hist, use_block_tables=use_block_tables, seed=seed)
    return _fill_values(w, device)


def restrict(w: Workload, seq_ids: List[int], device: str = "cpu", values: bool = True) -> Workload:
    """A workload with only the sequences ``seq_ids`` of ``w`` (same shapes,
    block ids renumbered compactly in order of first use, fresh values drawn
    from w's seed). Used to take a bounded sample of a large preset."""
    remap = {}
    tables = []
    for s in seq_ids:
        t = []
        for b in w.block_tables[s]:
            remap.setdefault(b, len(remap))
            t.append(remap[b])
        tables.append(t)
    hist, seen = [], set()
    for i, s in enumerate(seq_ids):
        c = w.num_cached[s]
        if c > 0:
            key = tuple(tables[i][:_blocks_for(c, w.block_size)])
            if key not in seen:
                seen.add(key)
                hist.append((i, 0, c))
    r = dataclasses.replace(
        w, seq_lens=[w.seq_lens[s] for s in seq_ids], num_cached=[w.num_cached[s] for s in seq_ids],
        block_tables=tables, num_blocks=len(remap), hist=hist,
        q=None, k_new=None, v_new=None, k_hist=None, v_hist=None)
    return _fill_values(r, device) if values else r
