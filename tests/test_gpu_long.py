"""Long-context prefill parity: one 16384-token prompt, 16 query heads over 8
kv heads, d 128, bf16 (256 key tiles per query block, 128 query blocks per
head). The oracle is too slow for every row at this size, so two samples are
checked, each against an exact oracle result:

- the first 1024 rows: by causality they equal the prefill of the first 1024
  tokens alone;
- the last 64 rows: the oracle's bottom-right-aligned attention of 64 queries
  over all 16384 keys, which crosses every key tile.

Both the contiguous keys and the paged pool (block size 256, permuted block
ids) are run."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_125_amd as pkv
from gpu_helpers import max_abs_err, say

pytestmark = pytest.mark.gpu

N, HQ, HKV, D, BS = 16384, 16, 8, 128, 256


@pytest.fixture(scope="module")
def inputs():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    pkv.lib()
    gen = torch.Generator().manual_seed(16384)
    q = torch.randn(N, HQ, D, generator=gen).to(torch.bfloat16)
    k = torch.randn(N, HKV, D, generator=gen).to(torch.bfloat16)
    v = torch.randn(N, HKV, D, generator=gen).to(torch.bfloat16)
    return q, k, v


def _check(out, q, k, v, scale):
    head = oracle.attention(q[:1024], [1024], [1024], HKV, scale, k=k[:1024], v=v[:1024])
    tail = oracle.attention(q[N - 64:], [64], [N], HKV, scale, k=k, v=v)
    e_head, e_tail = max_abs_err(out[:1024], head), max_abs_err(out[N - 64:], tail)
    say(f"  first 1024 rows: max |err| {e_head:.3e}; last 64 rows: max |err| {e_tail:.3e}")
    assert e_head <= 2e-2 and e_tail <= 2e-2


def test_long_prefill_contiguous(inputs):
    say(f"[gpu] long prefill: one {N}-token prompt, contiguous k/v")
    q, k, v = inputs
    scale = D ** -0.5
    cu = torch.tensor([0, N], dtype=torch.int32, device="cuda")
    out = pkv.prefill_attention_varlen(q.cuda(), cu, cu, N, N, scale, k=k.cuda(), v=v.cuda())
    torch.cuda.synchronize()
    _check(out, q, k, v, scale)


def test_long_prefill_paged(inputs):
    say(f"[gpu] long prefill: one {N}-token prompt through a permuted block table")
    q, k, v = inputs
    scale = D ** -0.5
    nb = N // BS
    perm = np.random.default_rng(7).permutation(nb + 5)[:nb]
    meta = pkv.pack_prefill([N], [0], [[int(b) for b in perm]], BS, device="cuda")
    kc = torch.zeros(nb + 5, BS, HKV, D, dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    pkv.store_kvcache(k.cuda(), v.cuda(), kc, vc, meta["slot_mapping"])
    # read back through the pool (a prefill without a cached prefix packs no
    # table; the decode packer builds the same table)
    bt = pkv.pack_decode([N], [[int(b) for b in perm]], BS, device="cuda")["block_tables"]
    out = pkv.prefill_attention_varlen(q.cuda(), meta["cu_seqlens_q"], meta["cu_seqlens_k"], N, N, scale,
                                       k_cache=kc, v_cache=vc, block_tables=bt)
    torch.cuda.synchronize()
    _check(out, q, k, v, scale)
