"""pkv_decode_attention_paged_noalloc against pkv_decode_attention_paged: the
same kernels with the library's static scratch instead of a caller workspace.
Two calls in a row share the scratch, the second on a smaller input; each must
equal the workspace entry point's output bit for bit (the same kernels on the
same inputs) and the oracle within the bf16 bar. A call whose plan needs more
than the scratch holds is refused on the host before anything is launched."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_125_amd as pkv
from gpu_helpers import max_abs_err, say, to_device
from paged_kv_cache_125_amd.step import alloc_pool, write_ranges
from workloads import custom_workload, make_workload

pytestmark = pytest.mark.gpu


def _setup(w):
    kc, vc = alloc_pool(w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim, w.dtype, "cuda")
    write_ranges(w.hist, w.block_tables, w.block_size, w.k_hist, w.v_hist, kc, vc)
    meta = pkv.pack_decode(w.seq_lens, w.block_tables, w.block_size, device="cuda")
    pkv.store_kvcache(w.k_new, w.v_new, kc, vc, meta["slot_mapping"])
    return kc, vc, meta


def test_noalloc_decode_matches_the_workspace_entry_point():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    pkv.lib()
    big = to_device(make_workload(2), "cuda")              # balanced split over all waves
    small = to_device(custom_workload(phase="decode", seq_lens=[700, 33, 1, 257],
                                      num_cached=[699, 32, 0, 256], num_q_heads=8, num_kv_heads=2,
                                      head_dim=128, block_size=16, seed=5), "cuda")
    cases = [(big, 0), (small, 64)]                        # the second: fixed partitions of 64
    setups = [_setup(w) for w, _ in cases]
    outs = []
    for (w, part), (kc, vc, meta) in zip(cases, setups):
        say(f"[gpu] noalloc decode: {w.name}, {w.num_seqs} seqs, partition {part}, "
            f"scratch need {pkv.decode_workspace_bytes(w.num_seqs, max(w.seq_lens), w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size, w.dtype, part)} B")
        out = torch.full_like(w.q, float("nan"))
        pkv.decode_attention_paged_noalloc(w.q, kc, vc, meta["block_tables"], meta["context_lens"],
                                           meta["max_seqlen_k"], w.scale, out, partition_size=part)
        outs.append(out)
    torch.cuda.synchronize()
    for (w, part), (kc, vc, meta), got in zip(cases, setups, outs):
        ref = pkv.decode_attention_paged(w.q, kc, vc, meta["block_tables"], meta["context_lens"],
                                         meta["max_seqlen_k"], w.scale, partition_size=part)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), f"{w.name}: noalloc output differs from the workspace entry point"
        want, *_ = oracle.run_workload(to_device(w, "cpu"))
        err = max_abs_err(got, want)
        say(f"  {w.name}: bit-identical to decode_attention_paged; max |err| vs oracle {err:.3e}")
        assert err <= 2e-2


def test_noalloc_decode_refuses_a_plan_beyond_its_scratch():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    B, hq, hkv, d, bs, ctx = 512, 32, 8, 128, 256, 32768
    need = pkv.decode_workspace_bytes(B, ctx, hq, hkv, d, bs, torch.bfloat16, 16)
    assert need > pkv.NOALLOC_SCRATCH_BYTES
    q = torch.zeros(B, hq, d, dtype=torch.bfloat16, device="cuda")
    kc = torch.zeros(4, bs, hkv, d, dtype=torch.bfloat16, device="cuda")
    bt = torch.zeros(B, ctx // bs, dtype=torch.int32, device="cuda")
    cl = torch.ones(B, dtype=torch.int32, device="cuda")
    out = torch.empty_like(q)
    with pytest.raises(pkv.PkvError, match="scratch"):
        pkv.decode_attention_paged_noalloc(q, kc, kc, bt, cl, ctx, d ** -0.5, out, partition_size=16)
    say(f"[gpu] noalloc decode: a plan needing {need} B is refused before launch")
