"""Regression tests for memory the binding allocates and for bad step metadata.

1. Staging lifetime. The binding packs a step's metadata into a pinned host
   buffer and uploads it with pkv_upload (hipMemcpyAsync). When the binding
   allocated that buffer itself and the caller keeps only the device views,
   the buffer used to be freed at once; torch's pinned-memory cache then gave
   it to the next pack of the same size class, which overwrote it before the
   queued copy had run, so the earlier step's device metadata held the later
   step's values. The binding now holds such buffers until the copy has run.
2. Prefill bounds. The prefill kernels index q, out and contiguous k/v rows
   with cu_seqlens read on the device. A sequence whose rows do not fit in
   [0, total_q) is now skipped instead of read and written out of range.
3. Other streams. Device memory the binding allocates (decode workspace, out,
   packed metadata) comes from torch's caching allocator on the current
   stream. When the kernels go to another stream, the binding records the
   tensors on it, so that the allocator does not hand that memory to the
   current stream's next allocation before the kernels have run.

Only packs, uploads, spin kernels, decode calls on valid inputs and prefill
calls whose out-of-range rows lie inside memory the test itself allocated run
here: q, k, v and out are allocated with rows to spare past the claimed range,
filled with a sentinel, and the call is handed views of their first total_q
rows. A regressed guard would then read and write those spare rows, which the
test owns and checks, instead of memory past an allocation."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_125_amd as pkv
from gpu_helpers import max_abs_err, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def cuda():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    pkv.lib()
    return torch.device("cuda")


def test_staging_buffer_outlives_its_queued_upload(cuda):
    say("[gpu] pinned staging buffer held until its upload has run")
    bs = 16
    lens = [100 + i for i in range(32)]
    tables_a = [list(range(i * 80, i * 80 + -(-n // bs))) for i, n in enumerate(lens)]
    tables_b = [list(range(5000 + i * 80, 5000 + i * 80 + -(-n // bs))) for i, n in enumerate(lens)]
    for trial in range(3):
        torch.cuda.synchronize()
        torch.cuda._sleep(20_000_000)       # the uploads queue behind a few ms of spinning
        m = pkv.pack_decode(lens, tables_a, bs, device="cuda")
        bt_a = m["block_tables"]             # keep only the device view, as a step does
        del m
        m2 = pkv.pack_decode(lens, tables_b, bs, device="cuda")   # same layout size
        torch.cuda.synchronize()
        got = bt_a.cpu()
        for i, t in enumerate(tables_a):
            assert got[i, :len(t)].tolist() == t, f"trial {trial}: sequence {i}'s table overwritten"
        say(f"  trial {trial}: first step's block tables intact")
        del m2, bt_a


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16-mfma", "f32-generic"])
@pytest.mark.parametrize("paged", [False, True], ids=["contiguous", "paged"])
def test_prefill_skips_sequence_outside_total_q(cuda, dtype, paged):
    say(f"[gpu] prefill: a sequence whose cu_seqlens overrun total_q is skipped ({dtype}, paged={paged})")
    hq, hkv, d, bs = 8, 4, 128, 16
    total, n0, spare = 200, 100, 256
    gen = torch.Generator().manual_seed(11)
    q = torch.randn(spare, hq, d, generator=gen).to(dtype)
    k = torch.randn(spare, hkv, d, generator=gen).to(dtype)
    v = torch.randn(spare, hkv, d, generator=gen).to(dtype)
    # sequence 1 claims rows [100, 230) of a 200-row batch; the tensors hold
    # 256 rows, of which the call sees the first 200
    cu = torch.tensor([0, n0, n0 + 130], dtype=torch.int32, device="cuda")
    sentinel = 7.0
    out_all = torch.full((spare, hq, d), sentinel, dtype=dtype, device="cuda")
    out = out_all[:total]
    qd, kd, vd = q.cuda()[:total], k.cuda()[:total], v.cuda()[:total]
    scale = d ** -0.5
    if paged:
        nb = 2 * (-(-230 // bs)) + 2
        kc = torch.zeros(nb, bs, hkv, d, dtype=dtype)
        vc = torch.zeros(nb, bs, hkv, d, dtype=dtype)
        kc.view(-1, hkv, d)[:n0] = k[:n0]
        vc.view(-1, hkv, d)[:n0] = v[:n0]
        w = -(-230 // bs)
        tables = torch.full((2, w), -1, dtype=torch.int32)
        tables[0, :-(-n0 // bs)] = torch.arange(-(-n0 // bs), dtype=torch.int32)
        tables[1] = torch.arange(w, 2 * w, dtype=torch.int32)
        pkv.prefill_attention_varlen(qd, cu, cu, 130, 130, scale, k_cache=kc.cuda(),
                                     v_cache=vc.cuda(), block_tables=tables.cuda(), out=out)
    else:
        pkv.prefill_attention_varlen(qd, cu, cu, 130, 130, scale, k=kd, v=vd, out=out)
    torch.cuda.synchronize()
    want = oracle.attention(q[:n0], [n0], [n0], hkv, scale, k=k[:n0], v=v[:n0])
    err = max_abs_err(out[:n0], want)
    bar = 2e-2 if dtype == torch.bfloat16 else 1e-4
    say(f"  sequence 0: max |err| = {err:.3e}")
    assert err <= bar
    # rows [100, 200) belong to the skipped sequence; [200, 256) lie past total_q
    assert bool((out_all[n0:].float() == sentinel).all()), "rows of the skipped sequence were written"


def test_binding_allocations_survive_work_on_another_stream(cuda):
    say("[gpu] decode on a side stream: the binding's workspace is not reused before it has run")
    bs, hq, hkv, d, B = 16, 8, 4, 128, 8
    lens = [300 + 37 * i for i in range(B)]
    counts = [-(-n // bs) for n in lens]
    tables, at = [], 0
    for c in counts:
        tables.append(list(range(at, at + c)))
        at += c
    gen = torch.Generator().manual_seed(21)
    kc = torch.randn(at, bs, hkv, d, generator=gen).to(torch.bfloat16).cuda()
    vc = torch.randn(at, bs, hkv, d, generator=gen).to(torch.bfloat16).cuda()
    q = torch.randn(B, hq, d, generator=gen).to(torch.bfloat16).cuda()
    meta = pkv.pack_decode(lens, tables, bs, device="cuda")
    args = (q, kc, vc, meta["block_tables"], meta["context_lens"], max(lens), d ** -0.5)
    need = pkv.decode_workspace_bytes(B, max(lens), hq, hkv, d, bs, torch.bfloat16, 64)
    assert need > 0
    ref = pkv.decode_attention_paged(*args, partition_size=64)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    for trial in range(3):
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            torch.cuda._sleep(20_000_000)      # the side stream's decode runs a few ms late
        got = pkv.decode_attention_paged(*args, partition_size=64, stream=side)
        # the current stream allocates and overwrites memory of the workspace's size at once
        junk = [torch.empty(need, dtype=torch.uint8, device="cuda").fill_(255) for _ in range(4)]
        torch.cuda.synchronize()
        assert torch.equal(got, ref), f"trial {trial}: side-stream decode differs"
        say(f"  trial {trial}: side-stream decode identical to the current-stream one")
        del junk, got


@pytest.mark.parametrize("partition", [-1, 0, 64, 512],
                         ids=["balanced", "library-choice", "fixed-5-parts", "fixed-1-part"])
def test_decode_cuts_contexts_past_max_context_len(cuda, partition):
    say(f"[gpu] decode: context_lens past max_context_len are cut to it (partition {partition})")
    bs, hq, hkv, d = 64, 8, 4, 128
    ctx = [1000, 200, 300, 64]
    cap = 300
    counts = [-(-n // bs) for n in ctx]
    tables, at = [], 0
    for c in counts:
        tables.append(list(range(at, at + c)))
        at += c
    gen = torch.Generator().manual_seed(33)
    kc = torch.randn(at, bs, hkv, d, generator=gen).to(torch.bfloat16)
    vc = torch.randn(at, bs, hkv, d, generator=gen).to(torch.bfloat16)
    q = torch.randn(len(ctx), hq, d, generator=gen).to(torch.bfloat16)
    meta = pkv.pack_decode(ctx, tables, bs, device="cuda")
    scale = d ** -0.5
    want_part = pkv.decode_partition_size(len(ctx), cap, hq, hkv, d, bs, torch.bfloat16, partition)
    say(f"  plan: partition size {want_part} ({'balanced' if want_part == 0 else 'fixed'})")
    out = pkv.decode_attention_paged(q.cuda(), kc.cuda(), vc.cuda(), meta["block_tables"],
                                     meta["context_lens"], cap, scale, partition_size=partition)
    torch.cuda.synchronize()
    cut = [min(n, cap) for n in ctx]
    want = oracle.attention(q, [1] * len(ctx), cut, hkv, scale, k_cache=kc, v_cache=vc,
                            tables=tables, block_size=bs)
    err = max_abs_err(out, want)
    say(f"  max |err| against the oracle on the cut contexts = {err:.3e}")
    assert err <= 2e-2


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16-mfma", "f32-generic"])
@pytest.mark.parametrize("lk1", [5000, 50], ids=["keys-past-max_seqlen_k", "fewer-keys-than-queries"])
def test_prefill_skips_sequence_with_key_count_out_of_range(cuda, dtype, lk1):
    say(f"[gpu] prefill: a sequence claiming {lk1} keys for 100 queries (max_seqlen_k 100) is skipped")
    hq, hkv, d, bs = 8, 4, 128, 16
    n0 = 100
    gen = torch.Generator().manual_seed(13)
    q = torch.randn(2 * n0, hq, d, generator=gen).to(dtype)
    k = torch.randn(n0, hkv, d, generator=gen).to(dtype)
    v = torch.randn(n0, hkv, d, generator=gen).to(dtype)
    nb = -(-n0 // bs)
    kc = torch.zeros(2 * nb, bs, hkv, d, dtype=dtype)
    vc = torch.zeros(2 * nb, bs, hkv, d, dtype=dtype)
    kc.view(-1, hkv, d)[:n0] = k
    vc.view(-1, hkv, d)[:n0] = v
    tables = torch.stack([torch.arange(nb, dtype=torch.int32), torch.arange(nb, 2 * nb, dtype=torch.int32)])
    cu_q = torch.tensor([0, n0, 2 * n0], dtype=torch.int32, device="cuda")
    cu_k = torch.tensor([0, n0, n0 + lk1], dtype=torch.int32, device="cuda")
    sentinel = 7.0
    out = torch.full((2 * n0, hq, d), sentinel, dtype=dtype, device="cuda")
    scale = d ** -0.5
    pkv.prefill_attention_varlen(q.cuda(), cu_q, cu_k, n0, n0, scale, k_cache=kc.cuda(), v_cache=vc.cuda(),
                                 block_tables=tables.cuda(), out=out)
    torch.cuda.synchronize()
    want = oracle.attention(q[:n0], [n0], [n0], hkv, scale, k=k, v=v)
    err = max_abs_err(out[:n0], want)
    say(f"  sequence 0: max |err| = {err:.3e}")
    assert err <= (2e-2 if dtype == torch.bfloat16 else 1e-4)
    assert bool((out[n0:].float() == sentinel).all()), "rows of the skipped sequence were written"
