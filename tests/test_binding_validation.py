"""CPU tests of the binding's tensor checks: a call whose tensors disagree in
dtype, shape, layout or device raises ValueError before any C call, so no
kernel is ever launched with row sizes that do not match its buffers. The
tensors here live on the CPU; every check on dtype, shape and layout runs
before the device check, and the device check itself is what a well-formed
call on the CPU trips."""
import pytest
import torch

import paged_kv_cache_125_amd as pkv

BF, F32, I32 = torch.bfloat16, torch.float32, torch.int32


def _decode_args(dt=BF):
    B, hq, hkv, d, nb, bs = 3, 8, 2, 128, 6, 16
    return dict(
        q=torch.zeros(B, hq, d, dtype=dt),
        k_cache=torch.zeros(nb, bs, hkv, d, dtype=dt),
        v_cache=torch.zeros(nb, bs, hkv, d, dtype=dt),
        block_tables=torch.zeros(B, 2, dtype=I32),
        context_lens=torch.ones(B, dtype=I32),
    )


def _decode(a, **kw):
    return pkv.decode_attention_paged(a["q"], a["k_cache"], a["v_cache"], a["block_tables"],
                                      a["context_lens"], 32, 0.1, **kw)


@pytest.mark.parametrize("change, msg", [
    (lambda a: a.update(q=a["q"].float()), "dtype"),                       # fp32 q, bf16 pool
    (lambda a: a.update(v_cache=a["v_cache"][:, :8]), "shape"),            # pools differ
    (lambda a: a.update(k_cache=torch.zeros(6, 16, 2, 256, dtype=BF)[..., ::2]), "contiguous"),
    (lambda a: a.update(block_tables=a["block_tables"].long()), "int32"),
    (lambda a: a.update(context_lens=a["context_lens"][:2]), "entries"),   # fewer than B
    (lambda a: a.update(block_tables=a["block_tables"][:2]), "rows"),
    (lambda a: a.update(q=a["q"][..., :64]), "head_dim"),                  # q d != cache d
    (lambda a: a.update(q=torch.zeros(3, 128, 8, dtype=BF).transpose(1, 2)), "contiguous rows"),
])
def test_decode_rejects_disagreeing_tensors(change, msg):
    a = _decode_args()
    change(a)
    with pytest.raises(ValueError, match=msg):
        _decode(a)


def test_decode_rejects_bad_out_and_workspace():
    a = _decode_args()
    with pytest.raises(ValueError, match="out dtype"):
        _decode(a, out=torch.empty(3, 8, 128, dtype=F32))
    with pytest.raises(ValueError, match="out has shape"):
        _decode(a, out=torch.empty(3, 8, 64, dtype=BF))
    with pytest.raises(ValueError, match="contiguous"):
        _decode(a, out=torch.empty(8, 3, 128, dtype=BF).transpose(0, 1))
    with pytest.raises(ValueError, match="workspace"):
        _decode(a, workspace=torch.empty(64, dtype=torch.int32))


def test_decode_well_formed_call_stops_at_the_device_check():
    with pytest.raises(ValueError, match="GPU"):
        _decode(_decode_args())


def _prefill_args(paged, dt=BF):
    T, hq, hkv, d = 40, 4, 2, 128
    a = dict(q=torch.zeros(T, hq, d, dtype=dt),
             cu_seqlens_q=torch.tensor([0, 15, 40], dtype=I32),
             cu_seqlens_k=torch.tensor([0, 15, 40], dtype=I32))
    if paged:
        a.update(k_cache=torch.zeros(5, 16, hkv, d, dtype=dt), v_cache=torch.zeros(5, 16, hkv, d, dtype=dt),
                 block_tables=torch.zeros(2, 3, dtype=I32))
    else:
        a.update(k=torch.zeros(T, hkv, d, dtype=dt), v=torch.zeros(T, hkv, d, dtype=dt))
    return a


def _prefill(a, **kw):
    a = dict(a)
    q, cq, ck = a.pop("q"), a.pop("cu_seqlens_q"), a.pop("cu_seqlens_k")
    return pkv.prefill_attention_varlen(q, cq, ck, 25, 25, 0.1, **a, **kw)


@pytest.mark.parametrize("paged, change, msg", [
    (False, lambda a: a.update(k=a["k"].float(), v=a["v"].float()), "dtype"),
    (False, lambda a: a.update(k=a["k"][:30], v=a["v"][:30]), "rows"),       # fewer rows than q
    (False, lambda a: a.update(v=torch.zeros(40, 2, 64, dtype=BF)), "shape"),
    (False, lambda a: a.update(cu_seqlens_q=a["cu_seqlens_q"].long()), "int32"),
    (False, lambda a: a.update(cu_seqlens_k=torch.tensor([0, 40], dtype=I32)), "one entry"),
    (True, lambda a: a.update(k_cache=a["k_cache"].float()), "dtype"),
    (True, lambda a: a.update(block_tables=a["block_tables"][:1]), "rows"),
    (True, lambda a: a.update(block_tables=a["block_tables"].long()), "int32"),
    (True, lambda a: a.update(v_cache=torch.zeros(5, 16, 2, 64, dtype=BF)), "shape"),
])
def test_prefill_rejects_disagreeing_tensors(paged, change, msg):
    a = _prefill_args(paged)
    change(a)
    with pytest.raises(ValueError, match=msg):
        _prefill(a)


def test_prefill_rejects_bad_out_and_stops_at_the_device_check():
    a = _prefill_args(False)
    with pytest.raises(ValueError, match="out dtype"):
        _prefill(a, out=torch.empty(40, 4, 128, dtype=F32))
    with pytest.raises(ValueError, match="out has shape"):
        _prefill(a, out=torch.empty(39, 4, 128, dtype=BF))
    with pytest.raises(ValueError, match="GPU"):
        _prefill(a)
    with pytest.raises(ValueError, match="GPU"):
        _prefill(_prefill_args(True))


def _fused_args():
    T, hq, hkv, d = 40, 4, 2, 128
    return dict(q=torch.zeros(T, hq, d, dtype=BF), k=torch.zeros(T, hkv, d, dtype=BF),
                v=torch.zeros(T, hkv, d, dtype=BF), k_cache=torch.zeros(5, 16, hkv, d, dtype=BF),
                v_cache=torch.zeros(5, 16, hkv, d, dtype=BF), slot_mapping=torch.arange(T, dtype=I32),
                cu_seqlens_q=torch.tensor([0, 15, 40], dtype=I32),
                cu_seqlens_k=torch.tensor([0, 15, 40], dtype=I32))


@pytest.mark.parametrize("change, msg", [
    (lambda a: a.update(k=a["k"].float(), v=a["v"].float()), "dtype"),    # fp32 rows, bf16 q and pool
    (lambda a: a.update(k_cache=a["k_cache"].float()), "dtype"),
    (lambda a: a.update(v=a["v"][:30]), "rows"),                          # fewer rows than q
    (lambda a: a.update(slot_mapping=a["slot_mapping"][:39]), "entries"),  # a slot short
    (lambda a: a.update(slot_mapping=a["slot_mapping"].long()), "int32"),
    (lambda a: a.update(cu_seqlens_q=a["cu_seqlens_q"].long()), "int32"),
    (lambda a: a.update(cu_seqlens_k=torch.tensor([0, 40], dtype=I32)), "one entry"),
    (lambda a: a.update(block_tables=torch.zeros(1, 3, dtype=I32)), "rows"),    # fewer rows than sequences
    (lambda a: a.update(block_tables=torch.zeros(2, 3, dtype=torch.int64)), "int32"),
    (lambda a: a.update(v_cache=torch.zeros(5, 16, 2, 64, dtype=BF)), "shape"),
    (lambda a: a.update(k_cache=torch.zeros(5, 16, 2, 64, dtype=BF),
                        v_cache=torch.zeros(5, 16, 2, 64, dtype=BF)), "head_dim"),
])
def test_fused_store_prefill_rejects_disagreeing_tensors(change, msg):
    a = _fused_args()
    change(a)
    with pytest.raises(ValueError, match=msg):
        pkv.prefill_store_attention_varlen(max_seqlen_q=25, max_seqlen_k=25, scale=0.1, **a)
    with pytest.raises(ValueError, match="GPU"):
        pkv.prefill_store_attention_varlen(max_seqlen_q=25, max_seqlen_k=25, scale=0.1, **_fused_args())
    with pytest.raises(ValueError, match="GPU"):
        pkv.prefill_store_attention_varlen(max_seqlen_q=25, max_seqlen_k=25, scale=0.1,
                                           block_tables=torch.zeros(2, 3, dtype=I32), **_fused_args())


def _store_args():
    N, hkv, d = 7, 2, 128
    return dict(k=torch.zeros(N, hkv, d, dtype=BF), v=torch.zeros(N, hkv, d, dtype=BF),
                k_cache=torch.zeros(4, 16, hkv, d, dtype=BF), v_cache=torch.zeros(4, 16, hkv, d, dtype=BF),
                slot_mapping=torch.arange(N, dtype=I32))


@pytest.mark.parametrize("change, msg", [
    (lambda a: a.update(k=a["k"].float()), "dtype"),                 # fp32 rows into a bf16 pool
    (lambda a: a.update(v=a["v"][:5]), "rows"),                      # fewer rows than slots
    (lambda a: a.update(k=torch.zeros(7, 4, 128, dtype=BF)), "shape"),
    (lambda a: a.update(slot_mapping=a["slot_mapping"].long()), "int32"),
    (lambda a: a.update(v_cache=a["v_cache"].float()), "dtype"),
])
def test_store_rejects_disagreeing_tensors(change, msg):
    a = _store_args()
    change(a)
    with pytest.raises(ValueError, match=msg):
        pkv.store_kvcache(**a)
    with pytest.raises(ValueError, match="GPU"):
        pkv.store_kvcache(**_store_args())


def test_rope_store_rejects_disagreeing_tensors():
    a = _store_args()
    q = torch.zeros(7, 4, 128, dtype=BF)
    pos = torch.arange(7, dtype=I32)
    cs = torch.zeros(64, 128, dtype=F32)
    with pytest.raises(ValueError, match="dtype"):
        pkv.rope_store_kvcache(q.float(), a["k"], a["v"], a["k_cache"], a["v_cache"],
                               a["slot_mapping"], pos, cs)
    with pytest.raises(ValueError, match="positions"):
        pkv.rope_store_kvcache(q, a["k"], a["v"], a["k_cache"], a["v_cache"],
                               a["slot_mapping"], pos[:3], cs)
    with pytest.raises(ValueError, match="one row per token"):
        pkv.rope_store_kvcache(q, torch.zeros(9, 2, 128, dtype=BF), a["v"], a["k_cache"],
                               a["v_cache"], a["slot_mapping"], pos, cs)
    with pytest.raises(ValueError, match="GPU"):
        pkv.rope_store_kvcache(q, a["k"], a["v"], a["k_cache"], a["v_cache"],
                               a["slot_mapping"], pos, cs)
