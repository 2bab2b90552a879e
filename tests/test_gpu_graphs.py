"""Decode steps captured as HIP graphs (paged_kv_cache_125_amd.graphs) against
the same steps run eagerly and against the oracle: several batch sizes per
bucket (padding rows: slot -1, context 0), two layers, and repeated replays
with eager work and synchronizations between them, every replay checked."""
import copy

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_125_amd as pkv
from gpu_helpers import max_abs_err, raw, say
from paged_kv_cache_125_amd.graphs import DecodeGraphs, bucket_for
from paged_kv_cache_125_amd.step import alloc_pool, write_ranges
from workloads import custom_workload

pytestmark = pytest.mark.gpu

HQ, HKV, D, BS = 16, 8, 128, 256


@pytest.fixture(scope="module")
def setup():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    pkv.lib()
    rng = np.random.default_rng(91)
    B = 40
    lens = [int(x) for x in rng.integers(1, 3000, B)]
    # two layers sharing lengths and block tables; the second layer's values
    # are the first's with K and V swapped and q negated
    w0 = custom_workload(phase="decode", seq_lens=lens, num_cached=[n - 1 for n in lens],
                         num_q_heads=HQ, num_kv_heads=HKV, head_dim=D, block_size=BS, seed=500)
    w1 = copy.copy(w0)
    w1.q, w1.k_new, w1.v_new = -w0.q, w0.v_new, w0.k_new
    w1.k_hist, w1.v_hist = w0.v_hist, w0.k_hist
    ws = [w0, w1]
    tables = w0.block_tables
    layers = []
    for w in ws:
        kc, vc = alloc_pool(w.num_blocks, BS, HKV, D, torch.bfloat16, "cuda")
        write_ranges(w.hist, tables, BS, w.k_hist.cuda(), w.v_hist.cuda(), kc, vc)
        layers.append((kc, vc))
    maxb = max(len(t) for t in tables)
    graphs = DecodeGraphs(layers, HQ, max_context_len=4096, max_blocks_per_seq=maxb + 2,
                          scale=ws[0].scale, buckets=[1, 8, 16, 48])
    return ws, layers, graphs


def _batch(ws, rows):
    """Inputs of a decode step over the sequences ``rows`` of the workloads."""
    w0 = ws[0]
    lens = [w0.seq_lens[r] for r in rows]
    tables = [w0.block_tables[r] for r in rows]
    meta = pkv.pack_decode(lens, tables, BS, device="cuda")
    q = [w.q[rows].cuda() for w in ws]
    k = [w.k_new[rows].cuda() for w in ws]
    v = [w.v_new[rows].cuda() for w in ws]
    return q, k, v, meta


def _want(ws, rows):
    from gpu_helpers import subset
    outs = []
    for w in ws:
        sub = subset(w, rows)
        o, *_ = oracle.run_workload(sub)
        outs.append(o)
    return outs


@pytest.mark.parametrize("rows", [[3], [0, 5, 7], list(range(8)), list(range(9)), list(range(40))],
                         ids=lambda r: f"B{len(r)}")
def test_graph_step_matches_eager_and_oracle(setup, rows):
    ws, layers, graphs = setup
    b = bucket_for(len(rows), graphs.buckets)
    say(f"[gpu] graph decode, batch {len(rows)} in bucket {b}")
    q, k, v, meta = _batch(ws, rows)
    got = [o.clone() for o in graphs.run(q, k, v, meta["slot_mapping"], meta["context_lens"],
                                           meta["block_tables"])]
    torch.cuda.synchronize()
    pools_g = [(raw(kc).copy(), raw(vc).copy()) for kc, vc in layers]
    eager = graphs.run_eager(q, k, v, meta["slot_mapping"], meta["context_lens"], meta["block_tables"],
                             max_context_len=meta["max_seqlen_k"])
    torch.cuda.synchronize()
    for (kc, vc), (kg, vg) in zip(layers, pools_g):     # the store is idempotent
        assert np.array_equal(raw(kc), kg) and np.array_equal(raw(vc), vg)
    want = _want(ws, rows)
    for l in range(len(layers)):
        e_g, e_o = max_abs_err(got[l], want[l]), (got[l].float() - eager[l].float()).abs().max().item()
        say(f"  layer {l}: graph vs oracle {e_g:.3e}, graph vs eager {e_o:.3e}")
        assert e_g <= 2e-2 and e_o <= 2e-2
    # padding rows of the bucket hold zeros
    if b > len(rows):
        assert graphs.out[:, len(rows):b].abs().max().item() == 0.0


def test_repeated_replays_with_eager_work_between(setup):
    ws, layers, graphs = setup
    say("[gpu] one captured bucket replayed 4 times, eager steps and syncs in between")
    rows_a, rows_b = list(range(10, 25)), list(range(20, 36))    # both in bucket 16
    qa, ka, va, ma = _batch(ws, rows_a)
    qb, kb, vb, mb = _batch(ws, rows_b)
    ref_a = [o.clone() for o in graphs.run_eager(qa, ka, va, ma["slot_mapping"], ma["context_lens"],
                                                  ma["block_tables"], ma["max_seqlen_k"])]
    ref_b = [o.clone() for o in graphs.run_eager(qb, kb, vb, mb["slot_mapping"], mb["context_lens"],
                                                  mb["block_tables"], mb["max_seqlen_k"])]
    torch.cuda.synchronize()
    for it in range(4):
        rows, (q, k, v, m), ref = ((rows_a, (qa, ka, va, ma), ref_a) if it % 2 == 0
                                   else (rows_b, (qb, kb, vb, mb), ref_b))
        got = graphs.run(q, k, v, m["slot_mapping"], m["context_lens"], m["block_tables"])
        torch.cuda.synchronize()
        for l in range(len(layers)):
            d = (got[l].float() - ref[l].float()).abs().max().item()
            say(f"  replay {it} layer {l}: max |graph - eager| = {d:.3e}")
            assert d <= 2e-2
        # eager work between replays
        graphs.run_eager(q, k, v, m["slot_mapping"], m["context_lens"], m["block_tables"],
                         m["max_seqlen_k"])
        torch.cuda.synchronize()

