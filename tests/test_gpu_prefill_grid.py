"""GPU tests of the prefill grids. The persistent grid (a fixed set of
workgroups claiming items from counters in the caller's workspace) against
the oracle and against the one-workgroup-per-item grid; the workspace left
zeroed after every call, so it is reused without clearing; batches past
the persistent grid's table limits, which take the fixed grid; and the
hardware's workgroup-to-XCD placement both grids' orders assume."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_125_amd as pkv
from gpu_helpers import gpu_run, max_abs_err, say, to_device
from paged_kv_cache_125_amd.step import alloc_pool, step_inputs_of, write_ranges
from workloads import custom_workload, make_workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def cuda():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    pkv.lib()
    return torch.device("cuda")


def _prefill(w, kc, vc, meta, **kw):
    if meta["block_tables"] is not None:
        return pkv.prefill_attention_varlen(w.q, meta["cu_seqlens_q"], meta["cu_seqlens_k"],
                                            meta["max_seqlen_q"], meta["max_seqlen_k"], w.scale,
                                            k_cache=kc, v_cache=vc, block_tables=meta["block_tables"], **kw)
    return pkv.prefill_attention_varlen(w.q, meta["cu_seqlens_q"], meta["cu_seqlens_k"],
                                        meta["max_seqlen_q"], meta["max_seqlen_k"], w.scale,
                                        k=w.k_new, v=w.v_new, **kw)


def _setup(w):
    kc, vc = alloc_pool(w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim, w.dtype, "cuda")
    write_ranges(w.hist, w.block_tables, w.block_size, w.k_hist, w.v_hist, kc, vc)
    meta = pkv.pack_prefill(w.seq_lens, w.num_cached, w.block_tables, w.block_size, device="cuda")
    pkv.store_kvcache(w.k_new, w.v_new, kc, vc, meta["slot_mapping"])
    return kc, vc, meta


@pytest.mark.parametrize("preset", [3, 4, 7])
def test_persistent_grid_matches_fixed_grid_and_resets_its_workspace(cuda, preset):
    say(f"[gpu] preset {preset}: persistent grid vs one workgroup per item, workspace reuse")
    w = to_device(make_workload(preset), "cuda")
    kc, vc, meta = _setup(w)
    ws = torch.zeros(pkv.lib().pkv_prefill_workspace_bytes(0, 0, 0, 0, 0, 0), dtype=torch.uint8, device="cuda")
    ref = _prefill(w, kc, vc, meta)
    for call in range(3):   # the same workspace, never cleared by the caller
        got = _prefill(w, kc, vc, meta, workspace=ws)
        torch.cuda.synchronize()
        assert bool((ws == 0).all()), f"call {call}: workspace not reset"
        assert torch.equal(got, ref), f"call {call}: persistent grid differs from the fixed grid"
    say("  3 calls on one workspace: bit-identical to the fixed grid, workspace zero after each")


def test_persistent_grid_against_the_oracle_on_ragged_shapes(cuda):
    rng = np.random.default_rng(77)
    ws = torch.zeros(pkv.prefill_workspace_bytes(), dtype=torch.uint8, device="cuda")
    for trial in range(4):
        S = int(rng.integers(1, 24))
        lens = [int(rng.integers(1, 700)) for _ in range(S)]
        cached = [int(rng.integers(0, n // 64 + 1)) * 64 if trial % 2 else 0 for n in lens]
        cached = [min(c, n - 1) if c else 0 for c, n in zip(cached, lens)]
        hq, hkv = [(16, 8), (8, 8), (32, 8), (12, 4)][trial]
        w = custom_workload(phase="prefill", seq_lens=lens, num_cached=cached, num_q_heads=hq,
                            num_kv_heads=hkv, head_dim=128, block_size=64, seed=900 + trial)
        say(f"[gpu] persistent grid trial {trial}: {S} seqs, Hq {hq}/Hkv {hkv}, cached {sum(cached)}")
        wd = to_device(w, "cuda")
        kc, vc, meta = _setup(wd)
        got = _prefill(wd, kc, vc, meta, workspace=ws)
        fixed = _prefill(wd, kc, vc, meta)
        torch.cuda.synchronize()
        want, *_ = oracle.run_workload(w)
        err = max_abs_err(got, want)
        say(f"  max |err| = {err:.3e}")
        assert err <= 2e-2
        assert torch.equal(got, fixed) and bool((ws == 0).all())


def test_batch_past_the_table_limit_takes_the_fixed_grid(cuda):
    # 300 sequences x 8 kv heads = 2400 (sequence, kv head) pairs: more than the
    # persistent grid's 256 per XCD, so the fixed grid runs and the workspace
    # is not touched
    rng = np.random.default_rng(5)
    lens = [int(x) for x in rng.integers(1, 40, size=300)]
    w = custom_workload(phase="prefill", seq_lens=lens, num_cached=[0] * 300, num_q_heads=16,
                        num_kv_heads=8, head_dim=128, block_size=16, seed=31)
    say(f"[gpu] 300 sequences ({sum(lens)} tokens): fixed-grid fallback")
    wd = to_device(w, "cuda")
    kc, vc, meta = _setup(wd)
    ws = torch.zeros(pkv.prefill_workspace_bytes(), dtype=torch.uint8, device="cuda")
    got = _prefill(wd, kc, vc, meta, workspace=ws)
    torch.cuda.synchronize()
    want, *_ = oracle.run_workload(w)
    err = max_abs_err(got, want)
    say(f"  max |err| = {err:.3e}")
    assert err <= 2e-2 and bool((ws == 0).all())


@pytest.mark.parametrize("n", [512, 1000, 4096])
def test_workgroups_land_on_xcd_blockidx_mod_8(cuda, n):
    # The grid order of both prefill grids puts a (sequence, kv head) pair's
    # items on one XCD by assuming the hardware deals a launch's workgroups to
    # the 8 XCDs round robin, so that workgroups with equal b % 8 share an XCD
    # and its L2. The first workgroup's XCD carries over from earlier launches
    # (the rotation does not restart at 0), so the check is that the XCD of
    # workgroup b is (b + s) % 8 for one s. libpkv_probe reads each
    # workgroup's XCC_ID register.
    import ctypes
    from paged_kv_cache_125_amd.build import PROBE_LIB
    lib = ctypes.CDLL(PROBE_LIB)
    lib.pkv_probe_xcc.restype = ctypes.c_int
    lib.pkv_probe_xcc.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p]
    say(f"[gpu] XCD of each of {n} workgroups")
    out = torch.full((n,), -1, dtype=torch.int32, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    assert lib.pkv_probe_xcc(ctypes.c_void_p(out.data_ptr()), n, stream) == 0
    got = out.cpu().numpy()
    assert ((got >= 0) & (got < 8)).all(), got[:32]
    shift = (got - np.arange(n)) % 8
    assert (shift == shift[0]).all(), got[:32]
    say(f"  workgroup b on XCD (b + {int(shift[0])}) % 8")
