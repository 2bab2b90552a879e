"""Pins for the oracle: it is checked here against what the pages and the
mathematics fix, never against itself or the HIP path.

* worked slot examples from the pages (tests/golden/slot_examples.json);
* the decode slot rule and the prefill block walk, as the pages state them,
  against the oracle's per-token slot formula;
* the store as a bit copy that touches nothing else;
* closed forms of softmax attention (one key, equal scores, two keys);
* a dense formulation with an explicit -inf mask matrix through library
  routines (numpy matmul, scipy softmax) on tiny inputs, enumerated;
* invariants the method rests on: paged == contiguous, cached-prefix prefill ==
  full recompute, decode == last prefill row, GQA == repeated-head MHA, masked
  positions contribute exactly nothing, split-context LSE combine == unsplit.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import oracle
from workloads import custom_workload, make_workload

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def f64(x):
    """Exact upcast of a torch tensor (fp32 or bf16) to float64 numpy."""
    return x.detach().cpu().to(torch.float64).numpy()


def logical_kv(w):
    """Per-sequence contiguous K and V ([n, Hkv, d] float64) assembled from the
    generator's history and new rows, by plain indexing (no slots)."""
    hist_rows, at = {}, 0
    for (s, b, e) in w.hist:
        hist_rows[s] = (at, b, e, w.block_tables[s])
        at += e - b
    new_at, out = 0, []
    kh, vh, kn, vn = f64(w.k_hist), f64(w.v_hist), f64(w.k_new), f64(w.v_new)
    for s, (n, c) in enumerate(zip(w.seq_lens, w.num_cached)):
        parts_k, parts_v = [], []
        if c > 0:
            owner = s if s in hist_rows else None
            if owner is None:  # shares another sequence's prefix blocks
                nb = -(-c // w.block_size)
                for o, (_, _, _, t) in hist_rows.items():
                    if t[:nb] == w.block_tables[s][:nb]:
                        owner = o
                        break
            r0, b, e, _ = hist_rows[owner]
            assert b == 0 and e >= c
            parts_k.append(kh[r0:r0 + c])
            parts_v.append(vh[r0:r0 + c])
        parts_k.append(kn[new_at:new_at + n - c])
        parts_v.append(vn[new_at:new_at + n - c])
        new_at += n - c
        out.append((np.concatenate(parts_k), np.concatenate(parts_v)))
    return out


def dense_reference(w):
    """softmax(scale * Q K^T + M) V per sequence and head, M the explicit mask
    matrix (0 where key j <= the query's absolute position, -inf elsewhere),
    through numpy matmul and scipy's softmax."""
    kv = logical_kv(w)
    q = f64(w.q)
    g = w.num_q_heads // w.num_kv_heads
    out = np.zeros_like(q)
    at = 0
    for s, (n, c) in enumerate(zip(w.seq_lens, w.num_cached)):
        lq = n - c
        K, V = kv[s]
        pos = c + np.arange(lq)
        M = np.where(np.arange(n)[None, :] <= pos[:, None], 0.0, -np.inf)
        for h in range(w.num_q_heads):
            S = w.scale * (q[at:at + lq, h, :] @ K[:, h // g, :].T) + M
            out[at:at + lq, h, :] = scipy.special.softmax(S, axis=1) @ V[:, h // g, :]
        at += lq
    return out


# ---------------------------------------------------------------- slots

def test_slot_worked_examples():
    with open(os.path.join(GOLDEN, "slot_examples.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        for p, want in zip(c["positions"], c["slots"]):
            got = oracle.slot(c["block_table"], c["block_size"], p)
            assert got == (-1 if want is None else want), (c["source"][:40], p)


def test_slot_matches_decode_rule():
    # nano-vLLM-1, "5. deocde 输入打包" and the Sequence properties: the token at
    # position len-1 goes to table[-1] * bs + last_block_num_tokens - 1, where
    # num_blocks = ceil(len / bs), last_block_num_tokens = len - (num_blocks-1)*bs.
    rng = np.random.default_rng(3)
    for _ in range(500):
        bs = int(rng.choice([1, 2, 4, 16, 256]))
        n = int(rng.integers(1, 5000))
        nblk = -(-n // bs)
        table = [int(x) for x in rng.permutation(nblk + 7)[:nblk]]
        last_n = n - (nblk - 1) * bs
        assert oracle.slot(table, bs, n - 1) == table[-1] * bs + last_n - 1


def test_slots_match_prefill_block_walk():
    # nano-vLLM-1, "4. prefill 输入打包": the uncached tokens of a sequence fill
    # its blocks from the first uncached one onward, each block from its first
    # slot, the last block only up to the sequence's length. The cached part is
    # always whole blocks (allocate only advances num_cached_tokens by bs).
    rng = np.random.default_rng(4)
    for _ in range(300):
        bs = int(rng.choice([1, 4, 16, 256]))
        n = int(rng.integers(1, 3000))
        nblk = -(-n // bs)
        cached = int(rng.integers(0, nblk)) * bs
        table = [int(x) for x in rng.permutation(nblk + 5)[:nblk]]
        walk = []
        for i in range(cached // bs, nblk):
            fill = bs if i < nblk - 1 else n - (nblk - 1) * bs
            walk.append(table[i] * bs + np.arange(fill))
        walk = np.concatenate(walk)
        got = oracle.slots([(0, cached, n)], [table], bs)
        assert np.array_equal(got, walk)


def test_slots_decode_batch_order():
    # one slot per sequence, in batch order, each the sequence's newest position
    tables = [[3, 9], [4], [0, 1, 2]]
    lens = [20, 5, 33]
    got = oracle.slots([(s, n - 1, n) for s, n in enumerate(lens)], tables, 16)
    assert list(got) == [9 * 16 + 3, 4 * 16 + 4, 2 * 16 + 0]


# ---------------------------------------------------------------- store

@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_store_is_bit_copy_and_touches_nothing_else(dtype):
    rng = np.random.default_rng(5)
    nb, bs, H, d = 9, 4, 2, 8
    code = oracle.BF16 if dtype == torch.bfloat16 else oracle.F32
    pattern = (np.arange(nb * bs * H * d) % 251).astype(np.uint16 if code else np.float32)
    pool = pattern.reshape(nb, bs, H, d).copy()
    n = 13
    src = torch.randn(n, H, d).to(dtype)
    ids = rng.choice(nb * bs, size=n, replace=False).astype(np.int64)
    ids[[2, 7]] = -1  # padding rows: no write
    oracle.store(src, pool, ids)
    s, _ = oracle.as_storage(src)
    flat = pool.reshape(nb * bs, H, d)
    ref = pattern.reshape(nb * bs, H, d)
    written = set()
    for i in range(n):
        if ids[i] >= 0:
            assert flat[ids[i]].tobytes() == s[i].tobytes()
            written.add(int(ids[i]))
    for r in range(nb * bs):
        if r not in written:
            assert flat[r].tobytes() == ref[r].tobytes()


def test_store_rejects_out_of_pool_and_duplicate():
    pool = np.zeros((2, 2, 1, 4), dtype=np.float32)
    src = torch.ones(2, 1, 4)
    with pytest.raises(ValueError):
        oracle.store(src, pool, np.array([0, 4]))
    with pytest.raises(ValueError):
        oracle.store(src, pool, np.array([1, 1]))


# ---------------------------------------------------------------- closed forms

def _contig(q, k, v, q_lens, k_lens, hkv, scale):
    return oracle.attention(torch.tensor(q, dtype=torch.float32), q_lens, k_lens, hkv, scale,
                            k=torch.tensor(k, dtype=torch.float32),
                            v=torch.tensor(v, dtype=torch.float32))


def test_single_key_returns_its_value_exactly():
    rng = np.random.default_rng(6)
    q = rng.standard_normal((1, 1, 8)).astype(np.float32)
    k = rng.standard_normal((1, 1, 8)).astype(np.float32)
    v = rng.standard_normal((1, 1, 8)).astype(np.float32)
    out = _contig(q, k, v, [1], [1], 1, 0.3)
    assert np.array_equal(out[0, 0], v[0, 0].astype(np.float64))


def test_zero_query_averages_exactly_the_visible_values():
    # q = 0 gives equal scores, so each row is the mean of the values it can
    # see: keys 0..p for query position p (the diagonal included).
    rng = np.random.default_rng(7)
    L, d = 6, 4
    q = np.zeros((L, 1, d), np.float32)
    k = rng.standard_normal((L, 1, d)).astype(np.float32)
    v = rng.standard_normal((L, 1, d)).astype(np.float32)
    out = _contig(q, k, v, [L], [L], 1, 1.0)
    for p in range(L):
        np.testing.assert_allclose(out[p, 0], v[:p + 1, 0].astype(np.float64).mean(0),
                                   rtol=0, atol=1e-15)
    # prefix hit: 2 queries over 6 keys sit at positions 4 and 5
    out2 = _contig(q[:2], k, v, [2], [L], 1, 1.0)
    np.testing.assert_allclose(out2[0, 0], v[:5, 0].astype(np.float64).mean(0), atol=1e-15)
    np.testing.assert_allclose(out2[1, 0], v[:6, 0].astype(np.float64).mean(0), atol=1e-15)


@pytest.mark.parametrize("a", [-3.0, -0.5, 0.25, 2.0])
def test_two_keys_logistic_weights(a):
    # scores x0 = scale*a*1, x1 = scale*a*2 -> gap D = scale*a, and
    # o = (v0 + e^D v1) / (1 + e^D)
    scale = 0.75
    q = np.array([[[a, 0, 0, 0]]], np.float32)
    k = np.array([[[1, 0, 0, 0]], [[2, 0, 0, 0]]], np.float32)
    v = np.array([[[1, 2, 3, 4]], [[-5, 6, 0.5, 8]]], np.float32)
    out = _contig(q, k, v, [1], [2], 1, scale)
    D = scale * a
    v64 = v.astype(np.float64)
    want = (v64[0, 0] + math.exp(D) * v64[1, 0]) / (1 + math.exp(D))
    np.testing.assert_allclose(out[0, 0], want, rtol=0, atol=1e-14)


def test_scale_multiplies_the_scores():
    rng = np.random.default_rng(8)
    q = rng.standard_normal((5, 2, 8)).astype(np.float32)
    k = rng.standard_normal((5, 1, 8)).astype(np.float32)
    v = rng.standard_normal((5, 1, 8)).astype(np.float32)
    a = _contig(q, k, v, [5], [5], 1, 0.5)
    b = _contig(q * 0.5, k, v, [5], [5], 1, 1.0)   # exact: power-of-two scale
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-14)


def test_empty_context_row_is_zero():
    q = np.ones((1, 1, 4), np.float32)
    z = np.zeros((0, 1, 4), np.float32)
    out = oracle.attention(torch.tensor(q), [1], [0], 1, 1.0, k=torch.tensor(z), v=torch.tensor(z))
    assert np.array_equal(out, np.zeros((1, 1, 4)))


# ---------------------------------------------------------------- brute force

@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_brute_force_against_dense_library_softmax(dtype):
    cases = 0
    for lk, bs, g in itertools.product(range(1, 9), [1, 2, 4], [1, 2]):
        for lq in range(1, lk + 1):
            cached = lk - lq
            if cached % bs:          # cached prefixes are whole blocks
                continue
            w = custom_workload(phase="prefill", seq_lens=[lk, max(1, lk - 1)],
                                num_cached=[cached, 0], num_q_heads=2 * g, num_kv_heads=2,
                                head_dim=8, block_size=bs, dtype=dtype,
                                seed=lk * 100 + lq * 10 + bs + g, use_block_tables=True)
            got, *_ = oracle.run_workload(w)
            np.testing.assert_allclose(got, dense_reference(w), rtol=0, atol=1e-12)
            cases += 1
    assert cases > 50


# ---------------------------------------------------------------- invariants

def test_paged_equals_contiguous():
    w = custom_workload(phase="prefill", seq_lens=[37, 100, 5], num_cached=[0, 0, 0],
                        num_q_heads=4, num_kv_heads=2, head_dim=16, block_size=16,
                        dtype=torch.float32, seed=11, use_block_tables=True)
    paged, *_ = oracle.run_workload(w)
    w.use_block_tables = False
    contig, *_ = oracle.run_workload(w)
    np.testing.assert_allclose(paged, contig, rtol=0, atol=1e-12)


def test_prefix_prefill_equals_full_recompute():
    # the causal mask makes a token's K/V independent of later tokens, so a
    # prefill that reads a cached prefix through the block table gives the same
    # rows as recomputing the whole prompt.
    full = custom_workload(phase="prefill", seq_lens=[70, 48], num_cached=[0, 0],
                           num_q_heads=4, num_kv_heads=1, head_dim=16, block_size=16,
                           dtype=torch.bfloat16, seed=12, use_block_tables=False)
    ref, *_ = oracle.run_workload(full)
    part = custom_workload(phase="prefill", seq_lens=[70, 48], num_cached=[32, 16],
                           num_q_heads=4, num_kv_heads=1, head_dim=16, block_size=16,
                           dtype=torch.bfloat16, seed=12)
    # reuse the full run's values: prefix rows become history, the rest are new
    part.q = torch.cat([full.q[32:70], full.q[70 + 16:]])
    part.k_new = torch.cat([full.k_new[32:70], full.k_new[70 + 16:]])
    part.v_new = torch.cat([full.v_new[32:70], full.v_new[70 + 16:]])
    part.k_hist = torch.cat([full.k_new[0:32], full.k_new[70:70 + 16]])
    part.v_hist = torch.cat([full.v_new[0:32], full.v_new[70:70 + 16]])
    got, *_ = oracle.run_workload(part)
    want = np.concatenate([ref[32:70], ref[70 + 16:]])
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_decode_equals_last_prefill_row():
    w = custom_workload(phase="decode", seq_lens=[45, 17], num_cached=[44, 16],
                        num_q_heads=4, num_kv_heads=2, head_dim=16, block_size=8,
                        dtype=torch.float32, seed=13)
    dec, *_ = oracle.run_workload(w)
    kv = logical_kv(w)
    for s, n in enumerate(w.seq_lens):
        k, v = kv[s]
        q = torch.zeros(n, 4, 16)
        q[n - 1] = w.q[s]
        full = oracle.attention(q, [n], [n], 2, w.scale,
                                k=torch.tensor(k, dtype=torch.float32),
                                v=torch.tensor(v, dtype=torch.float32))
        np.testing.assert_allclose(dec[s], full[n - 1], rtol=0, atol=1e-12)


def test_mixed_batch_rows_equal_decode_and_full_recompute():
    # A chunked-prefill step mixes, in one varlen call, sequences with Lq = 1
    # (decode), Lq < Lk with a cache boundary inside a block (a prompt chunk)
    # and Lq = Lk (a fresh prompt). Bottom-right alignment makes each row the
    # row of the same position in a full recomputation of its sequence, and an
    # Lq = 1 row the decode result for that sequence.
    lens, cached = [45, 70, 30, 17], [44, 50, 0, 16]
    kw = dict(num_q_heads=4, num_kv_heads=2, head_dim=16, block_size=16,
              dtype=torch.float32, seed=21)
    mixed = custom_workload(phase="prefill", seq_lens=lens, num_cached=cached, **kw)
    got, *_ = oracle.run_workload(mixed)
    kv = logical_kv(mixed)
    qo = np.concatenate([[0], np.cumsum([n - c for n, c in zip(lens, cached)])])
    for s, (n, c) in enumerate(zip(lens, cached)):
        k, v = kv[s]
        q = torch.zeros(n, 4, 16)
        q[c:] = mixed.q[qo[s]:qo[s + 1]]
        full = oracle.attention(q, [n], [n], 2, mixed.scale,
                                k=torch.tensor(k, dtype=torch.float32),
                                v=torch.tensor(v, dtype=torch.float32))
        np.testing.assert_allclose(got[qo[s]:qo[s + 1]], full[c:], rtol=0, atol=1e-12)
    # the Lq = 1 rows against the decode phase on the same cache and queries
    dec = custom_workload(phase="decode", seq_lens=[45, 17], num_cached=[44, 16], **kw)
    dec_pre = custom_workload(phase="prefill", seq_lens=[45, 17], num_cached=[44, 16], **kw)
    a, *_ = oracle.run_workload(dec)
    b, *_ = oracle.run_workload(dec_pre)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)


def test_gqa_equals_mha_with_repeated_kv_heads():
    w = custom_workload(phase="prefill", seq_lens=[23, 9], num_cached=[0, 0], num_q_heads=6,
                        num_kv_heads=2, head_dim=8, block_size=4, dtype=torch.float32, seed=14,
                        use_block_tables=False)
    gqa, *_ = oracle.run_workload(w)
    k = w.k_new.repeat_interleave(3, dim=1)
    v = w.v_new.repeat_interleave(3, dim=1)
    mha = oracle.attention(w.q, w.q_lens, w.seq_lens, 6, w.scale, k=k, v=v)
    np.testing.assert_allclose(gqa, mha, rtol=0, atol=1e-13)


def test_masked_positions_contribute_exactly_nothing():
    # contiguous: change every key/value after the last query's position of a
    # shorter view; paged: the pool outside written slots is NaN and results
    # stay finite and bit-identical when that garbage changes.
    w = custom_workload(phase="decode", seq_lens=[30, 7], num_cached=[29, 6], num_q_heads=2,
                        num_kv_heads=1, head_dim=8, block_size=16, dtype=torch.bfloat16,
                        seed=15)
    a, kp, vp, _ = oracle.run_workload(w)
    assert np.isfinite(a).all()
    # overwrite the NaN garbage with huge values and re-attend
    kp2 = kp.copy()
    vp2 = vp.copy()
    kp2[kp2 == 0x7FC0] = 0x7F00   # bf16 ~1.7e38
    vp2[vp2 == 0x7FC0] = 0xFF00
    b = oracle.attention(w.q, w.q_lens, w.seq_lens, 1, w.scale, k_cache=kp2, v_cache=vp2,
                         tables=w.block_tables, block_size=w.block_size)
    assert np.array_equal(a, b)


def test_split_context_lse_combine_equals_unsplit():
    # Flash-decoding: split the keys into parts; each part yields an
    # unnormalised sum acc_p, its max m_p and its weight sum l_p; with
    # M = max m_p the result is sum e^(m_p-M) acc_p / sum e^(m_p-M) l_p.
    rng = np.random.default_rng(16)
    n, d = 97, 16
    q = rng.standard_normal((1, 1, d)).astype(np.float32)
    k = rng.standard_normal((n, 1, d)).astype(np.float32)
    v = rng.standard_normal((n, 1, d)).astype(np.float32)
    scale = 1 / 4
    want = _contig(q, k, v, [1], [n], 1, scale)[0, 0]
    cuts = np.sort(rng.choice(np.arange(1, n), size=5, replace=False))
    bounds = [0, *cuts.tolist(), n]
    accs, ms, ls = [], [], []
    for b, e in zip(bounds[:-1], bounds[1:]):
        x = scale * (k[b:e, 0].astype(np.float64) @ q[0, 0].astype(np.float64))
        m = x.max()
        w_ = np.exp(x - m)
        accs.append(w_ @ v[b:e, 0].astype(np.float64))
        ms.append(m)
        ls.append(w_.sum())
    M = max(ms)
    num = sum(math.exp(m - M) * a for m, a in zip(ms, accs))
    den = sum(math.exp(m - M) * l for m, l in zip(ms, ls))
    np.testing.assert_allclose(num / den, want, rtol=0, atol=1e-12)


# ---------------------------------------------------------------- workloads

def test_presets_shapes():
    w1p = make_workload(1, "prefill", values=False)
    w1d = make_workload(1, "decode", values=False)
    assert w1p.seq_lens == [37, 100] and w1d.seq_lens == [38, 101]
    assert sorted(sum(w1p.block_tables, [])) == sorted(set(sum(w1p.block_tables, [])))
    w2 = make_workload(2, values=False)
    assert len(w2.seq_lens) == 64 and min(w2.seq_lens) >= 512 and max(w2.seq_lens) <= 4096
    assert w2.num_blocks == 2048
    w3 = make_workload(3, values=False)
    assert sum(w3.seq_lens) <= 16384 and len(w3.seq_lens) == 16
    assert all(128 <= n <= 2048 for n in w3.seq_lens)
    w4 = make_workload(4, values=False)
    assert w4.total_q == 16 * 1024 + 16 * 2048
    shared = {tuple(t[:4]) for s, t in enumerate(w4.block_tables) if s % 2 == 0}
    assert len(shared) == 1
    w5 = make_workload(5, values=False)
    assert len(w5.seq_lens) == 512 and min(w5.seq_lens) >= 256 and max(w5.seq_lens) <= 32768
    used = sum(w5.block_tables, [])
    assert len(used) == w5.num_blocks == len(set(used))
    w6 = make_workload(6, values=False)
    assert w6.phase == "prefill" and w6.seq_lens == w2.seq_lens and w6.block_tables == w2.block_tables
    assert w6.total_q == 64 and all(n - c == 1 for n, c in zip(w6.seq_lens, w6.num_cached))
    w7 = make_workload(7, values=False)
    assert w7.total_q == 64 + 2 * 512 and w7.num_cached[-2:] == [1536, 1536]
    used = sum(w7.block_tables, [])
    assert len(used) == len(set(used)) and max(used) < w7.num_blocks


def test_bf16_rounding_is_round_to_nearest_even():
    x = torch.randn(4096)
    u = x.view(torch.int32).numpy().astype(np.int64) & 0xFFFFFFFF
    want = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    got = x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, want)


# ---------------------------------------------------------------- rotary embedding
# The pages feed positions to RoPE without fixing its form; the oracle follows
# RoFormer (Su et al., 2021). Pinned by closed forms (worked angles, position
# zero), the rotation's invariants (pair norms, relative-position dot
# products) and numpy's complex exponential.

def _rand_heads(T, H, d, seed):
    return np.random.default_rng(seed).standard_normal((T, H, d)).astype(np.float32)


@pytest.mark.parametrize("style", [0, 1])
def test_rope_worked_angles(style):
    # base 10000, rot_dim 4: pair 0 turns by p rad, pair 1 by p / 100 rad
    x = np.zeros((2, 1, 6), dtype=np.float32)
    x[:, 0, 0] = 1.0                      # first element of pair 0
    x[:, 0, 5] = 3.0                      # past rot_dim: untouched
    got = oracle.rope(x, [1, 50], 4, 10000.0, style)
    b0 = 2 if style == 0 else 1           # partner of element 0
    for t, p in enumerate([1, 50]):
        want = np.zeros(6)
        want[0], want[b0], want[5] = math.cos(p), math.sin(p), 3.0
        np.testing.assert_allclose(got[t, 0], want, rtol=0, atol=1e-15)
    y = np.zeros((1, 1, 4), dtype=np.float32)
    y[0, 0, 1] = 1.0                      # first element of pair 1 (style 0) / second of pair 0 (style 1)
    got = oracle.rope(y, [100], 4, 10000.0, style)[0, 0]
    if style == 0:
        np.testing.assert_allclose(got, [0, math.cos(1.0), 0, math.sin(1.0)], rtol=0, atol=1e-15)
    else:
        np.testing.assert_allclose(got, [-math.sin(100.0), math.cos(100.0), 0, 0], rtol=0, atol=1e-15)


@pytest.mark.parametrize("style", [0, 1])
def test_rope_position_zero_is_identity_and_pairs_keep_their_norm(style):
    x = _rand_heads(5, 3, 64, 31)
    np.testing.assert_array_equal(oracle.rope(x, [0] * 5, 64, 1e6, style), x.astype(np.float64))
    pos = [1, 7, 300, 4095, 32767]
    got = oracle.rope(x, pos, 48, 1e6, style)
    xf = x.astype(np.float64)
    idx = (np.arange(24), np.arange(24) + 24) if style == 0 else (np.arange(0, 48, 2), np.arange(1, 48, 2))
    n_in = xf[..., idx[0]] ** 2 + xf[..., idx[1]] ** 2
    n_out = got[..., idx[0]] ** 2 + got[..., idx[1]] ** 2
    np.testing.assert_allclose(n_out, n_in, rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(got[..., 48:], xf[..., 48:])


@pytest.mark.parametrize("style", [0, 1])
def test_rope_dot_products_depend_only_on_relative_position(style):
    q, k = _rand_heads(1, 2, 32, 32), _rand_heads(1, 2, 32, 33)
    def dots(pq, pk):
        a = oracle.rope(q, [pq], 32, 500.0, style)
        b = oracle.rope(k, [pk], 32, 500.0, style)
        return (a * b).sum(-1)
    ref = dots(10, 3)
    for shift in (1, 17, 1000):
        np.testing.assert_allclose(dots(10 + shift, 3 + shift), ref, rtol=1e-9, atol=1e-9)
    assert np.abs(dots(11, 3) - ref).max() > 1e-3   # and they do depend on it


@pytest.mark.parametrize("style", [0, 1])
def test_rope_equals_complex_multiplication(style):
    x = _rand_heads(4, 2, 16, 34)
    pos = np.array([0, 3, 1000, 77])
    got = oracle.rope(x, pos, 16, 10000.0, style)
    xf = x.astype(np.float64)
    a, b = (xf[..., :8], xf[..., 8:]) if style == 0 else (xf[..., 0::2], xf[..., 1::2])
    freq = np.power(10000.0, -np.arange(8) * 2.0 / 16)
    z = (a + 1j * b) * np.exp(1j * pos[:, None, None] * freq)
    ga, gb = (got[..., :8], got[..., 8:]) if style == 0 else (got[..., 0::2], got[..., 1::2])
    np.testing.assert_allclose(ga, z.real, rtol=0, atol=1e-12)
    np.testing.assert_allclose(gb, z.imag, rtol=0, atol=1e-12)
