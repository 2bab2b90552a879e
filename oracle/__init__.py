"""The oracle -- TEST INFRASTRUCTURE ONLY.

A plain CPU implementation (``oracle.c``, fp64, OpenMP) of what the paged-KV
attention path computes: the slot of a token, the bit-copy cache write, and
causal attention with explicit block-table gathers. Only ``tests/``, the smoke
check in ``__graft_entry__`` and the cpu_baseline leg of ``bench.py`` may import
it. It shares no code with the HIP library and never imports it.

Every function here is pinned by ``tests/test_oracle_pins.py`` against facts
the pages and mathematics fix (worked examples, closed forms, invariants, a
library softmax on tiny inputs).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import List, Optional, Sequence, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

F32, BF16 = 0, 1


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc (-O2 -fopenmp). Building the checker is not
    using it."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                               _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def lib():
    global _lib
    if _lib is None:
        path = os.environ.get("PKV_ORACLE_LIB")  # a mutated build, for the mutation test
        if not path:
            path = _LIB_PATH
            if not os.path.exists(path):
                build(force=True)
        L = ctypes.CDLL(path)
        P = ctypes.c_void_p
        i32, i64, dbl = ctypes.c_int32, ctypes.c_int64, ctypes.c_double
        L.orc_slot.restype = i64
        L.orc_slot.argtypes = [P, i64, i32, i64]
        L.orc_slots.restype = i64
        L.orc_slots.argtypes = [i32, P, P, P, P, P, i32, P]
        L.orc_store.restype = ctypes.c_int
        L.orc_store.argtypes = [P, i64, i64, i64, P, i64, P]
        L.orc_attention.restype = ctypes.c_int
        L.orc_attention.argtypes = [i32, P, P, P, i32, i32, i32, dbl, ctypes.c_int,
                                    ctypes.c_int, P, P, P, P, P, P, i32, i64, P, ctypes.c_int]
        L.orc_rope.restype = ctypes.c_int
        L.orc_rope.argtypes = [P, i64, i32, i32, P, i32, dbl, i32]
        L.orc_max_threads.restype = ctypes.c_int
        _lib = L
    return _lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _csr(tables: Sequence[Sequence[int]]) -> Tuple[np.ndarray, np.ndarray]:
    off = np.zeros(len(tables) + 1, dtype=np.int64)
    for i, t in enumerate(tables):
        off[i + 1] = off[i] + len(t)
    flat = np.zeros(max(1, int(off[-1])), dtype=np.int32)
    for i, t in enumerate(tables):
        flat[off[i]:off[i + 1]] = np.asarray(t, dtype=np.int32)
    return flat, off


def as_storage(x) -> Tuple[np.ndarray, int]:
    """A torch CPU tensor or numpy array -> (contiguous numpy storage, dtype code).
    bf16 is carried as its uint16 bit pattern; values are never rounded here."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().cpu().contiguous()
            if x.dtype == torch.bfloat16:
                return x.view(torch.int16).numpy().view(np.uint16), BF16
            if x.dtype == torch.float32:
                return x.numpy(), F32
            raise TypeError(f"unsupported dtype {x.dtype}")
    except ImportError:  # pragma: no cover
        pass
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        return x, BF16
    if x.dtype == np.float32:
        return x, F32
    raise TypeError(f"unsupported dtype {x.dtype}")


def to_f64(x) -> np.ndarray:
    """The exact float64 values of a bf16 / fp32 tensor or array."""
    s, code = as_storage(x)
    if code == BF16:
        return (s.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return s.astype(np.float64)


def rope(x, positions, rot_dim: int, base: float, style: int = 0) -> np.ndarray:
    """Rotary position embedding of head vectors x [T, H, d] at int positions
    [T] (``orc_rope``: pair j turns by positions[t] * base**(-2j/rot_dim);
    style 0 pairs (j, j + rot_dim/2), style 1 pairs (2j, 2j+1)). fp64 result."""
    v = np.ascontiguousarray(to_f64(x))
    T, H, d = v.shape
    pos = np.ascontiguousarray(positions, dtype=np.int32)
    assert pos.shape == (T,)
    if lib().orc_rope(_ptr(v), T, H, d, _ptr(pos), int(rot_dim), float(base), int(style)) != 0:
        raise ValueError("bad rotary arguments")
    return v


def slot(table: Sequence[int], block_size: int, pos: int) -> int:
    """Slot of position ``pos`` of a sequence whose block table is ``table``."""
    t = np.asarray(table, dtype=np.int32)
    return int(lib().orc_slot(_ptr(t), len(t), block_size, pos))


def slots(ranges: Sequence[Tuple[int, int, int]], tables, block_size: int) -> np.ndarray:
    """Slots of positions [b, e) of sequence s for each (s, b, e), in order."""
    flat, off = _csr(tables)
    n = sum(e - b for _, b, e in ranges)
    rs = np.array([r[0] for r in ranges] or [0], dtype=np.int32)
    rb = np.array([r[1] for r in ranges] or [0], dtype=np.int32)
    re = np.array([r[2] for r in ranges] or [0], dtype=np.int32)
    out = np.zeros(max(1, n), dtype=np.int64)
    got = lib().orc_slots(len(ranges), _ptr(rs), _ptr(rb), _ptr(re), _ptr(flat), _ptr(off),
                          block_size, _ptr(out))
    if got < 0:
        raise ValueError("position without a block-table entry")
    return out[:n]


def store(src, cache: np.ndarray, slot_ids: np.ndarray) -> None:
    """Bit-copy row i of ``src`` [N, ...] into row slot_ids[i] of ``cache``
    viewed as [num_slots, row]; negative slots are skipped. In place."""
    s, _ = as_storage(src)
    n = s.shape[0]
    row_bytes = s[0].nbytes if n else 0
    num_slots = cache.shape[0] * cache.shape[1]
    assert cache.flags.c_contiguous and cache[0, 0].nbytes == row_bytes or n == 0
    ids = np.ascontiguousarray(slot_ids, dtype=np.int64)
    assert ids.shape[0] == n
    rc = lib().orc_store(_ptr(s), n, row_bytes, row_bytes, _ptr(cache), num_slots, _ptr(ids))
    if rc == -1:
        raise ValueError("slot past the end of the pool")
    if rc == -2:
        raise ValueError("two rows target one slot")
    if rc != 0:
        raise MemoryError("oracle store failed")


def attention(q, q_lens, k_lens, num_kv_heads: int, scale: float, *,
              k=None, v=None, k_cache=None, v_cache=None, tables=None,
              block_size: int = 0, nthreads: int = 0) -> np.ndarray:
    """Causal attention over a ragged batch, fp64 output [sum q_lens, Hq, d].

    Keys come from contiguous ``k``/``v`` [sum k_lens, Hkv, d] or, when
    ``tables`` is given, from the pool ``k_cache``/``v_cache``
    [num_blocks, bs, Hkv, d] through the block tables."""
    qs, dt = as_storage(q)
    Tq, Hq, d = qs.shape
    ql = np.ascontiguousarray(q_lens, dtype=np.int32)
    kl = np.ascontiguousarray(k_lens, dtype=np.int32)
    assert int(ql.sum()) == Tq
    out = np.zeros((max(Tq, 1), Hq, d), dtype=np.float64)
    paged = tables is not None
    if paged:
        kc, dt2 = as_storage(k_cache)
        vc, _ = as_storage(v_cache)
        ks = vs = None
        flat, off = _csr(tables)
        nb = kc.shape[0]
    else:
        ks, dt2 = as_storage(k)
        vs, _ = as_storage(v)
        kc = vc = flat = off = None
        nb = 0
    assert dt2 == dt
    rc = lib().orc_attention(len(ql), _ptr(ql), _ptr(kl), _ptr(qs), Hq, num_kv_heads, d,
                             float(scale), dt, int(paged), _ptr(ks), _ptr(vs), _ptr(kc),
                             _ptr(vc), _ptr(flat), _ptr(off), block_size, nb, _ptr(out),
                             nthreads)
    if rc == -1:
        raise ValueError("key position without a valid block-table entry")
    if rc != 0:
        raise ValueError(f"oracle attention failed ({rc})")
    return out[:Tq]


def new_pool(num_blocks: int, block_size: int, num_kv_heads: int, head_dim: int,
             dtype_code: int) -> np.ndarray:
    """A pool [num_blocks, bs, Hkv, d] with every element NaN, so that a read
    of a slot nobody wrote shows up in the result."""
    if dtype_code == BF16:
        return np.full((num_blocks, block_size, num_kv_heads, head_dim), 0x7FC0, dtype=np.uint16)
    return np.full((num_blocks, block_size, num_kv_heads, head_dim), np.nan, dtype=np.float32)


def run_workload(w, nthreads: int = 0):
    """The whole path on one seeded workload: write the history K/V into a
    NaN-filled pool, write this call's new K/V, then attend.

    Returns (out fp64 [Tq, Hq, d], k_pool, v_pool, new-token slots)."""
    _, dt = as_storage(w.q[:0])
    kp = new_pool(w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim, dt)
    vp = new_pool(w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim, dt)
    if w.hist:
        hs = slots(w.hist, w.block_tables, w.block_size)
        store(w.k_hist, kp, hs)
        store(w.v_hist, vp, hs)
    new_ranges = [(s, c, n) for s, (n, c) in enumerate(zip(w.seq_lens, w.num_cached))]
    ns = slots(new_ranges, w.block_tables, w.block_size)
    store(w.k_new, kp, ns)
    store(w.v_new, vp, ns)
    if w.phase == "decode" or w.use_block_tables:
        out = attention(w.q, w.q_lens, w.seq_lens, w.num_kv_heads, w.scale,
                        k_cache=kp, v_cache=vp, tables=w.block_tables,
                        block_size=w.block_size, nthreads=nthreads)
    else:
        out = attention(w.q, w.q_lens, w.seq_lens, w.num_kv_heads, w.scale,
                        k=w.k_new, v=w.v_new, nthreads=nthreads)
    return out, kp, vp, ns


def max_threads() -> int:
    return int(lib().orc_max_threads())


def pools_after_store(w):
    """The pools after this step's writes (history, then the new tokens),
    without attending: (k_pool, v_pool, new-token slots)."""
    _, dt = as_storage(w.q[:0])
    kp = new_pool(w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim, dt)
    vp = new_pool(w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim, dt)
    if w.hist:
        hs = slots(w.hist, w.block_tables, w.block_size)
        store(w.k_hist, kp, hs)
        store(w.v_hist, vp, hs)
    ns = slots([(s, c, n) for s, (n, c) in enumerate(zip(w.seq_lens, w.num_cached))],
               w.block_tables, w.block_size)
    store(w.k_new, kp, ns)
    store(w.v_new, vp, ns)
    return kp, vp, ns
