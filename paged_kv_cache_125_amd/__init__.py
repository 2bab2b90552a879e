"""paged_kv_cache_125_amd -- Python binding of libpkv, the MI355X (gfx950)
paged-KV attention hot path.

Thin ctypes marshalling over the C ABI in ``include/pkv.h``: every step of the
path runs in the HIP kernels of ``libpkv.so``. PyTorch only provides device
memory (tensors) and the current HIP stream. If the library is not built this
module raises on use -- there is no fallback path.

Entry points (same names as the C functions, without the ``pkv_`` prefix):
``store_kvcache``, ``prefill_attention_varlen``, ``decode_attention_paged``,
``decode_attention_paged_noalloc``, ``decode_workspace_bytes``,
``decode_partition_size``, ``pack_prefill``, ``pack_decode``.

Streams: every call queues its work on ``stream`` (torch's current stream
when None). Device buffers the binding allocates itself for that work
(packed metadata, an output or workspace not given by the caller) are
allocated in that stream's context, and pinned staging buffers are held until
their upload has run; buffers the caller passes stay the caller's to order.
"""
from __future__ import annotations

import ctypes
import os
import threading
from typing import Dict, List, Optional, Sequence, Tuple

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libpkv.so")
ABI_VERSION = 6

PKV_F32, PKV_BF16 = 0, 1
# partition_size for decode_attention_paged: force the balanced split where the shape allows it
PARTITION_BALANCED = -1
_STATUS = {0: "PKV_OK", 1: "PKV_EINVAL", 2: "PKV_EUNSUPPORTED", 3: "PKV_ELAUNCH", 4: "PKV_ENOSPACE"}

EXPORTED = [
    "pkv_abi_version", "pkv_last_error", "pkv_store_kvcache", "pkv_prefill_attention_varlen",
    "pkv_decode_attention_paged", "pkv_decode_partition_size", "pkv_decode_workspace_bytes",
    "pkv_decode_attention_paged_noalloc", "pkv_decode_store_attention_paged", "pkv_prefill_workspace_bytes",
    "pkv_prefill_store_attention_varlen",
    "pkv_plan_prefill", "pkv_pack_prefill", "pkv_plan_decode", "pkv_pack_decode", "pkv_upload",
    "pkv_rope_cos_sin_table", "pkv_rope_store_kvcache",
    "pkv_xxh64", "pkv_block_hash", "pkv_bm_create", "pkv_bm_destroy", "pkv_bm_num_free",
    "pkv_bm_can_allocate", "pkv_bm_allocate", "pkv_bm_append_token", "pkv_bm_can_append",
    "pkv_bm_may_append", "pkv_bm_deallocate", "pkv_bm_block_table", "pkv_bm_gather",
]


class PkvError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_STATUS.get(status, status)}: {message}")
        self.status = status


class BatchLayout(ctypes.Structure):
    _fields_ = [
        ("num_seqs", ctypes.c_int32), ("total_q", ctypes.c_int32), ("total_k", ctypes.c_int64),
        ("max_seqlen_q", ctypes.c_int32), ("max_seqlen_k", ctypes.c_int32),
        ("max_blocks_per_seq", ctypes.c_int32), ("has_block_tables", ctypes.c_int32),
        ("num_slots", ctypes.c_int32), ("is_prefill", ctypes.c_int32),
        ("off_slot_mapping", ctypes.c_int64), ("off_cu_seqlens_q", ctypes.c_int64),
        ("off_cu_seqlens_k", ctypes.c_int64), ("off_context_lens", ctypes.c_int64),
        ("off_block_tables", ctypes.c_int64), ("off_positions", ctypes.c_int64),
        ("total_bytes", ctypes.c_int64),
    ]


_lib = None


def lib():
    """The loaded libpkv (ctypes.CDLL); raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                           "(or python -m paged_kv_cache_125_amd.build)")
    L = ctypes.CDLL(LIB_PATH)
    P, i32, i64, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    L.pkv_abi_version.restype = ctypes.c_int
    L.pkv_last_error.restype = ctypes.c_char_p
    L.pkv_store_kvcache.restype = ctypes.c_int
    L.pkv_store_kvcache.argtypes = [P, P, i64, i64, P, P, P, i32, i32, i32, i32, i32, i32, P]
    L.pkv_prefill_attention_varlen.restype = ctypes.c_int
    L.pkv_prefill_attention_varlen.argtypes = [P, i64, P, P, i64, P, P, P, i32, P, P, i32, i32, i32,
                                               i32, i32, i32, i32, i32, i32, f32, i32, P, P, sz, P]
    L.pkv_prefill_store_attention_varlen.restype = ctypes.c_int
    L.pkv_prefill_store_attention_varlen.argtypes = [P, i64, P, P, i64, P, P, P, P, i32, P, P, i32, i32,
                                                     i32, i32, i32, i32, i32, i32, i32, f32, i32, P, P]
    L.pkv_prefill_workspace_bytes.restype = sz
    L.pkv_prefill_workspace_bytes.argtypes = [i32] * 6
    L.pkv_decode_attention_paged.restype = ctypes.c_int
    L.pkv_decode_attention_paged.argtypes = [P, i64, P, P, P, i32, P, i32, i32, i32, i32, i32, i32,
                                             i32, f32, i32, P, i32, P, sz, P]
    L.pkv_decode_store_attention_paged.restype = ctypes.c_int
    L.pkv_decode_store_attention_paged.argtypes = [P, i64, P, P, i64, P, P, P, P, i32, P, i32, i32, i32,
                                                   i32, i32, i32, i32, f32, i32, P, i32, P, sz, P]
    L.pkv_decode_attention_paged_noalloc.restype = ctypes.c_int
    L.pkv_decode_attention_paged_noalloc.argtypes = [P, i64, P, P, P, i32, P, i32, i32, i32, i32, i32,
                                                     i32, i32, f32, i32, P, i32, P]
    L.pkv_decode_partition_size.restype = i32
    L.pkv_decode_partition_size.argtypes = [i32] * 8
    L.pkv_decode_workspace_bytes.restype = sz
    L.pkv_decode_workspace_bytes.argtypes = [i32] * 8
    L.pkv_plan_prefill.restype = ctypes.c_int
    L.pkv_plan_prefill.argtypes = [i32, P, P, P, i32, ctypes.POINTER(BatchLayout)]
    L.pkv_pack_prefill.restype = ctypes.c_int
    L.pkv_pack_prefill.argtypes = [i32, P, P, P, P, i32, ctypes.POINTER(BatchLayout), P, sz]
    L.pkv_plan_decode.restype = ctypes.c_int
    L.pkv_plan_decode.argtypes = [i32, P, P, i32, ctypes.POINTER(BatchLayout)]
    L.pkv_pack_decode.restype = ctypes.c_int
    L.pkv_pack_decode.argtypes = [i32, P, P, P, i32, ctypes.POINTER(BatchLayout), P, sz]
    L.pkv_upload.restype = ctypes.c_int
    L.pkv_upload.argtypes = [P, P, sz, P]
    u64 = ctypes.c_uint64
    L.pkv_xxh64.restype = u64
    L.pkv_xxh64.argtypes = [P, sz, u64]
    L.pkv_block_hash.restype = u64
    L.pkv_block_hash.argtypes = [P, i32, i32, u64]
    L.pkv_bm_create.restype = ctypes.c_int
    L.pkv_bm_create.argtypes = [i32, i32, ctypes.POINTER(P)]
    L.pkv_bm_destroy.restype = None
    L.pkv_bm_destroy.argtypes = [P]
    L.pkv_bm_num_free.restype = i32
    L.pkv_bm_num_free.argtypes = [P]
    L.pkv_bm_can_allocate.restype = ctypes.c_int
    L.pkv_bm_can_allocate.argtypes = [P, i32]
    L.pkv_bm_allocate.restype = ctypes.c_int
    L.pkv_bm_allocate.argtypes = [P, i64, P, i32, ctypes.POINTER(i32)]
    L.pkv_bm_append_token.restype = ctypes.c_int
    L.pkv_bm_append_token.argtypes = [P, i64, i64]
    L.pkv_bm_can_append.restype = ctypes.c_int
    L.pkv_bm_can_append.argtypes = [P, i64]
    L.pkv_bm_may_append.restype = ctypes.c_int
    L.pkv_bm_may_append.argtypes = [P, i64]
    L.pkv_bm_deallocate.restype = ctypes.c_int
    L.pkv_bm_deallocate.argtypes = [P, i64]
    L.pkv_bm_block_table.restype = i32
    L.pkv_bm_block_table.argtypes = [P, i64, P, i32]
    L.pkv_bm_gather.restype = ctypes.c_int
    L.pkv_bm_gather.argtypes = [P, i32, P, P, P, P, P, i64]
    L.pkv_rope_cos_sin_table.restype = ctypes.c_int
    L.pkv_rope_cos_sin_table.argtypes = [P, i32, i32, ctypes.c_double]
    L.pkv_rope_store_kvcache.restype = ctypes.c_int
    L.pkv_rope_store_kvcache.argtypes = [P, i64, P, P, i64, i64, P, P, P, P, P, i32, i32, i32, i32,
                                         i32, i32, i32, i32, i32, i32, i32, P]
    if L.pkv_abi_version() != ABI_VERSION:
        raise RuntimeError(f"libpkv ABI {L.pkv_abi_version()} != binding ABI {ABI_VERSION}")
    _lib = L
    return L


def _check(rc: int) -> None:
    if rc != 0:
        raise PkvError(rc, lib().pkv_last_error().decode())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return PKV_BF16
    if t.dtype == torch.float32:
        return PKV_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _alloc_on(stream, *shape, **kw) -> torch.Tensor:
    """A device tensor the binding allocates itself for work it queues on
    ``stream``: allocated in that stream's context, so that torch's caching
    allocator orders any later reuse of its memory after that stream's work.
    Allocated on the current stream instead (and only marked with
    record_stream), it could receive a block that work still queued on the
    current stream reads -- a block freed there is handed out again at once
    -- and the upload or kernel on ``stream`` would overwrite it first."""
    if stream is None or stream == torch.cuda.current_stream():
        return torch.empty(*shape, **kw)
    with torch.cuda.stream(stream):
        return torch.empty(*shape, **kw)


def _token_stride(t: torch.Tensor) -> int:
    # [tokens, heads, d] with each token's heads*d elements contiguous
    if t.dim() != 3 or t.stride(2) != 1 or t.stride(1) != t.shape[2]:
        raise ValueError("expected [tokens, heads, head_dim] with contiguous rows")
    return int(t.stride(0))


# ----------------------------------------------------------------- validation
# The C ABI validates sizes and alignment, but it sees only pointers: it cannot
# tell that two tensors disagree in dtype or shape, or live on different
# devices. A kernel then indexes with the wrong row size and leaves its
# buffers. Every entry point below checks that its tensors agree before any C
# call, and raises ValueError when they do not.

_ATTN_DTYPES = (torch.bfloat16, torch.float32)


def _need(cond: bool, msg) -> None:
    """Raise ValueError(msg) unless cond; msg may be a callable that formats
    the message, so that a passing check formats nothing."""
    if not cond:
        raise ValueError(msg() if callable(msg) else msg)


def _one_gpu(**tensors) -> None:
    """All given tensors on one device, and that device a GPU."""
    dev = None
    for t in tensors.values():
        if t is None:
            continue
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError("tensors on different devices: " + ", ".join(
                f"{n} on {x.device}" for n, x in tensors.items() if x is not None))
    _need(dev is not None and dev.type == "cuda", "the tensors must be on a GPU")


def _int32_vec(t: torch.Tensor, name: str, min_len: int) -> None:
    _need(t.dtype == torch.int32, lambda: f"{name} must be int32, got {t.dtype}")
    _need(t.dim() == 1 and t.is_contiguous(), lambda: f"{name} must be a contiguous 1-D tensor")
    _need(t.numel() >= min_len, lambda: f"{name} has {t.numel()} entries, needs {min_len}")


def _int32_table(t: torch.Tensor, name: str, min_rows: int) -> None:
    _need(t.dtype == torch.int32, lambda: f"{name} must be int32, got {t.dtype}")
    _need(t.dim() == 2 and t.is_contiguous(), lambda: f"{name} must be a contiguous 2-D tensor")
    _need(t.shape[0] >= min_rows and t.shape[1] >= 1,
          lambda: f"{name} has shape {tuple(t.shape)}, needs at least {min_rows} rows")


def _pool(k_cache: torch.Tensor, v_cache: torch.Tensor, dtype: torch.dtype) -> None:
    _need(k_cache.dim() == 4, "caches must be [num_blocks, block_size, num_kv_heads, head_dim]")
    _need(k_cache.shape == v_cache.shape, "k_cache and v_cache differ in shape")
    _need(k_cache.dtype == dtype and v_cache.dtype == dtype,
          lambda: f"cache dtype {k_cache.dtype}/{v_cache.dtype} differs from {dtype}")
    _need(k_cache.is_contiguous() and v_cache.is_contiguous(), "caches must be contiguous")


def _rows(t: torch.Tensor, name: str, heads: int, head_dim: int, dtype: torch.dtype,
          min_rows: int) -> None:
    """[tokens, heads, head_dim] with contiguous rows, of the given dtype."""
    _need(t.dtype == dtype, lambda: f"{name} dtype {t.dtype} differs from {dtype}")
    _need(t.dim() == 3 and t.shape[1] == heads and t.shape[2] == head_dim,
          lambda: f"{name} has shape {tuple(t.shape)}, expected [tokens, {heads}, {head_dim}]")
    _need(t.shape[0] >= min_rows, lambda: f"{name} has {t.shape[0]} rows, needs {min_rows}")
    _token_stride(t)


def _out(out: torch.Tensor, like: torch.Tensor) -> None:
    _need(out.dtype == like.dtype, lambda: f"out dtype {out.dtype} differs from q's {like.dtype}")
    _need(tuple(out.shape) == tuple(like.shape),
          lambda: f"out has shape {tuple(out.shape)}, expected {tuple(like.shape)}")
    _need(out.is_contiguous(), "out must be contiguous")


def store_kvcache(k: torch.Tensor, v: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                  slot_mapping: torch.Tensor, stream=None) -> None:
    """pkv_store_kvcache: k/v [N, Hkv, d] -> caches [num_blocks, bs, Hkv, d] at slot_mapping."""
    _pool(k_cache, v_cache, k_cache.dtype)
    nb, bs, hkv, d = k_cache.shape
    _int32_vec(slot_mapping, "slot_mapping", 0)
    n = int(slot_mapping.numel())
    _rows(k, "k", hkv, d, k_cache.dtype, n)
    _rows(v, "v", hkv, d, k_cache.dtype, n)
    _one_gpu(k=k, v=v, k_cache=k_cache, v_cache=v_cache, slot_mapping=slot_mapping)
    _check(lib().pkv_store_kvcache(_ptr(k), _ptr(v), _token_stride(k), _token_stride(v),
                                   _ptr(k_cache), _ptr(v_cache), _ptr(slot_mapping),
                                   int(slot_mapping.numel()), nb, bs, hkv, d, _dtype_code(k_cache),
                                   _stream(stream)))


def xxh64(data: bytes, seed: int = 0) -> int:
    """pkv_xxh64 of a byte string."""
    buf = ctypes.create_string_buffer(bytes(data), len(data))
    return int(lib().pkv_xxh64(ctypes.cast(buf, ctypes.c_void_p), len(data), seed))


def block_hash(token_ids: Sequence[int], prefix: Optional[int] = None) -> int:
    """pkv_block_hash: the chained hash of one full block."""
    import numpy as np
    t = np.ascontiguousarray(token_ids, dtype=np.int64)
    return int(lib().pkv_block_hash(ctypes.c_void_p(t.ctypes.data), len(t), prefix is not None,
                                    0 if prefix is None else int(prefix)))


class BlockManager:
    """The host block manager (pkv_bm_*): block tables and cached-prefix
    counts for sequences identified by integer ids."""

    def __init__(self, num_blocks: int, block_size: int):
        L = lib()
        h = ctypes.c_void_p()
        _check(L.pkv_bm_create(int(num_blocks), int(block_size), ctypes.byref(h)))
        self._h, self._lib = h, L
        self.num_blocks, self.block_size = int(num_blocks), int(block_size)

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value:
            self._lib.pkv_bm_destroy(h)
            self._h = None

    @property
    def num_free(self) -> int:
        return int(self._lib.pkv_bm_num_free(self._h))

    def can_allocate(self, num_tokens: int) -> bool:
        return bool(self._lib.pkv_bm_can_allocate(self._h, int(num_tokens)))

    def allocate(self, seq_id: int, token_ids: Sequence[int]) -> int:
        """Block table for a new sequence; returns its cached-token count."""
        import numpy as np
        t = np.ascontiguousarray(token_ids, dtype=np.int64)
        cached = ctypes.c_int32(0)
        _check(self._lib.pkv_bm_allocate(self._h, int(seq_id), ctypes.c_void_p(t.ctypes.data),
                                         len(t), ctypes.byref(cached)))
        return int(cached.value)

    def append_token(self, seq_id: int, token_id: int) -> None:
        _check(self._lib.pkv_bm_append_token(self._h, int(seq_id), int(token_id)))

    def can_append(self, seq_id: int) -> bool:
        return bool(self._lib.pkv_bm_can_append(self._h, int(seq_id)))

    def may_append(self, seq_id: int) -> None:
        _check(self._lib.pkv_bm_may_append(self._h, int(seq_id)))

    def deallocate(self, seq_id: int) -> None:
        _check(self._lib.pkv_bm_deallocate(self._h, int(seq_id)))

    def block_table(self, seq_id: int) -> List[int]:
        import numpy as np
        n = int(self._lib.pkv_bm_block_table(self._h, int(seq_id), None, 0))
        if n < 0:
            raise KeyError(seq_id)
        out = np.zeros(max(1, n), dtype=np.int32)
        self._lib.pkv_bm_block_table(self._h, int(seq_id), ctypes.c_void_p(out.ctypes.data), n)
        return [int(x) for x in out[:n]]

    def gather(self, seq_ids: Sequence[int]):
        """(seq_lens, num_cached_tokens, block_tables) of the sequences, in order."""
        import numpy as np
        ids = np.ascontiguousarray(seq_ids, dtype=np.int64)
        n = len(ids)
        lens = np.zeros(max(1, n), dtype=np.int32)
        cached = np.zeros(max(1, n), dtype=np.int32)
        off = np.zeros(n + 1, dtype=np.int64)
        cap = sum(max(0, int(self._lib.pkv_bm_block_table(self._h, int(i), None, 0))) for i in ids)
        bt = np.zeros(max(1, cap), dtype=np.int32)
        P = ctypes.c_void_p
        _check(self._lib.pkv_bm_gather(self._h, n, P(ids.ctypes.data), P(lens.ctypes.data),
                                       P(cached.ctypes.data), P(off.ctypes.data), P(bt.ctypes.data),
                                       cap))
        tables = [[int(x) for x in bt[off[s]:off[s + 1]]] for s in range(n)]
        return [int(x) for x in lens[:n]], [int(x) for x in cached[:n]], tables


ROPE_HALF, ROPE_INTERLEAVED = 0, 1


def rope_cos_sin_table(max_positions: int, rot_dim: int, base: float,
                       device="cuda") -> torch.Tensor:
    """pkv_rope_cos_sin_table: float [max_positions, rot_dim] (cos | sin),
    filled on the host and copied to ``device``."""
    t = torch.empty((max_positions, rot_dim), dtype=torch.float32)
    _check(lib().pkv_rope_cos_sin_table(ctypes.c_void_p(t.data_ptr()), int(max_positions),
                                        int(rot_dim), float(base)))
    return t.to(device)


def rope_store_kvcache(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, k_cache: torch.Tensor,
                       v_cache: torch.Tensor, slot_mapping: torch.Tensor, positions: torch.Tensor,
                       cos_sin: torch.Tensor, style: int = ROPE_HALF, write_k: bool = True,
                       stream=None) -> None:
    """pkv_rope_store_kvcache: rotate q (in place) and k by ``positions``,
    store the rotated k and v into the caches at ``slot_mapping`` (and the
    rotated k back into ``k`` when ``write_k``)."""
    _pool(k_cache, v_cache, k_cache.dtype)
    nb, bs, hkv, d = k_cache.shape
    _need(q.dim() == 3, "q must be [tokens, num_q_heads, head_dim]")
    n, hq, _ = q.shape
    _rows(q, "q", hq, d, k_cache.dtype, n)
    _rows(k, "k", hkv, d, k_cache.dtype, n)
    _rows(v, "v", hkv, d, k_cache.dtype, n)
    _need(k.shape[0] == n and v.shape[0] == n, "q, k and v must have one row per token")
    _int32_vec(slot_mapping, "slot_mapping", n)
    _int32_vec(positions, "positions", n)
    _need(slot_mapping.numel() == n and positions.numel() == n,
          "slot_mapping and positions must have one entry per token")
    if cos_sin.dtype != torch.float32 or cos_sin.dim() != 2 or not cos_sin.is_contiguous():
        raise TypeError("cos_sin must be a contiguous float32 [max_positions, rot_dim] table")
    _one_gpu(q=q, k=k, v=v, k_cache=k_cache, v_cache=v_cache, slot_mapping=slot_mapping,
             positions=positions, cos_sin=cos_sin)
    _check(lib().pkv_rope_store_kvcache(
        _ptr(q), _token_stride(q), _ptr(k), _ptr(v), _token_stride(k), _token_stride(v),
        _ptr(k_cache), _ptr(v_cache), _ptr(slot_mapping), _ptr(positions), _ptr(cos_sin),
        int(cos_sin.shape[0]), int(cos_sin.shape[1]), int(style), int(bool(write_k)), n, nb, bs,
        hq, hkv, d, _dtype_code(q), _stream(stream)))


def prefill_workspace_bytes() -> int:
    """pkv_prefill_workspace_bytes: the size of the workspace that selects the
    persistent prefill grid."""
    return int(lib().pkv_prefill_workspace_bytes(0, 0, 0, 0, 0, 0))


def prefill_attention_varlen(q: torch.Tensor, cu_seqlens_q: torch.Tensor, cu_seqlens_k: torch.Tensor,
                             max_seqlen_q: int, max_seqlen_k: int, scale: float, *,
                             k: Optional[torch.Tensor] = None, v: Optional[torch.Tensor] = None,
                             k_cache: Optional[torch.Tensor] = None,
                             v_cache: Optional[torch.Tensor] = None,
                             block_tables: Optional[torch.Tensor] = None,
                             num_kv_heads: Optional[int] = None,
                             out: Optional[torch.Tensor] = None,
                             workspace: Optional[torch.Tensor] = None,
                             stream=None) -> torch.Tensor:
    """pkv_prefill_attention_varlen. Keys from k/v, or from the caches through
    block_tables when given. Without ``workspace`` one workgroup runs per
    item; a ``workspace`` (uint8, >= prefill_workspace_bytes(), zeroed once
    when allocated and left zeroed by every call) selects the persistent grid
    and must not be shared by calls that may overlap."""
    _need(q.dim() == 3, "q must be [tokens, num_q_heads, head_dim]")
    _need(q.dtype in _ATTN_DTYPES, lambda: f"unsupported dtype {q.dtype}")
    total_q, hq, d = q.shape
    _rows(q, "q", hq, d, q.dtype, 0)
    _int32_vec(cu_seqlens_q, "cu_seqlens_q", 1)
    _int32_vec(cu_seqlens_k, "cu_seqlens_k", 1)
    _need(cu_seqlens_k.numel() == cu_seqlens_q.numel(),
          "cu_seqlens_q and cu_seqlens_k must have one entry per sequence plus one")
    num_seqs = int(cu_seqlens_q.numel()) - 1
    if block_tables is not None:
        _need(k_cache is not None and v_cache is not None, "block_tables need k_cache and v_cache")
        _pool(k_cache, v_cache, q.dtype)
        nb, bs, hkv, _ = k_cache.shape
        _need(k_cache.shape[3] == d, "cache head_dim differs from q's")
        _int32_table(block_tables, "block_tables", num_seqs)
        maxb = int(block_tables.shape[1])
        kv_stride = 0
    else:
        _need(k is not None and v is not None, "k and v are needed without block_tables")
        nb, bs, maxb = 0, 1, 0
        _need(k.dim() == 3, "k must be [tokens, num_kv_heads, head_dim]")
        hkv = k.shape[1]
        _rows(k, "k", hkv, d, q.dtype, total_q)
        _rows(v, "v", hkv, d, q.dtype, total_q)
        kv_stride = _token_stride(k)
        if _token_stride(v) != kv_stride:
            raise ValueError("k and v must share a token stride")
    if num_kv_heads is not None and num_kv_heads != hkv:
        raise ValueError("num_kv_heads does not match the key tensors")
    if out is not None:
        _out(out, q)
    _one_gpu(q=q, k=k, v=v, k_cache=k_cache if block_tables is not None else None,
             v_cache=v_cache if block_tables is not None else None, block_tables=block_tables,
             cu_seqlens_q=cu_seqlens_q, cu_seqlens_k=cu_seqlens_k, out=out)
    if workspace is not None:
        _need(workspace.dtype == torch.uint8 and workspace.is_contiguous()
              and workspace.device == q.device, "workspace must be a contiguous uint8 tensor on q's device")
    if out is None:
        out = _alloc_on(stream, (total_q, hq, d), dtype=q.dtype, device=q.device)
    _need(workspace is None or workspace.numel() >= prefill_workspace_bytes(),
          "workspace is smaller than prefill_workspace_bytes()")
    _check(lib().pkv_prefill_attention_varlen(
        _ptr(q), _token_stride(q), _ptr(k), _ptr(v), kv_stride, _ptr(k_cache), _ptr(v_cache),
        _ptr(block_tables), maxb, _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), num_seqs, total_q,
        int(max_seqlen_q), int(max_seqlen_k), nb, bs, hq, hkv, d, float(scale), _dtype_code(q),
        _ptr(out), _ptr(workspace), 0 if workspace is None else workspace.numel(), _stream(stream)))
    return out


def prefill_store_attention_varlen(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                                   k_cache: torch.Tensor, v_cache: torch.Tensor,
                                   slot_mapping: torch.Tensor, cu_seqlens_q: torch.Tensor,
                                   cu_seqlens_k: torch.Tensor, max_seqlen_q: int, max_seqlen_k: int,
                                   scale: float, *, block_tables: Optional[torch.Tensor] = None,
                                   out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """pkv_prefill_store_attention_varlen: store_kvcache(k, v, k_cache, v_cache,
    slot_mapping) and prefill_attention_varlen in one launch on the bf16
    head_dim-128 path. Without ``block_tables`` the keys are the call's own
    k/v rows; with them, cached positions come from the pool and this call's
    positions from its k/v rows."""
    _need(q.dim() == 3, "q must be [tokens, num_q_heads, head_dim]")
    _need(q.dtype in _ATTN_DTYPES, lambda: f"unsupported dtype {q.dtype}")
    total_q, hq, d = q.shape
    _rows(q, "q", hq, d, q.dtype, 0)
    _pool(k_cache, v_cache, q.dtype)
    nb, bs, hkv, _ = k_cache.shape
    _need(k_cache.shape[3] == d, "cache head_dim differs from q's")
    _rows(k, "k", hkv, d, q.dtype, total_q)
    _rows(v, "v", hkv, d, q.dtype, total_q)
    kv_stride = _token_stride(k)
    if _token_stride(v) != kv_stride:
        raise ValueError("k and v must share a token stride")
    _int32_vec(slot_mapping, "slot_mapping", total_q)
    _int32_vec(cu_seqlens_q, "cu_seqlens_q", 1)
    _int32_vec(cu_seqlens_k, "cu_seqlens_k", 1)
    _need(cu_seqlens_k.numel() == cu_seqlens_q.numel(),
          "cu_seqlens_q and cu_seqlens_k must have one entry per sequence plus one")
    num_seqs = int(cu_seqlens_q.numel()) - 1
    maxb = 0
    if block_tables is not None:
        _int32_table(block_tables, "block_tables", num_seqs)
        maxb = int(block_tables.shape[1])
    if out is not None:
        _out(out, q)
    _one_gpu(q=q, k=k, v=v, k_cache=k_cache, v_cache=v_cache, slot_mapping=slot_mapping,
             cu_seqlens_q=cu_seqlens_q, cu_seqlens_k=cu_seqlens_k, block_tables=block_tables, out=out)
    if out is None:
        out = _alloc_on(stream, (total_q, hq, d), dtype=q.dtype, device=q.device)
    _check(lib().pkv_prefill_store_attention_varlen(
        _ptr(q), _token_stride(q), _ptr(k), _ptr(v), kv_stride, _ptr(k_cache), _ptr(v_cache),
        _ptr(slot_mapping), _ptr(block_tables), maxb, _ptr(cu_seqlens_q), _ptr(cu_seqlens_k),
        num_seqs, total_q, int(max_seqlen_q), int(max_seqlen_k), nb, bs, hq, hkv, d, float(scale),
        _dtype_code(q), _ptr(out), _stream(stream)))
    return out


def decode_partition_size(num_seqs: int, max_context_len: int, num_q_heads: int, num_kv_heads: int,
                          head_dim: int, block_size: int, dtype: torch.dtype,
                          partition_size: int = 0) -> int:
    code = PKV_BF16 if dtype == torch.bfloat16 else PKV_F32
    return int(lib().pkv_decode_partition_size(num_seqs, max_context_len, num_q_heads, num_kv_heads,
                                               head_dim, block_size, code, partition_size))


def decode_workspace_bytes(num_seqs: int, max_context_len: int, num_q_heads: int, num_kv_heads: int,
                           head_dim: int, block_size: int, dtype: torch.dtype,
                           partition_size: int = 0) -> int:
    code = PKV_BF16 if dtype == torch.bfloat16 else PKV_F32
    return int(lib().pkv_decode_workspace_bytes(num_seqs, max_context_len, num_q_heads, num_kv_heads,
                                                head_dim, block_size, code, partition_size))


def decode_attention_paged(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                           block_tables: torch.Tensor, context_lens: torch.Tensor,
                           max_context_len: int, scale: float, *,
                           out: Optional[torch.Tensor] = None, partition_size: int = 0,
                           workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """pkv_decode_attention_paged: q [B, Hq, d] against context_lens keys per
    sequence. ``workspace`` (uint8, >= decode_workspace_bytes) is allocated
    through torch when not given."""
    _need(q.dim() == 3, "q must be [num_seqs, num_q_heads, head_dim]")
    _need(q.dtype in _ATTN_DTYPES, lambda: f"unsupported dtype {q.dtype}")
    B, hq, d = q.shape
    _rows(q, "q", hq, d, q.dtype, 0)
    _pool(k_cache, v_cache, q.dtype)
    nb, bs, hkv, _ = k_cache.shape
    _need(k_cache.shape[3] == d, "cache head_dim differs from q's")
    _int32_table(block_tables, "block_tables", B)
    _int32_vec(context_lens, "context_lens", B)
    if out is not None:
        _out(out, q)
    if workspace is not None:
        _need(workspace.dtype == torch.uint8 and workspace.is_contiguous(),
              "workspace must be a contiguous uint8 tensor")
    _one_gpu(q=q, k_cache=k_cache, v_cache=v_cache, block_tables=block_tables,
             context_lens=context_lens, out=out, workspace=workspace)
    if out is None:
        out = _alloc_on(stream, (B, hq, d), dtype=q.dtype, device=q.device)
    need = decode_workspace_bytes(B, max_context_len, hq, hkv, d, bs, q.dtype, partition_size)
    if workspace is None and need > 0:
        workspace = _alloc_on(stream, need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().pkv_decode_attention_paged(
        _ptr(q), _token_stride(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
        int(block_tables.shape[1]), _ptr(context_lens), B, int(max_context_len), nb, bs, hq, hkv, d,
        float(scale), _dtype_code(q), _ptr(out), int(partition_size), _ptr(workspace), ws_bytes,
        _stream(stream)))
    return out


def decode_store_attention_paged(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                                 k_cache: torch.Tensor, v_cache: torch.Tensor,
                                 slot_mapping: torch.Tensor, block_tables: torch.Tensor,
                                 context_lens: torch.Tensor, max_context_len: int, scale: float, *,
                                 out: Optional[torch.Tensor] = None, partition_size: int = 0,
                                 workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """pkv_decode_store_attention_paged: store_kvcache of k/v [B, Hkv, d] at
    slot_mapping, then decode_attention_paged, in one call (one launch on the
    fixed-partition path). k and v must share one token stride."""
    _need(q.dim() == 3, "q must be [num_seqs, num_q_heads, head_dim]")
    _need(q.dtype in _ATTN_DTYPES, lambda: f"unsupported dtype {q.dtype}")
    B, hq, d = q.shape
    _rows(q, "q", hq, d, q.dtype, 0)
    _pool(k_cache, v_cache, q.dtype)
    nb, bs, hkv, _ = k_cache.shape
    _need(k_cache.shape[3] == d, "cache head_dim differs from q's")
    _rows(k, "k", hkv, d, q.dtype, B)
    _rows(v, "v", hkv, d, q.dtype, B)
    _need(_token_stride(k) == _token_stride(v), "k and v must share one token stride")
    _int32_vec(slot_mapping, "slot_mapping", B)
    _int32_table(block_tables, "block_tables", B)
    _int32_vec(context_lens, "context_lens", B)
    if out is not None:
        _out(out, q)
    if workspace is not None:
        _need(workspace.dtype == torch.uint8 and workspace.is_contiguous(),
              "workspace must be a contiguous uint8 tensor")
    _one_gpu(q=q, k=k, v=v, k_cache=k_cache, v_cache=v_cache, slot_mapping=slot_mapping,
             block_tables=block_tables, context_lens=context_lens, out=out, workspace=workspace)
    if out is None:
        out = _alloc_on(stream, (B, hq, d), dtype=q.dtype, device=q.device)
    need = decode_workspace_bytes(B, max_context_len, hq, hkv, d, bs, q.dtype, partition_size)
    if workspace is None and need > 0:
        workspace = _alloc_on(stream, need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().pkv_decode_store_attention_paged(
        _ptr(q), _token_stride(q), _ptr(k), _ptr(v), _token_stride(k), _ptr(k_cache), _ptr(v_cache),
        _ptr(slot_mapping), _ptr(block_tables), int(block_tables.shape[1]), _ptr(context_lens), B,
        int(max_context_len), nb, bs, hq, hkv, d, float(scale), _dtype_code(q), _ptr(out),
        int(partition_size), _ptr(workspace), ws_bytes, _stream(stream)))
    return out


NOALLOC_SCRATCH_BYTES = 16 << 20   # PKV_NOALLOC_SCRATCH_BYTES


def decode_attention_paged_noalloc(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                                   block_tables: torch.Tensor, context_lens: torch.Tensor,
                                   max_context_len: int, scale: float, out: torch.Tensor, *,
                                   partition_size: int = 0, stream=None) -> torch.Tensor:
    """pkv_decode_attention_paged_noalloc: decode_attention_paged with the
    library's own device scratch as workspace, for callers that cannot
    allocate. ``out`` must be given; nothing is allocated on the path. Calls
    that may overlap on one GPU race on its scratch."""
    _need(q.dim() == 3, "q must be [num_seqs, num_q_heads, head_dim]")
    _need(q.dtype in _ATTN_DTYPES, lambda: f"unsupported dtype {q.dtype}")
    B, hq, d = q.shape
    _rows(q, "q", hq, d, q.dtype, 0)
    _pool(k_cache, v_cache, q.dtype)
    nb, bs, hkv, _ = k_cache.shape
    _need(k_cache.shape[3] == d, "cache head_dim differs from q's")
    _int32_table(block_tables, "block_tables", B)
    _int32_vec(context_lens, "context_lens", B)
    _out(out, q)
    _one_gpu(q=q, k_cache=k_cache, v_cache=v_cache, block_tables=block_tables,
             context_lens=context_lens, out=out)
    _check(lib().pkv_decode_attention_paged_noalloc(
        _ptr(q), _token_stride(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
        int(block_tables.shape[1]), _ptr(context_lens), B, int(max_context_len), nb, bs, hq, hkv, d,
        float(scale), _dtype_code(q), _ptr(out), int(partition_size), _stream(stream)))
    return out


def _csr(block_tables: Sequence[Sequence[int]]):
    """The per-sequence tables as one int32 id array plus int64 offsets, built
    in two passes over the Python lists (no per-row temporary arrays)."""
    import itertools
    import numpy as np
    n = len(block_tables)
    off = np.empty(n + 1, dtype=np.int64)
    off[0] = 0
    np.cumsum(np.fromiter(map(len, block_tables), dtype=np.int64, count=n), out=off[1:])
    total = int(off[-1])
    if total == 0:
        return np.zeros(1, dtype=np.int32), off
    ids = np.fromiter(itertools.chain.from_iterable(block_tables), dtype=np.int32, count=total)
    return ids, off


def _views(layout: BatchLayout, dev: torch.Tensor) -> Dict[str, object]:
    def arr(off, n):
        return None if off < 0 else dev[off:off + 4 * n].view(torch.int32)
    out = {
        "slot_mapping": arr(layout.off_slot_mapping, layout.num_slots),
        "cu_seqlens_q": arr(layout.off_cu_seqlens_q, layout.num_seqs + 1),
        "cu_seqlens_k": arr(layout.off_cu_seqlens_k, layout.num_seqs + 1),
        "context_lens": arr(layout.off_context_lens, layout.num_seqs),
        "positions": arr(layout.off_positions, layout.num_slots),
        "block_tables": None,
        "max_seqlen_q": layout.max_seqlen_q, "max_seqlen_k": layout.max_seqlen_k,
        "total_q": layout.total_q, "max_blocks_per_seq": layout.max_blocks_per_seq,
        "buffer": dev,
    }
    if layout.off_block_tables >= 0:
        n = layout.num_seqs * layout.max_blocks_per_seq
        out["block_tables"] = dev[layout.off_block_tables:layout.off_block_tables + 4 * n] \
            .view(torch.int32).view(layout.num_seqs, layout.max_blocks_per_seq)
    return out


# Pinned staging buffers that the binding allocated itself, each held until an
# event recorded right after its upload has completed. torch's pinned-memory
# cache knows nothing of a hipMemcpyAsync issued through the C ABI: a buffer
# freed while such a copy is still queued goes straight back to its free list,
# the next pinned allocation of the same size class receives it, and the
# packer then overwrites the bytes the queued copy has yet to read (the device
# metadata of the earlier step would hold the later step's values).
_staging: List[Tuple[torch.Tensor, object]] = []
_staging_lock = threading.Lock()


def _hold_until_uploaded(host: torch.Tensor, stream) -> None:
    ev = torch.cuda.Event()
    ev.record(torch.cuda.current_stream() if stream is None else stream)
    with _staging_lock:
        _staging[:] = [(h, e) for h, e in _staging if not e.query()]
        _staging.append((host, ev))


def _pack(prefill: bool, seq_lens, num_cached, block_tables, block_size: int, device,
          stream=None, host_buffer: Optional[torch.Tensor] = None,
          dev_buffer: Optional[torch.Tensor] = None) -> Dict[str, object]:
    import numpy as np
    L = lib()
    lens = np.ascontiguousarray(seq_lens, dtype=np.int32)
    ids, off = _csr(block_tables)
    layout = BatchLayout()
    P = ctypes.c_void_p
    if prefill:
        cached = np.ascontiguousarray(num_cached, dtype=np.int32)
        _check(L.pkv_plan_prefill(len(lens), P(lens.ctypes.data), P(cached.ctypes.data),
                                  P(off.ctypes.data), block_size, ctypes.byref(layout)))
    else:
        _check(L.pkv_plan_decode(len(lens), P(lens.ctypes.data), P(off.ctypes.data), block_size,
                                 ctypes.byref(layout)))
    nbytes = layout.total_bytes
    if host_buffer is None:
        host = torch.empty(nbytes, dtype=torch.uint8, pin_memory=torch.cuda.is_available())
    else:
        if host_buffer.dtype != torch.uint8 or host_buffer.device.type != "cpu" \
                or not host_buffer.is_contiguous() or host_buffer.numel() < nbytes:
            raise ValueError(f"host_buffer must be a contiguous CPU uint8 tensor of >= {nbytes} bytes")
        host = host_buffer[:nbytes]
    if prefill:
        _check(L.pkv_pack_prefill(len(lens), P(lens.ctypes.data), P(cached.ctypes.data),
                                  P(ids.ctypes.data), P(off.ctypes.data), block_size,
                                  ctypes.byref(layout), P(host.data_ptr()), nbytes))
    else:
        _check(L.pkv_pack_decode(len(lens), P(lens.ctypes.data), P(ids.ctypes.data),
                                 P(off.ctypes.data), block_size, ctypes.byref(layout),
                                 P(host.data_ptr()), nbytes))
    if device is None or torch.device(device).type == "cpu":
        dev = host
    else:
        if dev_buffer is None:
            dev = _alloc_on(stream, nbytes, dtype=torch.uint8, device=device)
        else:
            if dev_buffer.dtype != torch.uint8 or dev_buffer.device.type != "cuda" \
                    or not dev_buffer.is_contiguous() or dev_buffer.numel() < nbytes:
                raise ValueError(f"dev_buffer must be a contiguous device uint8 tensor of >= {nbytes} bytes")
            dev = dev_buffer[:nbytes]
        _check(L.pkv_upload(P(host.data_ptr()), P(dev.data_ptr()), nbytes, _stream(stream)))
        if host_buffer is None:
            _hold_until_uploaded(host, stream)
    res = _views(layout, dev)
    res["host_buffer"] = host
    res["layout"] = layout
    return res


def pack_prefill(seq_lens: Sequence[int], num_cached: Sequence[int],
                 block_tables: Sequence[Sequence[int]], block_size: int,
                 device="cuda", stream=None, host_buffer: Optional[torch.Tensor] = None,
                 dev_buffer: Optional[torch.Tensor] = None) -> Dict[str, object]:
    """pkv_plan_prefill + pkv_pack_prefill + pkv_upload: the step's metadata in
    one buffer. Returns device views slot_mapping, cu_seqlens_q/_k,
    block_tables (or None) and the host scalars.

    ``host_buffer`` (pinned CPU uint8) and ``dev_buffer`` (device uint8), when
    given, are used as the staging and destination buffers instead of new
    allocations; the caller must not reuse or free ``host_buffer`` before the
    stream has run the copy. A staging buffer the binding allocates itself is
    held by the binding until the copy has run."""
    return _pack(True, seq_lens, num_cached, block_tables, block_size, device, stream,
                 host_buffer, dev_buffer)


def pack_decode(seq_lens: Sequence[int], block_tables: Sequence[Sequence[int]], block_size: int,
                device="cuda", stream=None, host_buffer: Optional[torch.Tensor] = None,
                dev_buffer: Optional[torch.Tensor] = None) -> Dict[str, object]:
    """pkv_plan_decode + pkv_pack_decode + pkv_upload (buffers as in pack_prefill)."""
    return _pack(False, seq_lens, None, block_tables, block_size, device, stream,
                 host_buffer, dev_buffer)
