// pack.cpp -- host metadata packing for one prefill or decode step.
//
// "nano-vLLM-1", "4. prefill 输入打包" and "5. deocde 输入打包" build the kernel
// metadata as Python lists and ship each as its own pinned tensor. Here the
// same arrays are written by one C++ pass into a single caller-provided host
// buffer (pinned for an asynchronous copy), at 256-byte-aligned offsets, so the
// whole step's metadata reaches the device in one hipMemcpyAsync (pkv_upload).
//
// Prefill: the uncached tokens of each sequence fill its blocks from the first
// uncached position on; each block contributes a run of consecutive slots
// starting at physical_block * bs (the first one at the cached offset, the
// last one ending at the sequence length). cu_seqlens_q / cu_seqlens_k are the
// prefix sums of the query and key lengths; block tables, padded with -1 to the
// longest one ("prepare_block_tables"), are packed only when the batch reads a
// cached prefix (total keys > total queries).
// Decode: one slot per sequence -- the slot of its newest position --, the
// context length, and the padded block tables. Both also pack the position of
// every slot (the rotary embedding's input).
#include <limits.h>
#include <string.h>

#include "pkv.h"

int pkv_internal_fail(int code, const char *msg);

namespace {

int64_t align256(int64_t x) { return (x + 255) & ~int64_t(255); }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

void finish_layout(pkv_batch_layout *L, bool prefill) {
    int64_t at = 0;
    L->off_slot_mapping = at;
    at = align256(at + (int64_t)L->num_slots * 4);
    if (prefill) {
        L->off_cu_seqlens_q = at;
        at = align256(at + (int64_t)(L->num_seqs + 1) * 4);
        L->off_cu_seqlens_k = at;
        at = align256(at + (int64_t)(L->num_seqs + 1) * 4);
        L->off_context_lens = -1;
    } else {
        L->off_cu_seqlens_q = L->off_cu_seqlens_k = -1;
        L->off_context_lens = at;
        at = align256(at + (int64_t)L->num_seqs * 4);
    }
    if (L->has_block_tables) {
        L->off_block_tables = at;
        at = align256(at + (int64_t)L->num_seqs * L->max_blocks_per_seq * 4);
    } else {
        L->off_block_tables = -1;
    }
    L->off_positions = at;
    at = align256(at + (int64_t)L->num_slots * 4);
    L->total_bytes = at > 0 ? at : 256;
}

void write_tables(const pkv_batch_layout *L, const int32_t *bt_ids, const int64_t *bt_off,
                  char *buf) {
    int32_t *bt = (int32_t *)(buf + L->off_block_tables);
    for (int32_t s = 0; s < L->num_seqs; ++s) {
        const int64_t n = bt_off[s + 1] - bt_off[s];
        int32_t *row = bt + (int64_t)s * L->max_blocks_per_seq;
        for (int64_t i = 0; i < n; ++i) row[i] = bt_ids[bt_off[s] + i];
        for (int64_t i = n; i < L->max_blocks_per_seq; ++i) row[i] = -1;
    }
}

}  // namespace

extern "C" int pkv_plan_prefill(int32_t num_seqs, const int32_t *seq_lens,
                                const int32_t *num_cached_tokens, const int64_t *bt_offsets,
                                int32_t block_size, pkv_batch_layout *layout) {
    if (!layout || num_seqs < 0 || block_size <= 0 || (num_seqs > 0 && (!seq_lens || !num_cached_tokens || !bt_offsets)))
        return pkv_internal_fail(PKV_EINVAL, "pkv_plan_prefill: bad arguments");
    pkv_batch_layout L;
    memset(&L, 0, sizeof L);
    L.num_seqs = num_seqs;
    L.is_prefill = 1;
    int64_t total_q = 0, total_k = 0;
    for (int32_t s = 0; s < num_seqs; ++s) {
        const int64_t n = seq_lens[s], c = num_cached_tokens[s];
        if (n < 0 || c < 0 || c > n)
            return pkv_internal_fail(PKV_EINVAL, "pkv_plan_prefill: lengths out of range");
        const int64_t tlen = bt_offsets[s + 1] - bt_offsets[s];
        if (tlen < ceil_div(n, block_size))
            return pkv_internal_fail(PKV_EINVAL, "pkv_plan_prefill: block table shorter than the sequence");
        total_q += n - c;
        total_k += n;
        if (n - c > L.max_seqlen_q) L.max_seqlen_q = (int32_t)(n - c);
        if (n > L.max_seqlen_k) L.max_seqlen_k = (int32_t)n;
        if (tlen > L.max_blocks_per_seq) {
            if (tlen > INT32_MAX) return pkv_internal_fail(PKV_EINVAL, "pkv_plan_prefill: table too long");
            L.max_blocks_per_seq = (int32_t)tlen;
        }
    }
    if (total_q > INT32_MAX || total_k > INT32_MAX)
        return pkv_internal_fail(PKV_EINVAL, "pkv_plan_prefill: batch has more than 2^31-1 tokens");
    L.total_q = (int32_t)total_q;
    L.total_k = total_k;
    L.num_slots = (int32_t)total_q;
    L.has_block_tables = total_k > total_q && L.max_blocks_per_seq > 0;
    finish_layout(&L, true);
    *layout = L;
    return PKV_OK;
}

extern "C" int pkv_pack_prefill(int32_t num_seqs, const int32_t *seq_lens,
                                const int32_t *num_cached_tokens, const int32_t *bt_ids,
                                const int64_t *bt_offsets, int32_t block_size,
                                const pkv_batch_layout *layout, void *host_buf,
                                size_t host_bytes) {
    if (!layout || !host_buf || layout->num_seqs != num_seqs || !layout->is_prefill)
        return pkv_internal_fail(PKV_EINVAL, "pkv_pack_prefill: layout does not match the batch");
    if ((int64_t)host_bytes < layout->total_bytes)
        return pkv_internal_fail(PKV_ENOSPACE, "pkv_pack_prefill: host buffer too small");
    char *buf = (char *)host_buf;
    int32_t *slots = (int32_t *)(buf + layout->off_slot_mapping);
    int32_t *cu_q = (int32_t *)(buf + layout->off_cu_seqlens_q);
    int32_t *cu_k = (int32_t *)(buf + layout->off_cu_seqlens_k);
    int32_t *pos = (int32_t *)(buf + layout->off_positions);
    int64_t at = 0;
    cu_q[0] = cu_k[0] = 0;
    for (int32_t s = 0; s < num_seqs; ++s) {
        const int64_t n = seq_lens[s], c = num_cached_tokens[s];
        const int32_t *table = bt_ids + bt_offsets[s];
        const int64_t nblk = ceil_div(n, block_size);
        for (int64_t i = c / block_size; i < nblk; ++i) {
            const int64_t lo = i * block_size < c ? c - i * block_size : 0;
            const int64_t hi = i == nblk - 1 ? n - i * block_size : block_size;
            const int64_t base = (int64_t)table[i] * block_size;
            if (table[i] < 0 || base + hi - 1 > INT32_MAX)
                return pkv_internal_fail(PKV_EINVAL, "pkv_pack_prefill: block id out of range");
            for (int64_t o = lo; o < hi; ++o) {
                pos[at] = (int32_t)(i * block_size + o);
                slots[at++] = (int32_t)(base + o);
            }
        }
        cu_q[s + 1] = cu_q[s] + (int32_t)(n - c);
        cu_k[s + 1] = cu_k[s] + (int32_t)n;
    }
    if (at != layout->num_slots || cu_q[num_seqs] != layout->total_q)
        return pkv_internal_fail(PKV_EINVAL, "pkv_pack_prefill: layout does not match the batch");
    if (layout->has_block_tables) write_tables(layout, bt_ids, bt_offsets, buf);
    return PKV_OK;
}

extern "C" int pkv_plan_decode(int32_t num_seqs, const int32_t *seq_lens,
                               const int64_t *bt_offsets, int32_t block_size,
                               pkv_batch_layout *layout) {
    if (!layout || num_seqs < 0 || block_size <= 0 || (num_seqs > 0 && (!seq_lens || !bt_offsets)))
        return pkv_internal_fail(PKV_EINVAL, "pkv_plan_decode: bad arguments");
    pkv_batch_layout L;
    memset(&L, 0, sizeof L);
    L.num_seqs = num_seqs;
    L.total_q = num_seqs;
    L.num_slots = num_seqs;
    L.max_seqlen_q = num_seqs > 0 ? 1 : 0;
    for (int32_t s = 0; s < num_seqs; ++s) {
        const int64_t n = seq_lens[s];
        const int64_t tlen = bt_offsets[s + 1] - bt_offsets[s];
        if (n < 1) return pkv_internal_fail(PKV_EINVAL, "pkv_plan_decode: a sequence has no token");
        if (tlen < ceil_div(n, block_size))
            return pkv_internal_fail(PKV_EINVAL, "pkv_plan_decode: block table shorter than the sequence");
        if (tlen > INT32_MAX) return pkv_internal_fail(PKV_EINVAL, "pkv_plan_decode: table too long");
        L.total_k += n;
        if (n > L.max_seqlen_k) L.max_seqlen_k = (int32_t)n;
        if (tlen > L.max_blocks_per_seq) L.max_blocks_per_seq = (int32_t)tlen;
    }
    L.has_block_tables = num_seqs > 0;
    finish_layout(&L, false);
    *layout = L;
    return PKV_OK;
}

extern "C" int pkv_pack_decode(int32_t num_seqs, const int32_t *seq_lens, const int32_t *bt_ids,
                               const int64_t *bt_offsets, int32_t block_size,
                               const pkv_batch_layout *layout, void *host_buf,
                               size_t host_bytes) {
    if (!layout || !host_buf || layout->num_seqs != num_seqs || layout->is_prefill)
        return pkv_internal_fail(PKV_EINVAL, "pkv_pack_decode: layout does not match the batch");
    if ((int64_t)host_bytes < layout->total_bytes)
        return pkv_internal_fail(PKV_ENOSPACE, "pkv_pack_decode: host buffer too small");
    char *buf = (char *)host_buf;
    int32_t *slots = (int32_t *)(buf + layout->off_slot_mapping);
    int32_t *ctx = (int32_t *)(buf + layout->off_context_lens);
    int32_t *pos = (int32_t *)(buf + layout->off_positions);
    for (int32_t s = 0; s < num_seqs; ++s) {
        const int64_t n = seq_lens[s];
        const int64_t last_block = (n - 1) / block_size;       // logical block of position n-1
        const int64_t in_block = n - last_block * block_size;  // tokens in that block
        const int32_t blk = bt_ids[bt_offsets[s] + last_block];
        const int64_t slot = (int64_t)blk * block_size + in_block - 1;
        if (blk < 0 || slot > INT32_MAX)
            return pkv_internal_fail(PKV_EINVAL, "pkv_pack_decode: block id out of range");
        slots[s] = (int32_t)slot;
        ctx[s] = (int32_t)n;
        pos[s] = (int32_t)(n - 1);
    }
    if (layout->has_block_tables) write_tables(layout, bt_ids, bt_offsets, buf);
    return PKV_OK;
}
