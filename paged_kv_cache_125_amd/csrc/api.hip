// api.hip -- the extern "C" entry points of libpkv (declared in include/pkv.h):
// host-side validation, launch configuration and workspace layout. No device
// memory is allocated and nothing synchronises; the one library-owned device
// buffer is the static decode scratch below.
#include <stdarg.h>
#include <stdio.h>

#include <mutex>

#include <math.h>

#include "pkv.h"
#include "pkv_internal.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return code;
}

int launched(hipError_t e, const char *what) {
    if (e == hipErrorNotSupported)
        return fail(PKV_EUNSUPPORTED, "%s: no kernel for this dtype/shape", what);
    if (e != hipSuccess) return fail(PKV_ELAUNCH, "%s: launch failed: %s", what, hipGetErrorString(e));
    return PKV_OK;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }
bool is_pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }
int ilog2(int64_t x) {
    int r = 0;
    while ((int64_t(1) << r) < x) ++r;
    return r;
}
int elem_size(int32_t dtype) { return dtype == PKV_F32 ? 4 : 2; }
bool dtype_ok(int32_t dtype) { return dtype == PKV_F32 || dtype == PKV_BF16; }

int64_t align256(int64_t x) { return (x + 255) & ~int64_t(255); }

}  // namespace

extern "C" int pkv_abi_version(void) { return PKV_ABI_VERSION; }

extern "C" const char *pkv_last_error(void) { return g_err; }

extern "C" int pkv_store_kvcache(const void *k, const void *v, int64_t k_token_stride,
                                 int64_t v_token_stride, void *k_cache, void *v_cache,
                                 const int32_t *slot_mapping, int32_t num_tokens,
                                 int32_t num_blocks, int32_t block_size, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t dtype, void *stream) {
    const char *fn = "pkv_store_kvcache";
    if (!dtype_ok(dtype)) return fail(PKV_EINVAL, "%s: unknown dtype %d", fn, dtype);
    if (num_tokens < 0) return fail(PKV_EINVAL, "%s: num_tokens < 0", fn);
    if (num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || num_blocks <= 0)
        return fail(PKV_EINVAL, "%s: non-positive shape", fn);
    const int64_t num_slots = (int64_t)num_blocks * block_size;
    if (num_slots > INT32_MAX) return fail(PKV_EINVAL, "%s: pool has more than 2^31-1 slots", fn);
    const int es = elem_size(dtype);
    const int64_t row = (int64_t)num_kv_heads * head_dim;
    if ((row * es) % 16) return fail(PKV_EUNSUPPORTED, "%s: row bytes not a multiple of 16", fn);
    if (k_token_stride < row || v_token_stride < row)
        return fail(PKV_EINVAL, "%s: token stride smaller than a row", fn);
    if ((k_token_stride * es) % 16 || (v_token_stride * es) % 16)
        return fail(PKV_EINVAL, "%s: token strides must be multiples of 16 bytes", fn);
    if (num_tokens == 0) return PKV_OK;
    if (!k || !v || !k_cache || !v_cache || !slot_mapping)
        return fail(PKV_EINVAL, "%s: null pointer", fn);
    if (!aligned16(k) || !aligned16(v) || !aligned16(k_cache) || !aligned16(v_cache))
        return fail(PKV_EINVAL, "%s: pointers must be 16-byte aligned", fn);
    pkv::StoreArgs a;
    a.k = (const uint8_t *)k;
    a.v = (const uint8_t *)v;
    a.k_stride_bytes = k_token_stride * es;
    a.v_stride_bytes = v_token_stride * es;
    a.kc = (uint8_t *)k_cache;
    a.vc = (uint8_t *)v_cache;
    a.slots = slot_mapping;
    a.num_tokens = num_tokens;
    a.chunks_per_row = (int32_t)(row * es / 16);
    a.num_slots = num_slots;
    return launched(pkv::launch_store(a, (hipStream_t)stream), fn);
}

extern "C" int pkv_rope_cos_sin_table(float *host_out, int32_t max_positions, int32_t rot_dim,
                                      double base) {
    const char *fn = "pkv_rope_cos_sin_table";
    if (!host_out) return fail(PKV_EINVAL, "%s: null pointer", fn);
    if (max_positions < 1 || rot_dim < 2 || (rot_dim & 1))
        return fail(PKV_EINVAL, "%s: need max_positions >= 1 and an even rot_dim >= 2", fn);
    if (!(base > 0.0) || base == INFINITY) return fail(PKV_EINVAL, "%s: base must be positive", fn);
    const int half = rot_dim / 2;
    for (int32_t j = 0; j < half; ++j) {
        // theta_j(p) = p * base^(-2j / rot_dim), in double
        const double inv_freq = pow(base, -(2.0 * j) / rot_dim);
        for (int64_t p = 0; p < max_positions; ++p) {
            const double ang = (double)p * inv_freq;
            host_out[p * rot_dim + j] = (float)cos(ang);
            host_out[p * rot_dim + half + j] = (float)sin(ang);
        }
    }
    return PKV_OK;
}

extern "C" int pkv_rope_store_kvcache(void *q, int64_t q_token_stride, void *k, const void *v,
                                      int64_t k_token_stride, int64_t v_token_stride,
                                      void *k_cache, void *v_cache, const int32_t *slot_mapping,
                                      const int32_t *positions, const float *cos_sin,
                                      int32_t max_positions, int32_t rot_dim, int32_t style,
                                      int32_t write_k, int32_t num_tokens, int32_t num_blocks,
                                      int32_t block_size, int32_t num_q_heads,
                                      int32_t num_kv_heads, int32_t head_dim, int32_t dtype,
                                      void *stream) {
    const char *fn = "pkv_rope_store_kvcache";
    if (!dtype_ok(dtype)) return fail(PKV_EINVAL, "%s: unknown dtype %d", fn, dtype);
    if (num_tokens < 0) return fail(PKV_EINVAL, "%s: num_tokens < 0", fn);
    if (num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || num_blocks <= 0)
        return fail(PKV_EINVAL, "%s: non-positive shape", fn);
    if (style != PKV_ROPE_HALF && style != PKV_ROPE_INTERLEAVED)
        return fail(PKV_EINVAL, "%s: unknown style %d", fn, style);
    if (max_positions < 1) return fail(PKV_EINVAL, "%s: max_positions < 1", fn);
    const int es = elem_size(dtype);
    const int V = 16 / es;   // elements per 16-byte chunk
    if (rot_dim < 2 || (rot_dim & 1) || rot_dim > head_dim)
        return fail(PKV_EINVAL, "%s: rot_dim must be even and in [2, head_dim]", fn);
    if ((head_dim * es) % 16 || rot_dim % (style == PKV_ROPE_HALF ? 2 * V : V))
        return fail(PKV_EUNSUPPORTED, "%s: head_dim or rot_dim not a whole number of 16-byte chunks", fn);
    const int64_t num_slots = (int64_t)num_blocks * block_size;
    if (num_slots > INT32_MAX) return fail(PKV_EINVAL, "%s: pool has more than 2^31-1 slots", fn);
    const int64_t qrow = (int64_t)num_q_heads * head_dim, kvrow = (int64_t)num_kv_heads * head_dim;
    if (q_token_stride < qrow || k_token_stride < kvrow || v_token_stride < kvrow)
        return fail(PKV_EINVAL, "%s: token stride smaller than a row", fn);
    if ((q_token_stride * es) % 16 || (k_token_stride * es) % 16 || (v_token_stride * es) % 16)
        return fail(PKV_EINVAL, "%s: token strides must be multiples of 16 bytes", fn);
    if (num_tokens == 0) return PKV_OK;
    if (!q || !k || !v || !k_cache || !v_cache || !slot_mapping || !positions || !cos_sin)
        return fail(PKV_EINVAL, "%s: null pointer", fn);
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(k_cache) ||
        !aligned16(v_cache) || !aligned16(cos_sin))
        return fail(PKV_EINVAL, "%s: pointers must be 16-byte aligned", fn);
    pkv::RopeStoreArgs a;
    a.q = (uint8_t *)q;
    a.k = (uint8_t *)k;
    a.v = (const uint8_t *)v;
    a.q_stride_bytes = q_token_stride * es;
    a.k_stride_bytes = k_token_stride * es;
    a.v_stride_bytes = v_token_stride * es;
    a.kc = (uint8_t *)k_cache;
    a.vc = (uint8_t *)v_cache;
    a.slots = slot_mapping;
    a.positions = positions;
    a.cos_sin = cos_sin;
    a.max_positions = max_positions;
    a.rot_dim = rot_dim;
    a.style = style;
    a.write_k = write_k != 0;
    a.d = head_dim;
    a.row_bytes = kvrow * es;
    a.num_slots = num_slots;
    a.r_items = style == PKV_ROPE_HALF ? rot_dim / (2 * V) : rot_dim / V;
    a.p_items = (head_dim - rot_dim) / V;
    a.q_items = num_q_heads * a.r_items;
    a.k_items = num_kv_heads * (a.r_items + a.p_items);
    a.items_per_token = a.q_items + a.k_items + (int32_t)(kvrow * es / 16);
    a.total_items = (int64_t)num_tokens * a.items_per_token;
    return launched(pkv::launch_rope_store(a, dtype, (hipStream_t)stream), fn);
}

static int check_attention_shape(const char *fn, int32_t dtype, int32_t Hq, int32_t Hkv,
                                 int32_t d, int32_t num_seqs, float scale) {
    if (!dtype_ok(dtype)) return fail(PKV_EINVAL, "%s: unknown dtype %d", fn, dtype);
    if (!(scale > 0.f) || scale == INFINITY) return fail(PKV_EINVAL, "%s: scale must be positive and finite", fn);
    if (Hq <= 0 || Hkv <= 0 || Hq % Hkv)
        return fail(PKV_EINVAL, "%s: num_q_heads must be a positive multiple of num_kv_heads", fn);
    if (d != 64 && d != 128) return fail(PKV_EUNSUPPORTED, "%s: head_dim must be 64 or 128", fn);
    if (num_seqs < 0 || num_seqs > 65535) return fail(PKV_EINVAL, "%s: num_seqs out of [0, 65535]", fn);
    return PKV_OK;
}

static int check_pool(const char *fn, const void *kc, const void *vc, const int32_t *bt,
                      int32_t maxb, int32_t num_blocks, int32_t bs) {
    if (!kc || !vc || !bt) return fail(PKV_EINVAL, "%s: null cache or block table", fn);
    if (!aligned16(kc) || !aligned16(vc)) return fail(PKV_EINVAL, "%s: caches must be 16-byte aligned", fn);
    if (!is_pow2(bs) || bs > 1024) return fail(PKV_EINVAL, "%s: block_size must be a power of two <= 1024", fn);
    if (num_blocks <= 0 || maxb <= 0) return fail(PKV_EINVAL, "%s: num_blocks and max_blocks_per_seq must be positive", fn);
    if ((int64_t)num_blocks * bs > INT32_MAX) return fail(PKV_EINVAL, "%s: pool has more than 2^31-1 slots", fn);
    return PKV_OK;
}

// The two prefill entry points; st is the fused store's destination (null
// for plain attention).
struct PrefillStore {
    void *kc, *vc;
    const int32_t *slots;
    int32_t num_slots;
};

static int prefill_call(
    const char *fn, const void *q, int64_t q_token_stride, const void *k, const void *v,
    int64_t kv_token_stride, const void *k_cache, const void *v_cache, const int32_t *block_tables,
    int32_t max_blocks_per_seq, const int32_t *cu_seqlens_q, const int32_t *cu_seqlens_k,
    int32_t num_seqs, int32_t total_q, int32_t max_seqlen_q, int32_t max_seqlen_k,
    int32_t num_blocks, int32_t block_size, int32_t num_q_heads, int32_t num_kv_heads,
    int32_t head_dim, float scale, int32_t dtype, void *out, void *workspace,
    size_t workspace_bytes, const PrefillStore *st, void *stream) {
    int rc = check_attention_shape(fn, dtype, num_q_heads, num_kv_heads, head_dim, num_seqs, scale);
    if (rc) return rc;
    if (total_q < 0 || max_seqlen_q < 0 || max_seqlen_k < 0)
        return fail(PKV_EINVAL, "%s: negative length", fn);
    if (max_seqlen_q > max_seqlen_k && block_tables)
        return fail(PKV_EINVAL, "%s: max_seqlen_q > max_seqlen_k", fn);
    if (num_seqs == 0 || total_q == 0 || max_seqlen_q == 0) return PKV_OK;
    if (!q || !out || !cu_seqlens_q || !cu_seqlens_k) return fail(PKV_EINVAL, "%s: null pointer", fn);
    const int es = elem_size(dtype);
    if (q_token_stride < (int64_t)num_q_heads * head_dim)
        return fail(PKV_EINVAL, "%s: q token stride smaller than a row", fn);
    if (!aligned16(q) || !aligned16(out) || (q_token_stride * es) % 16)
        return fail(PKV_EINVAL, "%s: q/out must be 16-byte aligned with 16-byte strides", fn);
    if (workspace) {
        if (workspace_bytes < pkv::kPrefillWorkspaceBytes)
            return fail(PKV_ENOSPACE, "%s: workspace needs %zu bytes", fn, pkv::kPrefillWorkspaceBytes);
        if ((uintptr_t)workspace & 255u) return fail(PKV_EINVAL, "%s: workspace must be 256-byte aligned", fn);
    } else if (workspace_bytes) {
        return fail(PKV_EINVAL, "%s: null workspace with a nonzero size", fn);
    }
    pkv::PrefillArgs a;
    a.work_ctr = (uint32_t *)workspace;
    a.q = q;
    a.q_stride = q_token_stride;
    a.paged = block_tables != nullptr;
    if (a.paged) {
        rc = check_pool(fn, k_cache, v_cache, block_tables, max_blocks_per_seq, num_blocks, block_size);
        if (rc) return rc;
    }
    if (a.paged && !st) {
        a.k = a.v = nullptr;
        a.kv_stride = 0;
    } else {
        // the keys' rows (no block tables), or the rows the fused store writes
        if (!k || !v) return fail(PKV_EINVAL, "%s: null k/v without block tables", fn);
        if (kv_token_stride < (int64_t)num_kv_heads * head_dim)
            return fail(PKV_EINVAL, "%s: kv token stride smaller than a row", fn);
        if (!aligned16(k) || !aligned16(v) || (kv_token_stride * es) % 16)
            return fail(PKV_EINVAL, "%s: k/v must be 16-byte aligned with 16-byte strides", fn);
        a.k = k;
        a.v = v;
        a.kv_stride = kv_token_stride;
    }
    a.kc = k_cache;
    a.vc = v_cache;
    a.bt = block_tables;
    a.maxb = max_blocks_per_seq;
    a.cu_q = cu_seqlens_q;
    a.cu_k = cu_seqlens_k;
    a.num_seqs = num_seqs;
    a.num_blocks = num_blocks;
    a.bs = a.paged ? block_size : 1;
    a.log2bs = ilog2(a.bs);
    a.Hq = num_q_heads;
    a.Hkv = num_kv_heads;
    a.d = head_dim;
    a.group = num_q_heads / num_kv_heads;
    a.scale_log2 = scale * 1.4426950408889634f;
    a.out = out;
    a.max_seqlen_q = max_seqlen_q;
    a.max_seqlen_k = max_seqlen_k;
    a.total_q = total_q;
    if (st) {
        a.store_kc = st->kc;
        a.store_vc = st->vc;
        a.slots = st->slots;
        a.num_slots = st->num_slots;
    }
    // Longest query blocks first across pairs when the batch's K/V fits in half
    // the 256 MB MALL: contiguous keys are the call's own rows, paged keys are
    // bounded by num_seqs * max_seqlen_k.
    {
        const int64_t keys = a.paged ? (int64_t)num_seqs * max_seqlen_k : (int64_t)total_q;
        a.by_rank = keys * num_kv_heads * head_dim * 2 * 2 <= (int64_t(128) << 20);
    }
    return launched(pkv::launch_prefill(a, dtype, (hipStream_t)stream), fn);
}

extern "C" int pkv_prefill_attention_varlen(
    const void *q, int64_t q_token_stride, const void *k, const void *v, int64_t kv_token_stride,
    const void *k_cache, const void *v_cache, const int32_t *block_tables,
    int32_t max_blocks_per_seq, const int32_t *cu_seqlens_q, const int32_t *cu_seqlens_k,
    int32_t num_seqs, int32_t total_q, int32_t max_seqlen_q, int32_t max_seqlen_k,
    int32_t num_blocks, int32_t block_size, int32_t num_q_heads, int32_t num_kv_heads,
    int32_t head_dim, float scale, int32_t dtype, void *out, void *workspace,
    size_t workspace_bytes, void *stream) {
    return prefill_call("pkv_prefill_attention_varlen", q, q_token_stride, k, v, kv_token_stride,
                        k_cache, v_cache, block_tables, max_blocks_per_seq, cu_seqlens_q,
                        cu_seqlens_k, num_seqs, total_q, max_seqlen_q, max_seqlen_k, num_blocks,
                        block_size, num_q_heads, num_kv_heads, head_dim, scale, dtype, out,
                        workspace, workspace_bytes, nullptr, stream);
}

extern "C" int pkv_prefill_store_attention_varlen(
    const void *q, int64_t q_token_stride, const void *k, const void *v, int64_t kv_token_stride,
    void *k_cache, void *v_cache, const int32_t *slot_mapping, const int32_t *block_tables,
    int32_t max_blocks_per_seq, const int32_t *cu_seqlens_q, const int32_t *cu_seqlens_k,
    int32_t num_seqs, int32_t total_q, int32_t max_seqlen_q, int32_t max_seqlen_k,
    int32_t num_blocks, int32_t block_size, int32_t num_q_heads, int32_t num_kv_heads,
    int32_t head_dim, float scale, int32_t dtype, void *out, void *stream) {
    const char *fn = "pkv_prefill_store_attention_varlen";
    if (!dtype_ok(dtype)) return fail(PKV_EINVAL, "%s: unknown dtype %d", fn, dtype);
    if (block_size <= 0 || num_blocks <= 0) return fail(PKV_EINVAL, "%s: non-positive pool shape", fn);
    const int64_t num_slots = (int64_t)num_blocks * block_size;
    if (num_slots > INT32_MAX) return fail(PKV_EINVAL, "%s: pool has more than 2^31-1 slots", fn);
    if (num_kv_heads > 0 && head_dim > 0 && ((int64_t)num_kv_heads * head_dim * elem_size(dtype)) % 16)
        return fail(PKV_EUNSUPPORTED, "%s: row bytes not a multiple of 16", fn);
    if (total_q > 0 && num_seqs > 0 && max_seqlen_q > 0) {
        if (!k || !v) return fail(PKV_EINVAL, "%s: null k/v", fn);
        if (!k_cache || !v_cache || !slot_mapping) return fail(PKV_EINVAL, "%s: null cache or slot_mapping", fn);
        if (!aligned16(k_cache) || !aligned16(v_cache))
            return fail(PKV_EINVAL, "%s: caches must be 16-byte aligned", fn);
    }
    const PrefillStore st = {k_cache, v_cache, slot_mapping, (int32_t)num_slots};
    // With block tables the attention reads the pool and the call's k/v rows
    // both; without, only the rows.
    return prefill_call(fn, q, q_token_stride, k, v, kv_token_stride, block_tables ? k_cache : nullptr,
                        block_tables ? v_cache : nullptr, block_tables, max_blocks_per_seq,
                        cu_seqlens_q, cu_seqlens_k, num_seqs, total_q, max_seqlen_q, max_seqlen_k,
                        num_blocks, block_size, num_q_heads, num_kv_heads, head_dim, scale, dtype,
                        out, nullptr, 0, &st, stream);
}

extern "C" size_t pkv_prefill_workspace_bytes(int32_t, int32_t, int32_t, int32_t, int32_t, int32_t) {
    return pkv::kPrefillWorkspaceBytes;
}

extern "C" int32_t pkv_decode_partition_size(int32_t num_seqs, int32_t max_context_len,
                                             int32_t num_q_heads, int32_t num_kv_heads,
                                             int32_t head_dim, int32_t block_size, int32_t dtype,
                                             int32_t partition_size) {
    const pkv::DecodePlan p = pkv::plan_decode(num_seqs, max_context_len, num_q_heads, num_kv_heads,
                                               head_dim, block_size, dtype, partition_size);
    return p.balanced ? 0 : p.P;
}

extern "C" size_t pkv_decode_workspace_bytes(int32_t num_seqs, int32_t max_context_len,
                                             int32_t num_q_heads, int32_t num_kv_heads,
                                             int32_t head_dim, int32_t block_size, int32_t dtype,
                                             int32_t partition_size) {
    if (num_seqs <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0) return 0;
    return (size_t)pkv::plan_decode(num_seqs, max_context_len, num_q_heads, num_kv_heads, head_dim,
                                    block_size, dtype, partition_size).total;
}

// ---------------------------------------------------------------------------
// Library-owned scratch for pkv_decode_attention_paged_noalloc: the decode
// workspace (partial results and the split's prefix sums) for callers that
// cannot allocate device memory. Each device holds one copy of this array for
// the life of the process. In host code `scratch` only names the array for the
// runtime; its address on a device comes from hipGetSymbolAddress, looked up
// once per device with that device current, and only that address reaches a
// kernel.
constexpr size_t kNoAllocScratchBytes = PKV_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_addr[kMaxDevices];   // device address of `scratch`, per device

// The current device's copy of `scratch`.
int scratch_address(const char *fn, void **out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(PKV_ELAUNCH, "%s: hipGetDevice: %s", fn, hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(PKV_EUNSUPPORTED, "%s: device %d", fn, dev);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_addr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(PKV_ELAUNCH, "%s: hipGetSymbolAddress: %s", fn, hipGetErrorString(e));
        g_scratch_addr[dev] = p;
    }
    *out = g_scratch_addr[dev];
    return PKV_OK;
}

// Shared body of the two decode entry points. With use_scratch the workspace
// is the current device's `scratch` (the plan must fit in it), otherwise the
// caller's.
int decode_call(const char *fn, const void *q, int64_t q_token_stride, const void *k_cache,
                const void *v_cache, const int32_t *block_tables, int32_t max_blocks_per_seq,
                const int32_t *context_lens, int32_t num_seqs, int32_t max_context_len,
                int32_t num_blocks, int32_t block_size, int32_t num_q_heads, int32_t num_kv_heads,
                int32_t head_dim, float scale, int32_t dtype, void *out, int32_t partition_size,
                void *workspace, size_t workspace_bytes, bool use_scratch, void *stream,
                const pkv::StoreArgs *st = nullptr) {
    int rc = check_attention_shape(fn, dtype, num_q_heads, num_kv_heads, head_dim, num_seqs, scale);
    if (rc) return rc;
    if (max_context_len < 0) return fail(PKV_EINVAL, "%s: negative max_context_len", fn);
    if ((partition_size < 0 && partition_size != PKV_PARTITION_BALANCED) || (partition_size > 0 && partition_size % 16))
        return fail(PKV_EINVAL, "%s: partition_size must be 0, PKV_PARTITION_BALANCED or a positive multiple of 16", fn);
    if (num_seqs == 0) return PKV_OK;
    if (!q || !out || !context_lens) return fail(PKV_EINVAL, "%s: null pointer", fn);
    rc = check_pool(fn, k_cache, v_cache, block_tables, max_blocks_per_seq, num_blocks, block_size);
    if (rc) return rc;
    const int es = elem_size(dtype);
    if (q_token_stride < (int64_t)num_q_heads * head_dim)
        return fail(PKV_EINVAL, "%s: q token stride smaller than a row", fn);
    if (!aligned16(q) || !aligned16(out) || (q_token_stride * es) % 16)
        return fail(PKV_EINVAL, "%s: q/out must be 16-byte aligned with 16-byte strides", fn);
    const pkv::DecodePlan ws = pkv::plan_decode(num_seqs, max_context_len, num_q_heads, num_kv_heads,
                                                head_dim, block_size, dtype, partition_size);
    if (use_scratch) {
        if (ws.total > (int64_t)kNoAllocScratchBytes)
            return fail(PKV_ENOSPACE, "%s: needs %lld bytes of scratch, more than the library's %zu",
                        fn, (long long)ws.total, kNoAllocScratchBytes);
        workspace = nullptr;
        workspace_bytes = kNoAllocScratchBytes;
        if (ws.total > 0) {
            rc = scratch_address(fn, &workspace);
            if (rc) return rc;
        }
    }
    if ((int64_t)workspace_bytes < ws.total)
        return fail(PKV_ENOSPACE, "%s: workspace needs %lld bytes", fn, (long long)ws.total);
    if (ws.total > 0 && (!workspace || ((uintptr_t)workspace & 255u)))
        return fail(PKV_EINVAL, "%s: workspace must be non-null and 256-byte aligned", fn);
    pkv::DecodeArgs a;
    a.q = q;
    a.q_stride = q_token_stride;
    a.kc = k_cache;
    a.vc = v_cache;
    a.bt = block_tables;
    a.maxb = max_blocks_per_seq;
    a.ctx = context_lens;
    a.ctx_cap = max_context_len;
    a.num_seqs = num_seqs;
    a.num_blocks = num_blocks;
    a.bs = block_size;
    a.log2bs = ilog2(block_size);
    a.Hq = num_q_heads;
    a.Hkv = num_kv_heads;
    a.d = head_dim;
    a.group = num_q_heads / num_kv_heads;
    a.scale_log2 = scale * 1.4426950408889634f;
    a.out = out;
    a.P = ws.P;
    a.maxparts = ws.maxparts;
    a.waves = ws.waves;
    a.ws_acc = ws.total ? (float *)workspace : nullptr;
    a.ws_ml = ws.total ? (float *)((char *)workspace + ws.acc_bytes) : nullptr;
    a.ws_cum = ws.cum_bytes ? (int32_t *)((char *)workspace + ws.acc_bytes + ws.ml_bytes) : nullptr;
    if (st) {
        // Fused where the fixed-partition kernel runs; otherwise the store
        // kernel first, on the same stream, then the attention.
        if (pkv::decode_store_fusable(a, ws, dtype)) {
            a.st_k = st->k;
            a.st_v = st->v;
            a.st_stride_bytes = st->k_stride_bytes;
            a.st_kc = st->kc;
            a.st_vc = st->vc;
            a.st_slots = st->slots;
            a.st_num_slots = st->num_slots;
        } else {
            rc = launched(pkv::launch_store(*st, (hipStream_t)stream), fn);
            if (rc) return rc;
        }
    }
    return launched(pkv::launch_decode(a, ws, dtype, (hipStream_t)stream), fn);
}

}  // namespace

extern "C" int pkv_decode_attention_paged(
    const void *q, int64_t q_token_stride, const void *k_cache, const void *v_cache,
    const int32_t *block_tables, int32_t max_blocks_per_seq, const int32_t *context_lens,
    int32_t num_seqs, int32_t max_context_len, int32_t num_blocks, int32_t block_size,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, float scale, int32_t dtype,
    void *out, int32_t partition_size, void *workspace, size_t workspace_bytes, void *stream) {
    return decode_call("pkv_decode_attention_paged", q, q_token_stride, k_cache, v_cache,
                       block_tables, max_blocks_per_seq, context_lens, num_seqs, max_context_len,
                       num_blocks, block_size, num_q_heads, num_kv_heads, head_dim, scale, dtype,
                       out, partition_size, workspace, workspace_bytes, false, stream);
}

extern "C" int pkv_decode_attention_paged_noalloc(
    const void *q, int64_t q_token_stride, const void *k_cache, const void *v_cache,
    const int32_t *block_tables, int32_t max_blocks_per_seq, const int32_t *context_lens,
    int32_t num_seqs, int32_t max_context_len, int32_t num_blocks, int32_t block_size,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, float scale, int32_t dtype,
    void *out, int32_t partition_size, void *stream) {
    return decode_call("pkv_decode_attention_paged_noalloc", q, q_token_stride, k_cache, v_cache,
                       block_tables, max_blocks_per_seq, context_lens, num_seqs, max_context_len,
                       num_blocks, block_size, num_q_heads, num_kv_heads, head_dim, scale, dtype,
                       out, partition_size, nullptr, 0, true, stream);
}

extern "C" int pkv_decode_store_attention_paged(
    const void *q, int64_t q_token_stride, const void *k, const void *v, int64_t kv_token_stride,
    void *k_cache, void *v_cache, const int32_t *slot_mapping, const int32_t *block_tables,
    int32_t max_blocks_per_seq, const int32_t *context_lens, int32_t num_seqs,
    int32_t max_context_len, int32_t num_blocks, int32_t block_size, int32_t num_q_heads,
    int32_t num_kv_heads, int32_t head_dim, float scale, int32_t dtype, void *out,
    int32_t partition_size, void *workspace, size_t workspace_bytes, void *stream) {
    const char *fn = "pkv_decode_store_attention_paged";
    if (!dtype_ok(dtype)) return fail(PKV_EINVAL, "%s: unknown dtype %d", fn, dtype);
    if (num_seqs > 0) {
        if (!k || !v || !slot_mapping) return fail(PKV_EINVAL, "%s: null k, v or slot_mapping", fn);
        if (num_kv_heads <= 0 || head_dim <= 0) return fail(PKV_EINVAL, "%s: non-positive shape", fn);
        const int es = elem_size(dtype);
        const int64_t row = (int64_t)num_kv_heads * head_dim;
        if ((row * es) % 16) return fail(PKV_EUNSUPPORTED, "%s: row bytes not a multiple of 16", fn);
        if (kv_token_stride < row) return fail(PKV_EINVAL, "%s: k/v token stride smaller than a row", fn);
        if ((kv_token_stride * es) % 16) return fail(PKV_EINVAL, "%s: k/v token stride not a multiple of 16 bytes", fn);
        if (!aligned16(k) || !aligned16(v)) return fail(PKV_EINVAL, "%s: k/v must be 16-byte aligned", fn);
        if (block_size <= 0 || num_blocks <= 0 || (int64_t)num_blocks * block_size > INT32_MAX)
            return fail(PKV_EINVAL, "%s: pool shape", fn);
    }
    pkv::StoreArgs st;
    const int es = elem_size(dtype);
    st.k = (const uint8_t *)k;
    st.v = (const uint8_t *)v;
    st.k_stride_bytes = st.v_stride_bytes = kv_token_stride * es;
    st.kc = (uint8_t *)k_cache;
    st.vc = (uint8_t *)v_cache;
    st.slots = slot_mapping;
    st.num_tokens = num_seqs;
    st.chunks_per_row = (int32_t)((int64_t)num_kv_heads * head_dim * es / 16);
    st.num_slots = (int64_t)num_blocks * block_size;
    return decode_call(fn, q, q_token_stride, k_cache, v_cache, block_tables, max_blocks_per_seq,
                       context_lens, num_seqs, max_context_len, num_blocks, block_size, num_q_heads,
                       num_kv_heads, head_dim, scale, dtype, out, partition_size, workspace,
                       workspace_bytes, false, stream, &st);
}

extern "C" int pkv_upload(const void *host_buf, void *dev_buf, size_t bytes, void *stream) {
    if (bytes == 0) return PKV_OK;
    if (!host_buf || !dev_buf) return fail(PKV_EINVAL, "pkv_upload: null pointer");
    hipError_t e = hipMemcpyAsync(dev_buf, host_buf, bytes, hipMemcpyHostToDevice, (hipStream_t)stream);
    if (e != hipSuccess) return fail(PKV_ELAUNCH, "pkv_upload: %s", hipGetErrorString(e));
    return PKV_OK;
}

// Used by the packers (pack.cpp) to report errors through pkv_last_error.
int pkv_internal_fail(int code, const char *msg) { return fail(code, "%s", msg); }
