/*
 * pkv.h -- C ABI of libpkv, the paged-KV attention hot path for AMD MI355X
 * (gfx950, CDNA4).
 *
 * The pages this follows (cited by title and section):
 *  [NV1] "nano-vLLM-1" (senjlearning.space): "3. KV cache 分配" (the per-layer
 *        cache view [num_blocks, block_size, kv_heads, head_dim]),
 *        "4. prefill 输入打包" (prepare_block_tables, prepare_prefill),
 *        "5. deocde 输入打包" (prepare_decode and why prefill needs block
 *        tables only on a prefix hit), BlockManager "3. 核心方法一：分配"
 *        (the slot of position p is block_table[p / bs] * bs + p % bs).
 *  [MR]  "Nano vLLM 解读（5）：解析 ModelRunner" (languisher.top):
 *        "FlashAttention Kernel 函参准备" (the three groups of kernel inputs),
 *        "prepare_prefill" / "prepare_decode" (cu_seqlens, slot_mapping,
 *        block_tables, context_lens), and the ModelRunner init (attention
 *        writes new K/V through slot_mapping and reads history through
 *        block_tables).
 *  [ES]  "【nano-vllm 学习】04 - 自顶向下的引擎调度层源码学习2" (kyonqi.github.io):
 *        "KV-Cache … 是什么？" (softmax(QK^T / sqrt(d_k)) V with a causal mask)
 *        and "PageAttention" (blocks as pages, block_table as page table).
 *
 * Conventions for every device entry point:
 *  - All device pointers are caller-owned and must stay valid until the stream
 *    reaches the call. The library never synchronises and allocates no device
 *    memory; the only device memory it owns is the fixed scratch array of
 *    pkv_decode_attention_paged_noalloc, the only state kept between calls.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *  - Tensors are row-major; strides are in ELEMENTS. The caches are the
 *    per-layer views [num_blocks, block_size, num_kv_heads, head_dim],
 *    contiguous.
 *  - Every call validates its host-side arguments and returns a pkv_status;
 *    on failure nothing is launched and pkv_last_error() describes why.
 *    Device-resident metadata (slots, block tables, lengths) is not read on
 *    the host. A slot outside [0, num_blocks*block_size) is skipped by the
 *    store; a block-table entry outside [0, num_blocks), or a length beyond
 *    what the table covers, makes the affected output rows unspecified but
 *    never causes an access outside the caches.
 *  - Thread-safe across host threads and streams; calls that overlap on one
 *    stream are ordered by it.
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PKV_ABI_VERSION 6

typedef enum {
    PKV_OK = 0,
    PKV_EINVAL = 1,        /* an argument is outside its documented range     */
    PKV_EUNSUPPORTED = 2,  /* valid, but no kernel for this dtype/shape        */
    PKV_ELAUNCH = 3,       /* the HIP runtime reported an error on launch      */
    PKV_ENOSPACE = 4       /* a caller-provided buffer is too small            */
} pkv_status;

typedef enum {
    PKV_F32 = 0,           /* IEEE binary32                                     */
    PKV_BF16 = 1           /* bfloat16; accumulation is fp32                    */
} pkv_dtype;

/* PKV_ABI_VERSION of the loaded library. */
int pkv_abi_version(void);

/* Message for the last non-OK status returned on the calling host thread.
 * The pointer stays valid until the next call on that thread. */
const char *pkv_last_error(void);

/* ---------------------------------------------------------------------------
 * store_kvcache  ([MR] ModelRunner init and "prepare_prefill": slot_mapping
 * says where each new token's K/V is written; [NV1] "3. KV cache 分配" fixes
 * the cache view.)
 *
 * For i in [0, num_tokens): s = slot_mapping[i]; if 0 <= s < num_blocks *
 * block_size, copy k row i ([num_kv_heads, head_dim] elements) bit for bit to
 * k_cache viewed as [num_blocks * block_size, num_kv_heads, head_dim] row s,
 * and likewise v -> v_cache. Negative slots (padding) are skipped: nothing is
 * written for them (their k/v rows must still be readable memory).
 *
 *  k, v            [num_tokens, num_kv_heads, head_dim] with token strides
 *                  k_token_stride / v_token_stride (elements; the rows of one
 *                  token are contiguous). May be slices of a fused QKV buffer.
 *  k_cache,v_cache [num_blocks, block_size, num_kv_heads, head_dim].
 *  slot_mapping    device int32 [num_tokens]. Slots must be unique within a
 *                  call (each token owns its slot); duplicates leave the row
 *                  with one of the written values.
 *  dtype           PKV_F32 or PKV_BF16 (a bit copy: dtype only sizes rows).
 * Requires head_dim * num_kv_heads * element_size and the token strides to be
 * multiples of 16 bytes and all pointers 16-byte aligned. num_tokens == 0 is a
 * no-op. */
int pkv_store_kvcache(const void *k, const void *v, int64_t k_token_stride,
                      int64_t v_token_stride, void *k_cache, void *v_cache,
                      const int32_t *slot_mapping, int32_t num_tokens, int32_t num_blocks,
                      int32_t block_size, int32_t num_kv_heads, int32_t head_dim,
                      int32_t dtype, void *stream);

/* ---------------------------------------------------------------------------
 * prefill_attention_varlen  ([MR] "FlashAttention Kernel 函参准备" and
 * "prepare_prefill"; [NV1] "5. deocde 输入打包", block tables on a prefix hit;
 * [ES] the attention equation and causal mask.)
 *
 * Sequence s owns query rows [cu_seqlens_q[s], cu_seqlens_q[s+1]) and keys
 * [0, Lk_s) with Lk_s = cu_seqlens_k[s+1] - cu_seqlens_k[s] >= Lq_s. Query i
 * of sequence s sits at position Lk_s - Lq_s + i and attends to keys 0..that
 * position (bottom-right causal alignment; the diagonal is visible). For each
 * q head h, kv head h / (num_q_heads / num_kv_heads):
 *     out[row, h, :] = softmax(scale * q[row, h, :] . K^T) V
 *
 * Keys and values come from
 *  - block_tables == NULL: the call's contiguous k, v rows
 *    [cu_seqlens_k[s] + j] ([total_k, num_kv_heads, head_dim], token stride
 *    kv_token_stride). Requires Lk_s == Lq_s (no cached prefix).
 *  - block_tables != NULL: the caches, position j of sequence s at slot
 *    block_tables[s * max_blocks_per_seq + j / block_size] * block_size +
 *    j % block_size. The K/V of this call's tokens must already have been
 *    stored (pkv_store_kvcache on the same stream, before this call).
 *
 *  q               [total_q, num_q_heads, head_dim], token stride q_token_stride.
 *  out             [total_q, num_q_heads, head_dim], contiguous, q's dtype.
 *  cu_seqlens_q/_k device int32 [num_seqs + 1], prefix sums starting at 0.
 *                  The kernels never touch q or out rows outside [0, total_q),
 *                  nor contiguous k/v rows outside it: a sequence whose range
 *                  does not fit, or whose key count lies outside
 *                  [Lq_s, max_seqlen_k], is skipped (its out rows are left
 *                  unwritten).
 *  max_seqlen_q/_k host upper bounds of Lq_s / Lk_s (size the launch grid).
 *  dtype           PKV_BF16 (MFMA path for head_dim 128) or PKV_F32.
 *  workspace       NULL (with workspace_bytes 0): one workgroup per
 *                  (sequence, kv head, query block, query head) item, laid
 *                  out longest first so that the hardware's own dispatch
 *                  balances the batch; when no sequence has more than 64
 *                  query rows (32 with a group of 4 or more), 2 (or 4)
 *                  query heads of a GQA group share an item and every K/V
 *                  tile it stages. Non-NULL: device memory of
 *                  pkv_prefill_workspace_bytes() bytes, 256-byte aligned,
 *                  ZEROED ONCE when it is allocated, holding the counters of
 *                  the persistent grid: two workgroups per CU whatever the
 *                  batch, which claim items as they go. Each call leaves it
 *                  zeroed again when it completes, so it is reused call after
 *                  call without clearing; calls that may run at the same time
 *                  (on different streams) need workspaces of their own.
 *                  Batches beyond the persistent grid's tables (more than
 *                  2048 (sequence, kv head) pairs or 512 query blocks), and
 *                  batches whose query heads share items, take one
 *                  workgroup per item and leave the workspace untouched.
 *                  Both grids give bit-identical results; on the batches
 *                  measured so far the one-workgroup-per-item grid is the
 *                  faster one. Only the bf16 head_dim-128 kernel has the
 *                  persistent grid; the others ignore the workspace.
 * Requires num_q_heads % num_kv_heads == 0, head_dim in {64, 128}, a
 * positive finite scale, and block_size a power of two in [1, 1024] when
 * block_tables != NULL. PKV_ENOSPACE if a non-NULL workspace is smaller than
 * pkv_prefill_workspace_bytes(). */
int pkv_prefill_attention_varlen(const void *q, int64_t q_token_stride, const void *k,
                                 const void *v, int64_t kv_token_stride, const void *k_cache,
                                 const void *v_cache, const int32_t *block_tables,
                                 int32_t max_blocks_per_seq, const int32_t *cu_seqlens_q,
                                 const int32_t *cu_seqlens_k, int32_t num_seqs,
                                 int32_t total_q, int32_t max_seqlen_q, int32_t max_seqlen_k,
                                 int32_t num_blocks, int32_t block_size, int32_t num_q_heads,
                                 int32_t num_kv_heads, int32_t head_dim, float scale,
                                 int32_t dtype, void *out, void *workspace,
                                 size_t workspace_bytes, void *stream);

/* Workspace bytes pkv_prefill_attention_varlen needs (a constant 256: the
 * persistent grid's counters; the arguments are those of the call). */
size_t pkv_prefill_workspace_bytes(int32_t num_seqs, int32_t max_seqlen_q, int32_t num_q_heads,
                                   int32_t num_kv_heads, int32_t head_dim, int32_t dtype);

/* ---------------------------------------------------------------------------
 * prefill_store_attention_varlen: store_kvcache and prefill_attention_varlen
 * of one prefill step in one call ([MR] the attention layer's forward, which
 * writes the step's K/V through slot_mapping and then runs varlen attention;
 * "prepare_prefill" for the metadata; [NV1] "5. deocde 输入打包" for the
 * block tables on a prefix hit).
 *
 * The result equals pkv_store_kvcache(k, v, kv_token_stride, kv_token_stride,
 * k_cache, v_cache, slot_mapping, total_q, num_blocks, block_size, ...)
 * followed on the same stream by pkv_prefill_attention_varlen(q, ..., k, v,
 * kv_token_stride, k_cache, v_cache, block_tables, ...) with the same
 * arguments, provided the metadata agree the way pkv_pack_prefill lays them
 * out:
 *  - block_tables == NULL: the keys of sequence s are its own rows of k/v
 *    (Lk_s == Lq_s), as in pkv_prefill_attention_varlen.
 *  - block_tables != NULL: positions below Lk_s - Lq_s are read from the
 *    caches through the block table; the later ones -- the tokens this call
 *    stores -- are read from the call's rows, position Lk_s - Lq_s + i from
 *    row cu_seqlens_q[s] + i, instead of from the slots they are stored to.
 *    The two forms agree when slot_mapping[cu_seqlens_q[s] + i] is the slot
 *    of that position under sequence s's block table.
 *
 * For bf16 and head_dim 128 (block_size >= 16 with block tables) this is one
 * launch: after its attention, each query block copies its own rows of k/v
 * into their slots (the group's query heads share the copy; the rows were
 * read for the block's last key tiles moments before). Other shapes run the
 * store kernel and then the attention kernel. Rows outside every sequence's
 * range, and rows of a sequence the attention skips (see
 * pkv_prefill_attention_varlen), may be left unstored; with metadata from
 * pkv_pack_prefill every row is stored. The call reads no slot it writes.
 *
 *  q, out, cu_seqlens_q/_k, max_seqlen_q/_k, block_tables, max_blocks_per_seq:
 *                  as in pkv_prefill_attention_varlen.
 *  k, v            [total_q, num_kv_heads, head_dim], token stride
 *                  kv_token_stride, q's dtype; row i is the token of q row i.
 *  k_cache,v_cache [num_blocks, block_size, num_kv_heads, head_dim].
 *  slot_mapping    device int32 [total_q]; slots unique within the call;
 *                  negative slots and slots past the pool are skipped.
 * Errors as in the two calls it combines. Uses no workspace (always one
 * workgroup per item). */
int pkv_prefill_store_attention_varlen(const void *q, int64_t q_token_stride, const void *k,
                                       const void *v, int64_t kv_token_stride, void *k_cache,
                                       void *v_cache, const int32_t *slot_mapping,
                                       const int32_t *block_tables, int32_t max_blocks_per_seq,
                                       const int32_t *cu_seqlens_q, const int32_t *cu_seqlens_k,
                                       int32_t num_seqs, int32_t total_q, int32_t max_seqlen_q,
                                       int32_t max_seqlen_k, int32_t num_blocks,
                                       int32_t block_size, int32_t num_q_heads,
                                       int32_t num_kv_heads, int32_t head_dim, float scale,
                                       int32_t dtype, void *out, void *stream);

/* ---------------------------------------------------------------------------
 * decode_attention_paged  ([MR] "prepare_decode": one query per sequence,
 * context_lens keys read through block_tables; split-context partitions and
 * their log-sum-exp combine follow Flash-Decoding (Dao et al., 2023).)
 *
 * For each sequence b with n = context_lens[b] and q head h:
 *     out[b, h, :] = softmax(scale * q[b, h, :] . K_b^T) V_b
 * over positions 0..n-1, position j at slot
 * block_tables[b * max_blocks_per_seq + j / block_size] * block_size +
 * j % block_size. The token being decoded must already be stored (its K/V is
 * position n-1). n == 0 (a padded row) gives an all-zero output row.
 *
 * Contexts are split so that every part of the GPU gets work, and the parts
 * are combined by a second kernel. With partition_size == 0 the library
 * chooses: for bf16, head_dim 128 and a block_size that is a multiple of 64
 * (nano-vLLM's 256 included) the (sequence, kv head, 64-position chunk) work
 * list is divided evenly over all waves the GPU holds at once, each wave
 * finishing the sequences it covers entirely and leaving at most two partial
 * results -- except for batches of at most 64 (sequence, kv head) pairs,
 * where fixed partitions of 64 to 512 positions are faster; other shapes use
 * fixed partitions. PKV_PARTITION_BALANCED forces the balanced split where
 * the shape allows it (the library's choice elsewhere). A positive multiple
 * of 16 forces fixed partitions of that many positions. The workspace must hold
 * pkv_decode_workspace_bytes(...) bytes (256-byte aligned), and may be NULL
 * when that is 0. pkv_decode_partition_size() reports the fixed partition
 * size, or 0 for the balanced split.
 *
 *  q               [num_seqs, num_q_heads, head_dim], token stride q_token_stride.
 *  out             [num_seqs, num_q_heads, head_dim], contiguous, q's dtype.
 *  block_tables    device int32 [num_seqs, max_blocks_per_seq], -1 padded.
 *  context_lens    device int32 [num_seqs].
 *  max_context_len host upper bound of context_lens (sizes the grid and the
 *                  workspace). The kernels read each context length as
 *                  min(max(context_lens[b], 0), max_context_len): a longer
 *                  context is cut to its first max_context_len positions.
 * Requires num_q_heads % num_kv_heads == 0, head_dim in {64, 128}, a positive
 * finite scale, and block_size a power of two in [1, 1024]. */
#define PKV_PARTITION_BALANCED (-1)

int pkv_decode_attention_paged(const void *q, int64_t q_token_stride, const void *k_cache,
                               const void *v_cache, const int32_t *block_tables,
                               int32_t max_blocks_per_seq, const int32_t *context_lens,
                               int32_t num_seqs, int32_t max_context_len, int32_t num_blocks,
                               int32_t block_size, int32_t num_q_heads, int32_t num_kv_heads,
                               int32_t head_dim, float scale, int32_t dtype, void *out,
                               int32_t partition_size, void *workspace, size_t workspace_bytes,
                               void *stream);

/* Fixed partition size the decode call will use for these arguments, or 0
 * when it balances the work over all waves instead. */
int32_t pkv_decode_partition_size(int32_t num_seqs, int32_t max_context_len,
                                  int32_t num_q_heads, int32_t num_kv_heads,
                                  int32_t head_dim, int32_t block_size, int32_t dtype,
                                  int32_t partition_size);

/* Workspace bytes pkv_decode_attention_paged needs for these arguments. */
size_t pkv_decode_workspace_bytes(int32_t num_seqs, int32_t max_context_len,
                                  int32_t num_q_heads, int32_t num_kv_heads,
                                  int32_t head_dim, int32_t block_size, int32_t dtype,
                                  int32_t partition_size);

/* ---------------------------------------------------------------------------
 * decode_attention_paged without a workspace argument, for callers that
 * cannot allocate device memory: code under HIP graph capture, serving loops
 * that allocate nothing per step, harnesses that forbid hipMalloc. The
 * computation, arguments and errors are those of pkv_decode_attention_paged;
 * the workspace is instead a scratch array of PKV_NOALLOC_SCRATCH_BYTES
 * (16 MiB) that the library holds on every device it runs on until the
 * process ends. The call allocates nothing itself (the caller still provides
 * q, the caches, the metadata and out).
 *  - PKV_ENOSPACE when pkv_decode_workspace_bytes(...) for these arguments
 *    exceeds PKV_NOALLOC_SCRATCH_BYTES (the balanced split needs about
 *    waves * 2 * group * (head_dim + 2) * 4 bytes: 4.3 MB at 1024 waves,
 *    group 4, head_dim 128; long fixed partitions can need more).
 *  - The scratch of a device is found once, on the first call made with that
 *    device current; `stream` must belong to the current device.
 *  - Every call on a device shares that device's scratch and leaves its
 *    contents behind (nothing in it needs to start zeroed). Calls that may
 *    run at the same time on one device -- on different streams, or from
 *    different host threads -- race on it; order them on one stream.
 * -------------------------------------------------------------------------*/
#define PKV_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)

int pkv_decode_attention_paged_noalloc(const void *q, int64_t q_token_stride, const void *k_cache,
                                       const void *v_cache, const int32_t *block_tables,
                                       int32_t max_blocks_per_seq, const int32_t *context_lens,
                                       int32_t num_seqs, int32_t max_context_len,
                                       int32_t num_blocks, int32_t block_size,
                                       int32_t num_q_heads, int32_t num_kv_heads,
                                       int32_t head_dim, float scale, int32_t dtype, void *out,
                                       int32_t partition_size, void *stream);

/* ---------------------------------------------------------------------------
 * store_kvcache and decode_attention_paged in one call: the decode step of a
 * layer writes each sequence's new K/V row through slot_mapping and then
 * attends over the context including it ([MR] ModelRunner init: attention
 * writes new K/V through slot_mapping and reads history through
 * block_tables; "prepare_decode": slot_mapping holds the slot of each
 * sequence's last position and context_lens counts it).
 *  k, v            the new tokens' rows [num_seqs, num_kv_heads, head_dim],
 *                  kv_token_stride elements between sequences (16-byte
 *                  aligned); row b is sequence b's token.
 *  slot_mapping    int32 [num_seqs]: the slot of row b, negative to skip it.
 *  The other arguments, the workspace and the errors are those of
 *  pkv_decode_attention_paged (the caches are written).
 * The result -- out and both caches -- equals pkv_store_kvcache(k, v,
 * kv_token_stride, kv_token_stride, k_cache, v_cache, slot_mapping, num_seqs,
 * ...) followed by pkv_decode_attention_paged(...) on the same stream,
 * provided slot_mapping[b] is the slot of position context_lens[b] - 1 of
 * sequence b through its block table (as pkv_pack_decode lays them out) or
 * negative. On the fixed-partition bf16 path (head_dim 128, block_size a
 * multiple of 64, the partition sizes small batches take) the store runs
 * inside the attention launch: the wave holding a sequence's last position
 * writes that token's row of its kv head before it reads the slot. Other
 * shapes and the balanced split run the store kernel, then the attention.
 * -------------------------------------------------------------------------*/
int pkv_decode_store_attention_paged(const void *q, int64_t q_token_stride, const void *k,
                                     const void *v, int64_t kv_token_stride, void *k_cache,
                                     void *v_cache, const int32_t *slot_mapping,
                                     const int32_t *block_tables, int32_t max_blocks_per_seq,
                                     const int32_t *context_lens, int32_t num_seqs,
                                     int32_t max_context_len, int32_t num_blocks,
                                     int32_t block_size, int32_t num_q_heads, int32_t num_kv_heads,
                                     int32_t head_dim, float scale, int32_t dtype, void *out,
                                     int32_t partition_size, void *workspace,
                                     size_t workspace_bytes, void *stream);

/* ---------------------------------------------------------------------------
 * Rotary embedding fused with store_kvcache (the step just before the KV write
 * in the attention layer: "Nano vLLM 解读（5）：解析 ModelRunner", the attention
 * layer's forward, and "nano-vLLM-1", "4. prefill 输入打包", where positions are
 * packed for it). The pages name RoPE but give neither its base nor its
 * variant, so both are parameters; the rotation itself is that of RoFormer
 * (Su et al., 2021): pair j of a head vector at position p turns by the angle
 *     theta_j(p) = p * base^(-2j / rot_dim),   j in [0, rot_dim / 2),
 *     (x, y) -> (x cos theta - y sin theta,  y cos theta + x sin theta).
 * style PKV_ROPE_HALF pairs elements (j, j + rot_dim/2) (the "rotate half"
 * layout of GPT-NeoX / Llama / Qwen); PKV_ROPE_INTERLEAVED pairs (2j, 2j+1)
 * (GPT-J). Elements at or past rot_dim are not rotated.
 *
 * pkv_rope_cos_sin_table fills, on the host (no GPU involved), the float table
 *     cos_sin[p * rot_dim + j]               = cos(theta_j(p))
 *     cos_sin[p * rot_dim + rot_dim / 2 + j] = sin(theta_j(p))
 * for p in [0, max_positions), computed in double and rounded to float. The
 * caller copies it to the device once (it depends only on the model).
 * Errors: PKV_EINVAL for a null pointer, max_positions < 1, rot_dim odd or
 * < 2, or base <= 0.
 *
 * pkv_rope_store_kvcache, for each token i in [0, num_tokens) with
 * p = positions[i] (device int32, 0 <= p < max_positions; a position outside
 * that range is clamped into it):
 *   - rotates q[i, h, :rot_dim] in place for every q head h;
 *   - rotates k row i, writes it to k_cache row slot_mapping[i] (skipped when
 *     the slot is negative or past the pool, as in pkv_store_kvcache) and, if
 *     write_k != 0, back into k in place (needed when the same step's prefill
 *     reads k/v directly rather than through the block tables);
 *   - copies v row i bit for bit to v_cache row slot_mapping[i].
 * Arithmetic in float with fused multiply-adds; results round to nearest even
 * in the storage dtype. Layouts as in pkv_store_kvcache, with q
 * [num_tokens, num_q_heads, head_dim] at token stride q_token_stride; cos_sin
 * is the device copy of the table above. Requires rot_dim even, <= head_dim,
 * and a multiple of 16 / element_size (2 * 16 / element_size for
 * PKV_ROPE_HALF), rows and strides multiples of 16 bytes, pointers 16-byte
 * aligned. num_tokens == 0 is a no-op. k and the caches must not overlap q.
 * -------------------------------------------------------------------------*/
typedef enum { PKV_ROPE_HALF = 0, PKV_ROPE_INTERLEAVED = 1 } pkv_rope_style;

int pkv_rope_cos_sin_table(float *host_out, int32_t max_positions, int32_t rot_dim, double base);

int pkv_rope_store_kvcache(void *q, int64_t q_token_stride, void *k, const void *v,
                           int64_t k_token_stride, int64_t v_token_stride, void *k_cache,
                           void *v_cache, const int32_t *slot_mapping, const int32_t *positions,
                           const float *cos_sin, int32_t max_positions, int32_t rot_dim,
                           int32_t style, int32_t write_k, int32_t num_tokens,
                           int32_t num_blocks, int32_t block_size, int32_t num_q_heads,
                           int32_t num_kv_heads, int32_t head_dim, int32_t dtype, void *stream);

/* ---------------------------------------------------------------------------
 * Host block manager with a hashed prefix cache ([NV1] BlockManager sections
 * "1. Block" through "6. 辅助查询方法"; [ES] "PageAttention / 内/显存管理").
 * Host memory only; no GPU call. Produces each sequence's block table and
 * cached-token count for pkv_plan_* / pkv_pack_* (pkv_bm_gather writes them
 * in the packers' CSR form).
 *
 * A pool of num_blocks blocks of block_size tokens. Free blocks form a FIFO:
 * allocation takes the front, release appends to the back. A full block is
 * identified by a chained hash: xxh64 (seed 0) of the previous block's hash
 * as 8 little-endian bytes (absent for a sequence's first block) followed by
 * the block's token ids as little-endian int64 (pkv_block_hash). A hash-table
 * hit is taken only when the block's recorded hash and tokens both match.
 *
 *  pkv_bm_create / pkv_bm_destroy   the manager; handles are not thread-safe.
 *  pkv_bm_can_allocate(n)           free blocks >= ceil(n / block_size).
 *  pkv_bm_allocate(seq, tokens, n)  block table for a new sequence (prefill):
 *      up to the first miss, full blocks found in the cache are shared and
 *      count as cached tokens (a multiple of block_size, written to
 *      *num_cached_tokens); every later block is fresh. Full blocks are
 *      (re)registered. PKV_ENOSPACE if the worst case (no hit) does not fit,
 *      before anything changes; PKV_EINVAL if seq already holds blocks.
 *  pkv_bm_append_token(seq, tok)    the sequence grows by one token (after a
 *      decode step samples it).
 *  pkv_bm_can_append(seq)           1 if the next pkv_bm_may_append fits.
 *  pkv_bm_may_append(seq)           before a decode step writes the KV of the
 *      sequence's newest token: a new block when that token opens one,
 *      registration of the last block when it fills it. PKV_ENOSPACE when no
 *      block is free; PKV_EINVAL when the sequence's state is inconsistent.
 *  pkv_bm_deallocate(seq)           one reference dropped per block, last
 *      block first; blocks reaching zero go to the back of the FIFO and keep
 *      their registration until reused. The sequence is forgotten.
 *  pkv_bm_block_table(seq, out, cap) length of the table (-1 if unknown);
 *      copied to out when cap is large enough.
 *  pkv_bm_gather(n, seq_ids, ...)   seq_lens[s], num_cached_tokens[s],
 *      bt_offsets[0..n] and bt_ids for the packers; PKV_ENOSPACE if
 *      bt_capacity is too small.
 * pkv_xxh64 is the hash itself (seed as given), exposed for testing.
 * -------------------------------------------------------------------------*/
typedef struct pkv_block_manager pkv_block_manager;

uint64_t pkv_xxh64(const void *data, size_t len, uint64_t seed);
uint64_t pkv_block_hash(const int64_t *token_ids, int32_t num_tokens, int32_t has_prefix,
                        uint64_t prefix);
int pkv_bm_create(int32_t num_blocks, int32_t block_size, pkv_block_manager **out);
void pkv_bm_destroy(pkv_block_manager *m);
int32_t pkv_bm_num_free(const pkv_block_manager *m);
int pkv_bm_can_allocate(const pkv_block_manager *m, int32_t num_tokens);
int pkv_bm_allocate(pkv_block_manager *m, int64_t seq_id, const int64_t *token_ids,
                    int32_t num_tokens, int32_t *num_cached_tokens);
int pkv_bm_append_token(pkv_block_manager *m, int64_t seq_id, int64_t token_id);
int pkv_bm_can_append(const pkv_block_manager *m, int64_t seq_id);
int pkv_bm_may_append(pkv_block_manager *m, int64_t seq_id);
int pkv_bm_deallocate(pkv_block_manager *m, int64_t seq_id);
int32_t pkv_bm_block_table(const pkv_block_manager *m, int64_t seq_id, int32_t *out,
                           int32_t capacity);
int pkv_bm_gather(const pkv_block_manager *m, int32_t num_seqs, const int64_t *seq_ids,
                  int32_t *seq_lens, int32_t *num_cached_tokens, int64_t *bt_offsets,
                  int32_t *bt_ids, int64_t bt_capacity);

/* ---------------------------------------------------------------------------
 * Host metadata packing ([NV1] "4. prefill 输入打包" and "5. deocde 输入打包":
 * prepare_block_tables, prepare_prefill, prepare_decode; pinned memory and
 * one asynchronous host-to-device copy.)
 *
 * A batch is described on the host by, per sequence s:
 *   seq_lens[s]          len(seq): tokens including this step's,
 *   num_cached_tokens[s] leading tokens whose K/V is already in the cache
 *                        (prefill; decode uses seq_lens[s] - 1 implicitly),
 *   block table          bt_ids[bt_offsets[s] .. bt_offsets[s+1]) (CSR).
 *
 * pkv_plan_* computes the layout of one packed buffer; pkv_pack_* fills a host
 * buffer (ideally pinned) with it; pkv_upload copies it to the device with one
 * hipMemcpyAsync. Each array starts at a 256-byte-aligned offset.
 *
 * Prefill packs, in this order:
 *   slot_mapping   int32 [num_slots]   slots of positions
 *                  [num_cached_tokens[s], seq_lens[s]) of each s, in order
 *   cu_seqlens_q   int32 [num_seqs+1]  prefix sums of seq_lens - num_cached
 *   cu_seqlens_k   int32 [num_seqs+1]  prefix sums of seq_lens
 *   block_tables   int32 [num_seqs, max_blocks_per_seq], -1 padded, present
 *                  only when the batch has a cached prefix (total_k > total_q)
 *   positions      int32 [num_slots]   the positions themselves, same order
 *                  ([NV1] "4. prefill 输入打包": positions start at
 *                  num_cached_tokens; they drive the rotary embedding)
 * Decode packs:
 *   slot_mapping   int32 [num_seqs]    slot of position seq_lens[s] - 1
 *   context_lens   int32 [num_seqs]    seq_lens[s]
 *   block_tables   int32 [num_seqs, max_blocks_per_seq], -1 padded (always)
 *   positions      int32 [num_seqs]    seq_lens[s] - 1
 * Errors: PKV_EINVAL if a sequence's table has fewer than ceil(len / bs)
 * entries, a length is negative (prefill) or < 1 (decode), num_cached exceeds
 * len, or a count overflows int32; PKV_ENOSPACE if the buffer is too small. */
typedef struct {
    int32_t num_seqs;
    int32_t total_q;             /* query rows (prefill) or num_seqs (decode)  */
    int64_t total_k;             /* sum of seq_lens                            */
    int32_t max_seqlen_q;
    int32_t max_seqlen_k;        /* also the decode max_context_len            */
    int32_t max_blocks_per_seq;
    int32_t has_block_tables;
    int32_t num_slots;
    int32_t is_prefill;
    int64_t off_slot_mapping;    /* byte offsets into the packed buffer; -1 if */
    int64_t off_cu_seqlens_q;    /* the array is absent                        */
    int64_t off_cu_seqlens_k;
    int64_t off_context_lens;
    int64_t off_block_tables;
    int64_t off_positions;
    int64_t total_bytes;
} pkv_batch_layout;

int pkv_plan_prefill(int32_t num_seqs, const int32_t *seq_lens,
                     const int32_t *num_cached_tokens, const int64_t *bt_offsets,
                     int32_t block_size, pkv_batch_layout *layout);
int pkv_pack_prefill(int32_t num_seqs, const int32_t *seq_lens,
                     const int32_t *num_cached_tokens, const int32_t *bt_ids,
                     const int64_t *bt_offsets, int32_t block_size,
                     const pkv_batch_layout *layout, void *host_buf, size_t host_bytes);
int pkv_plan_decode(int32_t num_seqs, const int32_t *seq_lens, const int64_t *bt_offsets,
                    int32_t block_size, pkv_batch_layout *layout);
int pkv_pack_decode(int32_t num_seqs, const int32_t *seq_lens, const int32_t *bt_ids,
                    const int64_t *bt_offsets, int32_t block_size,
                    const pkv_batch_layout *layout, void *host_buf, size_t host_bytes);

/* One asynchronous host-to-device copy of `bytes` from host_buf (pinned for
 * true asynchrony) to dev_buf on `stream`. */
int pkv_upload(const void *host_buf, void *dev_buf, size_t bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
