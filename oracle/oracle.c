/*
 * oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, obviously-correct CPU implementation of what the paged-KV
 * attention hot path computes. Only the test suite, the smoke check and the
 * bench's cpu_baseline leg may load it; the product library never does. It
 * shares no code, header, table or helper with the HIP library.
 *
 * Everything is computed from the definitions, in double precision, from inputs
 * upcast exactly (fp32 -> double, bf16 -> fp32 -> double). No blocking, fusion
 * or reordering beyond what the definitions state.
 *
 * Sources (pages as published; cited by title and section):
 *  [NV1] "nano-vLLM-1" (senjlearning.space), sections "3. KV cache 分配",
 *        "4. prefill 输入打包", "5. deocde 输入打包", BlockManager
 *        "3. 核心方法一：分配 (allocate)", and the Sequence derived properties.
 *  [MR]  "Nano vLLM 解读（5）：解析 ModelRunner" (languisher.top), sections
 *        "FlashAttention Kernel 函参准备", "prepare_prefill", "prepare_decode".
 *  [ES]  "【nano-vllm 学习】04 - 自顶向下的引擎调度层源码学习2" (kyonqi.github.io),
 *        "KV-Cache … 是什么？" (the attention equation and the causal mask) and
 *        "PageAttention / 内/显存管理" (pages = blocks, block_table = page table).
 *
 * Readings where the pages leave a step open (all chosen as the plainest one):
 *  - causal alignment when a sequence has fewer queries than keys (prefix hit):
 *    query i of a sequence with Lq queries and Lk keys sits at absolute
 *    position Lk - Lq + i, and sees keys 0 .. Lk - Lq + i, itself included
 *    ([NV1] prepare_prefill positions start at num_cached_tokens; [ES] the mask
 *    starts one past the current position).
 *  - grouped-query heads: q head h reads kv head h / (Hq / Hkv).
 *  - a sequence with zero keys produces an all-zero output row.
 *  - a negative slot means "no write" (padding rows).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORC_F32 = 0, ORC_BF16 = 1 };

/* Exact upcast of one stored element to double. A bf16 value is the upper 16
 * bits of an IEEE binary32, so widening is a shift. */
static double orc_elem(const void *base, int64_t idx, int dtype)
{
    if (dtype == ORC_F32)
        return (double)((const float *)base)[idx];
    uint32_t u = (uint32_t)((const uint16_t *)base)[idx] << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* [NV1] allocate / prepare_prefill: the token at position p of a sequence lives
 * in logical block p / bs, at offset p % bs inside it; the block table maps the
 * logical block to a physical one, and the flat slot index is
 * physical_block * bs + offset. Returns -1 if the table is too short. */
int64_t orc_slot(const int32_t *table, int64_t table_len, int32_t bs, int64_t p)
{
    int64_t lb = p / bs;
    if (p < 0 || lb >= table_len)
        return -1;
    return (int64_t)table[lb] * bs + p % bs;
}

/* Slots for a list of position ranges [begin, end) of sequences, in list order,
 * positions ascending -- the order in which prepare_prefill / prepare_decode
 * emit them. Tables are given in CSR form (bt_flat, bt_off[S+1]).
 * Returns the number of slots written, or -1 if a position has no table entry. */
int64_t orc_slots(int32_t n_ranges, const int32_t *rseq, const int32_t *rbegin,
                  const int32_t *rend, const int32_t *bt_flat, const int64_t *bt_off,
                  int32_t bs, int64_t *out)
{
    int64_t n = 0;
    for (int32_t r = 0; r < n_ranges; ++r) {
        const int32_t *table = bt_flat + bt_off[rseq[r]];
        int64_t tlen = bt_off[rseq[r] + 1] - bt_off[rseq[r]];
        for (int64_t p = rbegin[r]; p < rend[r]; ++p) {
            int64_t s = orc_slot(table, tlen, bs, p);
            if (s < 0)
                return -1;
            out[n++] = s;
        }
    }
    return n;
}

/* [MR] "FlashAttention Kernel 函参准备" (slot_mapping names where each new
 * token's K/V goes): row i of the new K (or V) is copied, bit for bit,
 * into the cache row numbered slots[i] of a cache viewed as
 * [num_blocks * block_size, row_bytes]. slots[i] < 0 is skipped.
 * Returns 0, or -1 for a slot past the pool, or -2 for a duplicate slot
 * (each token owns its slot; a batch never writes one slot twice). */
int orc_store(const void *src, int64_t n_rows, int64_t row_bytes, int64_t src_stride_bytes,
              void *cache, int64_t num_slots, const int64_t *slots)
{
    unsigned char *seen = (unsigned char *)calloc((size_t)(num_slots > 0 ? num_slots : 1), 1);
    if (!seen)
        return -3;
    int rc = 0;
    for (int64_t i = 0; i < n_rows; ++i) {
        int64_t s = slots[i];
        if (s < 0)
            continue;
        if (s >= num_slots) { rc = -1; break; }
        if (seen[s]) { rc = -2; break; }
        seen[s] = 1;
        memcpy((unsigned char *)cache + s * row_bytes,
               (const unsigned char *)src + i * src_stride_bytes, (size_t)row_bytes);
    }
    free(seen);
    return rc;
}

/* Where the keys of one sequence come from: either contiguous rows (the call's
 * own k/v, used when a prefill has no cached prefix), or the paged pool read
 * through the sequence's block table. */
typedef struct {
    int paged;
    const void *k, *v;          /* contiguous: [sum Lk, Hkv, d] */
    int64_t k_base;             /* first row of this sequence */
    const void *kc, *vc;        /* paged: [num_blocks, bs, Hkv, d] */
    const int32_t *table;
    int64_t table_len;
    int32_t bs;
    int64_t num_blocks;
} orc_keys;

/* Row index (in units of Hkv*d elements) of key position j, or -1 when the
 * table has no valid entry for it. [NV1]: physical block = table[j / bs],
 * offset j % bs; a padded (-1) entry is not a block. */
static int64_t orc_key_row(const orc_keys *ks, int64_t j)
{
    if (!ks->paged)
        return ks->k_base + j;
    int64_t lb = j / ks->bs;
    if (lb >= ks->table_len)
        return -1;
    int64_t pb = ks->table[lb];
    if (pb < 0 || pb >= ks->num_blocks)
        return -1;
    return pb * ks->bs + j % ks->bs;
}

/* [ES] Attention(Q,K,V) = softmax(Q K^T / sqrt(d_k)) V, for one query row over
 * keys 0 .. n_keys-1 of one kv head, with the caller's scale:
 *   x_j = scale * sum_e q_e k_je,  m = max_j x_j,  w_j = exp(x_j - m),
 *   o   = sum_j w_j v_j / sum_j w_j.
 * Positions past n_keys are never touched (the causal mask sets them to -inf,
 * whose weight is exactly 0). Returns -1 if a key has no valid table entry. */
static int orc_row(const void *q, int64_t q_off, const orc_keys *ks, int64_t n_keys,
                   int32_t Hkv, int32_t kvh, int32_t d, double scale, int dtype,
                   double *x, double *o)
{
    for (int32_t e = 0; e < d; ++e)
        o[e] = 0.0;
    if (n_keys <= 0)
        return 0;
    const void *kb = ks->paged ? ks->kc : ks->k;
    const void *vb = ks->paged ? ks->vc : ks->v;
    double m = -INFINITY;
    for (int64_t j = 0; j < n_keys; ++j) {
        int64_t row = orc_key_row(ks, j);
        if (row < 0)
            return -1;
        int64_t k_off = (row * Hkv + kvh) * d;
        double dot = 0.0;
        for (int32_t e = 0; e < d; ++e)
            dot += orc_elem(q, q_off + e, dtype) * orc_elem(kb, k_off + e, dtype);
        x[j] = scale * dot;
        if (x[j] > m)
            m = x[j];
    }
    double den = 0.0;
    for (int64_t j = 0; j < n_keys; ++j) {
        double w = exp(x[j] - m);
        den += w;
        int64_t v_off = (orc_key_row(ks, j) * Hkv + kvh) * d;
        for (int32_t e = 0; e < d; ++e)
            o[e] += w * orc_elem(vb, v_off + e, dtype);
    }
    for (int32_t e = 0; e < d; ++e)
        o[e] /= den;
    return 0;
}

/* Causal attention over a ragged batch ([MR] prepare_prefill: cu_seqlens_q /
 * cu_seqlens_k delimit each sequence; [MR] prepare_decode: one query per
 * sequence over context_lens keys).
 *
 * q_lens[s] / k_lens[s]: queries and keys of sequence s; its query i sits at
 * position k_lens[s] - q_lens[s] + i and sees keys 0 .. that position.
 * q: [sum q_lens, Hq, d]; out: [sum q_lens, Hq, d] (double).
 * Keys come from k/v rows [sum k_lens, Hkv, d] when paged == 0, else from the
 * pool k_cache / v_cache [num_blocks, bs, Hkv, d] through the block tables
 * (CSR: bt_flat, bt_off[S+1]).
 * A query row that sees no key (a decode row with context length 0, padded
 * in by a graph replay) produces zeros.
 * Returns 0, -1 for a key with no valid table entry, -2 for bad shapes. */
int orc_attention(int32_t num_seqs, const int32_t *q_lens, const int32_t *k_lens,
                  const void *q, int32_t Hq, int32_t Hkv, int32_t d, double scale, int dtype,
                  int paged, const void *k, const void *v,
                  const void *k_cache, const void *v_cache, const int32_t *bt_flat,
                  const int64_t *bt_off, int32_t bs, int64_t num_blocks,
                  double *out, int nthreads)
{
    if (Hkv <= 0 || Hq % Hkv != 0 || d <= 0)
        return -2;
    int32_t g = Hq / Hkv;
    int64_t *q_start = (int64_t *)malloc(sizeof(int64_t) * (size_t)(num_seqs + 1));
    int64_t *k_start = (int64_t *)malloc(sizeof(int64_t) * (size_t)(num_seqs + 1));
    int64_t max_k = 1;
    q_start[0] = k_start[0] = 0;
    for (int32_t s = 0; s < num_seqs; ++s) {
        if (q_lens[s] < 0 || k_lens[s] < 0) {
            free(q_start); free(k_start);
            return -2;
        }
        q_start[s + 1] = q_start[s] + q_lens[s];
        k_start[s + 1] = k_start[s] + k_lens[s];
        if (k_lens[s] > max_k)
            max_k = k_lens[s];
    }
    int64_t total_rows = q_start[num_seqs] * Hq;
    int err = 0;
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#endif
#pragma omp parallel
    {
        double *x = (double *)malloc(sizeof(double) * (size_t)max_k);
#pragma omp for schedule(dynamic, 16)
        for (int64_t r = 0; r < total_rows; ++r) {
            int64_t t = r / Hq;        /* flat query token */
            int32_t h = (int32_t)(r % Hq);
            int32_t s = 0;             /* sequence of token t (binary search) */
            int32_t lo = 0, hi = num_seqs - 1;
            while (lo < hi) {
                int32_t mid = (lo + hi + 1) / 2;
                if (q_start[mid] <= t) lo = mid; else hi = mid - 1;
            }
            s = lo;
            int64_t i = t - q_start[s];
            int64_t pos = (int64_t)k_lens[s] - q_lens[s] + i;
            orc_keys ks;
            memset(&ks, 0, sizeof ks);
            ks.paged = paged;
            ks.k = k; ks.v = v; ks.k_base = k_start[s];
            ks.kc = k_cache; ks.vc = v_cache; ks.bs = bs; ks.num_blocks = num_blocks;
            if (paged) {
                ks.table = bt_flat + bt_off[s];
                ks.table_len = bt_off[s + 1] - bt_off[s];
            }
            int rc = orc_row(q, (t * Hq + h) * (int64_t)d, &ks, pos + 1, Hkv, h / g, d, scale,
                             dtype, x, out + (t * Hq + h) * (int64_t)d);
            if (rc) {
#pragma omp atomic write
                err = rc;
            }
        }
        free(x);
    }
    free(q_start);
    free(k_start);
    return err;
}

/* Rotary position embedding, in place on fp64 head vectors x [T, H, d]
 * (row t, head h at x + (t * H + h) * d). The pages name the positions that
 * feed it ([NV1] "4. prefill 输入打包": positions start at
 * num_cached_tokens) but not the rotation; this is RoFormer's (Su et al.,
 * 2021, section 3.2 and its equation for the general case): pair j of the
 * vector at position p, j in [0, rot_dim / 2), turns by the angle
 *     theta_j = p * base^(-2j / rot_dim)
 * as the 2-D rotation (a, b) -> (a cos theta - b sin theta, b cos theta + a sin theta).
 * style 0 pairs elements (j, j + rot_dim / 2); style 1 pairs (2j, 2j + 1).
 * Elements at or past rot_dim are left alone. Returns 0, or -1 on bad arguments. */
int orc_rope(double *x, int64_t T, int32_t H, int32_t d, const int32_t *pos, int32_t rot_dim,
             double base, int32_t style) {
    if (rot_dim < 2 || rot_dim % 2 || rot_dim > d || !(base > 0.0) || (style != 0 && style != 1))
        return -1;
    const int32_t half = rot_dim / 2;
    for (int64_t t = 0; t < T; ++t)
        for (int32_t h = 0; h < H; ++h) {
            double *v = x + (t * H + h) * (int64_t)d;
            for (int32_t j = 0; j < half; ++j) {
                const double theta = (double)pos[t] * pow(base, -2.0 * j / rot_dim);
                const double c = cos(theta), sn = sin(theta);
                const int32_t ia = style == 0 ? j : 2 * j;
                const int32_t ib = style == 0 ? j + half : 2 * j + 1;
                const double a = v[ia], b = v[ib];
                v[ia] = a * c - b * sn;
                v[ib] = b * c + a * sn;
            }
        }
    return 0;
}

int orc_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
