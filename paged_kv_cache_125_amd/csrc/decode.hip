// decode.hip -- paged decode attention with split-context partitions.
//
// One query token per sequence attends to context_lens[b] keys gathered
// through the sequence's block table ("Nano vLLM 解读（5）：解析 ModelRunner",
// "prepare_decode"; "nano-vLLM-1", "5. deocde 输入打包"): position j lives at
// slot block_tables[b][j / bs] * bs + j % bs of the per-layer pool
// [num_blocks, bs, Hkv, d]. The output is softmax(scale * q K^T) V
// ("【nano-vllm 学习】04 - …源码学习2", "KV-Cache … 是什么？").
//
// Long contexts are cut into partitions of P tokens, each reduced to an
// unnormalised (acc, max, sum) triple and combined by a log-sum-exp rule
// afterwards (Flash-Decoding, Dao et al. 2023; online softmax, Milakov &
// Gimelshein 2018). A sequence that fits one partition is finished in place.
//
// Kernels:
//  decode_sk_kernel<G> + decode_sk_reduce_kernel<G>   the default for bf16,
//      head_dim 128, block size a multiple of 64: the (sequence, kv head,
//      64-position chunk) work list split evenly over one wave per SIMD
//      (stream-K), partials only where a wave's range cuts a segment, and
//      their combine. Used whenever no partition size is forced.
//  decode_blk_kernel<G, CH>       bf16, head_dim 128, block size a multiple of
//      CH (nano-vLLM's 256 included), G <= 16: both contractions on MFMA,
//      buffer loads range-checked by the hardware (see below).
//  decode_mfma_kernel<G, CHUNK>   bf16, head_dim 128, any block size, G <= 8. One
//      wave per (sequence, kv head, partition). The K/V rows of the kv head are
//      loaded once into registers with 16-byte loads and serve all G query
//      heads of the group: q.K^T runs on MFMA (16x16x32 bf16, the G heads as
//      rows), P.V on the VALU in fp32. Softmax statistics use DPP row
//      reductions; LDS carries only the slot rows, P and per-head statistics.
//  decode_generic_kernel<T, D>    any dtype/group, fp32 math, one wave per
//      (sequence, q head, partition); used for fp32 and small head dims.
//  decode_reduce_kernel<T>        the log-sum-exp combine of partitions.
// The fixed-partition kernels above serve forced partition sizes and the
// shapes outside the default kernel's range.
#include <stdlib.h>

#include <type_traits>

#include "pkv.h"
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

// A sequence's context length as the kernels use it: clamped to [0,
// max_context_len], so that a context_lens entry past the host's bound can
// neither address partitions the workspace does not hold nor overflow the
// balanced split's chunk count.
__device__ __forceinline__ int dec_ctx(const DecodeArgs &a, int b) {
    return min(max(a.ctx[b], 0), a.ctx_cap);
}

constexpr int kDecWaves = 4;    // kv heads (waves) per workgroup, MFMA kernel
constexpr int kDecChunk = 64;   // tokens per online-softmax step, MFMA kernel

// Slot row of position t of sequence b, or -1 for an entry outside the table
// or the pool (such positions read as zeros; outputs are then unspecified).
__device__ __forceinline__ int32_t decode_row(const DecodeArgs &a, int b, int t) {
    const int lb = t >> a.log2bs;
    if (lb >= a.maxb) return -1;
    const int blk = a.bt[(int64_t)b * a.maxb + lb];
    if (blk < 0 || blk >= a.num_blocks) return -1;
    return blk * a.bs + (t & (a.bs - 1));
}

template <int G, int CHUNK>
__global__ __launch_bounds__(64 * kDecWaves) void decode_mfma_kernel(DecodeArgs a) {
    constexpr int D = 128;
    constexpr int TILES = CHUNK / 16;   // 16-token MFMA tiles per chunk
    constexpr int TPL = CHUNK / 4;      // tokens each lane accumulates in P.V
    static_assert(G >= 1 && G <= 8, "group");
    __shared__ int32_t rows_s[kDecWaves][CHUNK];
    __shared__ float p_s[kDecWaves][CHUNK * G];
    __shared__ float st_s[kDecWaves][3][16];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int kvh = blockIdx.z * kDecWaves + wave;
    const int b = blockIdx.y, p = blockIdx.x;
    if (kvh >= a.Hkv) return;
    const int n = dec_ctx(a, b);
    const int t_begin = p * a.P;
    if (t_begin >= n && p > 0) return;
    const int nparts = (n + a.P - 1) / a.P;
    const int t_end = min(n, t_begin + a.P);
    const int lr = lane & 15, lg = lane >> 4;
    const int64_t row_bytes = (int64_t)a.Hkv * D * 2;
    const uint8_t *kbase = (const uint8_t *)a.kc + (int64_t)kvh * D * 2;
    const uint8_t *vbase = (const uint8_t *)a.vc + (int64_t)kvh * D * 2;

    // A operand: row = head lr of the group (zero rows above G), k = d.
    bf16x8 qa[4];
    {
        const uint16_t *q = (const uint16_t *)a.q + (int64_t)b * a.q_stride + (int64_t)kvh * G * D;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            u32x4 w = {0u, 0u, 0u, 0u};
            if (lr < G) w = ld16(q + lr * D + 32 * kk + 8 * lg);
            qa[kk] = __builtin_bit_cast(bf16x8, w);
        }
    }
    float m_run[4], l_run[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) { m_run[r] = -INFINITY; l_run[r] = 0.f; }
    float acc[G][8];
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;

    for (int t0 = t_begin; t0 < t_end; t0 += CHUNK) {
        for (int i = lane; i < CHUNK; i += 64) {
            const int t = t0 + i;
            rows_s[wave][i] = t < t_end ? decode_row(a, b, t) : -1;
        }
        wave_lds_fence();
        // K: lane (lr, lg) reads token 16*tile + lr, d = 32*kk + 8*lg .. +8.
        u32x4 kx[TILES][4];
#pragma unroll
        for (int tile = 0; tile < TILES; ++tile) {
            const int row = rows_s[wave][16 * tile + lr];
            const uint8_t *src = kbase + (int64_t)row * row_bytes + lg * 16;
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                u32x4 w = {0u, 0u, 0u, 0u};
                if (row >= 0) w = ld16(src + kk * 64);
                kx[tile][kk] = w;
            }
        }
        // V: lane (lr, lg) reads d = 8*lr .. +8 of tokens lg + 4*i.
        u32x4 vx[TPL];
#pragma unroll
        for (int i = 0; i < TPL; ++i) {
            const int row = rows_s[wave][lg + 4 * i];
            u32x4 w = {0u, 0u, 0u, 0u};
            if (row >= 0) w = ld16(vbase + (int64_t)row * row_bytes + lr * 16);
            vx[i] = w;
        }
        // S = q . K^T: lane holds S[head 4*lg + r][token 16*tile + lr].
        f32x4 s[TILES];
#pragma unroll
        for (int tile = 0; tile < TILES; ++tile) {
            s[tile] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
                s[tile] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    qa[kk], __builtin_bit_cast(bf16x8, kx[tile][kk]), s[tile], 0, 0, 0);
        }
        float alpha[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float mx = -INFINITY;
#pragma unroll
            for (int tile = 0; tile < TILES; ++tile) {
                const bool ok = t0 + 16 * tile + lr < t_end;
                const float x = ok ? s[tile][r] * a.scale_log2 : -INFINITY;
                s[tile][r] = x;
                mx = fmaxf(mx, x);
            }
            mx = row16_max(mx);
            const float m_new = fmaxf(m_run[r], mx);
            alpha[r] = fast_exp2(m_run[r] - m_new);
            float ls = 0.f;
#pragma unroll
            for (int tile = 0; tile < TILES; ++tile) {
                const float e = fast_exp2(s[tile][r] - m_new);
                s[tile][r] = e;
                ls += e;
            }
            l_run[r] = l_run[r] * alpha[r] + ls;
            m_run[r] = m_new;
        }
#pragma unroll
        for (int tile = 0; tile < TILES; ++tile)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int h = 4 * lg + r;
                if (h < G) p_s[wave][(16 * tile + lr) * G + h] = s[tile][r];
            }
        if (lr == 0) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int h = 4 * lg + r;
                if (h < G) st_s[wave][0][h] = alpha[r];
            }
        }
        wave_lds_fence();
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const float al = st_s[wave][0][h];
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[h][e] *= al;
        }
#pragma unroll
        for (int i = 0; i < TPL; ++i) {
            const int tl = lg + 4 * i;
            float v[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                v[2 * e] = bf16lo(vx[i][e]);
                v[2 * e + 1] = bf16hi(vx[i][e]);
            }
#pragma unroll
            for (int h = 0; h < G; ++h) {
                const float ph = p_s[wave][tl * G + h];
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[h][e] = fmaf(ph, v[e], acc[h][e]);
            }
        }
        wave_lds_fence();
    }

#pragma unroll
    for (int r = 0; r < 4; ++r) l_run[r] = row16_sum(l_run[r]);
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            acc[h][e] += shfl_xor(acc[h][e], 16);
            acc[h][e] += shfl_xor(acc[h][e], 32);
        }
    if (lr == 0) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int h = 4 * lg + r;
            if (h < G) {
                st_s[wave][1][h] = m_run[r];
                st_s[wave][2][h] = l_run[r];
            }
        }
    }
    wave_lds_fence();
    if (lane < 16) {
        const int c = lane;  // d = 8c .. 8c+7
        const int h0 = kvh * G;
        if (n == 0 || nparts == 1) {
#pragma unroll
            for (int h = 0; h < G; ++h) {
                const float inv = n == 0 ? 0.f : 1.f / st_s[wave][2][h];
                u32x4 w;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    w[e] = pack_bf16x2(acc[h][2 * e] * inv, acc[h][2 * e + 1] * inv);
                st16((uint16_t *)a.out + ((int64_t)b * a.Hq + h0 + h) * D + 8 * c, w);
            }
        } else {
#pragma unroll
            for (int h = 0; h < G; ++h) {
                float *dst = a.ws_acc + (((int64_t)b * a.maxparts + p) * a.Hq + h0 + h) * D + 8 * c;
                st16(dst, u32x4{__float_as_uint(acc[h][0]), __float_as_uint(acc[h][1]),
                                __float_as_uint(acc[h][2]), __float_as_uint(acc[h][3])});
                st16(dst + 4, u32x4{__float_as_uint(acc[h][4]), __float_as_uint(acc[h][5]),
                                    __float_as_uint(acc[h][6]), __float_as_uint(acc[h][7])});
                if (c == 0) {
                    float *ml = a.ws_ml + (((int64_t)b * a.maxparts + p) * a.Hq + h0 + h) * 2;
                    ml[0] = st_s[wave][1][h];
                    ml[1] = st_s[wave][2][h];
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// decode_blk_kernel<G, CH>: bf16, head_dim 128, block_size a multiple of CH.
//
// A chunk of CH consecutive positions then lies inside one pool block, so its
// K/V rows are CH consecutive slots: one block-table read per chunk (a scalar
// load, issued a chunk ahead) and unconditional 16-byte loads. One wave owns
// one (sequence, kv head, partition); its loads for chunk c+1 are in flight
// while chunk c is computed (K and V registers are refilled as soon as they
// are consumed).
//
// Both contractions run on v_mfma_f32_16x16x32_bf16 with the group's heads as
// the 16 MFMA columns (zero columns above G):
//   S^T = K q^T   A = K rows straight from the loads, B = q
//   O^T += V^T P^T  B = P^T straight from the S^T registers, A = V^T read
//                   from the chunk staged row-major in LDS with the gfx950
//                   transpose read (ds_read_b64_tr_b16)
// Each lane owns one head column: the running max, its rescale factor and the
// output accumulators are lane-local; only the max and the final sum cross
// the 4 lane rows of a column.
//
// STORE: store_kvcache fused into the launch. The wave that holds a
// sequence's last position (its last partition; partition 0 for an empty
// context) first writes that token's K and V rows of its kv head to the
// token's slot, and waits for the writes before it issues any load, so its
// own reads of that slot see them. Every kv head of every sequence is stored
// once; padding slots (negative) and slots past the pool are skipped.
template <int G, int CH, bool STORE>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void decode_blk_kernel(DecodeArgs a) {
    constexpr int D = 128;
    constexpr int TILES = CH / 16;   // 16-token MFMA tiles per chunk
    constexpr int VL = CH / 4;       // 16-byte V loads per lane per chunk
    constexpr int VP = 144;          // LDS row pitch of the staged V chunk (elements)
    static_assert(G >= 1 && G <= 16 && (TILES % 2) == 0, "shape");
    __shared__ __attribute__((aligned(16))) uint16_t vs_all[4][CH * VP];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
    const int kvh = blockIdx.x * 4 + wave;
    const int p = blockIdx.y, b = blockIdx.z;
    if (kvh >= a.Hkv) return;
    const int n = dec_ctx(a, b);
    const int t_begin = p * a.P;
    if (t_begin >= n && p > 0) return;
    if constexpr (STORE) {
        if (p == (n > 0 ? (n - 1) / a.P : 0)) {
            const int slot = a.st_slots[b];
            if ((uint32_t)slot < (uint64_t)a.st_num_slots && lane < D * 2 / 16) {
                const int64_t src = (int64_t)b * a.st_stride_bytes + (int64_t)kvh * D * 2 + 16 * lane;
                const int64_t dst = ((int64_t)slot * a.Hkv + kvh) * D * 2 + 16 * lane;
                st16(a.st_kc + dst, ld16(a.st_k + src));
                st16(a.st_vc + dst, ld16(a.st_v + src));
            }
            __builtin_amdgcn_s_waitcnt(0);   // the row is written before this wave reads the slot
        }
    }
    const int nparts = (n + a.P - 1) / a.P;
    const int t_end = min(n, t_begin + a.P);
    const int lr = lane & 15, lg = lane >> 4;
    const int64_t row_bytes = (int64_t)a.Hkv * D * 2;
    const uint32_t rb32 = (uint32_t)row_bytes;
    const uint8_t *kb = (const uint8_t *)a.kc + (int64_t)kvh * D * 2;
    const uint8_t *vb = (const uint8_t *)a.vc + (int64_t)kvh * D * 2;
    // Per-lane byte offsets inside a chunk (the chunk base is in the descriptor).
    const uint32_t k_lane = (uint32_t)lr * rb32 + (uint32_t)lg * 16u;
    const uint32_t v_lane = (uint32_t)lg * rb32 + (uint32_t)lr * 16u;
    const int32_t *bt_row = a.bt + (int64_t)b * a.maxb;
    uint16_t *vs = vs_all[wave];

    // B operand of S^T = K q^T: lane holds q[head lr][d = 32*kk + 8*lg .. +8].
    bf16x8 qb[4];
    {
        const uint16_t *q = (const uint16_t *)a.q + (int64_t)b * a.q_stride + (int64_t)(kvh * G + lr) * D + 8 * lg;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            u32x4 w = {0u, 0u, 0u, 0u};
            if (lr < G) w = ld16(q + 32 * kk);
            qb[kk] = __builtin_bit_cast(bf16x8, w);
        }
    }
    // Buffer descriptor of the chunk starting at position t: its CH rows are
    // consecutive slots of one block, and num_records covers only positions
    // < t_end, so the hardware returns zeros past the context, for a missing
    // block-table entry and for the prefetch past the partition's end.
    // The partition's block ids, one per lane, read once (a partition spans at
    // most 64 blocks: P <= 64 * block_size is checked on the host).
    const int lb0 = t_begin >> a.log2bs;
    const int nblk = ((t_end - 1) >> a.log2bs) - lb0 + 1;
    const int my_blk = (lane < nblk && lb0 + lane < a.maxb) ? bt_row[lb0 + lane] : -1;
    auto chunk_rsrc = [&](const uint8_t *pool, int t) -> __amdgpu_buffer_rsrc_t {
        const int valid = min(CH, t_end - t);
        const int idx = min((t >> a.log2bs) - lb0, 63);
        const int blk = valid > 0 ? __builtin_amdgcn_readlane(my_blk, idx) : -1;
        if (blk < 0 || blk >= a.num_blocks)
            return __builtin_amdgcn_make_buffer_rsrc((void *)pool, (short)0, 0, kBufWord3);
        const uint8_t *base = pool + ((int64_t)blk * a.bs + (t & (a.bs - 1))) * row_bytes;
        return __builtin_amdgcn_make_buffer_rsrc((void *)base, (short)0, valid * (int)rb32, kBufWord3);
    };
    u32x4 kx[TILES][4], vx[VL];
    auto load_k = [&](__amdgpu_buffer_rsrc_t r) {
#pragma unroll
        for (int tile = 0; tile < TILES; ++tile)
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
                kx[tile][kk] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                    r, (int)(k_lane + (uint32_t)(16 * tile) * rb32 + 64u * kk), 0, 0));
    };
    auto load_v = [&](__amdgpu_buffer_rsrc_t r) {
#pragma unroll
        for (int i = 0; i < VL; ++i)
            vx[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                r, (int)(v_lane + (uint32_t)(4 * i) * rb32), 0, 0));
    };

    f32x4 o[8];
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) o[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.f;

    load_v(chunk_rsrc(vb, t_begin));
    load_k(chunk_rsrc(kb, t_begin));
    for (int t0 = t_begin; t0 < t_end; t0 += CH) {
        // V(c) -> LDS (rows past the context arrive as zeros), then prefetch V(c+1).
#pragma unroll
        for (int i = 0; i < VL; ++i)
            *reinterpret_cast<u32x4 *>(vs + (lg + 4 * i) * VP + 8 * lr) = vx[i];
        load_v(chunk_rsrc(vb, t0 + CH));
        // S^T tiles: st[tile][r] = S[head lr][position t0 + 16*tile + 4*lg + r].
        f32x4 st[TILES];
#pragma unroll
        for (int tile = 0; tile < TILES; ++tile) {
            st[tile] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
                st[tile] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    __builtin_bit_cast(bf16x8, kx[tile][kk]), qb[kk], st[tile], 0, 0, 0);
        }
        load_k(chunk_rsrc(kb, t0 + CH));
        float mx = -INFINITY;
#pragma unroll
        for (int tile = 0; tile < TILES; ++tile)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float x = st[tile][r] * a.scale_log2;
                if (t0 + 16 * tile + 4 * lg + r >= t_end) x = -INFINITY;
                st[tile][r] = x;
                mx = fmaxf(mx, x);
            }
        mx = xor32_max(xor16_max(mx));
        const float m_new = fmaxf(m_run, mx);
        const float alpha = fast_exp2(m_run - m_new);
        float ls = 0.f;
#pragma unroll
        for (int tile = 0; tile < TILES; ++tile)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float e = fast_exp2(st[tile][r] - m_new);
                st[tile][r] = e;
                ls += e;
            }
        l_run = l_run * alpha + ls;
        m_run = m_new;
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) o[mt] *= alpha;
        wave_lds_fence();
        // O^T += V^T P^T, 32 positions per MFMA step: k-slot 8*lg + e holds
        // position 4*lg + e (e < 4) or 16 + 4*lg + e - 4 of the step.
#pragma unroll
        for (int s = 0; s < TILES / 2; ++s) {
            bf16x8 pb;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                pb[r] = (__bf16)st[2 * s][r];
                pb[4 + r] = (__bf16)st[2 * s + 1][r];
            }
            const uint16_t *src_lo = vs + (32 * s + 4 * lg + (lr >> 2)) * VP + 4 * (lr & 3);
            const uint16_t *src_hi = src_lo + 16 * VP;
#pragma unroll
            for (int mt = 0; mt < 8; ++mt) {
                typedef short s16x4 __attribute__((ext_vector_type(4)));
                const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) s16x4 *)(src_lo + 16 * mt));
                const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) s16x4 *)(src_hi + 16 * mt));
                typedef short s16x8 __attribute__((ext_vector_type(8)));
                const s16x8 av = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
                o[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av), pb,
                                                                o[mt], 0, 0, 0);
            }
        }
        wave_lds_fence();
    }

    l_run = xor32_sum(xor16_sum(l_run));
    if (lr < G) {
        const int h = kvh * G + lr;
        if (n == 0 || nparts == 1) {
            const float inv = n == 0 ? 0.f : 1.f / l_run;
            uint16_t *dst = (uint16_t *)a.out + ((int64_t)b * a.Hq + h) * D + 4 * lg;
#pragma unroll
            for (int mt = 0; mt < 8; ++mt) {
                u32x2 w;
                w[0] = pack_bf16x2(o[mt][0] * inv, o[mt][1] * inv);
                w[1] = pack_bf16x2(o[mt][2] * inv, o[mt][3] * inv);
                *reinterpret_cast<u32x2 *>(dst + 16 * mt) = w;
            }
        } else {
            const int64_t slot = ((int64_t)b * a.maxparts + p) * a.Hq + h;
            float *dst = a.ws_acc + slot * D + 4 * lg;
#pragma unroll
            for (int mt = 0; mt < 8; ++mt)
                st16(dst + 16 * mt, u32x4{__float_as_uint(o[mt][0]), __float_as_uint(o[mt][1]),
                                          __float_as_uint(o[mt][2]), __float_as_uint(o[mt][3])});
            if (lg == 0) {
                a.ws_ml[slot * 2] = m_run;
                a.ws_ml[slot * 2 + 1] = l_run;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// decode_sk_kernel<G>: the block-aligned kernel above, with the work balanced
// over exactly the waves the GPU holds at once (a stream-K style split).
//
// The work is the list of (sequence b, kv head, chunk of 64 positions) in
// that order: sequence b contributes Hkv * ceil(ctx_b / 64) chunks. Wave w of
// W owns chunks [floor(w*C/W), floor((w+1)*C/W)) of the C total and streams
// through them with the next chunk's loads always in flight, also across the
// boundary between two (sequence, kv head) segments. A segment that a wave
// covers entirely is finished in place; otherwise the wave stores an
// unnormalised partial (acc, max, sum) in one of its two workspace slots --
// slot 0 for a segment that starts where the wave's range starts, slot 1 for
// the one that ends where it ends -- and decode_sk_reduce combines them.
constexpr int kSkChunk = 64;

__device__ __forceinline__ int sk_nch(int ctx) { return (ctx + kSkChunk - 1) / kSkChunk; }
// The wave whose range holds chunk x, and where wave w's range starts.
__device__ __forceinline__ int64_t sk_owner(int64_t x, int64_t C, int64_t W) { return ((x + 1) * W - 1) / C; }
__device__ __forceinline__ int64_t sk_start(int64_t w, int64_t C, int64_t W) { return w * C / W; }
// Waves the split uses out of the W launched: all of them while each gets at
// least kSkMinChunks chunks, fewer for a small batch, so that a segment spans
// fewer waves and the combine gathers fewer partials. Both kernels derive it
// from the same chunk count.
constexpr int kSkMinChunks = 2;
__device__ __forceinline__ int64_t sk_waves(int64_t C, int64_t W) {
    return max((int64_t)1, min(W, C / kSkMinChunks));
}

// Position of one chunk in the work list (all wave-uniform).
struct SkCursor {
    int b, kvh, c, ctx;
};

template <int G>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void decode_sk_kernel(DecodeArgs a) {
    constexpr int D = 128;
    constexpr int CH = kSkChunk;
    constexpr int TILES = CH / 16;   // 16-position MFMA tiles per chunk
    constexpr int VL = CH / 4;       // 16-byte V loads per lane per chunk
    constexpr int VP = 144;          // LDS row pitch of the staged V chunk (elements)
    static_assert(G >= 1 && G <= 16, "group");
    __shared__ __attribute__((aligned(16))) uint16_t vs_all[4][CH * VP];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int w = blockIdx.x * 4 + wave;
    const int W = a.waves;
    const int B = a.num_seqs, Hkv = a.Hkv;
    const int lr = lane & 15, lg = lane >> 4;

    // Chunk counts of all sequences, 64 per pass; wave 0 records the prefix
    // sums for the combine kernel.
    int total = 0;
    for (int b0 = 0; b0 < B; b0 += 64) {
        const int bb = b0 + lane;
        const int n = bb < B ? sk_nch(dec_ctx(a, bb)) : 0;
        int incl = n;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int y = __shfl_up(incl, off);
            if (lane >= off) incl += y;
        }
        if (w == 0 && bb < B) a.ws_cum[bb] = total + incl - n;
        total += __builtin_amdgcn_readfirstlane(__shfl(incl, 63));
    }
    if (w == 0 && lane == 0) a.ws_cum[B] = total;
    const int64_t C = (int64_t)Hkv * total;
    const int64_t We = sk_waves(C, W);
    if (w >= We) return;
    const int64_t x0 = sk_start(w, C, We), x1 = sk_start(w + 1, C, We);
    if (x0 >= x1) return;

    // Locate chunk x0: the sequence b with Hkv*cum_b <= x0 < Hkv*cum_(b+1).
    SkCursor cur{0, 0, 0, 0};
    {
        int base = 0;
        for (int b0 = 0; b0 < B; b0 += 64) {
            const int bb = b0 + lane;
            const int ctxv = bb < B ? dec_ctx(a, bb) : 0;
            const int n = sk_nch(ctxv);
            int incl = n;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const int y = __shfl_up(incl, off);
                if (lane >= off) incl += y;
            }
            const int64_t lo = (int64_t)Hkv * (base + incl - n), hi = (int64_t)Hkv * (base + incl);
            const uint64_t hit = __builtin_amdgcn_ballot_w64(n > 0 && lo <= x0 && x0 < hi);
            if (hit) {
                const int src = __builtin_ctzll(hit);
                cur.b = b0 + src;
                cur.ctx = __shfl(ctxv, src);
                const int64_t rem = x0 - (int64_t)Hkv * __shfl(base + incl - n, src);
                const int nch = sk_nch(cur.ctx);
                cur.kvh = (int)(rem / nch);
                cur.c = (int)(rem - (int64_t)cur.kvh * nch);
                break;
            }
            base += __builtin_amdgcn_readfirstlane(__shfl(incl, 63));
        }
    }
    cur.b = __builtin_amdgcn_readfirstlane(cur.b);
    cur.kvh = __builtin_amdgcn_readfirstlane(cur.kvh);
    cur.c = __builtin_amdgcn_readfirstlane(cur.c);
    cur.ctx = __builtin_amdgcn_readfirstlane(cur.ctx);
    // The chunk after u in the work list (u itself past the end of the list).
    auto advance = [&](SkCursor u) -> SkCursor {
        if (++u.c == sk_nch(u.ctx)) {
            u.c = 0;
            if (++u.kvh == Hkv) {
                u.kvh = 0;
                do {
                    ++u.b;
                    u.ctx = u.b < B ? dec_ctx(a, u.b) : 0;
                } while (u.b < B && u.ctx == 0);
            }
        }
        return u;
    };

    const int64_t row_bytes = (int64_t)Hkv * D * 2;
    const uint32_t rb32 = (uint32_t)row_bytes;
    const uint32_t k_lane = (uint32_t)lr * rb32 + (uint32_t)lg * 16u;
    const uint32_t v_lane = (uint32_t)lg * rb32 + (uint32_t)lr * 16u;
    uint16_t *vs = vs_all[wave];

    // Descriptor of chunk u; ok == false gives an empty range (loads return
    // zeros and touch no memory).
    auto chunk_rsrc = [&](const void *pool, const SkCursor &u, bool ok) -> __amdgpu_buffer_rsrc_t {
        const int t = u.c * CH;
        const int valid = min(CH, u.ctx - t);
        const int lb = t >> a.log2bs;
        int blk = -1;
        if (ok && valid > 0 && lb < a.maxb) blk = a.bt[(int64_t)u.b * a.maxb + lb];
        if (blk < 0 || blk >= a.num_blocks)
            return __builtin_amdgcn_make_buffer_rsrc((void *)pool, (short)0, 0, kBufWord3);
        const uint8_t *base = (const uint8_t *)pool + (int64_t)u.kvh * D * 2 +
                              ((int64_t)blk * a.bs + (t & (a.bs - 1))) * row_bytes;
        return __builtin_amdgcn_make_buffer_rsrc((void *)base, (short)0, valid * (int)rb32, kBufWord3);
    };
    // Two register buffers per operand: chunks x+1 and x+2 are in flight while
    // chunk x is computed. One VGPR offset per lane; the row step goes in the
    // scalar offset. Rows past the context may read stale pool data: K scores
    // are masked by position and V rows are zeroed before they reach LDS.
    u32x4 kx[2][TILES][4], vx[2][VL];
    auto load_k = [&](u32x4 (&dst)[TILES][4], __amdgpu_buffer_rsrc_t r) {
#pragma unroll
        for (int tile = 0; tile < TILES; ++tile)
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
                dst[tile][kk] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                    r, (int)(k_lane + 64u * kk), (int)((uint32_t)(16 * tile) * rb32), 0));
    };
    auto load_v = [&](u32x4 (&dst)[VL], __amdgpu_buffer_rsrc_t r) {
#pragma unroll
        for (int i = 0; i < VL; ++i)
            dst[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                r, (int)v_lane, (int)((uint32_t)(4 * i) * rb32), 0));
    };
    // B operand of S^T = K q^T: lane holds q[head lr][d = 32*kk + 8*lg .. +8].
    bf16x8 qb[4];
    auto load_q = [&](const SkCursor &u) {
        const uint16_t *q = (const uint16_t *)a.q + (int64_t)u.b * a.q_stride + (int64_t)(u.kvh * G + lr) * D + 8 * lg;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            u32x4 wv = {0u, 0u, 0u, 0u};
            if (lr < G) wv = ld16(q + 32 * kk);
            qb[kk] = __builtin_bit_cast(bf16x8, wv);
        }
    };

    f32x4 o[8];
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) o[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.f;
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const bf16x2 ones = {(__bf16)1.f, (__bf16)1.f};
    int64_t seg_x = x0;   // where the current segment started in this wave's range
    int seg_c = cur.c;    // ... and at which chunk of its (sequence, kv head)

    // Process chunk x = cur from buffer `buf`, refilling it with chunk x + 2.
    auto step = [&](int64_t x, const SkCursor &n1, const SkCursor &n2, u32x4 (&kb)[TILES][4],
                    u32x4 (&vb)[VL]) {
        // V(x) -> LDS with rows past the context zeroed (the pool may hold NaN
        // there), then refill the V buffer with chunk x + 2.
        const bool partial = cur.ctx - cur.c * CH < CH;   // the segment's last, short chunk
        if (partial) {
            const int v_lim = cur.ctx - cur.c * CH - lg;
#pragma unroll
            for (int i = 0; i < VL; ++i) {
                u32x4 wv = vb[i];
                if (4 * i >= v_lim) wv = u32x4{0u, 0u, 0u, 0u};
                *reinterpret_cast<u32x4 *>(vs + (lg + 4 * i) * VP + 8 * lr) = wv;
            }
        } else {
#pragma unroll
            for (int i = 0; i < VL; ++i)
                *reinterpret_cast<u32x4 *>(vs + (lg + 4 * i) * VP + 8 * lr) = vb[i];
        }
        load_v(vb, chunk_rsrc(a.vc, n2, x + 2 < x1));
        f32x4 st[TILES];
#pragma unroll
        for (int tile = 0; tile < TILES; ++tile) {
            st[tile] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
                st[tile] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    __builtin_bit_cast(bf16x8, kb[tile][kk]), qb[kk], st[tile], 0, 0, 0);
        }
        load_k(kb, chunk_rsrc(a.kc, n2, x + 2 < x1));
        // Softmax over the chunk: st[tile][r] = S[head lr][position 64*c + 16*tile + 4*lg + r].
        float mx = -INFINITY;
#pragma unroll
        for (int tile = 0; tile < TILES; ++tile)
#pragma unroll
            for (int r = 0; r < 4; ++r) st[tile][r] *= a.scale_log2;
        if (partial) {
            const int t_lim = cur.ctx - cur.c * CH - 4 * lg;
#pragma unroll
            for (int tile = 0; tile < TILES; ++tile)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (16 * tile + r >= t_lim) st[tile][r] = -INFINITY;
        }
#pragma unroll
        for (int tile = 0; tile < TILES; ++tile)
#pragma unroll
            for (int r = 0; r < 4; ++r) mx = fmaxf(mx, st[tile][r]);
        mx = xor32_max(xor16_max(mx));
        const float m_new = fmaxf(m_run, mx);
        const float alpha = fast_exp2(m_run - m_new);
        l_run *= alpha;
        m_run = m_new;
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) o[mt] *= alpha;
        wave_lds_fence();
        // O^T += V^T P^T, 32 positions per MFMA step: k-slot 8*lg + e holds
        // position 4*lg + e (e < 4) or 16 + 4*lg + e - 4 of the step.
#pragma unroll
        for (int sp = 0; sp < TILES / 2; ++sp) {
            bf16x8 pb;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                pb[r] = (__bf16)fast_exp2(st[2 * sp][r] - m_new);
                pb[4 + r] = (__bf16)fast_exp2(st[2 * sp + 1][r] - m_new);
            }
#pragma unroll
            for (int e = 0; e < 8; e += 2)
                l_run = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pb[e], pb[e + 1]}, ones, l_run, false);
            const uint16_t *src_lo = vs + (32 * sp + 4 * lg + (lr >> 2)) * VP + 4 * (lr & 3);
            const uint16_t *src_hi = src_lo + 16 * VP;
#pragma unroll
            for (int mt = 0; mt < 8; ++mt) {
                typedef short s16x4 __attribute__((ext_vector_type(4)));
                typedef short s16x8 __attribute__((ext_vector_type(8)));
                const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) s16x4 *)(src_lo + 16 * mt));
                const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) s16x4 *)(src_hi + 16 * mt));
                const s16x8 av = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
                o[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av), pb,
                                                                o[mt], 0, 0, 0);
            }
        }
        wave_lds_fence();

        const bool has_next = x + 1 < x1;
        if (!has_next || n1.b != cur.b || n1.kvh != cur.kvh) {   // the segment ends here
            const float l_tot = xor32_sum(xor16_sum(l_run));
            const bool full = seg_c == 0 && cur.c == sk_nch(cur.ctx) - 1;
            if (lr < G) {
                const int h = cur.kvh * G + lr;
                if (full) {
                    const float inv = 1.f / l_tot;
                    uint16_t *dst = (uint16_t *)a.out + ((int64_t)cur.b * a.Hq + h) * D + 4 * lg;
#pragma unroll
                    for (int mt = 0; mt < 8; ++mt) {
                        u32x2 wv;
                        wv[0] = pack_bf16x2(o[mt][0] * inv, o[mt][1] * inv);
                        wv[1] = pack_bf16x2(o[mt][2] * inv, o[mt][3] * inv);
                        *reinterpret_cast<u32x2 *>(dst + 16 * mt) = wv;
                    }
                } else {
                    const int64_t slot = ((int64_t)w * 2 + (seg_x == x0 ? 0 : 1)) * G + lr;
                    float *dst = a.ws_acc + slot * D + 4 * lg;
#pragma unroll
                    for (int mt = 0; mt < 8; ++mt)
                        st16(dst + 16 * mt, u32x4{__float_as_uint(o[mt][0]), __float_as_uint(o[mt][1]),
                                                  __float_as_uint(o[mt][2]), __float_as_uint(o[mt][3])});
                    if (lg == 0) {
                        a.ws_ml[slot * 2] = m_run;
                        a.ws_ml[slot * 2 + 1] = l_tot;
                    }
                }
            }
            if (has_next) {
#pragma unroll
                for (int mt = 0; mt < 8; ++mt) o[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
                m_run = -INFINITY;
                l_run = 0.f;
                load_q(n1);
                seg_x = x + 1;
                seg_c = n1.c;
            }
        }
    };

    SkCursor n1 = advance(cur);
    load_q(cur);
    load_v(vx[0], chunk_rsrc(a.vc, cur, true));
    load_k(kx[0], chunk_rsrc(a.kc, cur, true));
    load_v(vx[1], chunk_rsrc(a.vc, n1, x0 + 1 < x1));
    load_k(kx[1], chunk_rsrc(a.kc, n1, x0 + 1 < x1));
    for (int64_t x = x0; x < x1; x += 2) {
        SkCursor n2 = advance(n1);
        step(x, n1, n2, kx[0], vx[0]);
        if (x + 1 >= x1) break;
        cur = n1;
        n1 = n2;
        n2 = advance(n1);
        step(x + 1, n1, n2, kx[1], vx[1]);
        cur = n1;
        n1 = n2;
    }
}

template <typename T>
__device__ __forceinline__ float load_elem(const T *p, int64_t i);
template <>
__device__ __forceinline__ float load_elem<float>(const float *p, int64_t i) { return p[i]; }
template <>
__device__ __forceinline__ float load_elem<uint16_t>(const uint16_t *p, int64_t i) {
    return __uint_as_float((uint32_t)p[i] << 16);
}
template <typename T>
__device__ __forceinline__ void store_elem(T *p, int64_t i, float x);
template <>
__device__ __forceinline__ void store_elem<float>(float *p, int64_t i, float x) { p[i] = x; }
template <>
__device__ __forceinline__ void store_elem<uint16_t>(uint16_t *p, int64_t i, float x) {
    p[i] = (uint16_t)f32_to_bf16(x);
}

template <typename T, int D>
__global__ __launch_bounds__(64) void decode_generic_kernel(DecodeArgs a) {
    constexpr int EPL = D / 64;
    const int lane = threadIdx.x;
    const int p = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int kvh = h / a.group;
    const int n = dec_ctx(a, b);
    const int t_begin = p * a.P;
    if (t_begin >= n && p > 0) return;
    const int nparts = (n + a.P - 1) / a.P;
    const int t_end = min(n, t_begin + a.P);
    const T *q = (const T *)a.q + (int64_t)b * a.q_stride + (int64_t)h * D;
    const T *kc = (const T *)a.kc;
    const T *vc = (const T *)a.vc;
    float qv[EPL], acc[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
        qv[e] = load_elem<T>(q, lane * EPL + e) * a.scale_log2;
        acc[e] = 0.f;
    }
    float m = -INFINITY, l = 0.f;
    for (int t = t_begin; t < t_end; ++t) {
        const int row = decode_row(a, b, t);
        float kv[EPL], vv[EPL];
        const int64_t off = ((int64_t)(row < 0 ? 0 : row) * a.Hkv + kvh) * D + lane * EPL;
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
            kv[e] = row >= 0 ? load_elem<T>(kc, off + e) : 0.f;
            vv[e] = row >= 0 ? load_elem<T>(vc, off + e) : 0.f;
        }
        float dot = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) dot = fmaf(qv[e], kv[e], dot);
        dot = wave_sum(dot);
        const float m_new = fmaxf(m, dot);
        const float alpha = fast_exp2(m - m_new);
        const float pw = fast_exp2(dot - m_new);
        l = l * alpha + pw;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[e] = fmaf(pw, vv[e], acc[e] * alpha);
        m = m_new;
    }
    if (n == 0 || nparts == 1) {
        const float inv = n == 0 ? 0.f : 1.f / l;
        T *o = (T *)a.out + ((int64_t)b * a.Hq + h) * D;
#pragma unroll
        for (int e = 0; e < EPL; ++e) store_elem<T>(o, lane * EPL + e, acc[e] * inv);
    } else {
        float *dst = a.ws_acc + (((int64_t)b * a.maxparts + p) * a.Hq + h) * D;
#pragma unroll
        for (int e = 0; e < EPL; ++e) dst[lane * EPL + e] = acc[e];
        if (lane == 0) {
            float *ml = a.ws_ml + (((int64_t)b * a.maxparts + p) * a.Hq + h) * 2;
            ml[0] = m;
            ml[1] = l;
        }
    }
}

// Combine: M = max_p m_p; out = sum_p 2^(m_p - M) acc_p / sum_p 2^(m_p - M) l_p.
// One wave per (sequence, q head). Lane p holds partition p's statistics (in
// passes of 64); the accumulator rows are then read with the partition loop
// unrolled so that many row loads are in flight at once.
template <typename T, int D>
__global__ __launch_bounds__(256) void decode_reduce_kernel(DecodeArgs a) {
    constexpr int EPL = D / 64;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int h = blockIdx.x * 4 + wave, b = blockIdx.y;
    if (h >= a.Hq) return;
    const int n = dec_ctx(a, b);
    const int nparts = (n + a.P - 1) / a.P;
    if (nparts <= 1) return;
    const int64_t pstride = (int64_t)a.Hq;
    const float *ml = a.ws_ml + ((int64_t)b * a.maxparts * a.Hq + h) * 2;
    const float *acc = a.ws_acc + ((int64_t)b * a.maxparts * a.Hq + h) * D + lane * EPL;
    float M = -INFINITY;
    for (int p = lane; p < nparts; p += 64) M = fmaxf(M, ml[p * pstride * 2]);
    M = wave_max(M);
    float o[EPL], den = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[e] = 0.f;
    for (int p0 = 0; p0 < nparts; p0 += 64) {
        const int p = p0 + lane;
        const float w = p < nparts ? fast_exp2(ml[p * pstride * 2] - M) : 0.f;
        den = fmaf(w, p < nparts ? ml[p * pstride * 2 + 1] : 0.f, den);
        const int cnt = min(64, nparts - p0);
        int i = 0;
        for (; i + 8 <= cnt; i += 8) {
            float v[8][EPL];
#pragma unroll
            for (int u = 0; u < 8; ++u)
#pragma unroll
                for (int e = 0; e < EPL; ++e) v[u][e] = acc[(p0 + i + u) * pstride * D + e];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const float wu = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), i + u));
#pragma unroll
                for (int e = 0; e < EPL; ++e) o[e] = fmaf(wu, v[u][e], o[e]);
            }
        }
        for (; i < cnt; ++i) {
            const float wu = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), i));
#pragma unroll
            for (int e = 0; e < EPL; ++e) o[e] = fmaf(wu, acc[(p0 + i) * pstride * D + e], o[e]);
        }
    }
    den = wave_sum(den);
    const float inv = 1.f / den;
    T *out = (T *)a.out + ((int64_t)b * a.Hq + h) * D;
#pragma unroll
    for (int e = 0; e < EPL; ++e) store_elem<T>(out, lane * EPL + e, o[e] * inv);
}

// Combine for decode_sk_kernel: one wave per (sequence, q head). A segment
// owned by one wave was finished in place; otherwise its partials sit in the
// slots of waves owner(G0) .. owner(G1-1) and are combined by the same
// log-sum-exp rule. Sequences with no context get zeros.
template <int G>
__global__ __launch_bounds__(256) void decode_sk_reduce_kernel(DecodeArgs a) {
    constexpr int D = 128, EPL = 2;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int h = blockIdx.x * 4 + wave, b = blockIdx.y;
    if (h >= a.Hq) return;
    const int kvh = h / G, r = h - kvh * G;
    const int nch = sk_nch(dec_ctx(a, b));
    uint16_t *out = (uint16_t *)a.out + ((int64_t)b * a.Hq + h) * D;
    if (nch == 0) {
        *reinterpret_cast<uint32_t *>(out + lane * EPL) = 0u;
        return;
    }
    const int64_t C = (int64_t)a.Hkv * a.ws_cum[a.num_seqs];
    const int64_t W = sk_waves(C, a.waves);
    const int64_t g0 = (int64_t)a.Hkv * a.ws_cum[b] + (int64_t)kvh * nch;
    const int64_t wf = sk_owner(g0, C, W), wl = sk_owner(g0 + nch - 1, C, W);
    if (wf == wl) return;
    const int first_slot = g0 == sk_start(wf, C, W) ? 0 : 1;
    // Candidate waves wf .. wl; those with an empty range (possible when there
    // are more waves than chunks) hold nothing and are skipped.
    const int n = (int)(wl - wf + 1);
    auto holds = [&](int i) -> bool {
        return i < n && sk_start(wf + i, C, W) < sk_start(wf + i + 1, C, W);
    };
    auto slot_of = [&](int i) -> int64_t {
        return ((wf + i) * 2 + (i == 0 ? first_slot : 0)) * G + r;
    };
    float M = -INFINITY;
    for (int i = lane; i < n; i += 64)
        if (holds(i)) M = fmaxf(M, a.ws_ml[slot_of(i) * 2]);
    M = wave_max(M);
    float o0 = 0.f, o1 = 0.f, den = 0.f;
    for (int i0 = 0; i0 < n; i0 += 64) {
        const int i = i0 + lane;
        const bool ok = holds(i);
        const float wgt = ok ? fast_exp2(a.ws_ml[slot_of(i) * 2] - M) : 0.f;
        if (ok) den = fmaf(wgt, a.ws_ml[slot_of(i) * 2 + 1], den);
        // Live candidates in batches whose accumulator rows load together: one
        // round trip per batch instead of one per partial. A small batch spreads
        // one segment over many waves (16 at a time then); otherwise a segment
        // has a few partials (4 at a time, fewer idle slots).
        auto gather = [&](auto width, uint64_t &lv) {
            constexpr int kBatch = decltype(width)::value;
            int kk[kBatch];
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                kk[u] = lv ? (int)__builtin_ctzll(lv) : -1;
                lv &= lv - 1;
            }
            float v0[kBatch], v1[kBatch];
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                v0[u] = 0.f;
                v1[u] = 0.f;
                if (kk[u] >= 0) {
                    const float *acc = a.ws_acc + slot_of(i0 + kk[u]) * D + lane * EPL;
                    v0[u] = acc[0];
                    v1[u] = acc[1];
                }
            }
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                if (kk[u] < 0) continue;
                const float wk = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wgt), kk[u]));
                o0 = fmaf(wk, v0[u], o0);
                o1 = fmaf(wk, v1[u], o1);
            }
        };
        uint64_t live = __builtin_amdgcn_ballot_w64(ok);
        if (__builtin_popcountll(live) <= 4) {
            gather(std::integral_constant<int, 4>{}, live);
        } else {
            while (live) gather(std::integral_constant<int, 16>{}, live);
        }
    }
    den = wave_sum(den);
    const float inv = 1.f / den;
    *reinterpret_cast<uint32_t *>(out + lane * EPL) = pack_bf16x2(o0 * inv, o1 * inv);
}

bool decode_has_mfma_path(int dtype, int32_t d, int32_t group) {
    return dtype == 1 && d == 128 && (group == 1 || group == 2 || group == 4 || group == 8);
}

constexpr int kBlkChunk = 64;   // positions per step of decode_blk_kernel

static bool blk_shape(int dtype, int32_t d, int32_t bs, int32_t group) {
    return dtype == 1 && d == 128 && bs % kBlkChunk == 0 &&
           (group == 1 || group == 2 || group == 4 || group == 8 || group == 16);
}

static bool decode_has_blk_path(const DecodeArgs &a, int dtype) {
    return blk_shape(dtype, a.d, a.bs, a.group) && a.P % kBlkChunk == 0 && a.P <= 64 * a.bs;
}

static int32_t decode_auto_partition(int32_t num_seqs, int32_t max_ctx, int32_t Hkv, int dtype,
                                     int32_t d) {
    if (!(dtype == 1 && d == 128)) return 256;
    // Enough (sequence, kv head, partition) waves to fill 256 CUs several times
    // over, but partitions long enough that the combine stays a small cost.
    const int64_t pairs = (int64_t)num_seqs * Hkv;
    const int64_t ctx = max_ctx > 0 ? max_ctx : 1;
    int32_t P = 256;
    while (P > 64 && pairs * ((ctx + P - 1) / P) < 4096) P /= 2;
    while (P < 512 && pairs * ((ctx + P - 1) / P) > 65536) P *= 2;
    return P;
}

// Waves of the balanced decode grid: one per SIMD on every CU of the current
// device (PKV_DECODE_WAVES, a positive multiple of 4, overrides it).
static int32_t balanced_waves() {
    if (const char *e = getenv("PKV_DECODE_WAVES")) {
        const int v = atoi(e);
        if (v >= 4 && v % 4 == 0) return v;
    }
    static int32_t cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 1024;
    if (!cached[dev]) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
            cus = 256;
        cached[dev] = cus * 4;   // one wave per SIMD
    }
    return cached[dev];
}

static int64_t align256(int64_t x) { return (x + 255) & ~int64_t(255); }

// Small batches take fixed partitions: up to 64 (sequence, kv head) pairs,
// the balanced split's fixed costs (every wave's scan of the context
// lengths, the split bookkeeping, its combine) outweigh its balance. The
// partition is the shortest of 64..512 positions that keeps pairs *
// partitions within 1024 (measured 16-35% faster than the split at 1-8
// sequences of up to 32k tokens; from 16 sequences on the two are within a
// few percent, and at 48 and more the split is faster). Only while the
// partials stay within 8 MiB; 0 when the split should be used.
static int32_t small_batch_partition(int32_t num_seqs, int32_t max_ctx, int32_t Hq, int32_t Hkv,
                                     int32_t d) {
    const int64_t pairs = (int64_t)num_seqs * Hkv;
    if (pairs > 64 || max_ctx <= 0) return 0;
    int32_t P = 64;
    while (P < 512 && pairs * (((int64_t)max_ctx + P - 1) / P) > 1024) P *= 2;
    const int64_t parts = ((int64_t)max_ctx + P - 1) / P;
    const int64_t bytes = (int64_t)num_seqs * parts * Hq * (d + 2) * 4;
    return bytes <= (int64_t(8) << 20) ? P : 0;
}

DecodePlan plan_decode(int32_t num_seqs, int32_t max_ctx, int32_t Hq, int32_t Hkv, int32_t d,
                       int32_t bs, int dtype, int32_t partition_size) {
    DecodePlan p{};
    const int32_t group = Hkv > 0 ? Hq / Hkv : 1;
    // The balanced split counts chunks in 32-bit integers: all of them,
    // num_seqs * Hkv * ceil(max_ctx / 64), must fit.
    const int64_t chunks = (int64_t)num_seqs * Hkv * (((int64_t)max(max_ctx, 0) + kSkChunk - 1) / kSkChunk);
    const bool can_balance = blk_shape(dtype, d, bs, group) && chunks <= INT32_MAX;
    const int32_t small_P =
        partition_size == 0 && can_balance ? small_batch_partition(num_seqs, max_ctx, Hq, Hkv, d) : 0;
    p.balanced = can_balance && (partition_size == PKV_PARTITION_BALANCED || (partition_size == 0 && small_P == 0));
    if (p.balanced) {
        p.waves = balanced_waves();
        p.P = 0;
        p.maxparts = 0;
        p.acc_bytes = align256((int64_t)p.waves * 2 * group * d * 4);
        p.ml_bytes = align256((int64_t)p.waves * 2 * group * 2 * 4);
        p.cum_bytes = align256((int64_t)(num_seqs + 1) * 4);
        p.total = p.acc_bytes + p.ml_bytes + p.cum_bytes;
        return p;
    }
    p.P = partition_size > 0 ? partition_size
          : small_P > 0      ? small_P
                             : decode_auto_partition(num_seqs, max_ctx, Hkv, dtype, d);
    p.maxparts = max_ctx > 0 ? (int32_t)((max_ctx + (int64_t)p.P - 1) / p.P) : 1;
    if (p.maxparts <= 1) {
        p.maxparts = 1;
        return p;
    }
    p.acc_bytes = align256((int64_t)num_seqs * p.maxparts * Hq * d * 4);
    p.ml_bytes = align256((int64_t)num_seqs * p.maxparts * Hq * 2 * 4);
    p.total = p.acc_bytes + p.ml_bytes;
    return p;
}

template <typename T, int D>
static void launch_generic(const DecodeArgs &a, hipStream_t stream) {
    hipLaunchKernelGGL((decode_generic_kernel<T, D>), dim3(a.maxparts, a.Hq, a.num_seqs),
                       dim3(64), 0, stream, a);
}

template <int G>
static void launch_sk(const DecodeArgs &a, hipStream_t stream) {
    hipLaunchKernelGGL((decode_sk_kernel<G>), dim3(a.waves / 4), dim3(256), 0, stream, a);
    hipLaunchKernelGGL((decode_sk_reduce_kernel<G>), dim3((a.Hq + 3) / 4, a.num_seqs), dim3(256), 0,
                       stream, a);
}

template <int G>
static void launch_blk(const DecodeArgs &a, hipStream_t stream) {
    const dim3 grid((a.Hkv + 3) / 4, a.maxparts, a.num_seqs);
    if (a.st_k)
        hipLaunchKernelGGL((decode_blk_kernel<G, kBlkChunk, true>), grid, dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL((decode_blk_kernel<G, kBlkChunk, false>), grid, dim3(256), 0, stream, a);
}

template <int G>
static void launch_mfma(const DecodeArgs &a, hipStream_t stream) {
    const dim3 grid(a.maxparts, a.num_seqs, (a.Hkv + kDecWaves - 1) / kDecWaves);
    hipLaunchKernelGGL((decode_mfma_kernel<G, kDecChunk>), grid, dim3(64 * kDecWaves), 0,
                       stream, a);
}

bool decode_store_fusable(const DecodeArgs &a, const DecodePlan &plan, int dtype) {
    return !plan.balanced && decode_has_blk_path(a, dtype) &&
           (a.group == 1 || a.group == 2 || a.group == 4 || a.group == 8 || a.group == 16);
}

hipError_t launch_decode(const DecodeArgs &a, const DecodePlan &plan, int dtype, hipStream_t stream) {
    if (a.num_seqs == 0) return hipSuccess;
    if (a.st_k && !decode_store_fusable(a, plan, dtype)) return hipErrorInvalidValue;
    if (plan.balanced) {
        switch (a.group) {
            case 1: launch_sk<1>(a, stream); break;
            case 2: launch_sk<2>(a, stream); break;
            case 4: launch_sk<4>(a, stream); break;
            case 8: launch_sk<8>(a, stream); break;
            case 16: launch_sk<16>(a, stream); break;
            default: return hipErrorNotSupported;
        }
        return hipGetLastError();
    }
    if (decode_has_blk_path(a, dtype)) {
        switch (a.group) {
            case 1: launch_blk<1>(a, stream); break;
            case 2: launch_blk<2>(a, stream); break;
            case 4: launch_blk<4>(a, stream); break;
            case 8: launch_blk<8>(a, stream); break;
            case 16: launch_blk<16>(a, stream); break;
            default: return hipErrorNotSupported;
        }
    } else if (decode_has_mfma_path(dtype, a.d, a.group)) {
        switch (a.group) {
            case 1: launch_mfma<1>(a, stream); break;
            case 2: launch_mfma<2>(a, stream); break;
            case 4: launch_mfma<4>(a, stream); break;
            case 8: launch_mfma<8>(a, stream); break;
            default: return hipErrorNotSupported;
        }
    } else if (dtype == 0 && a.d == 64) {
        launch_generic<float, 64>(a, stream);
    } else if (dtype == 0 && a.d == 128) {
        launch_generic<float, 128>(a, stream);
    } else if (dtype == 1 && a.d == 64) {
        launch_generic<uint16_t, 64>(a, stream);
    } else if (dtype == 1 && a.d == 128) {
        launch_generic<uint16_t, 128>(a, stream);
    } else {
        return hipErrorNotSupported;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.maxparts <= 1) return e;
    const dim3 grid((a.Hq + 3) / 4, a.num_seqs);
    if (dtype == 0 && a.d == 64)
        hipLaunchKernelGGL((decode_reduce_kernel<float, 64>), grid, dim3(256), 0, stream, a);
    else if (dtype == 0)
        hipLaunchKernelGGL((decode_reduce_kernel<float, 128>), grid, dim3(256), 0, stream, a);
    else if (a.d == 64)
        hipLaunchKernelGGL((decode_reduce_kernel<uint16_t, 64>), grid, dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL((decode_reduce_kernel<uint16_t, 128>), grid, dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace pkv
