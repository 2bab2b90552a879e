// prefill.hip -- varlen causal prefill attention over a flattened ragged batch.
//
// Sequence s owns query rows [cu_q[s], cu_q[s+1]) and keys [0, Lk); query i
// sits at position Lk - Lq + i and sees keys up to it ("Nano vLLM 解读（5）：
// 解析 ModelRunner", "FlashAttention Kernel 函参准备" and "prepare_prefill";
// "nano-vLLM-1", "4. prefill 输入打包": positions start at num_cached_tokens).
// Keys come from the call's contiguous k/v rows, or -- on a prefix-cache hit
// -- from the pool through the block table ("nano-vLLM-1", "5. deocde 输入打包",
// the block_table difference between prefill and decode). The result is
// softmax(scale * Q K^T + causal mask) V ("【nano-vllm 学习】04 - …源码学习2",
// "KV-Cache … 是什么？").
//
// prefill_mfma_kernel (bf16, head_dim 128) is a FlashAttention-2 style forward
// (Dao, 2023) laid out for CDNA4: a workgroup of 4 waves owns 128 query rows of
// one head (32 per wave) and streams 64-key tiles of K and V through two LDS
// buffers (the next tile's global loads are in flight while the current one
// is computed; one barrier per tile). Both contractions run on
// v_mfma_f32_32x32x16_bf16 in the transposed form
//     S^T = K Q^T        (keys as MFMA rows, the wave's queries as columns)
//     O^T += V^T P^T     (head dims as rows, queries as columns)
// so that every lane owns one query row: the row max needs a single
// cross-lane exchange, the rescale by exp2(m_old - m_new) is lane-local, and
// P^T is fed to the second MFMA straight from the registers the first one
// produced. V stays row-major in LDS; the V^T operand comes from the gfx950
// transpose read (ds_read_b64_tr_b16), two reads of 4 consecutive keys per
// MFMA. A wave skips key tiles that lie entirely above its causal diagonal.
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

constexpr int kPfD = 128;
constexpr int kPfBM = 128;     // query rows per workgroup
constexpr int kPfBN = 64;      // keys per tile
constexpr int kPitch = 144;    // LDS row pitch of the K and V tiles (elements)
constexpr float kLazy = 8.f;   // log2 headroom before the running max is moved

// Element offset of key `key` of sequence s in its source (k rows or the
// pool), for kv head kvh; -1 when the table entry is outside the pool.
__device__ __forceinline__ int64_t prefill_key_off(const PrefillArgs &a, int s, int k_start,
                                                   int key, int kvh, int D) {
    if (!a.paged) return (int64_t)(k_start + key) * a.kv_stride + (int64_t)kvh * D;
    const int lb = key >> a.log2bs;
    if (lb >= a.maxb) return -1;
    const int blk = a.bt[(int64_t)s * a.maxb + lb];
    if (blk < 0 || blk >= a.num_blocks) return -1;
    const int64_t row = (int64_t)blk * a.bs + (key & (a.bs - 1));
    return (row * a.Hkv + kvh) * D;
}

// Where a 64-key tile of K/V comes from.
enum KeySource {
    kContiguous = 0,   // the call's k/v rows: one descriptor per sequence
    kPoolBlocks = 1,   // the pool, block_size a multiple of 64: one descriptor per tile
    kPoolSmall = 2     // the pool, smaller blocks: a block-table read per key
};

template <int SRC>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void prefill_mfma_kernel(PrefillArgs a) {
    // Two LDS buffers, each a K tile and a V tile [64 keys][kPitch], row-major.
    __shared__ __attribute__((aligned(16))) uint16_t lds[2][2][kPfBN * kPitch];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int h = blockIdx.x, s = blockIdx.y;
    const int qt = gridDim.z - 1 - blockIdx.z;   // longest (last) query tiles first
    const int q_start = a.cu_q[s];
    const int Lq = a.cu_q[s + 1] - q_start;
    const int q0 = qt * kPfBM;
    if (q0 >= Lq) return;
    const int k_start = a.cu_k[s];
    const int Lk = a.cu_k[s + 1] - k_start;
    const int off = Lk - Lq;
    const int kvh = h / a.group;
    const int r32 = lane & 31, j = lane >> 5;
    const int my_row = q0 + 32 * wave + r32;
    const bool row_ok = my_row < Lq;
    const int my_pos = off + my_row;

    // B operand of S^T = K Q^T: lane holds Q[row r32][d = 16*kk + 8*j .. +8].
    bf16x8 qb[8];
    {
        const uint16_t *q = (const uint16_t *)a.q + (int64_t)(q_start + my_row) * a.q_stride +
                            (int64_t)h * kPfD + 8 * j;
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
            u32x4 w = {0u, 0u, 0u, 0u};
            if (row_ok) w = ld16(q + 16 * kk);
            qb[kk] = __builtin_bit_cast(bf16x8, w);
        }
    }
    const int kend = min(Lk, off + min(q0 + kPfBM, Lq));   // keys this block needs
    const int n_kt = (kend + kPfBN - 1) / kPfBN;
    const int wave_pos0 = off + q0 + 32 * wave;            // the wave's first row position
    const int wave_pos1 = wave_pos0 + 31;                  // ... and its last

    // Tile loader: thread -> keys (tid/16 + 16*it), 16-byte chunk tid%16, for
    // K and V. Keys at or past kend read as zeros (buffer range check).
    const uint8_t *kbase = (const uint8_t *)(SRC == kContiguous ? a.k : a.kc) + (int64_t)kvh * kPfD * 2;
    const uint8_t *vbase = (const uint8_t *)(SRC == kContiguous ? a.v : a.vc) + (int64_t)kvh * kPfD * 2;
    const uint32_t stride_b = (uint32_t)(SRC == kContiguous ? a.kv_stride * 2 : (int64_t)a.Hkv * kPfD * 2);
    const uint32_t lane_off = (uint32_t)(tid >> 4) * stride_b + (uint32_t)(tid & 15) * 16u;
    const int32_t *bt_row = a.bt + (int64_t)s * a.maxb;
    u32x4 kreg[4], vreg[4];
    auto load_tile = [&](int k0) {
        if constexpr (SRC == kPoolSmall) {
#pragma unroll
            for (int it = 0; it < 4; ++it) {
                const int key = k0 + (tid >> 4) + 16 * it;
                u32x4 kw = {0u, 0u, 0u, 0u}, vw = {0u, 0u, 0u, 0u};
                if (key < kend) {
                    const int64_t eo = prefill_key_off(a, s, k_start, key, kvh, kPfD);
                    if (eo >= 0) {
                        kw = ld16((const uint8_t *)a.kc + eo * 2 + (tid & 15) * 16);
                        vw = ld16((const uint8_t *)a.vc + eo * 2 + (tid & 15) * 16);
                    }
                }
                kreg[it] = kw;
                vreg[it] = vw;
            }
        } else {
            const int valid = min(kPfBN, kend - k0);
            int64_t row0;   // first row of the tile in its source
            bool ok = valid > 0;
            if constexpr (SRC == kContiguous) {
                row0 = (int64_t)k_start + k0;
            } else {
                const int lb = k0 >> a.log2bs;
                const int blk = (ok && lb < a.maxb) ? bt_row[lb] : -1;
                ok = ok && blk >= 0 && blk < a.num_blocks;
                row0 = (int64_t)blk * a.bs + (k0 & (a.bs - 1));
            }
            const int nrec = ok ? valid * (int)stride_b : 0;
            const int64_t rb = ok ? row0 * stride_b : 0;
            const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc((void *)(kbase + rb), (short)0, nrec, kBufWord3);
            const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc((void *)(vbase + rb), (short)0, nrec, kBufWord3);
#pragma unroll
            for (int it = 0; it < 4; ++it) {
                const int o = (int)(lane_off + (uint32_t)(16 * it) * stride_b);
                kreg[it] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, o, 0, 0));
                vreg[it] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rv, o, 0, 0));
            }
        }
    };
    auto store_tile = [&](int buf) {
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            const int o = ((tid >> 4) + 16 * it) * kPitch + 8 * (tid & 15);
            *reinterpret_cast<u32x4 *>(&lds[buf][0][o]) = kreg[it];
            *reinterpret_cast<u32x4 *>(&lds[buf][1][o]) = vreg[it];
        }
    };

    float m = -INFINITY, l = 0.f;
    f32x16 o[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[nt][r] = 0.f;
    const float c = a.scale_log2;
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const bf16x2 ones = {(__bf16)1.f, (__bf16)1.f};

    load_tile(0);
    store_tile(0);
    __syncthreads();
    for (int kt = 0; kt < n_kt; ++kt) {
        const int k0 = kt * kPfBN;
        const int buf = kt & 1;
        if (kt + 1 < n_kt) load_tile(k0 + kPfBN);
        const uint16_t *Ks = lds[buf][0];
        const uint16_t *Vs = lds[buf][1];
        if (k0 <= wave_pos1) {   // some key of the tile is visible to some row of the wave
            // S^T tiles: st[mt][r] = S[row r32][key k0 + 32*mt + 8*(r/4) + 4*j + r%4].
            f32x16 st[2];
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
                for (int r = 0; r < 16; ++r) st[mt][r] = 0.f;
#pragma unroll
                for (int kk = 0; kk < 8; ++kk) {
                    const u32x4 ka = *reinterpret_cast<const u32x4 *>(
                        &Ks[(32 * mt + r32) * kPitch + 16 * kk + 8 * j]);
                    st[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, ka),
                                                                     qb[kk], st[mt], 0, 0, 0);
                }
            }
            // Causal mask on the tiles that cross the wave's diagonal: key
            // k0 + 32*mt + 8*(r/4) + 4*j + r%4 is hidden when its in-tile
            // offset exceeds lim = my_pos - k0 - 4*j.
            if (row_ok && k0 + kPfBN - 1 > wave_pos0) {
                const int lim = my_pos - k0 - 4 * j;
#pragma unroll
                for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        if (32 * mt + 8 * (r >> 2) + (r & 3) > lim) st[mt][r] = -INFINITY;
            }
            // Online softmax in the exp2 domain on raw scores: the max is taken
            // on q.k, and p = exp2(q.k * c - m * c) with c = scale * log2(e) is
            // one FMA feeding v_exp_f32. The running max m is moved (and O, l
            // rescaled) only when some row's tile max exceeds it by more than
            // kLazy / c, so p <= 2^kLazy; the final division by l makes the
            // result independent of when the rescales happened.
            float mx = -INFINITY;
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int r = 0; r < 16; r += 2) mx = fmaxf(fmaxf(mx, st[mt][r]), st[mt][r + 1]);
            mx = xor32_max(mx);
            const bool grow = mx * c > m * c + kLazy;
            if (__builtin_amdgcn_ballot_w64(grow) != 0) {   // the decision is wave-wide
                const float m_new = fmaxf(m, mx);
                const float alpha = m == m_new ? 1.f : fast_exp2((m - m_new) * c);
                l *= alpha;
#pragma unroll
                for (int nt = 0; nt < 4; ++nt)
#pragma unroll
                    for (int r = 0; r < 16; ++r) o[nt][r] *= alpha;
                m = m_new;
            }
            const float mc = m * c;

            // O^T += V^T P^T over 4 steps of 16 keys. In step (mt, ap) lane
            // half j supplies keys 32*mt + 16*ap + 8*(e/4) + 4*j + e%4, e = 0..7:
            // its own S^T registers 8*ap .. 8*ap+7, and two transpose reads of
            // 4 consecutive V rows for the A operand. The row sum l adds the
            // same bf16-rounded weights that enter the MFMA (v_dot2 with ones).
            const int q16 = lane & 15, g2 = (lane >> 4) & 1;
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int ap = 0; ap < 2; ++ap) {
                    bf16x8 pb;
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        pb[e] = (__bf16)fast_exp2(__builtin_fmaf(st[mt][8 * ap + e], c, -mc));
#pragma unroll
                    for (int e = 0; e < 8; e += 2)
                        l = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pb[e], pb[e + 1]}, ones, l, false);
                    const int t_lo = 32 * mt + 16 * ap + 4 * j + (q16 >> 2);
                    const uint16_t *src_lo = Vs + t_lo * kPitch + 16 * g2 + 4 * (q16 & 3);
                    const uint16_t *src_hi = src_lo + 8 * kPitch;
#pragma unroll
                    for (int nt = 0; nt < 4; ++nt) {
                        typedef short s16x4 __attribute__((ext_vector_type(4)));
                        typedef short s16x8 __attribute__((ext_vector_type(8)));
                        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                            (__attribute__((address_space(3))) s16x4 *)(src_lo + 32 * nt));
                        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                            (__attribute__((address_space(3))) s16x4 *)(src_hi + 32 * nt));
                        const s16x8 av = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
                        o[nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                            __builtin_bit_cast(bf16x8, av), pb, o[nt], 0, 0, 0);
                    }
                }
        }
        if (kt + 1 < n_kt) store_tile(buf ^ 1);
        __syncthreads();
    }

    l = xor32_sum(l);
    if (row_ok) {
        const float inv = 1.f / l;
        uint16_t *out = (uint16_t *)a.out + ((int64_t)(q_start + my_row) * a.Hq + h) * kPfD;
        // o[nt][4*g + c] = O[row][d = 32*nt + 8*g + 4*j + c]
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                u32x2 w;
                w[0] = pack_bf16x2(o[nt][4 * g] * inv, o[nt][4 * g + 1] * inv);
                w[1] = pack_bf16x2(o[nt][4 * g + 2] * inv, o[nt][4 * g + 3] * inv);
                *reinterpret_cast<u32x2 *>(out + 32 * nt + 8 * g + 4 * j) = w;
            }
    }
}

template <typename T>
__device__ __forceinline__ float pf_load(const T *p, int64_t i);
template <>
__device__ __forceinline__ float pf_load<float>(const float *p, int64_t i) { return p[i]; }
template <>
__device__ __forceinline__ float pf_load<uint16_t>(const uint16_t *p, int64_t i) {
    return __uint_as_float((uint32_t)p[i] << 16);
}
template <typename T>
__device__ __forceinline__ void pf_store(T *p, int64_t i, float x);
template <>
__device__ __forceinline__ void pf_store<float>(float *p, int64_t i, float x) { p[i] = x; }
template <>
__device__ __forceinline__ void pf_store<uint16_t>(uint16_t *p, int64_t i, float x) {
    p[i] = (uint16_t)f32_to_bf16(x);
}

// One wave per (query row, q head): plain online softmax with wave reductions.
template <typename T, int D>
__global__ __launch_bounds__(256) void prefill_generic_kernel(PrefillArgs a) {
    constexpr int EPL = D / 64;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int row = blockIdx.x * 4 + wave, h = blockIdx.y, s = blockIdx.z;
    const int q_start = a.cu_q[s];
    const int Lq = a.cu_q[s + 1] - q_start;
    if (row >= Lq) return;
    const int k_start = a.cu_k[s];
    const int Lk = a.cu_k[s + 1] - k_start;
    const int pos = Lk - Lq + row;
    const int kvh = h / a.group;
    const T *q = (const T *)a.q + (int64_t)(q_start + row) * a.q_stride + (int64_t)h * D;
    const T *kb = (const T *)(a.paged ? a.kc : a.k);
    const T *vb = (const T *)(a.paged ? a.vc : a.v);
    float qv[EPL], acc[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
        qv[e] = pf_load<T>(q, lane * EPL + e) * a.scale_log2;
        acc[e] = 0.f;
    }
    float m = -INFINITY, l = 0.f;
    const int last = min(pos, Lk - 1);
    for (int key = 0; key <= last; ++key) {
        const int64_t eo = prefill_key_off(a, s, k_start, key, kvh, D);
        float kv[EPL], vv[EPL];
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
            kv[e] = eo >= 0 ? pf_load<T>(kb, eo + lane * EPL + e) : 0.f;
            vv[e] = eo >= 0 ? pf_load<T>(vb, eo + lane * EPL + e) : 0.f;
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
    const float inv = last >= 0 ? 1.f / l : 0.f;
    T *o = (T *)a.out + ((int64_t)(q_start + row) * a.Hq + h) * D;
#pragma unroll
    for (int e = 0; e < EPL; ++e) pf_store<T>(o, lane * EPL + e, acc[e] * inv);
}

hipError_t launch_prefill(const PrefillArgs &a, int dtype, hipStream_t stream) {
    if (a.num_seqs == 0 || a.max_seqlen_q == 0) return hipSuccess;
    if (dtype == 1 && a.d == 128) {
        const dim3 grid(a.Hq, a.num_seqs, (a.max_seqlen_q + kPfBM - 1) / kPfBM);
        if (!a.paged)
            hipLaunchKernelGGL(prefill_mfma_kernel<kContiguous>, grid, dim3(256), 0, stream, a);
        else if (a.bs % kPfBN == 0)
            hipLaunchKernelGGL(prefill_mfma_kernel<kPoolBlocks>, grid, dim3(256), 0, stream, a);
        else
            hipLaunchKernelGGL(prefill_mfma_kernel<kPoolSmall>, grid, dim3(256), 0, stream, a);
    } else {
        const dim3 grid((a.max_seqlen_q + 3) / 4, a.Hq, a.num_seqs);
        if (dtype == 0 && a.d == 64)
            hipLaunchKernelGGL((prefill_generic_kernel<float, 64>), grid, dim3(256), 0, stream, a);
        else if (dtype == 0 && a.d == 128)
            hipLaunchKernelGGL((prefill_generic_kernel<float, 128>), grid, dim3(256), 0, stream, a);
        else if (dtype == 1 && a.d == 64)
            hipLaunchKernelGGL((prefill_generic_kernel<uint16_t, 64>), grid, dim3(256), 0, stream,
                               a);
        else
            return hipErrorNotSupported;
    }
    return hipGetLastError();
}

}  // namespace pkv
