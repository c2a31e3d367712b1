// kvq_attn_common.h -- device code shared by the decode-attention kernels:
// the vector-ALU pass over a token range, the hand-off of per-workgroup
// partial results, and their log-sum-exp merge by the last workgroup of each
// stream to finish.
//
// Attention o = softmax(q K^T / sqrt(D)) V over one query token per sequence
// (KVTuner summary, A3 attention equation), in the log2 domain: q is
// prescaled by log2(e) / sqrt(D) and exp2 is used throughout.  Quantized
// tokens are dequantized on the fly, x^ = code * s + z (KVmix notes, key
// design 4); the query heads of one GQA group share each K/V read (KIVI notes,
// section 7.2).
#pragma once

#include <hip/hip_fp16.h>

#include "kvq_internal.h"
#include "kvq_layout.h"

namespace kvq {

constexpr int kAttnThreads = 256;
constexpr int kMaxG = 16;

// Page ids of up to 64 consecutive pages of one sequence, one per lane of a
// wave (paged layers).  A kernel loads them once for a run of tokens and then
// takes each block's page from a register (readlane for a wave-uniform token,
// bpermute for a per-lane one), so that no data load waits on a table read in
// the middle of a round.
struct WavePages {
    int first = 0;  // page index within the sequence held by lane 0
    int n = 0;      // pages held
    int id = 0;     // this lane's page id (first + lane), clamped into the pool

    // pages of tokens [t0, t1) all held?
    __device__ bool covers(const QAddr &qa, int t0, int t1) const
    {
        const int p0 = t0 >> qa.P_log2, p1 = (t1 - 1) >> qa.P_log2;
        return p0 >= first && p1 < first + n;
    }
    // hold the pages from token t0's on (up to 64, none past token t_end - 1)
    __device__ void load(const QAddr &qa, int lane, int t0, int t_end)
    {
        first = t0 >> qa.P_log2;
        const int last = (t_end - 1) >> qa.P_log2;
        n = min(64, last - first + 1);
        id = qa.clamp_page(qa.trow[first + min(lane, n - 1)]);
    }
    // row of token t: t the same in every lane / per lane (every lane active)
    __device__ size_t row_u(const QAddr &qa, int t) const
    {
        return qa.page_row(__builtin_amdgcn_readlane(id, (t >> qa.P_log2) - first), t);
    }
    __device__ size_t row_v(const QAddr &qa, int t) const
    {
        return qa.page_row(__builtin_amdgcn_ds_bpermute(((t >> qa.P_log2) - first) << 2, id), t);
    }
    __device__ size_t grp_v(const QAddr &qa, int gi) const
    {
        return qa.page_grp(__builtin_amdgcn_ds_bpermute((((gi * qa.G) >> qa.P_log2) - first) << 2, id), gi);
    }
};

// Partial entry of one (stream, workgroup, head): o[D], then m (log2 domain),
// l and two unused floats.  16-byte aligned (D is a multiple of 4).
__device__ __forceinline__ int part_stride(int D) { return D + 4; }

// Partials pass between workgroups of one launch, which may run on different
// XCDs with separate L2 caches.  They are written and read with device-coherent
// accesses (write-through stores, loads that bypass a possibly stale L2), so
// the hand-off needs no whole-cache write-back or invalidation.
__device__ __forceinline__ void part_store(float *p, float v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

typedef float f4_t __attribute__((ext_vector_type(4)));

// Cache-policy bit of a buffer access that makes it coherent across the
// device (the agent-scope bit; the accesses skip or write through L2).
constexpr int kDeviceCoherent = 16;

// Buffer view of the partial entries of one stream, with 16-byte coherent
// accesses (hardware range-checked against the stream's entries).
struct PartBuf {
    __amdgpu_buffer_rsrc_t r;

    __device__ PartBuf(const AttnArgs &a, int bh)
    {
        const size_t n = static_cast<size_t>(a.n_part) * part_entry_floats(a.g, a.D);
        r = __builtin_amdgcn_make_buffer_rsrc(a.part + static_cast<size_t>(bh) * n, 0,
                                              static_cast<int>(n * 4), 0x00020000);
    }
    // float offset of (entry, head, channel)
    __device__ int off(const AttnArgs &a, int entry, int h, int c) const
    {
        return entry * part_entry_floats(a.g, a.D) + h * part_stride(a.D) + c;
    }
    __device__ void store4(int off_f, f4_t v) const
    {
        __builtin_amdgcn_raw_buffer_store_b128(v, r, off_f * 4, 0, kDeviceCoherent);
    }
    __device__ f4_t load4(int off_f) const
    {
        return __builtin_amdgcn_raw_buffer_load_b128(r, off_f * 4, 0, kDeviceCoherent);
    }
    // when every writer ran on this workgroup's XCD: their write-through
    // stores passed this XCD's L2, so a load that only bypasses the L1 is
    // coherent with them (cache-policy bit sc0)
    __device__ f4_t load4_xcd(int off_f) const
    {
        return __builtin_amdgcn_raw_buffer_load_b128(r, off_f * 4, 0, 1);
    }
};

// Lengths of stream bh: those of the launch, or, for a ragged batch, those of
// the stream's sequence from the launch's tables.
struct StreamDims {
    int N, Tq, unit_groups, unit_extra, new_t;
};

__device__ __forceinline__ StreamDims stream_dims(const AttnArgs &a, const RaggedTables *rt, int bh)
{
    if (rt) {
        const int b = bh / a.Hkv;
        return StreamDims{rt->N[b], rt->Tq[b], rt->unit_groups[b], rt->unit_extra[b], rt->new_t[b]};
    }
    return StreamDims{a.N, a.Tq, a.unit_groups, a.unit_extra, a.new_t};
}

__device__ __forceinline__ float widen16(uint16_t x, int bf16)
{
    if (bf16)
        return __uint_as_float(static_cast<uint32_t>(x) << 16);
    return __half2float(__ushort_as_half(x));
}

__device__ __forceinline__ float load_q(const void *q, int dtype, size_t i)
{
    if (dtype == 0)
        return static_cast<const float *>(q)[i];
    return widen16(static_cast<const uint16_t *>(q)[i], dtype == 2);
}

__device__ __forceinline__ float wave_max(float v)
{
    for (int off = 32; off > 0; off >>= 1)
        v = fmaxf(v, __shfl_xor(v, off, 64));
    return v;
}

__device__ __forceinline__ float wave_sum(float v)
{
    for (int off = 32; off > 0; off >>= 1)
        v += __shfl_xor(v, off, 64);
    return v;
}

// Reductions over the four lanes l, l ^ 16, l ^ 32, l ^ 48 (one column of a
// 16-row matrix-core tile), with two VALU lane swaps instead of LDS shuffles:
// the 16-lane swap exchanges rows 0 <-> 1 and 2 <-> 3 of two copies of v, the
// 32-lane swap the two halves.
__device__ __forceinline__ float col_max(float v)
{
    const auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
    const auto t = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(t[0]), __uint_as_float(t[1]));
}

__device__ __forceinline__ float col_sum(float v)
{
    const auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(s[0]) + __uint_as_float(s[1]);
    const auto t = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(t[0]) + __uint_as_float(t[1]);
}

// K code of channel c in a token-major packed row.
__device__ __forceinline__ uint32_t row_code(const uint32_t *row, int bits, int c)
{
    if (bits == 3) {
        const int sl = c % 11;
        return (row[c / 11] >> (3 * sl)) & (sl == 10 ? 3u : 7u);
    }
    const int bitpos = c * bits;
    return (row[bitpos >> 5] >> (bitpos & 31)) & ((1u << bits) - 1u);
}

// Tokens per tile of the vector-ALU pass: 16 KB of 16-bit K (or V) per tile.
template <int D>
constexpr int valu_tile() { return 8192 / D; }

// Dynamic LDS bytes valu_range<D, GM>() needs: q[g][D], weights[g][TT],
// K tile (16 KB), V tile (16 KB), reductions.
__host__ __device__ inline int valu_lds_bytes(int g, int D)
{
    const int TT = 8192 / D;
    return (g * D + g * TT + 4 * 4 * kMaxG) * 4 + 2 * 16384;
}

// Cooperative copies into LDS.  Every thread first issues all of its global
// loads (up to MAXI 16-byte chunks, predicated), then stores them: one memory
// round trip per stage instead of one per loop iteration.  The chunks are
// native vectors, which stay in registers (an array of the struct-based uint4
// under predicated loads was kept in scratch memory, one round trip per load).
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// n 32-bit words from src (16-byte aligned when n is a multiple of 4).
template <int MAXI>
__device__ __forceinline__ void stage_words(uint32_t *dst, const uint32_t *src, int n)
{
    if ((n & 3) == 0 && (reinterpret_cast<uintptr_t>(src) & 15) == 0) {
        u32x4_t v[MAXI];
#pragma unroll
        for (int k = 0; k < MAXI; ++k) {
            const int i = threadIdx.x + k * kAttnThreads;
            v[k] = u32x4_t{0u, 0u, 0u, 0u};
            if (i < n / 4)
                v[k] = reinterpret_cast<const u32x4_t *>(src)[i];
        }
#pragma unroll
        for (int k = 0; k < MAXI; ++k) {
            const int i = threadIdx.x + k * kAttnThreads;
            if (i < n / 4)
                reinterpret_cast<u32x4_t *>(dst)[i] = v[k];
        }
    } else {
        uint32_t v[4 * MAXI];
#pragma unroll
        for (int k = 0; k < 4 * MAXI; ++k) {
            const int i = threadIdx.x + k * kAttnThreads;
            if (i < n)
                v[k] = src[i];
        }
#pragma unroll
        for (int k = 0; k < 4 * MAXI; ++k) {
            const int i = threadIdx.x + k * kAttnThreads;
            if (i < n)
                dst[i] = v[k];
        }
    }
}

// Ring rows of tokens [t0, t0 + n) into LDS [n][D] (n * D / 8 <= MAXI * 256).
// Token new_t, when in range, is read from new_row instead of the ring and
// also stored into its ring slot.
template <int D, int MAXI>
__device__ __forceinline__ void stage_ring(uint16_t *dst, uint16_t *ring, int R, int t0, int n,
                                           const uint16_t *new_row, int new_t)
{
    constexpr int CH = D / 8;  // 16-byte chunks per row
    u32x4_t v[MAXI];
#pragma unroll
    for (int k = 0; k < MAXI; ++k) {
        const int it = threadIdx.x + k * kAttnThreads;
        v[k] = u32x4_t{0u, 0u, 0u, 0u};
        if (it < n * CH) {
            const int t = t0 + it / CH;
            const uint16_t *row = (t == new_t) ? new_row : ring + static_cast<size_t>(t % R) * D;
            v[k] = reinterpret_cast<const u32x4_t *>(row)[it % CH];
        }
    }
#pragma unroll
    for (int k = 0; k < MAXI; ++k) {
        const int it = threadIdx.x + k * kAttnThreads;
        if (it < n * CH) {
            reinterpret_cast<u32x4_t *>(dst + (it / CH) * D)[it % CH] = v[k];
            const int t = t0 + it / CH;
            if (t == new_t)
                reinterpret_cast<u32x4_t *>(ring + static_cast<size_t>(t % R) * D)[it % CH] = v[k];
        }
    }
}

// q of the g heads of stream (b, kvh), prescaled, into LDS [g][D].
__device__ __forceinline__ void stage_q(const AttnArgs &a, int b, int kvh, float *q_l)
{
    constexpr int MAXQ = kMaxG * 256 / kAttnThreads;  // elements per thread at most
    const int n = a.g * a.D;
    const size_t base = (static_cast<size_t>(b) * a.Hkv * a.g + kvh * a.g) * a.D;
    float v[MAXQ];
#pragma unroll
    for (int k = 0; k < MAXQ; ++k) {
        const int i = threadIdx.x + k * kAttnThreads;
        if (i < n)
            v[k] = load_q(a.q, a.q_dtype, base + i);
    }
#pragma unroll
    for (int k = 0; k < MAXQ; ++k) {
        const int i = threadIdx.x + k * kAttnThreads;
        if (i < n)
            q_l[i] = v[k] * a.scale_log2;
    }
}

// Vector-ALU attention of one workgroup (256 threads) over tokens [t_beg, t_end)
// of stream bh; writes partial entry `slot` for each of the g heads.  Tiles of
// TT tokens, each all quantized or all recent, are staged in LDS with 16-byte
// loads.  Scores: P = 256 / TT threads per token, 32 channels each, reduced by
// lane shuffles.  P.V: one thread per (channel, head slot), the value scale
// folded into the weight, sum_t p_t (c_t s_t + z_t) = sum_t (p_t s_t) c_t +
// sum_t p_t z_t.
template <int D, int GM>
__device__ void valu_range(const AttnArgs &a, const RaggedTables *rt, int bh, int t_beg, int t_end, int slot,
                           float *smem, int h0)
{
    constexpr int TT = valu_tile<D>();
    constexpr int P = kAttnThreads / TT;  // threads per token in the score phase
    constexpr int CPT = D / P;            // channels per thread (32)
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = a.g;
    float *q_lds = smem;                         // [g][D]
    float *p_lds = smem + g * D;                 // [g][TT]
    float *red_lds = p_lds + g * TT;             // [4][4][kMaxG]
    uint32_t *k_tile = reinterpret_cast<uint32_t *>(red_lds + 4 * 4 * kMaxG);  // 16 KB
    uint32_t *v_tile = k_tile + 4096;                                           // 16 KB
#define q_l(h, c) q_lds[(h) * D + (c)]
#define p_l(h, i) p_lds[(h) * TT + (i)]
#define red(k, w, h) red_lds[((k) * 4 + (w)) * kMaxG + (h)]
    const int b = bh / a.Hkv, kvh = bh % a.Hkv;
    const LayerDev &L = a.L;
    const int bf = a.kv_bf16;
    const StreamDims sd = stream_dims(a, rt, bh);

    stage_q(a, b, kvh, q_lds);

    const int oc = tid % D, oh0 = tid / D, hstep = kAttnThreads / D;
    float o[GM], m[GM], l[GM];
#pragma unroll
    for (int k = 0; k < GM; ++k) {
        o[k] = 0.0f;
        m[k] = -INFINITY;
        l[k] = 0.0f;
    }

    const QAddr qa(L, bh);  // rows of the stream's tokens (through the page table when paged)
    for (int tile = t_beg; tile < t_end;) {
        const bool quant = tile < sd.Tq;
        const int tend = min(min(tile + TT, t_end), quant ? sd.Tq : t_end);
        const int nt = tend - tile;
        __syncthreads();  // previous tile's LDS reads are done (and q is staged)
        if (quant) {
            // a tile never crosses a page: tiles start at multiples of its
            // length, which divides the page length
            const size_t r0 = qa.row(tile);
            stage_words<4>(k_tile, L.k_words + r0 * L.wk, nt * L.wk);
            stage_words<4>(v_tile, L.v_words + r0 * L.wv, nt * L.wv);
        } else {
            stage_ring<D, 4>(reinterpret_cast<uint16_t *>(k_tile), L.ring_k + static_cast<size_t>(bh) * L.R * D,
                             L.R, tile, nt, a.new_k + static_cast<size_t>(bh) * D, sd.new_t);
            stage_ring<D, 4>(reinterpret_cast<uint16_t *>(v_tile), L.ring_v + static_cast<size_t>(bh) * L.R * D,
                             L.R, tile, nt, a.new_v + static_cast<size_t>(bh) * D, sd.new_t);
        }
        // per-thread metadata while the tile lands
        const int ti = tid / P, part = tid % P, c0 = part * CPT;
        const int t = tile + ti;
        const bool valid = ti < nt;
        float ks[CPT], kz[CPT];
        float vs = 1.0f, vz = 0.0f;
        if (quant && valid && L.k_tok) {
            // per-token Key: one scale and zero for the whole row
            const float2 k2 = *reinterpret_cast<const float2 *>(L.k_meta + qa.row(t) * 2);
#pragma unroll
            for (int i = 0; i < CPT; ++i) {
                ks[i] = k2.x;
                kz[i] = k2.y;
            }
        } else if (quant && valid) {
            const float *km = L.k_meta + qa.grp(t / L.G) * 2 * D + c0;
#pragma unroll
            for (int i = 0; i < CPT; i += 4) {
                const float4 s4 = *reinterpret_cast<const float4 *>(km + i);
                const float4 z4 = *reinterpret_cast<const float4 *>(km + D + i);
                ks[i] = s4.x; ks[i + 1] = s4.y; ks[i + 2] = s4.z; ks[i + 3] = s4.w;
                kz[i] = z4.x; kz[i + 1] = z4.y; kz[i + 2] = z4.z; kz[i + 3] = z4.w;
            }
        }
        if (quant && valid) {
            const float2 vm = *reinterpret_cast<const float2 *>(L.v_meta + qa.row(t) * 2);
            vs = vm.x;
            vz = vm.y;
        }
        __syncthreads();

        // ---- scores: this thread's 32 channels of token ti ----
        float sc[GM];
#pragma unroll
        for (int h = 0; h < GM; ++h)
            sc[h] = 0.0f;
        if (valid) {
            if (quant) {
                const uint32_t *row = k_tile + ti * L.wk;
#pragma unroll 8
                for (int i = 0; i < CPT; ++i) {
                    const int c = c0 + i;
                    const float x = __builtin_fmaf(static_cast<float>(row_code(row, L.kb, c)), ks[i], kz[i]);
#pragma unroll
                    for (int h = 0; h < GM; ++h)
                        if (h0 + h < g)
                            sc[h] = __builtin_fmaf(q_l(h0 + h, c), x, sc[h]);
                }
            } else {
                const uint16_t *row = reinterpret_cast<const uint16_t *>(k_tile) + ti * D + c0;
#pragma unroll 8
                for (int i = 0; i < CPT; ++i) {
                    const float x = widen16(row[i], bf);
#pragma unroll
                    for (int h = 0; h < GM; ++h)
                        if (h0 + h < g)
                            sc[h] = __builtin_fmaf(q_l(h0 + h, c0 + i), x, sc[h]);
                }
            }
        }
#pragma unroll
        for (int h = 0; h < GM; ++h)
            for (int off = 1; off < P; off <<= 1)
                sc[h] += __shfl_xor(sc[h], off, 64);

        // ---- tile maximum, weights, normalizer and z-term per head ----
#pragma unroll
        for (int h = 0; h < GM; ++h) {
            if (h0 + h < g) {
                const float w = wave_max(valid ? sc[h] : -INFINITY);
                if (lane == 0)
                    red(0, wave, h) = w;
            }
        }
        __syncthreads();
        float alpha[GM];
#pragma unroll
        for (int h = 0; h < GM; ++h) {
            if (h0 + h < g) {
                const float tm = fmaxf(fmaxf(red(0, 0, h), red(0, 1, h)), fmaxf(red(0, 2, h), red(0, 3, h)));
                const float mnew = fmaxf(m[h], tm);
                alpha[h] = exp2f(m[h] - mnew);
                if (tid == 0)
                    red(3, 0, h) = alpha[h];
                // one thread per token contributes to the sums
                const float p = (valid && part == 0) ? exp2f(sc[h] - mnew) : 0.0f;
                if (valid && part == 0)
                    p_l(h, ti) = p * vs;
                const float ps = wave_sum(p), pz = wave_sum(p * vz);
                if (lane == 0) {
                    red(1, wave, h) = ps;
                    red(2, wave, h) = pz;
                }
                m[h] = mnew;
            }
        }
        __syncthreads();
#pragma unroll
        for (int h = 0; h < GM; ++h)
            if (h0 + h < g)
                l[h] = l[h] * alpha[h] + (red(1, 0, h) + red(1, 1, h) + red(1, 2, h) + red(1, 3, h));
#pragma unroll
        for (int k = 0; k < GM; ++k) {
            const int h = oh0 + k * hstep;
            if (h < GM && h0 + h < g)
                o[k] = o[k] * red(3, 0, h) + (red(2, 0, h) + red(2, 1, h) + red(2, 2, h) + red(2, 3, h));
        }

        // ---- P.V from the staged V tile ----
        if (quant) {
            for (int i = 0; i < nt; ++i) {
                uint32_t code;
                if (L.v_tiled) {
                    int word, bit;
                    v_tile_pos(i & 31, oc, L.vb, D, &word, &bit);
                    code = (v_tile[(i & ~31) * L.wv + word] >> bit) & ((1u << L.vb) - 1u);
                } else {
                    code = row_code(v_tile + i * L.wv, L.vb, oc);
                }
                const float x = static_cast<float>(code);
#pragma unroll
                for (int k = 0; k < GM; ++k) {
                    const int h = oh0 + k * hstep;
                    if (h < GM && h0 + h < g)
                        o[k] = __builtin_fmaf(p_l(h, i), x, o[k]);
                }
            }
        } else {
            const uint16_t *vt = reinterpret_cast<const uint16_t *>(v_tile);
            for (int i = 0; i < nt; ++i) {
                const float x = widen16(vt[i * D + oc], bf);
#pragma unroll
                for (int k = 0; k < GM; ++k) {
                    const int h = oh0 + k * hstep;
                    if (h < GM && h0 + h < g)
                        o[k] = __builtin_fmaf(p_l(h, i), x, o[k]);
                }
            }
        }
        tile = tend;
    }

    const int ps = part_stride(D);
    float *part = a.part + (static_cast<size_t>(bh) * a.n_part + slot) * part_entry_floats(g, D);
#pragma unroll
    for (int k = 0; k < GM; ++k) {
        const int h = oh0 + k * hstep;
        if (h < GM && h0 + h < g) {
            part_store(part + (h0 + h) * ps + oc, o[k]);
            if (oc == 0) {
                part_store(part + (h0 + h) * ps + D, m[h]);
                part_store(part + (h0 + h) * ps + D + 1, l[h]);
            }
        }
    }
#undef q_l
#undef p_l
#undef red
}

// Workgroup-level merge: the waves of one workgroup have left their per-head
// results in LDS (o[g][D] at wave * region floats, m and l in pm / pl; m =
// -inf marks an empty one); the workgroup writes one partial entry per head,
// o = sum_w 2^(m_w - M) o_w, l = sum_w 2^(m_w - M) l_w, M = max_w m_w.
template <int D>
__device__ __forceinline__ void wg_merge_store(const AttnArgs &a, int bh, int entry, const float *lds,
                                               int region, const float (*pm)[kMaxG], const float (*pl)[kMaxG])
{
    constexpr int nc4 = D / 4;
    const PartBuf pb(a, bh);
    for (int it = threadIdx.x; it < a.g * nc4; it += kAttnThreads) {
        const int h = it / nc4, c4 = it % nc4;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < kAttnThreads / 64; ++w)
            M = fmaxf(M, pm[w][h]);
        f4_t o = {0.0f, 0.0f, 0.0f, 0.0f};
        float l = 0.0f;
        if (M != -INFINITY) {
#pragma unroll
            for (int w = 0; w < kAttnThreads / 64; ++w) {
                if (pm[w][h] == -INFINITY)
                    continue;
                const float f = exp2f(pm[w][h] - M);
                const f4_t v = *reinterpret_cast<const f4_t *>(lds + w * region + h * D + 4 * c4);
                o += f * v;
                l = __builtin_fmaf(f, pl[w][h], l);
            }
        }
        pb.store4(pb.off(a, entry, h, 4 * c4), o);
        if (c4 == 0)
            pb.store4(pb.off(a, entry, h, D), f4_t{M, l, 0.0f, 0.0f});
    }
}

// Merge of the n_part partial entries of stream bh by its last workgroup:
// out = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s, M = max_s m_s.
// Thread t owns four channels of one head (item tid_item) and the entries
// tid_sub, tid_sub + n_sub, ...  It issues the (m, l) and o loads of up to KC
// of its entries together (one memory round trip), merges them online, and
// the n_sub partial states of an item are merged through LDS (s_m, s_d,
// s_acc).  KC is instantiated to the entries a thread actually has, so that
// no masked-off entry slots are executed.
template <int D, int KC>
__device__ __forceinline__ void merge_stream(const AttnArgs &a, int bh, int n_sub, int tid_item, int tid_sub,
                                             float *s_m, float *s_d, f4_t *s_acc, bool xcd_local)
{
    const int tid = threadIdx.x;
    constexpr int nc4 = D / 4;
    const int g = a.g, P = a.n_part;
    const int n_items = g * nc4;  // <= 1024
    const PartBuf pb(a, bh);
    for (int it0 = 0; it0 < n_items; it0 += kAttnThreads) {
        const int item = it0 + tid_item;
        const int sub = tid_sub;
        const bool own = item < n_items && sub < n_sub;
        const int h = own ? item / nc4 : 0, c4 = own ? item % nc4 : 0;
        float M = -INFINITY, den = 0.0f;
        f4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
        for (int e0 = sub; e0 < P; e0 += KC * n_sub) {
            f4_t ml[KC], ov[KC];
#pragma unroll
            for (int k = 0; k < KC; ++k) {
                const int e = e0 + k * n_sub;
                if (own && e < P) {
                    ml[k] = xcd_local ? pb.load4_xcd(pb.off(a, e, h, D)) : pb.load4(pb.off(a, e, h, D));
                    ov[k] = xcd_local ? pb.load4_xcd(pb.off(a, e, h, 4 * c4)) : pb.load4(pb.off(a, e, h, 4 * c4));
                }
            }
            float Mc = M;
#pragma unroll
            for (int k = 0; k < KC; ++k)
                if (own && e0 + k * n_sub < P)
                    Mc = fmaxf(Mc, ml[k][0]);
            if (Mc == -INFINITY)
                continue;
            const float r = (M == -INFINITY) ? 0.0f : exp2f(M - Mc);
            acc *= r;
            den *= r;
            M = Mc;
#pragma unroll
            for (int k = 0; k < KC; ++k) {
                if (own && e0 + k * n_sub < P && ml[k][0] != -INFINITY) {
                    const float w = exp2f(ml[k][0] - M);
                    acc += w * ov[k];
                    den = __builtin_fmaf(w, ml[k][1], den);
                }
            }
        }
        if (n_sub > 1) {
            // merge the n_sub states of each item (entry sets of its threads)
            s_m[tid] = M;
            s_d[tid] = den;
            s_acc[tid] = acc;
            __syncthreads();
            if (own && sub == 0) {
                float Mt = M;
                for (int j = 1; j < n_sub; ++j)
                    Mt = fmaxf(Mt, s_m[tid + j * n_items]);
                const float r0 = (M == -INFINITY) ? 0.0f : exp2f(M - Mt);
                acc *= r0;
                den *= r0;
                for (int j = 1; j < n_sub; ++j) {
                    const float mj = s_m[tid + j * n_items];
                    if (mj == -INFINITY)
                        continue;
                    const float rj = exp2f(mj - Mt);
                    acc += rj * s_acc[tid + j * n_items];
                    den = __builtin_fmaf(rj, s_d[tid + j * n_items], den);
                }
            }
        }
        if (own && sub == 0)
            *reinterpret_cast<f4_t *>(a.out + (static_cast<size_t>(bh) * g + h) * D + 4 * c4) =
                acc * (1.0f / den);
    }
}

// XCD (accelerator complex die) this wave runs on.
__device__ __forceinline__ unsigned xcd_id()
{
    unsigned r;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(r));
    return r & 7u;
}

// Called by every workgroup at its end: the last one of stream bh to arrive
// merges the n_part partial entries (merge_stream) and re-arms the stream's
// counter.  With by_xcd (at most 15 workgroups per stream), each workgroup
// adds 1 to the 4-bit field of its XCD instead of 1: the last one then also
// knows whether every workgroup of the stream ran on its own XCD, and if so
// reads their partials through that XCD's L2.
template <int D>
__device__ __forceinline__ void arrive_and_merge(const AttnArgs &a, int bh, unsigned n_wgs, bool by_xcd = false)
{
    __shared__ int s_last;
    __shared__ float s_m[kAttnThreads], s_d[kAttnThreads];
    __shared__ f4_t s_acc[kAttnThreads];
    __builtin_amdgcn_s_waitcnt(0);  // this thread's partial stores are complete
    __syncthreads();
    if (threadIdx.x == 0) {
        if (by_xcd) {
            const unsigned x = xcd_id();
            const unsigned inc = 1u << (4 * x);
            const unsigned v =
                __hip_atomic_fetch_add(a.counters + bh * kCounterStride, inc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + inc;
            unsigned total = 0;
#pragma unroll
            for (int j = 0; j < 8; ++j)
                total += (v >> (4 * j)) & 15u;
            s_last = total == n_wgs ? (((v >> (4 * x)) & 15u) == n_wgs ? 2 : 1) : 0;
        } else {
            const unsigned prev =
                __hip_atomic_fetch_add(a.counters + bh * kCounterStride, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            s_last = (prev == n_wgs - 1);
        }
    }
    __syncthreads();
    if (!s_last)
        return;
    const bool xcd_local = s_last == 2;
    const int tid = threadIdx.x;
    const int n_items = a.g * (D / 4);  // <= 1024
    // n_sub = kAttnThreads / n_items threads per item (when items are fewer
    // than threads); thread tid = sub * n_items + item, found by subtraction
    int n_sub = 1, tid_item = tid, tid_sub = 0;
    if (n_items < kAttnThreads) {
        while ((n_sub + 1) * n_items <= kAttnThreads)
            ++n_sub;
        while (tid_item >= n_items) {
            tid_item -= n_items;
            ++tid_sub;
        }
    }
    const int P = a.n_part;  // entries per thread: ceil(P / n_sub)
    if (P <= 2 * n_sub)
        merge_stream<D, 2>(a, bh, n_sub, tid_item, tid_sub, s_m, s_d, s_acc, xcd_local);
    else if (P <= 4 * n_sub)
        merge_stream<D, 4>(a, bh, n_sub, tid_item, tid_sub, s_m, s_d, s_acc, xcd_local);
    else if (P <= 8 * n_sub)
        merge_stream<D, 8>(a, bh, n_sub, tid_item, tid_sub, s_m, s_d, s_acc, xcd_local);
    else
        merge_stream<D, 16>(a, bh, n_sub, tid_item, tid_sub, s_m, s_d, s_acc, xcd_local);
    if (tid == 0)
        __hip_atomic_store(a.counters + bh * kCounterStride, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace kvq
