// kvq_attn_prefill.hip -- matrix-core causal attention of a prefill chunk over
// the quantized cache, for one head_dim (KVQ_D, set by the build).
//
// The queries of the last n_q appended tokens attend to the cache as it is
// stored: query j, at position p = N - n_q + j, sees tokens 0..p (KVTuner
// summary, A3 attention equation: the query of step i attends to the keys of
// steps up to i), quantized tokens dequantized on the fly and recent tokens in
// 16 bits (KVTuner summary, A2: calibration runs prefill attention on the
// dequantized cache).
//
// One wave computes a tile of 16 / g queries of one (sequence, kv-head)
// stream: the 16 columns of each 16x16x32 product are (query, head) pairs,
// column jq * g + h carrying query head h of query jq.  Unlike decode, every
// column uses the same K group, so the products are dense: the B operand of
// q.K is (q_col * s_c) for the group's per-channel scales s (KVmix notes, key
// design 4: scale folded into the product, codes as exact fp16 integers), the
// z term sum_c q_c z_c stays in fp32, and P.V takes the weights p_t s_t of
// every column against the V code fragments (z term sum_t p_t z_t in fp32).
// Causality is a per-column mask on the scores.  The wave walks the stream's
// tokens once, quantized blocks first, then the recent 16-bit tokens, with one
// online softmax per column; no split and no merge.
#include "kvq_mfma_ops.h"

#ifndef KVQ_D
#error "KVQ_D (head_dim) must be defined"
#endif

#define KVQ_CAT2(x, y) x##y
#define KVQ_CAT(x, y) KVQ_CAT2(x, y)

namespace kvq {
namespace {

// Per-wave state of one tile: the column's online softmax (log2 domain) and
// its output accumulators.
template <int MT>
struct ColState {
    float m_run = -INFINITY, l_run = 0.0f;
    f4_t O[MT];
};

// Recent 16-bit tokens [t_beg, t_end) of stream bh for the tile's columns
// (fp16 or bfloat16 operands, as in decode); V rows staged transposed in the
// wave's LDS tile vt ([D][32]).  O is in units of 2^kWShift on entry and exit.
template <int D, bool BF>
__device__ __forceinline__ void prefill_recent(const PrefillArgs &a, int bh, size_t qrow, bool act, int p_col,
                                               int t_beg, int t_end, int lane, uint16_t *vt,
                                               ColState<D / 16> &st)
{
    constexpr int NC = D / 32;
    constexpr int MT = D / 16;
    const LayerDev &L = a.L;
    const int col = lane & 15, q = lane >> 4;
    const uint16_t *rk = L.ring_k + static_cast<size_t>(bh) * L.R * D;
    const uint16_t *rv = L.ring_v + static_cast<size_t>(bh) * L.R * D;

    // B operand of q.K: this column's q, chunk k, quad q -> channels 32k + 8q + i
    Frag b1[NC], b2[NC], b3[NC];
    int sh;
    {
        float qv[NC][8];
        float amax = 0.0f;
        load_q_runs<NC>(a.q, a.q_dtype, qrow + 8 * q, 32, qv);
#pragma unroll
        for (int k = 0; k < NC; ++k)
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                qv[k][i] = act ? qv[k][i] * a.scale_log2 : 0.0f;
                amax = fmaxf(amax, fabsf(qv[k][i]));
            }
        amax = col_max(amax);
        const int qexp = amax > 0.0f ? __builtin_amdgcn_frexp_expf(amax) : 0;
        sh = BF ? 0 : 14 - qexp;
#pragma unroll
        for (int k = 0; k < NC; ++k)
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const float x0 = ldexpf(qv[k][2 * p], sh), x1 = ldexpf(qv[k][2 * p + 1], sh);
                if constexpr (BF)
                    split3_bf16(x0, x1, b1[k].u[p], b2[k].u[p], b3[k].u[p]);
                else
                    split_pair(x0, x1, b1[k].u[p], b2[k].u[p]);
            }
    }
    const float kscale = ldexpf(1.0f, -sh);

    for (int t0 = t_beg; t0 < t_end; t0 += 32) {
        const int ta = min(t0 + col, t_end - 1), tb = min(t0 + 16 + col, t_end - 1);
        uint4 ka[NC], kb2[NC];
        const uint16_t *ra = rk + static_cast<size_t>(ta % L.R) * D;
        const uint16_t *rb = rk + static_cast<size_t>(tb % L.R) * D;
#pragma unroll
        for (int k = 0; k < NC; ++k) {
            ka[k] = *reinterpret_cast<const uint4 *>(ra + 32 * k + 8 * q);
            kb2[k] = *reinterpret_cast<const uint4 *>(rb + 32 * k + 8 * q);
        }
        // V rows -> LDS [channel][token]: lane handles token (lane & 31), half a row
        {
            const int tt = lane & 31, half = lane >> 5;
            const int tv = min(t0 + tt, t_end - 1);
            const uint4 *src = reinterpret_cast<const uint4 *>(rv + static_cast<size_t>(tv % L.R) * D + half * (D / 2));
            uint4 v[D / 16];
#pragma unroll
            for (int i = 0; i < D / 16; ++i)
                v[i] = src[i];
#pragma unroll
            for (int i = 0; i < D / 16; ++i) {
                const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int c = half * (D / 2) + 8 * i + e;
                    vt[c * 32 + tt] = static_cast<uint16_t>((e & 1) ? (w[e >> 1] >> 16) : (w[e >> 1] & 0xFFFFu));
                }
            }
        }
        f4_t acc0 = {0.0f, 0.0f, 0.0f, 0.0f}, acc1 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int k = 0; k < NC; ++k) {
            Frag a0, a1;
            a0.u[0] = ka[k].x; a0.u[1] = ka[k].y; a0.u[2] = ka[k].z; a0.u[3] = ka[k].w;
            a1.u[0] = kb2[k].x; a1.u[1] = kb2[k].y; a1.u[2] = kb2[k].z; a1.u[3] = kb2[k].w;
            if constexpr (BF) {
                acc0 = mfma_bf16(a0, b1[k], acc0);
                acc0 = mfma_bf16(a0, b2[k], acc0);
                acc0 = mfma_bf16(a0, b3[k], acc0);
                acc1 = mfma_bf16(a1, b1[k], acc1);
                acc1 = mfma_bf16(a1, b2[k], acc1);
                acc1 = mfma_bf16(a1, b3[k], acc1);
            } else {
                acc0 = mfma(a0, b1[k], acc0);
                acc0 = mfma(a0, b2[k], acc0);
                acc1 = mfma(a1, b1[k], acc1);
                acc1 = mfma(a1, b2[k], acc1);
            }
        }
        // scores of tokens 4q + j and 16 + 4q + j; causal mask t <= p_col
        float sc[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int t1 = t0 + 4 * q + j, t2 = t0 + 16 + 4 * q + j;
            sc[j] = (t1 < t_end && t1 <= p_col) ? acc0[j] * kscale : -INFINITY;
            sc[4 + j] = (t2 < t_end && t2 <= p_col) ? acc1[j] * kscale : -INFINITY;
        }
        float tmax = fmaxf(fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])),
                           fmaxf(fmaxf(sc[4], sc[5]), fmaxf(sc[6], sc[7])));
        tmax = col_max(tmax);
        const bool need = act && (tmax > st.m_run + kTau);
        if (__builtin_amdgcn_ballot_w64(need) != 0) {
            const float m_new = need ? tmax : st.m_run;
            const float alpha = (m_new == st.m_run) ? 1.0f : exp2f(st.m_run - m_new);
#pragma unroll
            for (int m = 0; m < MT; ++m)
                st.O[m] *= alpha;
            st.l_run *= alpha;
            st.m_run = m_new;
        }
        const float mo = act ? st.m_run : INFINITY;
        float p[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            p[j] = weight_exp2(sc[j] - mo);
            st.l_run += p[j];
        }
        Frag w1, w2, w3;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float x0 = ldexpf(p[2 * r], kWShift), x1 = ldexpf(p[2 * r + 1], kWShift);
            if constexpr (BF)
                split3_bf16(x0, x1, w1.u[r], w2.u[r], w3.u[r]);
            else
                split_pair(x0, x1, w1.u[r], w2.u[r]);
        }
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            const uint16_t *row = vt + (16 * m + col) * 32;
            const uint2 lo = *reinterpret_cast<const uint2 *>(row + 4 * q);
            const uint2 hi = *reinterpret_cast<const uint2 *>(row + 16 + 4 * q);
            Frag av;
            av.u[0] = lo.x; av.u[1] = lo.y; av.u[2] = hi.x; av.u[3] = hi.y;
            if constexpr (BF) {
                st.O[m] = mfma_bf16(av, w1, st.O[m]);
                st.O[m] = mfma_bf16(av, w2, st.O[m]);
                st.O[m] = mfma_bf16(av, w3, st.O[m]);
            } else {
                st.O[m] = mfma(av, w1, st.O[m]);
                st.O[m] = mfma(av, w2, st.O[m]);
            }
        }
        asm volatile("" ::: "memory");  // this block's V tile reads stay before the next block's writes
    }
}

// Workgroups of kPrefillWaves waves, all on one stream: wave w takes query
// tile wg * kPrefillWaves + w.  The quantized tokens are walked once per
// workgroup, 32 at a time: the workgroup dequantizes the block's K into LDS
// (k^ = s code + z in fp32, as fp16 hi and lo halves, token-major) and unpacks
// its V codes into each lane's P.V operand registers (exact fp16 integers, the
// V scale going into the weights), and every wave then reads them as matrix
// operands for its own tile.  The block's dequantization is paid once per
// workgroup instead of once per tile, and q.K needs no per-group rebuild of its
// q operand (the scales are on the K side).
constexpr int kPrefillWaves = 8;
constexpr int kPrefillThreads = 64 * kPrefillWaves;
// Query tiles per wave (each LDS operand read feeds all of them): two up to
// head_dim 128 (one beyond: registers), or one when two would leave compute
// units without a workgroup; each count is its own instantiation, so that the
// tiles' independent products interleave in straight-line code.

// A block's bytes as stored (K codes, V codes, V scales and zeros, K scales
// and zeros: the group's [2][D] floats, or per-token Key [32][2]), in the order
// they are staged in LDS.  Every segment is a whole number of 16-byte pieces.
template <int KB, int VB, int D, bool KT>
struct PfRaw {
    static constexpr int WK = KB == 3 ? 4 * ((D + 43) / 44) : D * KB / 32;  // K words per row
    static constexpr int K_BYTES = 32 * WK * 4;
    static constexpr int V_BYTES = 32 * (D * VB / 32) * 4;
    static constexpr int VM_OFF = K_BYTES + V_BYTES;
    static constexpr int KM_OFF = VM_OFF + 32 * 8;
    static constexpr int KM_BYTES = KT ? 32 * 8 : 2 * D * 4;
    static constexpr int BYTES = KM_OFF + KM_BYTES;
    static constexpr int PIECES = BYTES / 16;
    static constexpr int NP = (PIECES + kPrefillThreads - 1) / kPrefillThreads;  // pieces per thread
    static constexpr int SLOT = NP * kPrefillThreads * 16;                        // bytes of a ring slot
};

template <int KB, int VB, int D, bool KT>
struct PfLds {
    static constexpr int KROW = D + 8;                 // halves per K row (padding: no bank conflicts)
    static constexpr int KPLANE = 32 * KROW;           // halves per plane (hi, then lo)
    static constexpr int MT = D / 16;
    static constexpr int VROW = 4 * MT + 4;            // u32 per lane of V operand registers (padded)
    static constexpr int K_BYTES = 2 * KPLANE * 2;
    static constexpr int BUF_BYTES = K_BYTES + 64 * VROW * 4;
    static constexpr int RAW_OFF = 2 * BUF_BYTES;      // three ring slots of stored block bytes follow
    static constexpr int QUANT_BYTES = RAW_OFF + 3 * PfRaw<KB, VB, D, KT>::SLOT;
    static constexpr int RECENT_BYTES = kPrefillWaves * D * 32 * 2;  // per-wave V tiles of the recent phase
    static constexpr int BYTES = QUANT_BYTES > RECENT_BYTES ? QUANT_BYTES : RECENT_BYTES;
};

template <int KB, int VB, int D, bool KT, bool PG, int TW>
__device__ __forceinline__ void prefill_wg(const PrefillArgs &a, int bh, int wg_in, int wave, int lane, char *lds)
{
    constexpr int KW = D * KB / 128;  // (unused for the K side here: rows are read per item)
    (void)KW;
    constexpr int NC = D / 32;        // 32-channel chunks of q.K
    constexpr int MT = D / 16;        // 16-channel tiles of P.V
    constexpr int FW = D * VB / 64;   // V words per fragment (lane) of a block
    constexpr int P = 16 / VB;        // V operand registers per word
    using Lay = PfLds<KB, VB, D, KT>;
    using Raw = PfRaw<KB, VB, D, KT>;
    constexpr int TILES = kPrefillWaves * TW;  // tiles per workgroup

    const LayerDev &L = a.L;
    const int g = a.g, G = L.G;
    const int tid = threadIdx.x;
    const int col = lane & 15, q = lane >> 4;
    const int jq = col / g, h = col - jq * g;
    const int sb = a.ragged ? bh / a.Hkv : 0;
    const int N = a.ragged ? a.seqN[sb] : a.N;
    const int Tq = a.ragged ? a.seqTq[sb] : a.Tq;
    // the wave's tiles: wg_in * TILES + wave * TW + i
    int tile[TW], p_col[TW], p_first[TW];
    bool act[TW];
    size_t qrow[TW];
#pragma unroll
    for (int i = 0; i < TW; ++i) {
        tile[i] = wg_in * TILES + wave * TW + i;
        const int qi = tile[i] * a.QT + jq;
        act[i] = tile[i] < a.n_tiles && jq < a.QT && qi < a.n_q;
        p_col[i] = act[i] ? N - a.n_q + qi : -1;  // last token this column sees
        qrow[i] = (static_cast<size_t>(bh * g + (act[i] ? h : 0)) * a.n_q + (act[i] ? qi : 0)) * D;
        // first token any column of the tile sees: blocks past it need the mask
        p_first[i] = N - a.n_q + min(a.n_q - 1, tile[i] * a.QT);
    }
    // the workgroup's tokens [0, t_end): those of its last query (uniform)
    const int qi_last = min(a.n_q - 1, (wg_in + 1) * TILES * a.QT - 1);
    const int t_end = N - a.n_q + qi_last + 1;
    const int tq_end = min(Tq, (t_end + 31) & ~31);  // quantized blocks to visit (Tq: whole blocks)

    ColState<MT> st[TW];
#pragma unroll
    for (int i = 0; i < TW; ++i)
#pragma unroll
        for (int m = 0; m < MT; ++m)
            st[i].O[m] = f4_t{0.0f, 0.0f, 0.0f, 0.0f};

    if (tq_end > 0) {
        const QAddr qa(L, bh);
        WavePages wp;
        const int nb = tq_end / 32;

        // B operand of q.K: this column's q (times log2(e) / sqrt(D) and 2^sh),
        // chunk k, quad q -> channels 32k + 8q + i, as hi/lo fp16
        Frag bhi[TW][NC], blo[TW][NC];
        float kscale[TW];
#pragma unroll
        for (int t = 0; t < TW; ++t) {
            float qv[NC][8];
            float amax = 0.0f;
            load_q_runs<NC>(a.q, a.q_dtype, qrow[t] + 8 * q, 32, qv);
#pragma unroll
            for (int k = 0; k < NC; ++k)
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    qv[k][i] = act[t] ? qv[k][i] * a.scale_log2 : 0.0f;
                    amax = fmaxf(amax, fabsf(qv[k][i]));
                }
            amax = col_max(amax);
            const int sh = amax > 0.0f ? 14 - __builtin_amdgcn_frexp_expf(amax) : 0;
#pragma unroll
            for (int k = 0; k < NC; ++k)
#pragma unroll
                for (int p = 0; p < 4; ++p)
                    split_pair(ldexpf(qv[k][2 * p], sh), ldexpf(qv[k][2 * p + 1], sh), bhi[t][k].u[p],
                               blo[t][k].u[p]);
            kscale[t] = ldexpf(1.0f, -sh);
        }

        // first row of the block of token t0 (same in every lane)
        auto block_row = [&](int t0) -> size_t {
            if constexpr (PG) {
                if (!wp.covers(qa, t0, t0 + 32))
                    wp.load(qa, lane, t0, tq_end);
                return wp.row_u(qa, t0);
            } else {
                return qa.base + t0;
            }
        };
        // this thread's 16-byte pieces of a block's stored bytes: segment
        // (0 K codes, 1 V codes, 2 V meta, 3 K meta) and offset in it, fixed for
        // the walk.  Pieces past the block's bytes re-read its last piece, so
        // that every thread issues the same loads in every step.
        int pseg[Raw::NP], poff[Raw::NP];
#pragma unroll
        for (int ip = 0; ip < Raw::NP; ++ip) {
            const int o = min(16 * (tid + kPrefillThreads * ip), Raw::BYTES - 16);
            pseg[ip] = o < Raw::K_BYTES ? 0 : o < Raw::VM_OFF ? 1 : o < Raw::KM_OFF ? 2 : 3;
            poff[ip] = o - (o < Raw::K_BYTES ? 0 : o < Raw::VM_OFF ? Raw::K_BYTES : o < Raw::KM_OFF ? Raw::VM_OFF
                                                                                                   : Raw::KM_OFF);
        }
        // block t0's pieces, into registers
        auto issue = [&](u32x4_t (&r)[Raw::NP], int t0) {
            const size_t r0 = block_row(t0);
            const char *ksrc = reinterpret_cast<const char *>(L.k_words + r0 * L.wk);
            const char *vsrc = reinterpret_cast<const char *>(L.v_words + r0 * L.wv);
            const char *vmsrc = reinterpret_cast<const char *>(L.v_meta + r0 * 2);
            const char *kmsrc;
            if constexpr (KT) {
                kmsrc = reinterpret_cast<const char *>(L.k_meta + r0 * 2);
            } else {
                const int gi = t0 / G;
                size_t gr;
                if constexpr (PG)
                    gr = qa.page_grp(__builtin_amdgcn_readlane(wp.id, (t0 >> qa.P_log2) - wp.first), gi);
                else
                    gr = qa.gbase + gi;
                kmsrc = reinterpret_cast<const char *>(L.k_meta + gr * 2 * D);
            }
#pragma unroll
            for (int ip = 0; ip < Raw::NP; ++ip) {
                const char *base = pseg[ip] == 0 ? ksrc : pseg[ip] == 1 ? vsrc : pseg[ip] == 2 ? vmsrc : kmsrc;
                r[ip] = *reinterpret_cast<const u32x4_t *>(base + poff[ip]);
            }
        };
        // ring slot of block b's stored bytes
        auto raw_slot = [&](int b) { return lds + Lay::RAW_OFF + (b % 3) * Raw::SLOT; };
        // (every thread stores all its pieces: the slot has room for them, and
        // the pieces past the block's bytes land in its unused tail)
        auto stage = [&](const u32x4_t (&r)[Raw::NP], int b) {
            char *dst = raw_slot(b);
#pragma unroll
            for (int ip = 0; ip < Raw::NP; ++ip)
                *reinterpret_cast<u32x4_t *>(dst + 16 * (tid + kPrefillThreads * ip)) = r[ip];
        };
        // the dequantized block in LDS buffer buf
        auto kplane = [&](int buf) { return reinterpret_cast<_Float16 *>(lds + buf * Lay::BUF_BYTES); };
        auto vregs = [&](int buf) {
            return reinterpret_cast<uint32_t *>(lds + buf * Lay::BUF_BYTES + Lay::K_BYTES);
        };
        // this thread's share of block b's dequantization, from its ring slot
        // into buffer b & 1
        auto dequant = [&](int b) {
            const char *raw = raw_slot(b);
            const int buf = b & 1;
            _Float16 *khi = kplane(buf), *klo = khi + Lay::KPLANE;
            const float *km = reinterpret_cast<const float *>(raw + Raw::KM_OFF);
            constexpr int ITEMS = KB == 3 ? 32 * 12 : 32 * D / 8;
            constexpr int NI = (ITEMS + kPrefillThreads - 1) / kPrefillThreads;
#pragma unroll
            for (int ii = 0; ii < NI; ++ii) {
                const int i = tid + kPrefillThreads * ii;
                if (i < ITEMS) {
                    if constexpr (KB == 3) {
                        // one word: channels 11 wi + j (j < 10: 3 bits at 3j; j = 10: 2 bits at 30)
                        const int tok = i / 12, wi = i - tok * 12, c0 = 11 * wi;
                        const uint32_t w = reinterpret_cast<const uint32_t *>(raw)[tok * Raw::WK + wi];
#pragma unroll
                        for (int j = 0; j < 11; ++j) {
                            const int c = c0 + j;
                            if (c < D) {
                                const uint32_t code = j < 10 ? (w >> (3 * j)) & 7u : w >> 30;
                                const float x = __builtin_fmaf(km[c], static_cast<float>(code), km[D + c]);
                                const _Float16 hv = static_cast<_Float16>(x);
                                khi[tok * Lay::KROW + c] = hv;
                                klo[tok * Lay::KROW + c] = static_cast<_Float16>(x - static_cast<float>(hv));
                            }
                        }
                    } else {
                        // eight channels c0 .. c0 + 7 of one token (8 KB bits)
                        const int tok = i / (D / 8), c0 = 8 * (i - tok * (D / 8));
                        const char *row = raw + tok * Raw::WK * 4;
                        uint32_t w0, w1 = 0;
                        if constexpr (KB == 2) {
                            w0 = *reinterpret_cast<const uint16_t *>(row + c0 / 4);
                        } else if constexpr (KB == 4) {
                            w0 = *reinterpret_cast<const uint32_t *>(row + c0 / 2);
                        } else {
                            const uint2 v = *reinterpret_cast<const uint2 *>(row + c0);
                            w0 = v.x;
                            w1 = v.y;
                        }
                        float sc[8], zc[8];
                        if constexpr (KT) {
                            const float2 m = reinterpret_cast<const float2 *>(km)[tok];
#pragma unroll
                            for (int j = 0; j < 8; ++j) {
                                sc[j] = m.x;
                                zc[j] = m.y;
                            }
                        } else {
                            const float4 s0 = *reinterpret_cast<const float4 *>(km + c0);
                            const float4 s1 = *reinterpret_cast<const float4 *>(km + c0 + 4);
                            const float4 z0 = *reinterpret_cast<const float4 *>(km + D + c0);
                            const float4 z1 = *reinterpret_cast<const float4 *>(km + D + c0 + 4);
                            sc[0] = s0.x; sc[1] = s0.y; sc[2] = s0.z; sc[3] = s0.w;
                            sc[4] = s1.x; sc[5] = s1.y; sc[6] = s1.z; sc[7] = s1.w;
                            zc[0] = z0.x; zc[1] = z0.y; zc[2] = z0.z; zc[3] = z0.w;
                            zc[4] = z1.x; zc[5] = z1.y; zc[6] = z1.z; zc[7] = z1.w;
                        }
                        float x[8];
#pragma unroll
                        for (int j = 0; j < 8; ++j) {
                            uint32_t code;
                            if constexpr (KB == 8)
                                code = ((j < 4 ? w0 : w1) >> (8 * (j & 3))) & 0xFFu;
                            else
                                code = (w0 >> (KB * j)) & ((1u << KB) - 1u);
                            x[j] = __builtin_fmaf(sc[j], static_cast<float>(code), zc[j]);
                        }
                        uint4 hi, lo;
                        split_pair(x[0], x[1], hi.x, lo.x);
                        split_pair(x[2], x[3], hi.y, lo.y);
                        split_pair(x[4], x[5], hi.z, lo.z);
                        split_pair(x[6], x[7], hi.w, lo.w);
                        *reinterpret_cast<uint4 *>(khi + tok * Lay::KROW + c0) = hi;
                        *reinterpret_cast<uint4 *>(klo + tok * Lay::KROW + c0) = lo;
                    }
                }
            }
            // V: word w of the block's tiled codes -> lane w / FW's operand
            // registers (w % FW) * P .. + P - 1
            uint32_t *vr = vregs(buf);
            constexpr int VWORDS = D * VB;
            constexpr int NV = (VWORDS + kPrefillThreads - 1) / kPrefillThreads;
#pragma unroll
            for (int vi = 0; vi < NV; ++vi) {
                const int w = tid + kPrefillThreads * vi;
                if (w < VWORDS) {
                    const int f = w / FW, wi = w - f * FW;
                    const uint32_t word = reinterpret_cast<const uint32_t *>(raw + Raw::K_BYTES)[w];
                    const uint32_t ww[1] = {word}, w8[1] = {word >> 8};
                    uint32_t o[P];
#pragma unroll
                    for (int j = 0; j < P; ++j)
                        o[j] = code_reg<VB>(ww, w8, j);
                    uint32_t *dst = vr + f * Lay::VROW + wi * P;
                    if constexpr (P == 8) {
                        reinterpret_cast<uint4 *>(dst)[0] = uint4{o[0], o[1], o[2], o[3]};
                        reinterpret_cast<uint4 *>(dst)[1] = uint4{o[P > 4 ? 4 : 0], o[P > 5 ? 5 : 0], o[P > 6 ? 6 : 0],
                                                                  o[P > 7 ? 7 : 0]};
                    } else if constexpr (P == 4) {
                        *reinterpret_cast<uint4 *>(dst) = uint4{o[0], o[1], o[2], o[3]};
                    } else {
                        *reinterpret_cast<uint2 *>(dst) = uint2{o[0], o[1]};
                    }
                }
            }
        };

        float zb_run[TW];
        int E[TW];  // running V-scale exponent: the weights carry 2^(kWShift - E)
#pragma unroll
        for (int t = 0; t < TW; ++t) {
            zb_run[t] = 0.0f;
            E[t] = -1000;
        }
        // one block of the wave's tiles from buffer buf
        auto compute = [&](int b) {
            const int t0 = 32 * b, buf = b & 1;
            const _Float16 *khi = kplane(buf), *klo = khi + Lay::KPLANE;
            f4_t acc0[TW], acc1[TW];
#pragma unroll
            for (int t = 0; t < TW; ++t) {
                acc0[t] = f4_t{0.0f, 0.0f, 0.0f, 0.0f};
                acc1[t] = f4_t{0.0f, 0.0f, 0.0f, 0.0f};
            }
#pragma unroll
            for (int k = 0; k < NC; ++k) {
                Frag ah0, al0, ah1, al1;
                const int off0 = col * Lay::KROW + 32 * k + 8 * q, off1 = off0 + 16 * Lay::KROW;
                ah0.h = *reinterpret_cast<const half8_t *>(khi + off0);
                al0.h = *reinterpret_cast<const half8_t *>(klo + off0);
                ah1.h = *reinterpret_cast<const half8_t *>(khi + off1);
                al1.h = *reinterpret_cast<const half8_t *>(klo + off1);
#pragma unroll
                for (int t = 0; t < TW; ++t) {
                    acc0[t] = mfma(ah0, bhi[t][k], acc0[t]);
                    acc1[t] = mfma(ah1, bhi[t][k], acc1[t]);
                    acc0[t] = mfma(ah0, blo[t][k], acc0[t]);
                    acc1[t] = mfma(ah1, blo[t][k], acc1[t]);
                    acc0[t] = mfma(al0, bhi[t][k], acc0[t]);
                    acc1[t] = mfma(al1, bhi[t][k], acc1[t]);
                }
            }
            const float4 *vmp = reinterpret_cast<const float4 *>(raw_slot(b) + Raw::VM_OFF);
            const float4 vm0 = vmp[2 * q], vm1 = vmp[2 * q + 1], vm2 = vmp[8 + 2 * q], vm3 = vmp[8 + 2 * q + 1];
            const float vs[8] = {vm0.x, vm0.z, vm1.x, vm1.z, vm2.x, vm2.z, vm3.x, vm3.z};
            const float vz[8] = {vm0.y, vm0.w, vm1.y, vm1.w, vm2.y, vm2.w, vm3.y, vm3.w};
            float vmax = fmaxf(fmaxf(fmaxf(vs[0], vs[1]), fmaxf(vs[2], vs[3])),
                               fmaxf(fmaxf(vs[4], vs[5]), fmaxf(vs[6], vs[7])));
            vmax = col_max(vmax);
            const int eb = vmax > 0.0f ? __builtin_amdgcn_frexp_expf(vmax) : -1000;
            // B operands of P.V: weights p s 2^(kWShift - E), k-slot pairs, each
            // divided by its code class factor
            Frag whi[TW], wlo[TW];
#pragma unroll
            for (int t = 0; t < TW; ++t) {
                float sc[8];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    sc[j] = acc0[t][j] * kscale[t];
                    sc[4 + j] = acc1[t][j] * kscale[t];
                }
                if (t0 + 31 > p_first[t]) {  // causal mask (uniform: only blocks that reach the tile's queries)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        sc[j] = (t0 + 4 * q + j <= p_col[t]) ? sc[j] : -INFINITY;
                        sc[4 + j] = (t0 + 16 + 4 * q + j <= p_col[t]) ? sc[4 + j] : -INFINITY;
                    }
                }
                float tmax = fmaxf(fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])),
                                   fmaxf(fmaxf(sc[4], sc[5]), fmaxf(sc[6], sc[7])));
                tmax = col_max(tmax);
                ColState<MT> &c = st[t];
                const bool need_m = act[t] && (tmax > c.m_run + kTau);
                const bool need_e = act[t] && (eb > E[t]);
                if (__builtin_amdgcn_ballot_w64(need_m || need_e) != 0) {
                    const float m_new = need_m ? tmax : c.m_run;
                    const int E_new = need_e ? eb : E[t];
                    const float alpha = (m_new == c.m_run) ? 1.0f : exp2f(c.m_run - m_new);
                    const float f = ldexpf(alpha, E[t] - E_new);
#pragma unroll
                    for (int m = 0; m < MT; ++m)
                        c.O[m] *= f;
                    c.l_run *= alpha;
                    zb_run[t] *= alpha;
                    c.m_run = m_new;
                    E[t] = E_new;
                }
                const float mo = act[t] ? c.m_run : INFINITY;
                float p[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    p[j] = weight_exp2(sc[j] - mo);
                    c.l_run += p[j];
                    zb_run[t] = __builtin_fmaf(p[j], vz[j], zb_run[t]);
                }
                const int wsh = kWShift - E[t];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int e = wsh - class_exp<VB>(r);
                    split_pair(ldexpf(p[2 * r] * vs[2 * r], e), ldexpf(p[2 * r + 1] * vs[2 * r + 1], e),
                               whi[t].u[r], wlo[t].u[r]);
                }
            }
            const uint32_t *vr = vregs(buf) + lane * Lay::VROW;
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                Frag av;
                const uint4 v = *reinterpret_cast<const uint4 *>(vr + 4 * m);
                av.u[0] = v.x; av.u[1] = v.y; av.u[2] = v.z; av.u[3] = v.w;
#pragma unroll
                for (int t = 0; t < TW; ++t) {
                    st[t].O[m] = mfma(av, whi[t], st[t].O[m]);
                    st[t].O[m] = mfma(av, wlo[t], st[t].O[m]);
                }
            }
        };

        // Pipeline, one workgroup barrier per block.  In step b: block b is
        // computed (dequantized LDS buffer b & 1), block b + 1 is dequantized
        // from its ring slot into the other buffer, block b + 2's stored bytes
        // (loaded into registers kRegSets steps earlier) are staged into the
        // ring, and the loads of block b + 2 + kRegSets are issued into the
        // registers that frees.  Loads past the last block re-read it (in
        // bounds).
        // register sets: four blocks in flight, two when a block takes two or
        // more pieces per thread (registers)
        constexpr int kRegSets = Raw::NP == 1 ? 4 : 2;
        // (a native vector type: the struct type's copies are memcpys, which keep
        // an array of two pieces in scratch)
        u32x4_t rs0[Raw::NP], rs1[Raw::NP], rs2[Raw::NP], rs3[Raw::NP];
        issue(rs0, 0);
        issue(rs1, 32 * min(1, nb - 1));
        if constexpr (kRegSets == 4) {
            issue(rs2, 32 * min(2, nb - 1));
            issue(rs3, 32 * min(3, nb - 1));
        }
        stage(rs0, 0);
        issue(rs0, 32 * min(kRegSets, nb - 1));
        stage(rs1, 1);  // block 1 (a re-read of block 0 when nb == 1: unused)
        issue(rs1, 32 * min(kRegSets + 1, nb - 1));
        __syncthreads();
        dequant(0);
        __syncthreads();
        // one step; block b + 2 sits in set rs ((b + 2) % kRegSets).  The
        // steps past the last block only stage re-reads into free slots: the
        // sets are loaded and consumed unconditionally, so that their loads
        // stay in flight across steps.
        // The two waves that share a SIMD (w and w + 4) take the step's two
        // halves in opposite orders, so that one's matrix products overlap the
        // other's dequantization (the halves touch different buffers).
        const bool deq_first = wave >= kPrefillWaves / 2;
        auto step = [&](int b, u32x4_t (&rs)[Raw::NP]) {
            if (deq_first && b + 1 < nb)
                dequant(b + 1);
            if (b < nb)  // uniform
                compute(b);
            if (!deq_first && b + 1 < nb)
                dequant(b + 1);
            stage(rs, b + 2);
            issue(rs, 32 * min(b + 2 + kRegSets, nb - 1));
            __syncthreads();
        };
        for (int b0 = 0; b0 < nb; b0 += kRegSets) {
            if constexpr (kRegSets == 4) {
                step(b0, rs2);
                step(b0 + 1, rs3);
                step(b0 + 2, rs0);
                step(b0 + 3, rs1);
            } else {
                step(b0, rs0);
                step(b0 + 1, rs1);
            }
        }
        // into the recent-token units (2^kWShift): o = O 2^(E - kWShift) + sum_t p_t z_t
#pragma unroll
        for (int t = 0; t < TW; ++t) {
            const float ZB = ldexpf(col_sum(zb_run[t]), kWShift);
#pragma unroll
            for (int m = 0; m < MT; ++m)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    st[t].O[m][j] = ldexpf(st[t].O[m][j], E[t]) + ZB;
        }
    }

    // recent tokens and the output, one tile at a time (no barrier follows)
    uint16_t *vt = reinterpret_cast<uint16_t *>(lds) + wave * D * 32;
#pragma unroll
    for (int t = 0; t < TW; ++t) {
        if (tile[t] >= a.n_tiles)
            break;
        if (Tq < t_end) {
            if (a.kv_bf16)
                prefill_recent<D, true>(a, bh, qrow[t], act[t], p_col[t], Tq, t_end, lane, vt, st[t]);
            else
                prefill_recent<D, false>(a, bh, qrow[t], act[t], p_col[t], Tq, t_end, lane, vt, st[t]);
        }
        const float Lc = col_sum(st[t].l_run);
        if (act[t]) {
            const float inv = ldexpf(1.0f / Lc, -kWShift);
            float *o = a.out + qrow[t] + 4 * q;
#pragma unroll
            for (int m = 0; m < MT; ++m)
                *reinterpret_cast<f4_t *>(o + 16 * m) = st[t].O[m] * inv;
        }
    }
}

template <int KB, int VB, int D, bool KT, bool PG, int TW>
__global__ __launch_bounds__(kPrefillThreads, 1) void attn_prefill_kernel(PrefillArgs a)
{
    extern __shared__ __align__(16) char lds_pf[];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    // Workgroups are dealt to the eight XCDs in turn; number them so that
    // consecutive slots (workgroups of one stream, which read the same cache
    // rows) land on the same XCD and share its L2.
    const int id = blockIdx.x;
    const int slot = (a.n_wg % 8 == 0) ? (id % 8) * (a.n_wg / 8) + id / 8 : id;
    const int bh = slot / a.wg_per_stream, wg_in = slot - bh * a.wg_per_stream;
    prefill_wg<KB, VB, D, KT, PG, TW>(a, bh, wg_in, wave, lane, lds_pf);
}

template <int KB, int VB, bool KT, bool PG>
hipError_t launch_prefill_pair(const PrefillArgs &a, hipStream_t st)
{
    constexpr size_t lds = PfLds<KB, VB, KVQ_D, KT>::BYTES;
#if KVQ_D <= 128
    if (a.tw == 2) {
        hipLaunchKernelGGL((attn_prefill_kernel<KB, VB, KVQ_D, KT, PG, 2>), dim3(a.n_wg), dim3(kPrefillThreads), lds,
                           st, a);
        return hipGetLastError();
    }
#endif
    hipLaunchKernelGGL((attn_prefill_kernel<KB, VB, KVQ_D, KT, PG, 1>), dim3(a.n_wg), dim3(kPrefillThreads), lds, st, a);
    return hipGetLastError();
}

}  // namespace

hipError_t KVQ_CAT(launch_prefill_d, KVQ_D)(const PrefillArgs &a, hipStream_t st)
{
    const int kb = a.L.kb, vb = a.L.vb;
    const bool pg = a.L.table != nullptr;  // paged layer: its own instantiation
    if (kb == 16)  // recent tokens only: any instantiation serves
        return launch_prefill_pair<2, 2, false, false>(a, st);
#define KVQ_PAIR(K, V)                                                                                   \
    if (kb == K && vb == V)                                                                              \
        return pg ? (a.L.k_tok ? launch_prefill_pair<K, V, true, true>(a, st)                              \
                               : launch_prefill_pair<K, V, false, true>(a, st))                            \
                  : (a.L.k_tok ? launch_prefill_pair<K, V, true, false>(a, st)                             \
                               : launch_prefill_pair<K, V, false, false>(a, st));
    KVQ_PAIR(2, 2) KVQ_PAIR(2, 4) KVQ_PAIR(2, 8)
    KVQ_PAIR(4, 2) KVQ_PAIR(4, 4) KVQ_PAIR(4, 8)
    KVQ_PAIR(8, 2) KVQ_PAIR(8, 4) KVQ_PAIR(8, 8)
#undef KVQ_PAIR
#if KVQ_D == 128
    // 3-bit rows (per-channel Key only): twelve words, three per lane quad
    if (kb == 3 && vb == 2) return pg ? launch_prefill_pair<3, 2, false, true>(a, st) : launch_prefill_pair<3, 2, false, false>(a, st);
    if (kb == 3 && vb == 4) return pg ? launch_prefill_pair<3, 4, false, true>(a, st) : launch_prefill_pair<3, 4, false, false>(a, st);
    if (kb == 3 && vb == 8) return pg ? launch_prefill_pair<3, 8, false, true>(a, st) : launch_prefill_pair<3, 8, false, false>(a, st);
#endif
    return hipErrorInvalidValue;
}

}  // namespace kvq
