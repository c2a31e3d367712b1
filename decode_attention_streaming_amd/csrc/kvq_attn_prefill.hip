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

// q of this lane's column, channels c0 .. c0 + QC - 1 (16-byte aligned runs),
// widened to fp32
template <int QC>
__device__ __forceinline__ void load_q_slice(const void *q, int dtype, size_t i0, float (&r)[QC])
{
    if (dtype == 0) {
        float4 v[QC / 4];
#pragma unroll
        for (int i = 0; i < QC / 4; ++i)
            v[i] = reinterpret_cast<const float4 *>(static_cast<const float *>(q) + i0)[i];
#pragma unroll
        for (int i = 0; i < QC / 4; ++i) {
            r[4 * i] = v[i].x;
            r[4 * i + 1] = v[i].y;
            r[4 * i + 2] = v[i].z;
            r[4 * i + 3] = v[i].w;
        }
    } else {
        const int bf = dtype == 2;
        uint4 v[QC / 8];
#pragma unroll
        for (int i = 0; i < QC / 8; ++i)
            v[i] = reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(q) + i0)[i];
#pragma unroll
        for (int i = 0; i < QC / 8; ++i) {
            const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                r[8 * i + 2 * k] = widen16(static_cast<uint16_t>(w[k] & 0xFFFFu), bf);
                r[8 * i + 2 * k + 1] = widen16(static_cast<uint16_t>(w[k] >> 16), bf);
            }
        }
    }
}

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

// One tile: queries tile * QT .. tile * QT + QT - 1 of stream bh.
template <int KB, int VB, int D, bool KT>
__device__ void prefill_tile(const PrefillArgs &a, int bh, int tile, int lane, uint16_t *vt, float *meta_lds)
{
    constexpr int KW = D * KB / 128;  // K words per lane per token (3 bits: D / 11 rounded up, / 4)
    constexpr int PK = KB == 3 ? 1 : 16 / KB;   // K code pairs per word
    constexpr int CW = KB == 3 ? 11 : 32 / KB;  // K channels per word
    // channels of a quad's K words (3 bits: 11 per word, some past D), and
    // 32-position chunks of q.K (3 bits: six registers per word, padded)
    constexpr int QC = KB == 3 ? 11 * KW : D / 4;
    constexpr int NC = KB == 3 ? (6 * KW + 3) / 4 : D / 32;
    constexpr int FW = D * VB / 64;   // V words per lane per 32-token block
    constexpr int MT = D / 16;        // 16-channel tiles of P.V

    const LayerDev &L = a.L;
    const int g = a.g, G = L.G;
    const int col = lane & 15, q = lane >> 4;
    const int jq = col / g, h = col - jq * g;
    const int qi = tile * a.QT + jq;
    const bool act = jq < a.QT && qi < a.n_q;
    // this stream's sequence length and quantized tokens (per sequence when ragged)
    const int sb = a.ragged ? bh / a.Hkv : 0;
    const int N = a.ragged ? a.seqN[sb] : a.N;
    const int Tq = a.ragged ? a.seqTq[sb] : a.Tq;
    const int p_col = act ? N - a.n_q + qi : -1;  // last token this column sees
    const size_t qrow = (static_cast<size_t>(bh * g + (act ? h : 0)) * a.n_q + (act ? qi : 0)) * D;
    // tokens [0, t_end) cover every column of the tile (uniform)
    const int qi_last = min(a.n_q - 1, tile * a.QT + a.QT - 1);
    const int t_end = N - a.n_q + qi_last + 1;
    const int tq_end = min(Tq, (t_end + 31) & ~31);  // quantized blocks to visit

    ColState<MT> st;
#pragma unroll
    for (int m = 0; m < MT; ++m)
        st.O[m] = f4_t{0.0f, 0.0f, 0.0f, 0.0f};

    if (tq_end > 0) {
        const QAddr qa(L, bh);  // rows of the stream's tokens (through the page table when paged)
        float zb_run = 0.0f;
        int E = -1000;  // running V-scale exponent: the weights carry 2^(kWShift - E)
        Frag bhi[NC], blo[NC];
        float bias = 0.0f, kscale = 0.0f;

        // this column's q over the quad's channels, times log2(e) / sqrt(D)
        float qq[QC];
        if constexpr (KB == 3) {
            // channels 11 * KW * q + i; those past D weigh 0
#pragma unroll
            for (int i = 0; i < QC; ++i) {
                const int c = QC * q + i;
                qq[i] = c < D ? load_q(a.q, a.q_dtype, qrow + (c < D ? c : 0)) : 0.0f;
            }
        } else {
            load_q_slice<QC>(a.q, a.q_dtype, qrow + q * QC, qq);
        }
        {
            const float qscale = act ? a.scale_log2 : 0.0f;
#pragma unroll
            for (int i = 0; i < QC; ++i)
                qq[i] *= qscale;
        }

        // K scales and zeros of group gi ([2][D] floats) into LDS slot gi & 1
        // with direct-to-LDS loads: no registers held while they fly
        auto meta_issue = [&](int gi) {
            const float *src = L.k_meta + qa.grp(gi) * 2 * D;
            float *dst = meta_lds + (gi & 1) * 2 * D;
            constexpr int n16 = D / 2;  // 16-byte pieces
#pragma unroll
            for (int i0 = 0; i0 < n16; i0 += 64) {
                if (i0 + lane < n16)
                    __builtin_amdgcn_global_load_lds(src + 4 * (i0 + lane), dst + 4 * i0, 16, 0, 0);
            }
        };
        // B operand of q.K for group gi (per-token Key: q alone, built once):
        // q * s as hi/lo fp16 in the code-register order of the quad's words
        auto build_b = [&](int gi) {
            // the group's direct-to-LDS loads (issued one block earlier) must have
            // landed: wait for them explicitly, the compiler does not always
            // order LDS reads after them
            if constexpr (!KT)
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            float qs[QC];
            float amax = 0.0f;
            bias = 0.0f;
            if constexpr (KB == 3) {
                const float *sp = meta_lds + (gi & 1) * 2 * D;
#pragma unroll
                for (int i = 0; i < QC; ++i) {
                    const int c = QC * q + i;
                    const int cc = c < D ? c : 0;  // qq is 0 past D
                    qs[i] = qq[i] * sp[cc];
                    bias = __builtin_fmaf(qq[i], sp[D + cc], bias);
                    amax = fmaxf(amax, fabsf(qs[i]));
                }
            }
            const float *sp = meta_lds + (gi & 1) * 2 * D + q * QC;
            const float *zp = sp + D;
#pragma unroll
            for (int i = 0; i < (KB == 3 ? 0 : QC); i += 4) {
                const float4 one = {1.0f, 1.0f, 1.0f, 1.0f};
                const float4 s4 = KT ? one : *reinterpret_cast<const float4 *>(sp + i);
                const float4 z4 = KT ? one : *reinterpret_cast<const float4 *>(zp + i);
                const float sv[4] = {s4.x, s4.y, s4.z, s4.w};
                const float zv[4] = {z4.x, z4.y, z4.z, z4.w};
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    qs[i + k] = qq[i + k] * sv[k];
                    bias = __builtin_fmaf(qq[i + k], zv[k], bias);
                    amax = fmaxf(amax, fabsf(qs[i + k]));
                }
            }
            // the slot may be loaded again only after these reads
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            bias = col_sum(bias);
            amax = col_max(amax);
            const int sexp = amax > 0.0f ? __builtin_amdgcn_frexp_expf(amax) : 0;
            const int sh = 14 - sexp;  // |q s| * 2^sh < 2^14
#pragma unroll
            for (int k = 0; k < NC; ++k)
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    const int R = 4 * k + p;
                    if constexpr (KB == 3) {
                        // register r of word w: the lo slot (and the hi slot) of the
                        // 3-bit map, each divided by its bit offset
                        if (R < 6 * KW) {
                            const int w = R / 6, r = R % 6;
                            const float xlo = ldexpf(qs[11 * w + r], sh - k3_lo_e(r));
                            const float xhi =
                                k3_hi_slot(r) < 0 ? 0.0f : ldexpf(qs[11 * w + k3_hi_slot(r)], sh - k3_hi_e(r));
                            split_pair(xlo, xhi, bhi[k].u[p], blo[k].u[p]);
                        } else {
                            bhi[k].u[p] = 0u;
                            blo[k].u[p] = 0u;
                        }
                    } else {
                        const int clo = (R / PK) * CW + (R % PK), chi = clo + PK;
                        const int e = sh - class_exp<KB>(R);
                        split_pair(ldexpf(qs[clo], e), ldexpf(qs[chi], e), bhi[k].u[p], blo[k].u[p]);
                    }
                }
            kscale = ldexpf(1.0f, -sh);
        };
        if constexpr (KT)
            build_b(0);

        // one 32-token block: K rows of both 16-token tiles, the V fragment, the
        // V meta of this lane's eight tokens (and their K meta, per-token Key)
        struct Blk {
            uint32_t k0[KW], k1[KW], vw[FW];
            float4 vm[4], km[4];
        };
        auto load_blk = [&](Blk &b, int t0) {
            const size_t r0 = qa.row(t0);  // the block's 32 rows are consecutive
            load_words(L.k_words + (r0 + col) * L.wk + q * KW, b.k0);
            load_words(L.k_words + (r0 + 16 + col) * L.wk + q * KW, b.k1);
            load_words(L.v_words + r0 * L.wv + lane * FW, b.vw);
            const float4 *m0 = reinterpret_cast<const float4 *>(L.v_meta + (r0 + 4 * q) * 2);
            const float4 *m1 = reinterpret_cast<const float4 *>(L.v_meta + (r0 + 16 + 4 * q) * 2);
            b.vm[0] = m0[0];
            b.vm[1] = m0[1];
            b.vm[2] = m1[0];
            b.vm[3] = m1[1];
            if constexpr (KT) {
                const float4 *c0 = reinterpret_cast<const float4 *>(L.k_meta + (r0 + 4 * q) * 2);
                const float4 *c1 = reinterpret_cast<const float4 *>(L.k_meta + (r0 + 16 + 4 * q) * 2);
                b.km[0] = c0[0];
                b.km[1] = c0[1];
                b.km[2] = c1[0];
                b.km[3] = c1[1];
            }
        };

        // Software pipeline, one block ahead: while block t0 is computed, the
        // loads of block t0 + 32 (and of its group's meta when it starts a
        // group) are in flight.  The last iteration reloads its own block
        // (in bounds, unused) so that every iteration issues the same loads.
        Blk cur, nxt;
        if constexpr (!KT)
            meta_issue(0);
        load_blk(cur, 0);
        for (int t0 = 0; t0 < tq_end; t0 += 32) {
            if constexpr (!KT) {
                if (t0 % G == 0)  // G is a multiple of 32: a group starts on a block
                    build_b(t0 / G);
            }
            const int t1 = min(t0 + 32, tq_end - 32);
            if constexpr (!KT) {
                if (t1 > t0 && t1 % G == 0)
                    meta_issue(t1 / G);
            }
            load_blk(nxt, t1);

            // q.K for tokens 4q + j (acc0) and 16 + 4q + j (acc1)
            uint32_t k08[KW], k18[KW];
            shift8(cur.k0, k08);
            shift8(cur.k1, k18);
            f4_t acc0 = {0.0f, 0.0f, 0.0f, 0.0f}, acc1 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int k = 0; k < NC; ++k) {
                Frag a0, a1;
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    const int R = 4 * k + p;
                    if constexpr (KB == 3) {
                        a0.u[p] = R < 6 * KW ? code_reg3(cur.k0, k08, R) : 0u;
                        a1.u[p] = R < 6 * KW ? code_reg3(cur.k1, k18, R) : 0u;
                    } else {
                        a0.u[p] = code_reg<KB>(cur.k0, k08, R);
                        a1.u[p] = code_reg<KB>(cur.k1, k18, R);
                    }
                }
                acc0 = mfma(a0, bhi[k], acc0);
                acc0 = mfma(a0, blo[k], acc0);
                acc1 = mfma(a1, bhi[k], acc1);
                acc1 = mfma(a1, blo[k], acc1);
            }
            float sc[8];
            if constexpr (KT) {
                // score_t = s_t sum_c q_c code_tc + z_t sum_c q_c
                const float4 *km = cur.km;
                const float ks[8] = {km[0].x, km[0].z, km[1].x, km[1].z, km[2].x, km[2].z, km[3].x, km[3].z};
                const float kz[8] = {km[0].y, km[0].w, km[1].y, km[1].w, km[2].y, km[2].w, km[3].y, km[3].w};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    sc[j] = __builtin_fmaf(acc0[j] * kscale, ks[j], kz[j] * bias);
                    sc[4 + j] = __builtin_fmaf(acc1[j] * kscale, ks[4 + j], kz[4 + j] * bias);
                }
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    sc[j] = __builtin_fmaf(acc0[j], kscale, bias);
                    sc[4 + j] = __builtin_fmaf(acc1[j], kscale, bias);
                }
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {  // causal mask
                sc[j] = (t0 + 4 * q + j <= p_col) ? sc[j] : -INFINITY;
                sc[4 + j] = (t0 + 16 + 4 * q + j <= p_col) ? sc[4 + j] : -INFINITY;
            }
            const float4 *vm = cur.vm;
            const float vs[8] = {vm[0].x, vm[0].z, vm[1].x, vm[1].z, vm[2].x, vm[2].z, vm[3].x, vm[3].z};
            const float vz[8] = {vm[0].y, vm[0].w, vm[1].y, vm[1].w, vm[2].y, vm[2].w, vm[3].y, vm[3].w};
            float tmax = fmaxf(fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])),
                               fmaxf(fmaxf(sc[4], sc[5]), fmaxf(sc[6], sc[7])));
            tmax = col_max(tmax);
            float vmax = fmaxf(fmaxf(fmaxf(vs[0], vs[1]), fmaxf(vs[2], vs[3])),
                               fmaxf(fmaxf(vs[4], vs[5]), fmaxf(vs[6], vs[7])));
            vmax = col_max(vmax);
            const int eb = vmax > 0.0f ? __builtin_amdgcn_frexp_expf(vmax) : -1000;
            const bool need_m = act && (tmax > st.m_run + kTau);
            const bool need_e = act && (eb > E);
            if (__builtin_amdgcn_ballot_w64(need_m || need_e) != 0) {
                const float m_new = need_m ? tmax : st.m_run;
                const int E_new = need_e ? eb : E;
                const float alpha = (m_new == st.m_run) ? 1.0f : exp2f(st.m_run - m_new);
                const float f = ldexpf(alpha, E - E_new);
#pragma unroll
                for (int m = 0; m < MT; ++m)
                    st.O[m] *= f;
                st.l_run *= alpha;
                zb_run *= alpha;
                st.m_run = m_new;
                E = E_new;
            }
            const float mo = act ? st.m_run : INFINITY;
            float p[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                p[j] = weight_exp2(sc[j] - mo);
                st.l_run += p[j];
                zb_run = __builtin_fmaf(p[j], vz[j], zb_run);
            }
            // B operand of P.V: weights p s 2^(kWShift - E), k-slot pairs, each
            // divided by its code class factor
            Frag whi, wlo;
            const int wsh = kWShift - E;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int e = wsh - class_exp<VB>(r);
                split_pair(ldexpf(p[2 * r] * vs[2 * r], e), ldexpf(p[2 * r + 1] * vs[2 * r + 1], e), whi.u[r],
                           wlo.u[r]);
            }
            uint32_t v8[FW];
            shift8(cur.vw, v8);
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                Frag av;
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    av.u[r] = code_reg<VB>(cur.vw, v8, 4 * m + r);
                st.O[m] = mfma(av, whi, st.O[m]);
                st.O[m] = mfma(av, wlo, st.O[m]);
            }
            cur = nxt;
        }
        // into the recent-token units (2^kWShift): o = O 2^(E - kWShift) + sum_t p_t z_t
        const float ZB = ldexpf(col_sum(zb_run), kWShift);
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                st.O[m][j] = ldexpf(st.O[m][j], E) + ZB;
    }

    if (Tq < t_end) {
        if (a.kv_bf16)
            prefill_recent<D, true>(a, bh, qrow, act, p_col, Tq, t_end, lane, vt, st);
        else
            prefill_recent<D, false>(a, bh, qrow, act, p_col, Tq, t_end, lane, vt, st);
    }

    const float Lc = col_sum(st.l_run);
    if (act) {
        const float inv = ldexpf(1.0f / Lc, -kWShift);
        float *o = a.out + qrow + 4 * q;
#pragma unroll
        for (int m = 0; m < MT; ++m)
            *reinterpret_cast<f4_t *>(o + 16 * m) = st.O[m] * inv;
    }
}

// LDS floats per wave: V tile (D * 32 halves = D * 16 floats) + 2 * 2 * D
constexpr int kPrefillWaveFloats = KVQ_D * 16 + 4 * KVQ_D;

template <int KB, int VB, int D, bool KT>
__global__ __launch_bounds__(256, 2) void attn_prefill_kernel(PrefillArgs a)
{
    // per wave: a [D][32] 16-bit V tile (recent tokens), then two [2][D]
    // float slots of K scales and zeros (quantized tokens)
    extern __shared__ float lds_all[];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    // Workgroups are dealt to the eight XCDs in turn; number them so that
    // consecutive slots (tiles of one stream, which read the same cache rows)
    // land on the same XCD and share its L2.
    const int id = blockIdx.x;
    const int slot = (a.n_wg % 8 == 0) ? (id % 8) * (a.n_wg / 8) + id / 8 : id;
    const int unit = slot * 4 + wave;
    if (unit >= a.BH * a.n_tiles)
        return;  // no workgroup barrier follows: a wave may leave alone
    const int bh = unit / a.n_tiles, tile = unit - bh * a.n_tiles;
    float *region = lds_all + wave * kPrefillWaveFloats;
    prefill_tile<KB, VB, D, KT>(a, bh, tile, lane, reinterpret_cast<uint16_t *>(region), region + D * 16);
}

template <int KB, int VB, bool KT>
hipError_t launch_prefill_pair(const PrefillArgs &a, hipStream_t st)
{
    const size_t lds = 4 * kPrefillWaveFloats * sizeof(float);
    hipLaunchKernelGGL((attn_prefill_kernel<KB, VB, KVQ_D, KT>), dim3(a.n_wg), dim3(256), lds, st, a);
    return hipGetLastError();
}

}  // namespace

hipError_t KVQ_CAT(launch_prefill_d, KVQ_D)(const PrefillArgs &a, hipStream_t st)
{
    const int kb = a.L.kb, vb = a.L.vb;
    if (kb == 16)  // recent tokens only: any instantiation serves
        return launch_prefill_pair<2, 2, false>(a, st);
#define KVQ_PAIR(K, V)                                                        \
    if (kb == K && vb == V)                                                   \
        return a.L.k_tok ? launch_prefill_pair<K, V, true>(a, st) : launch_prefill_pair<K, V, false>(a, st);
    KVQ_PAIR(2, 2) KVQ_PAIR(2, 4) KVQ_PAIR(2, 8)
    KVQ_PAIR(4, 2) KVQ_PAIR(4, 4) KVQ_PAIR(4, 8)
    KVQ_PAIR(8, 2) KVQ_PAIR(8, 4) KVQ_PAIR(8, 8)
#undef KVQ_PAIR
#if KVQ_D == 128
    // 3-bit rows (per-channel Key only): twelve words, three per lane quad
    if (kb == 3 && vb == 2) return launch_prefill_pair<3, 2, false>(a, st);
    if (kb == 3 && vb == 4) return launch_prefill_pair<3, 4, false>(a, st);
    if (kb == 3 && vb == 8) return launch_prefill_pair<3, 8, false>(a, st);
#endif
    return hipErrorInvalidValue;
}

}  // namespace kvq
