// kvq_attn_mfma.hip -- matrix-core (MFMA) split-sequence decode attention over
// the quantized cache for one head_dim (KVQ_D, set by the build: 64, 128, 256).
//
// Both products of o = softmax(q K^T / sqrt(D)) V (KVTuner summary, A3
// attention equation) run on v_mfma_f32_16x16x32_f16 with fp32 accumulation,
// dequantization folded into the operands (KVmix notes, key design 4):
//   score_t = sum_c (q_c s_c) code_tc + sum_c q_c z_c      (K per channel, per group)
//   o_c     = sum_t (p_t s_t) code_tc + sum_t p_t z_t      (V per token)
// Codes enter the matrix core as fp16 integers: a code k is masked into the
// mantissa of 1024.0 (fp16 bits 0x6400 | k = 1024 + k) and 1024 is subtracted
// with a packed fp16 add, both exact.  (Feeding k as the fp16 subnormal
// k * 2^-24 would save the subtraction, but the matrix core multiplies
// subnormal operands with only about 13 bits of precision.)  The fp32 factors
// (q s and p s) are split into two fp16 halves, hi + lo, and both are
// multiplied (about 22 significant bits), after scaling by a power of two into
// fp16 range.  The z terms stay in fp32 on the vector ALU.
//
// One wave processes one unit (a run of whole K groups of one stream).  The 16
// columns of each product are (head, group-slot) pairs: with g query heads per
// kv-head, NG (the largest power of two <= 16 / g) consecutive groups are
// processed per window, column j*S + h (S = 16 / NG) carrying head h over the
// tokens of group j.  Every column keeps its own online-softmax state, so each
// lane's B operand is useful and no data moves between the two products; the
// NG columns of a head are merged at the end of the unit by row rotations.
// The four waves of a workgroup then merge their results through LDS into one
// partial entry per head.  Query heads of a GQA group share every K/V read
// (KIVI notes, section 7.2).
#include <type_traits>

#include "kvq_mfma_ops.h"

#ifndef KVQ_D
#error "KVQ_D (head_dim) must be defined"
#endif

namespace kvq {
namespace {

// Windows (groups) of the double-buffered walk: it serves windows of at most
// this many groups.
constexpr int kPipeGroups = 2;

// Types with a double-buffered instantiation, whose rounds take half the
// blocks of the plain walk's (two rounds in registers, as many as one round
// there): 3-bit Key excluded, per-token Key with four-block rounds only for
// narrow codes (wider ones spill), and K8V8, whose plain two-block rounds
// (16 KB per wave in flight) beat overlapped one-block rounds (Qwen2.5-7B
// shape: 39.7 against 41.6 us per call).
__host__ __device__ constexpr bool mfma_pipe_ok(int kb, int vb, int D, bool kt)
{
    return D <= 128 && mfma_round_blocks(kb, vb, D) >= 2 && kb != 3 && !(kb == 8 && vb == 8) &&
           (!kt || kb + vb <= 8 || mfma_round_blocks(kb, vb, D) == 2);
}

// End of a quantized unit: this lane's column state (l, z-term, o; weights
// carry 2^(kWShift - E)); the S-strided columns of one head are rescaled to
// their common max and summed, and slot 0 of head h < g writes o[h][D], m, l
// to LDS.
template <int S, int D, int MT>
__device__ __forceinline__ void finish_unit(float m_run, float l_run, float zb_run, int E, const f4_t (&O)[MT],
                                            int col, int q, int g, float *po, float *pm, float *pl)
{
    const float Lcol = col_sum(l_run);
    const float ZB = col_sum(zb_run);
    const float M = coset_max<S>(m_run);
    const float alpha = (m_run == -INFINITY) ? 0.0f : exp2f(m_run - M);
    const float fo = ldexpf(alpha, E - kWShift), fz = alpha * ZB;
    const float Lh = coset_sum<S>(alpha * Lcol);
    float o[MT][4];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            o[m][j] = coset_sum<S>(__builtin_fmaf(O[m][j], fo, fz));
    if (col < g) {  // slot 0 of head col
#pragma unroll
        for (int m = 0; m < MT; ++m)
            *reinterpret_cast<f4_t *>(po + col * D + 16 * m + 4 * q) = f4_t{o[m][0], o[m][1], o[m][2], o[m][3]};
        if (q == 0) {
            pm[col] = M;
            pl[col] = Lh;
        }
    }
}

// Data of one round: for each of its blocks the K rows of both 16-token tiles
// and the V fragment; the V meta (s, z) of this lane's eight k-slot tokens in
// its own block.
template <int NB, int KW, int FW>
struct RoundData {
    static constexpr int N = NB;
    uint32_t k0[NB][KW], k1[NB][KW], v[NB][FW];
    float4 vm[4];
    float4 km[4];  // per-token Key: (scale, zero) of the same eight tokens
};

// One unit: groups [g_beg, g_end) of stream bh, in windows of NG groups (one
// per column slot).  Inside a window, round (r, u) takes block r of the groups
// in slots u .. u + nb - 1: every block's q.K product is computed for all 16
// columns, and each lane keeps the scores of the block of its own slot, so the
// softmax work of one round serves nb blocks.  In the P.V products a lane's
// weights enter only its own block's product (zeros elsewhere).
// Results for head h < g go to po[h * D + c], pm[h], pl[h] (LDS).
template <int KB, int VB, int D, bool KT, bool PG, bool PP>
__device__ void mfma_unit(const AttnArgs &a, const RaggedTables *rt, int bh, int unit, int lane, float *po, float *pm,
                          float *pl,
                          float *meta_lds)
{
    constexpr int QC = D / 4;           // channels owned by one lane quad (2, 4, 8 bits)
    constexpr int KW = D * KB / 128;    // K words per lane per token (3 bits: D / 11 rounded up, / 4)
    constexpr int PK = KB == 3 ? 1 : 16 / KB;  // K code pairs per word
    constexpr int CW = KB == 3 ? 11 : 32 / KB; // K channels per word
    // 32-position chunks of q.K: D / 32, or six registers per 3-bit word
    // (padded with zero registers to whole chunks)
    constexpr int NC = KB == 3 ? (6 * KW + 3) / 4 : D / 32;
    constexpr int QK = KB == 3 ? 11 * KW : QC;  // channels of a quad's K words (3 bits: some past D)
    constexpr int FW = D * VB / 64;     // V words per lane per 32-token block
    constexpr int MT = D / 16;          // 16-channel tiles of P.V
    constexpr int NB = mfma_round_blocks(KB, VB, D);

    const LayerDev &L = a.L;
    const int G = L.G, g = a.g;
    const int col = lane & 15, q = lane >> 4;
    // S = 2^s_log2 columns per group slot, NG = 16 / S slots (host-computed:
    // no division before the first loads)
    const int S = 1 << a.s_log2, NG = 16 >> a.s_log2;
    const bool used = (col & (S - 1)) < g;
    const int h = used ? (col & (S - 1)) : 0;
    const int jslot = used ? (col >> a.s_log2) : NG;
    const StreamDims sd = stream_dims(a, rt, bh);
    const int g_beg = unit * sd.unit_groups + min(unit, sd.unit_extra);
    const int g_end = g_beg + sd.unit_groups + (unit < sd.unit_extra ? 1 : 0);
    const int bpg = G / 32;  // blocks per group

    const QAddr qa(L, bh);  // rows of the stream's tokens (through the page table when paged)
    constexpr bool paged = PG;  // (the launch picks the instantiation by the layer's layout)
    WavePages wp;           // paged: page ids of the current window's tokens, one per lane
    constexpr bool ktok = KT;  // per-token Key (its meta: 2 floats per row)
    // this lane's word offsets in a block's K rows (tiles of tokens col and
    // 16 + col) and V fragments, from the block's first row
    const size_t koff0 = static_cast<size_t>(col) * L.wk + q * KW, koff1 = koff0 + 16 * static_cast<size_t>(L.wk);
    const int voff = lane * FW;

    float m_run = -INFINITY, l_run = 0.0f, zb_run = 0.0f;
    int E = -1000;  // running V-scale exponent of this column: its weights carry 2^-E
    f4_t O[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m)
        O[m] = f4_t{0.0f, 0.0f, 0.0f, 0.0f};

    Frag bhi[NC], blo[NC];
    float bias = 0.0f, kscale = 0.0f;

    // ---- window of groups [w0, w0 + nwin): its K scales and zeros go to this
    // wave's LDS with direct-to-LDS loads (no registers held while they fly), so
    // that the window's first round can load at the same time ----
    // The stream's q (g heads, fp32 or 16-bit) follows them, loaded the same way.
    const int qbytes = a.q_dtype == 0 ? 4 : 2;
    float *q_lds = meta_lds + NG * 2 * D;
    auto setup_issue = [&](int w0, int nwin) {
        constexpr int gp_log2 = __builtin_ctz(D / 2);  // 16-byte pieces per group: D / 2
        const int n16 = ktok ? 0 : nwin * D / 2;  // 16-byte pieces of nwin groups' [2][D] floats
        for (int i0 = 0; i0 < n16; i0 += 64) {
            const int i = i0 + lane, j = min(i >> gp_log2, nwin - 1);  // piece i of group w0 + j
            const size_t gr = paged ? wp.grp_v(qa, w0 + j) : qa.gbase + w0 + j;
            if (i < n16)
                __builtin_amdgcn_global_load_lds(L.k_meta + gr * 2 * D + 4 * (i & (D / 2 - 1)),
                                                 meta_lds + 4 * i0, 16, 0, 0);
        }
        const char *qsrc = static_cast<const char *>(a.q) + static_cast<size_t>(bh) * g * D * qbytes;
        const int nq16 = g * D * qbytes / 16;
        for (int i0 = 0; i0 < nq16; i0 += 64) {
            if (i0 + lane < nq16)
                __builtin_amdgcn_global_load_lds(qsrc + 16 * (i0 + lane), q_lds + 4 * i0, 16, 0, 0);
        }
    };
    // ---- B operand of q.K for this lane's column, q * s as hi/lo fp16; waits
    // for every load issued so far ----
    // (dma: the window's meta came by direct-to-LDS loads, which the
    // compiler does not wait for by itself)
    auto setup_compute = [&](int nwin, auto dma) {
        if (dma)
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        const bool act_win = jslot < nwin;
        const float qscale = act_win ? a.scale_log2 : 0.0f;
        float qs[QK];
        float amax = 0.0f;
        bias = 0.0f;
        if constexpr (KB == 3) {
            // the quad's 11 * KW channels from c0 (those past D weigh 0)
            const int c0 = QK * q;
            const float *sp = meta_lds + (act_win ? jslot : 0) * 2 * D;
            const float *zp = sp + D;
            const int bf = a.q_dtype == 2;
#pragma unroll
            for (int i = 0; i < QK; ++i) {
                const int c = c0 + i;
                const bool ok = c < D;
                const int cc = ok ? c : 0;
                const float qv = a.q_dtype == 0 ? q_lds[h * D + cc]
                                                : widen16(reinterpret_cast<const uint16_t *>(q_lds)[h * D + cc], bf);
                const float qq = ok ? qv * qscale : 0.0f;
                qs[i] = qq * sp[cc];
                bias = __builtin_fmaf(qq, zp[cc], bias);
                amax = fmaxf(amax, fabsf(qs[i]));
            }
        } else {
            const float *sp = meta_lds + (act_win ? jslot : 0) * 2 * D + q * QC;
            const float *zp = sp + D;
            float qv[QC];
            if (a.q_dtype == 0) {
                const float4 *qp = reinterpret_cast<const float4 *>(q_lds + h * D + q * QC);
#pragma unroll
                for (int i = 0; i < QC / 4; ++i) {
                    const float4 v = qp[i];
                    qv[4 * i] = v.x; qv[4 * i + 1] = v.y; qv[4 * i + 2] = v.z; qv[4 * i + 3] = v.w;
                }
            } else {
                const uint4 *qp = reinterpret_cast<const uint4 *>(reinterpret_cast<const uint16_t *>(q_lds) + h * D + q * QC);
                if (a.q_dtype == 2) {
#pragma unroll
                    for (int i = 0; i < QC / 8; ++i) {
                        const uint4 v = qp[i];
                        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                        for (int k = 0; k < 4; ++k)
                            widen_pair<true>(w[k], qv[8 * i + 2 * k], qv[8 * i + 2 * k + 1]);
                    }
                } else {
#pragma unroll
                    for (int i = 0; i < QC / 8; ++i) {
                        const uint4 v = qp[i];
                        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                        for (int k = 0; k < 4; ++k)
                            widen_pair<false>(w[k], qv[8 * i + 2 * k], qv[8 * i + 2 * k + 1]);
                    }
                }
            }
#pragma unroll
            for (int i = 0; i < QC; i += 4) {
                // per-token Key: no per-channel factors here (s = z = 1: bias is
                // then sum_c q_c, the z-term's factor); the token's scale and
                // zero apply to the scores
                const float4 one = {1.0f, 1.0f, 1.0f, 1.0f};
                const float4 s4 = ktok ? one : *reinterpret_cast<const float4 *>(sp + i);
                const float4 z4 = ktok ? one : *reinterpret_cast<const float4 *>(zp + i);
                const float sv[4] = {s4.x, s4.y, s4.z, s4.w};
                const float zv[4] = {z4.x, z4.y, z4.z, z4.w};
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const float qq = qv[i + k] * qscale;
                    qs[i + k] = qq * sv[k];
                    bias = __builtin_fmaf(qq, zv[k], bias);
                    amax = fmaxf(amax, fabsf(qs[i + k]));
                }
            }
        }
        bias = col_sum(bias);
        amax = col_max(amax);
        const int sexp = amax > 0.0f ? __builtin_amdgcn_frexp_expf(amax) : 0;
        const int sh = 14 - sexp;  // |q s| * 2^sh < 2^14
#pragma unroll
        for (int k = 0; k < NC; ++k) {
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const int R = 4 * k + p;
                if constexpr (KB == 3) {
                    if (R < 6 * KW) {
                        const int w = R / 6, r = R % 6;
                        const float xlo = ldexpf(qs[11 * w + r], sh - k3_lo_e(r));
                        const float xhi = k3_hi_slot(r) < 0 ? 0.0f
                                                            : ldexpf(qs[11 * w + k3_hi_slot(r)], sh - k3_hi_e(r));
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
        }
        kscale = ldexpf(1.0f, -sh);  // acc * 2^-sh
        // the next window's meta may overwrite this one only after these reads
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    };

    // ---- one round: nb blocks starting at tokens t_first + i * G ----
    // every_slot: all NB slots are loaded, those past nb with a re-read of
    // block nb - 1, so that the loads issued do not depend on nb (the
    // compiler then waits for exactly this round's loads, not for every load
    // in flight)
    auto load_round = [&](auto &d, int t_first, int nb, int my_b, auto every_slot) {
        constexpr int NB = std::decay_t<decltype(d)>::N;
        // each block's 32 rows are consecutive; its first row is the same in
        // every lane (one branch on the layout per round)
        size_t r0[NB];
        const int tm = t_first + my_b * G;
        size_t rm;
        if (paged) {
#pragma unroll
            for (int i = 0; i < NB; ++i)
                r0[i] = wp.row_u(qa, t_first + min(i, nb - 1) * G);
            rm = wp.row_v(qa, tm);
        } else {
#pragma unroll
            for (int i = 0; i < NB; ++i)
                r0[i] = qa.base + t_first + (every_slot ? min(i, nb - 1) : i) * G;
            rm = qa.base + tm;
        }
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            if (every_slot || i < nb) {
                const uint32_t *kr = L.k_words + r0[i] * L.wk;
                load_words(kr + koff0, d.k0[i]);
                load_words(kr + koff1, d.k1[i]);
                load_words(L.v_words + r0[i] * L.wv + voff, d.v[i]);
            }
        }
        const float4 *m0 = reinterpret_cast<const float4 *>(L.v_meta + (rm + 4 * q) * 2);
        const float4 *m1 = reinterpret_cast<const float4 *>(L.v_meta + (rm + 16 + 4 * q) * 2);
        d.vm[0] = m0[0];
        d.vm[1] = m0[1];
        d.vm[2] = m1[0];
        d.vm[3] = m1[1];
        if constexpr (KT) {
            {
                const float4 *k0 = reinterpret_cast<const float4 *>(L.k_meta + (rm + 4 * q) * 2);
                const float4 *k1 = reinterpret_cast<const float4 *>(L.k_meta + (rm + 16 + 4 * q) * 2);
                d.km[0] = k0[0];
                d.km[1] = k0[1];
                d.km[2] = k1[0];
                d.km[3] = k1[1];
            }
        }
    };

    auto process_round = [&](const auto &d, int nb, bool mine, int my_b) {
        constexpr int NB = std::decay_t<decltype(d)>::N;
        // q.K for tokens 4q + j (acc0) and 16 + 4q + j (acc1) of each block;
        // this lane keeps its own block's scores
        float sc[8];
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            if (i < nb) {
                uint32_t k08[KW], k18[KW];
                shift8(d.k0[i], k08);
                shift8(d.k1[i], k18);
                f4_t acc0 = {0.0f, 0.0f, 0.0f, 0.0f}, acc1 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int k = 0; k < NC; ++k) {
                    Frag a0, a1;
#pragma unroll
                    for (int p = 0; p < 4; ++p) {
                        const int R = 4 * k + p;
                        if constexpr (KB == 3) {
                            a0.u[p] = R < 6 * KW ? code_reg3(d.k0[i], k08, R) : 0u;
                            a1.u[p] = R < 6 * KW ? code_reg3(d.k1[i], k18, R) : 0u;
                        } else {
                            a0.u[p] = code_reg<KB>(d.k0[i], k08, R);
                            a1.u[p] = code_reg<KB>(d.k1[i], k18, R);
                        }
                    }
                    acc0 = mfma(a0, bhi[k], acc0);
                    acc0 = mfma(a0, blo[k], acc0);
                    acc1 = mfma(a1, bhi[k], acc1);
                    acc1 = mfma(a1, blo[k], acc1);
                }
                const bool take = (i == 0) | (my_b == i);  // selects, not a branch
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    sc[j] = take ? acc0[j] : sc[j];
                    sc[4 + j] = take ? acc1[j] : sc[4 + j];
                }
            }
        }
        if constexpr (KT) {
            // score_t = s_t sum_c q_c code_tc + z_t sum_c q_c
            const float ks[8] = {d.km[0].x, d.km[0].z, d.km[1].x, d.km[1].z,
                                 d.km[2].x, d.km[2].z, d.km[3].x, d.km[3].z};
            const float kz[8] = {d.km[0].y, d.km[0].w, d.km[1].y, d.km[1].w,
                                 d.km[2].y, d.km[2].w, d.km[3].y, d.km[3].w};
#pragma unroll
            for (int j = 0; j < 8; ++j)
                sc[j] = __builtin_fmaf(sc[j] * kscale, ks[j], kz[j] * bias);
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j)
                sc[j] = __builtin_fmaf(sc[j], kscale, bias);
        }
        const float vs[8] = {d.vm[0].x, d.vm[0].z, d.vm[1].x, d.vm[1].z,
                             d.vm[2].x, d.vm[2].z, d.vm[3].x, d.vm[3].z};
        const float vz[8] = {d.vm[0].y, d.vm[0].w, d.vm[1].y, d.vm[1].w,
                             d.vm[2].y, d.vm[2].w, d.vm[3].y, d.vm[3].w};
        float tmax = fmaxf(fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])),
                           fmaxf(fmaxf(sc[4], sc[5]), fmaxf(sc[6], sc[7])));
        tmax = col_max(tmax);
        // V-scale exponent of this column's block: s < 2^eb for every token
        float vmax = fmaxf(fmaxf(fmaxf(vs[0], vs[1]), fmaxf(vs[2], vs[3])),
                           fmaxf(fmaxf(vs[4], vs[5]), fmaxf(vs[6], vs[7])));
        vmax = col_max(vmax);
        const int eb = vmax > 0.0f ? __builtin_amdgcn_frexp_expf(vmax) : -1000;
        const bool need_m = mine && (tmax > m_run + kTau);
        const bool need_e = mine && (eb > E);
        if (__builtin_amdgcn_ballot_w64(need_m || need_e) != 0) {
            const float m_new = need_m ? tmax : m_run;
            const int E_new = need_e ? eb : E;
            const float alpha = (m_new == m_run) ? 1.0f : exp2f(m_run - m_new);
            const float f = ldexpf(alpha, E - E_new);
#pragma unroll
            for (int m = 0; m < MT; ++m)
                O[m] *= f;
            l_run *= alpha;
            zb_run *= alpha;
            m_run = m_new;
            E = E_new;
        }
        const float mo = mine ? m_run : INFINITY;  // columns without a block here: weights 0
        float p[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            p[j] = weight_exp2(sc[j] - mo);
            l_run += p[j];
            zb_run = __builtin_fmaf(p[j], vz[j], zb_run);
        }
        // B operand of P.V: weights p s 2^(kWShift - E), k-slot pairs (0,1) (2,3)
        // (4,5) (6,7), each divided by its code class factor
        Frag whi, wlo;
        const int wsh = kWShift - E;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int e = wsh - class_exp<VB>(r);
            split_pair(ldexpf(p[2 * r] * vs[2 * r], e), ldexpf(p[2 * r + 1] * vs[2 * r + 1], e), whi.u[r],
                       wlo.u[r]);
        }
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            if (i < nb) {
                Frag bh_, bl_;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    bh_.u[r] = (my_b == i) ? whi.u[r] : 0u;
                    bl_.u[r] = (my_b == i) ? wlo.u[r] : 0u;
                }
                uint32_t v8[FW];
                shift8(d.v[i], v8);
#pragma unroll
                for (int m = 0; m < MT; ++m) {
                    Frag av;
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        av.u[r] = code_reg<VB>(d.v[i], v8, 4 * m + r);
                    O[m] = mfma(av, bh_, O[m]);
                    O[m] = mfma(av, bl_, O[m]);
                }
            }
        }
    };

    static_assert(!PP || mfma_pipe_ok(KB, VB, D, KT), "no double-buffered walk for this type");
    if constexpr (PP) {
        // Windows of at most kPipeGroups groups (g > 16 / kPipeGroups), rounds
        // of PB = NB / 2 blocks: two round buffers (no more registers than one
        // round of NB), and the loads of the next round -- with the K scales and zeros
        // of the window it belongs to -- are issued before this round is
        // processed, so that the memory round trip overlaps the processing.
        // Those scales come into registers (a pending direct-to-LDS load would
        // make the compiler wait for every load before this round's products)
        // and go to LDS after them, when the next round starts a window; q
        // stays in LDS from the unit's first set-up.
        constexpr int PB = NB / 2;
        RoundData<PB, KW, FW> dA, dB;
        // round (w0, r, u): block r of groups w0 + u .. w0 + u + nb - 1
        int w0 = g_beg, r = 0, u = 0;
        int nwin = __builtin_amdgcn_readfirstlane(min(NG, g_end - w0));
        int nb = min(PB, nwin);
        bool mine = jslot < nb;
        if (paged && !wp.covers(qa, w0 * G, (w0 + nwin) * G))
            wp.load(qa, lane, w0 * G, g_end * G);
        setup_issue(w0, nwin);
        load_round(dA, w0 * G, nb, mine ? jslot : 0, std::true_type{});
        setup_compute(nwin, std::true_type{});
        // a window's [nwin][2][D] floats as 16-byte pieces, lane + 64 i (those
        // past the window re-read its last pieces)
        constexpr int MP = KT ? 1 : (kPipeGroups * D / 2 + 63) / 64;
        u32x4_t mreg[MP];
        auto meta_load = [&](int w1, int nwin1) {
            if constexpr (!KT) {
                constexpr int gp_log2 = __builtin_ctz(D / 2);
#pragma unroll
                for (int ip = 0; ip < MP; ++ip) {
                    const int i = min(64 * ip + lane, nwin1 * D / 2 - 1), j = i >> gp_log2;
                    const size_t gr = paged ? wp.grp_v(qa, w1 + j) : qa.gbase + w1 + j;
                    mreg[ip] = *reinterpret_cast<const u32x4_t *>(L.k_meta + gr * 2 * D + 4 * (i & (D / 2 - 1)));
                }
            }
        };
        auto meta_store = [&](int nwin1) {
            if constexpr (!KT) {
#pragma unroll
                for (int ip = 0; ip < MP; ++ip)
                    if (64 * ip + lane < nwin1 * D / 2)
                        *reinterpret_cast<u32x4_t *>(meta_lds + 4 * (64 * ip + lane)) = mreg[ip];
            }
        };
        // one round from cur (round (w0, r, u)) with the loads of the next into
        // nxt; false after the unit's last round.  The loads are issued
        // unconditionally (after the last round: a re-read of this one, from
        // L2), so that the wait before the products is for cur's loads only.
        auto pipe_step = [&](auto &cur, auto &nxt) -> bool {
            int w1 = w0, r1 = r, u1 = u + PB, nwin1 = nwin;
            if (u1 >= nwin) {
                u1 = 0;
                ++r1;
            }
            const bool new_win = r1 == bpg;
            if (new_win) {
                w1 = w0 + NG;
                r1 = 0;
                nwin1 = __builtin_amdgcn_readfirstlane(min(NG, g_end - w1));
            }
            const bool more = w1 < g_end;  // uniform
            if (!more) {
                w1 = w0;
                r1 = r;
                u1 = u;
                nwin1 = nwin;
            }
            const int nb1 = min(PB, nwin1 - u1);
            const bool mine1 = jslot >= u1 && jslot < u1 + nb1;
            if (paged && more && new_win && !wp.covers(qa, w1 * G, (w1 + nwin1) * G))
                wp.load(qa, lane, w1 * G, g_end * G);  // (its own wait: once per 64 pages)
            meta_load(w1, nwin1);
            load_round(nxt, (w1 + u1) * G + r1 * 32, nb1, mine1 ? jslot - u1 : 0, std::true_type{});
            process_round(cur, nb, mine, mine ? jslot - u : 0);
            if (more && new_win) {
                meta_store(nwin1);
                setup_compute(nwin1, std::false_type{});
            }
            w0 = w1;
            r = r1;
            u = u1;
            nwin = nwin1;
            nb = nb1;
            mine = mine1;
            return more;
        };
        while (pipe_step(dA, dB) && pipe_step(dB, dA)) {
        }
    } else {
        for (int w0 = g_beg; w0 < g_end; w0 += NG) {
            const int nwin = __builtin_amdgcn_readfirstlane(min(NG, g_end - w0));  // uniform
            const bool in_win = jslot < nwin;
            if (paged && !wp.covers(qa, w0 * G, (w0 + nwin) * G))
                wp.load(qa, lane, w0 * G, g_end * G);  // once per 64 pages of the unit
            setup_issue(w0, nwin);
            for (int r = 0; r < bpg; ++r) {
                for (int u = 0; u < nwin; u += NB) {
                    const int nb = __builtin_amdgcn_readfirstlane(min(NB, nwin - u));
                    const bool mine = in_win && jslot >= u && jslot < u + nb;
                    const int my_b = mine ? jslot - u : 0;
                    RoundData<NB, KW, FW> d;
                    load_round(d, (w0 + u) * G + r * 32, nb, my_b, std::false_type{});
                    if (r == 0 && u == 0)  // one memory round trip for the set-up and the first round
                        setup_compute(nwin, std::true_type{});
                    process_round(d, nb, mine, my_b);
                }
            }
        }
    }

    switch (a.s_log2) {
    case 0: finish_unit<1, D>(m_run, l_run, zb_run, E, O, col, q, g, po, pm, pl); break;
    case 1: finish_unit<2, D>(m_run, l_run, zb_run, E, O, col, q, g, po, pm, pl); break;
    case 2: finish_unit<4, D>(m_run, l_run, zb_run, E, O, col, q, g, po, pm, pl); break;
    case 3: finish_unit<8, D>(m_run, l_run, zb_run, E, O, col, q, g, po, pm, pl); break;
    default: finish_unit<16, D>(m_run, l_run, zb_run, E, O, col, q, g, po, pm, pl); break;
    }
}

// Recent (16-bit) tokens [Tq + runit * res_tokens, ...) of one stream on the
// matrix core, one wave.  Column h < g carries head h.  q.K reads the K rows as
// fp16 or bf16 operands directly (q split into hi/lo fp16, or three bfloat16
// parts); P.V reads V through a per-wave LDS tile written transposed
// ([channel][token]) so that each lane's operand (eight tokens of one channel)
// is two 8-byte LDS reads.
template <int D, bool BF>
__device__ void mfma_residual_unit(const AttnArgs &a, const RaggedTables *rt, int bh, int runit, int lane, float *po,
                                   float *pm, float *pl)
{
    constexpr int NC = D / 32;
    constexpr int MT = D / 16;
    const LayerDev &L = a.L;
    const int g = a.g;
    const int col = lane & 15, q = lane >> 4;
    const bool act = col < g;
    const int h = act ? col : 0;
    constexpr bool bf = BF;  // bfloat16 recent tokens (instantiated per dtype: no branches)
    const StreamDims sd = stream_dims(a, rt, bh);
    const int t_beg = sd.Tq + runit * a.res_tokens;
    const int t_end = min(sd.N, t_beg + a.res_tokens);
    uint16_t *vt = reinterpret_cast<uint16_t *>(po);  // [D][32] tile, then the results
    uint16_t *rk = L.ring_k + static_cast<size_t>(bh) * L.R * D;
    uint16_t *rv = L.ring_v + static_cast<size_t>(bh) * L.R * D;
    // row of token t: the ring, or the just-appended token's own row
    const int new_t = sd.new_t;
    auto k_row = [&](int t) {
        return (t == new_t) ? a.new_k + static_cast<size_t>(bh) * D : rk + static_cast<size_t>(t % L.R) * D;
    };
    auto v_row = [&](int t) {
        return (t == new_t) ? a.new_v + static_cast<size_t>(bh) * D : rv + static_cast<size_t>(t % L.R) * D;
    };

    // B operand of q.K: q of head h, chunk k, quad q -> channels 32k + 8q + i
    Frag b1[NC], b2[NC], b3[NC];
    int sh;
    {
        float qv[NC][8];
        const size_t base = (static_cast<size_t>(bh) * g + h) * D;  // stream bh = (b, kv head)
        float amax = 0.0f;
        load_q_runs<NC>(a.q, a.q_dtype, base + 8 * q, 32, qv);
#pragma unroll
        for (int k = 0; k < NC; ++k) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                qv[k][i] = act ? qv[k][i] * a.scale_log2 : 0.0f;
                amax = fmaxf(amax, fabsf(qv[k][i]));
            }
        }
        amax = col_max(amax);
        const int qexp = amax > 0.0f ? __builtin_amdgcn_frexp_expf(amax) : 0;
        sh = bf ? 0 : 14 - qexp;  // fp16 operands need the fp16 range
#pragma unroll
        for (int k = 0; k < NC; ++k)
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const float x0 = ldexpf(qv[k][2 * p], sh), x1 = ldexpf(qv[k][2 * p + 1], sh);
                if constexpr (bf)
                    split3_bf16(x0, x1, b1[k].u[p], b2[k].u[p], b3[k].u[p]);
                else
                    split_pair(x0, x1, b1[k].u[p], b2[k].u[p]);
            }
    }
    const float kscale = ldexpf(1.0f, -sh);

    float m_run = -INFINITY, l_run = 0.0f;
    f4_t O[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m)
        O[m] = f4_t{0.0f, 0.0f, 0.0f, 0.0f};

    for (int t0 = t_beg; t0 < t_end; t0 += 32) {
        // K rows of the two 16-token tiles (rows past the end repeat the last token)
        const int ta = min(t0 + col, t_end - 1), tb = min(t0 + 16 + col, t_end - 1);
        uint4 ka[NC], kb2[NC];
        const uint16_t *ra = k_row(ta), *rb = k_row(tb);
#pragma unroll
        for (int k = 0; k < NC; ++k) {
            ka[k] = *reinterpret_cast<const uint4 *>(ra + 32 * k + 8 * q);
            kb2[k] = *reinterpret_cast<const uint4 *>(rb + 32 * k + 8 * q);
        }
        // the just-appended token's K row goes to its ring slot
        if (t0 + col == new_t) {
            uint16_t *dst = rk + static_cast<size_t>(new_t % L.R) * D;
#pragma unroll
            for (int k = 0; k < NC; ++k)
                *reinterpret_cast<uint4 *>(dst + 32 * k + 8 * q) = ka[k];
        }
        if (t0 + 16 + col == new_t) {
            uint16_t *dst = rk + static_cast<size_t>(new_t % L.R) * D;
#pragma unroll
            for (int k = 0; k < NC; ++k)
                *reinterpret_cast<uint4 *>(dst + 32 * k + 8 * q) = kb2[k];
        }
        // V rows -> LDS [channel][token]: lane handles token (lane & 31), half of the row
        {
            const int tt = lane & 31, half = lane >> 5;
            const int tv = min(t0 + tt, t_end - 1);
            const uint4 *src = reinterpret_cast<const uint4 *>(v_row(tv) + half * (D / 2));
            uint4 v[D / 16];
#pragma unroll
            for (int i = 0; i < D / 16; ++i)
                v[i] = src[i];
            if (t0 + tt == new_t) {  // the just-appended token's V row goes to its ring slot
                uint4 *dst = reinterpret_cast<uint4 *>(rv + static_cast<size_t>(new_t % L.R) * D + half * (D / 2));
#pragma unroll
                for (int i = 0; i < D / 16; ++i)
                    dst[i] = v[i];
            }
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
            if constexpr (bf) {
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
        float sc[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            sc[j] = (t0 + 4 * q + j < t_end) ? acc0[j] * kscale : -INFINITY;
            sc[4 + j] = (t0 + 16 + 4 * q + j < t_end) ? acc1[j] * kscale : -INFINITY;
        }
        float tmax = fmaxf(fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])),
                           fmaxf(fmaxf(sc[4], sc[5]), fmaxf(sc[6], sc[7])));
        tmax = col_max(tmax);
        const bool need = act && (tmax > m_run + kTau);
        if (__builtin_amdgcn_ballot_w64(need) != 0) {
            const float m_new = need ? tmax : m_run;
            const float alpha = (m_new == m_run) ? 1.0f : exp2f(m_run - m_new);
#pragma unroll
            for (int m = 0; m < MT; ++m)
                O[m] *= alpha;
            l_run *= alpha;
            m_run = m_new;
        }
        const float mo = act ? m_run : INFINITY;
        float p[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            p[j] = weight_exp2(sc[j] - mo);
            l_run += p[j];
        }
        // weights p 2^kWShift (below 2^15) as hi/lo fp16 or three bfloat16 parts
        Frag w1, w2, w3;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float x0 = ldexpf(p[2 * r], kWShift), x1 = ldexpf(p[2 * r + 1], kWShift);
            if constexpr (bf)
                split3_bf16(x0, x1, w1.u[r], w2.u[r], w3.u[r]);
            else
                split_pair(x0, x1, w1.u[r], w2.u[r]);
        }
        // V^T operand of tile m: channel 16m + col, tokens 4q..4q+3 and 16+4q..16+4q+3
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            const uint16_t *row = vt + (16 * m + col) * 32;
            const uint2 lo = *reinterpret_cast<const uint2 *>(row + 4 * q);
            const uint2 hi = *reinterpret_cast<const uint2 *>(row + 16 + 4 * q);
            Frag av;
            av.u[0] = lo.x; av.u[1] = lo.y; av.u[2] = hi.x; av.u[3] = hi.y;
            if constexpr (bf) {
                O[m] = mfma_bf16(av, w1, O[m]);
                O[m] = mfma_bf16(av, w2, O[m]);
                O[m] = mfma_bf16(av, w3, O[m]);
            } else {
                O[m] = mfma(av, w1, O[m]);
                O[m] = mfma(av, w2, O[m]);
            }
        }
    }
    const float Lc = col_sum(l_run);
    asm volatile("" ::: "memory");  // the V tile's last reads stay before the result writes
    if (act) {
#pragma unroll
        for (int m = 0; m < MT; ++m)
            *reinterpret_cast<f4_t *>(po + col * D + 16 * m + 4 * q) =
                f4_t{ldexpf(O[m][0], -kWShift), ldexpf(O[m][1], -kWShift), ldexpf(O[m][2], -kWShift),
                     ldexpf(O[m][3], -kWShift)};
        if (q == 0) {
            pm[col] = m_run;
            pl[col] = Lc;
        }
    }
}

// Waves per SIMD the register allocation must allow: three for the narrow
// pairs (a few bytes of spill at most), two for the wider ones.
template <int KB, int VB>
constexpr int mfma_waves_per_simd() { return 2; }

__host__ __device__ inline int wave_region(const AttnArgs &a)
{
    return mfma_wave_region(a.D, a.g, a.units_q > 0, a.units_r > 0);
}

template <int KB, int VB, int D, bool KT, bool PG, bool PP>
__device__ __forceinline__ void attn_mfma_body(const AttnArgs &a, const RaggedTables *rt)
{
    extern __shared__ float lds[];
    __shared__ float s_pm[kAttnThreads / 64][kMaxG], s_pl[kAttnThreads / 64][kMaxG];
    // the wave index is uniform across the wave: keep it (and everything derived
    // from it) in scalar registers, so that unit bounds and branches are scalar
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    int bh, wx;  // stream, and this workgroup's place among the stream's
    if (a.xcd_shift > 0) {
        const int i = blockIdx.x, k = i >> 3;
        bh = (i & 7) + 8 * (k >> a.xcd_shift);
        wx = k & ((1 << a.xcd_shift) - 1);
    } else {
        bh = blockIdx.y;
        wx = blockIdx.x;
    }
    const int unit = wx * 4 + wave;
    const int region = wave_region(a);
    float *po = lds + wave * region;
    if (unit < a.units_q) {
        mfma_unit<KB, VB, D, KT, PG, PP>(a, rt, bh, unit, lane, po, s_pm[wave], s_pl[wave], po);
    } else if (unit < a.units_q + a.units_r) {
        if (a.kv_bf16)
            mfma_residual_unit<D, true>(a, rt, bh, unit - a.units_q, lane, po, s_pm[wave], s_pl[wave]);
        else
            mfma_residual_unit<D, false>(a, rt, bh, unit - a.units_q, lane, po, s_pm[wave], s_pl[wave]);
    } else if (lane < a.g) {
        s_pm[wave][lane] = -INFINITY;
        s_pl[wave][lane] = 0.0f;
    }
    __syncthreads();
    wg_merge_store<D>(a, bh, wx, lds, region, s_pm, s_pl);
    arrive_and_merge<D>(a, bh, a.mfma_wgs, a.xcd_shift > 0);
}

template <int KB, int VB, int D, bool KT, bool PG, bool PP>
__global__ __launch_bounds__(kAttnThreads, (mfma_waves_per_simd<KB, VB>())) void attn_mfma_kernel(AttnArgs a)
{
    attn_mfma_body<KB, VB, D, KT, PG, PP>(a, nullptr);
}

// ragged batches: per-sequence lengths in the argument block
template <int KB, int VB, int D, bool KT, bool PG, bool PP>
__global__ __launch_bounds__(kAttnThreads, (mfma_waves_per_simd<KB, VB>())) void attn_mfma_kernel_rg(
    RaggedAttnArgs r)
{
    attn_mfma_body<KB, VB, D, KT, PG, PP>(r.a, &r.t);
}

template <int KB, int VB, bool KT, bool PG, bool PP>
hipError_t launch_kernel(const AttnArgs &a, const RaggedTables *rt, hipStream_t st)
{
    const dim3 grid = a.xcd_shift > 0 ? dim3(a.mfma_wgs * a.BH) : dim3(a.mfma_wgs, a.BH);
    const size_t lds = (kAttnThreads / 64) * wave_region(a) * sizeof(float);
    if (rt) {
        const RaggedAttnArgs r{a, *rt};
        hipLaunchKernelGGL((attn_mfma_kernel_rg<KB, VB, KVQ_D, KT, PG, PP>), grid, dim3(kAttnThreads), lds, st, r);
    } else {
        hipLaunchKernelGGL((attn_mfma_kernel<KB, VB, KVQ_D, KT, PG, PP>), grid, dim3(kAttnThreads), lds, st, a);
    }
    return hipGetLastError();
}

// The double-buffered instantiation where the type has one and a window holds
// at most kPipeGroups groups (g > 16 / kPipeGroups); otherwise the plain one
// (separate kernels: the plain walk's code is not affected by the other's).
template <int KB, int VB, bool KT, bool PG>
hipError_t launch_pair(const AttnArgs &a, const RaggedTables *rt, hipStream_t st)
{
    if constexpr (mfma_pipe_ok(KB, VB, KVQ_D, KT)) {
        if (a.pipe && (16 >> a.s_log2) <= kPipeGroups)
            return launch_kernel<KB, VB, KT, PG, true>(a, rt, st);
    }
    return launch_kernel<KB, VB, KT, PG, false>(a, rt, st);
}

}  // namespace

#define KVQ_CAT2(x, y) x##y
#define KVQ_CAT(x, y) KVQ_CAT2(x, y)

hipError_t KVQ_CAT(launch_mfma_d, KVQ_D)(const AttnArgs &a, const RaggedTables *rt, hipStream_t st)
{
    const int kb = a.L.kb, vb = a.L.vb;
    const bool pg = a.L.table != nullptr;  // paged layer: its own instantiation
#define KVQ_PAIR(K, V)                                                        \
    if (kb == K && vb == V)                                                   \
        return pg ? (a.L.k_tok ? launch_pair<K, V, true, true>(a, rt, st) : launch_pair<K, V, false, true>(a, rt, st)) \
                  : (a.L.k_tok ? launch_pair<K, V, true, false>(a, rt, st) : launch_pair<K, V, false, false>(a, rt, st));
    KVQ_PAIR(2, 2) KVQ_PAIR(2, 4) KVQ_PAIR(2, 8)
    KVQ_PAIR(4, 2) KVQ_PAIR(4, 4) KVQ_PAIR(4, 8)
    KVQ_PAIR(8, 2) KVQ_PAIR(8, 4) KVQ_PAIR(8, 8)
#if KVQ_D == 128
    // 3-bit rows: twelve words, three per lane quad (head_dim 256 would need
    // more registers than two waves per SIMD leave)
    if (kb == 3 && vb == 2) return pg ? launch_pair<3, 2, false, true>(a, rt, st) : launch_pair<3, 2, false, false>(a, rt, st);
    if (kb == 3 && vb == 4) return pg ? launch_pair<3, 4, false, true>(a, rt, st) : launch_pair<3, 4, false, false>(a, rt, st);
    if (kb == 3 && vb == 8) return pg ? launch_pair<3, 8, false, true>(a, rt, st) : launch_pair<3, 8, false, false>(a, rt, st);
#endif
#undef KVQ_PAIR
    return hipErrorInvalidValue;
}

}  // namespace kvq
