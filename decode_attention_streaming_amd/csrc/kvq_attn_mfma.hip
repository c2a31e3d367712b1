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
// kv-head, NG = 16 / g consecutive groups are processed per window, column
// j*g + h carrying head h over the tokens of group j.  Every column keeps its
// own online-softmax state, so each lane's B operand is useful and no data
// moves between the two products; the NG columns of a head are merged at the
// end of the unit.  Query heads of a GQA group share every K/V read (KIVI
// notes, section 7.2).
#include "kvq_attn_common.h"

#ifndef KVQ_D
#error "KVQ_D (head_dim) must be defined"
#endif

namespace kvq {
namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float f4_t __attribute__((ext_vector_type(4)));

union Frag {
    uint32_t u[4];
    half8_t h;
};

// Lazy rescale threshold (log2 units): the running max only moves when a score
// exceeds it by more than this, so softmax weights stay below 2^kTau.
constexpr float kTau = 8.0f;
// P.V weights p s are scaled to p s 2^(kWShift - E) with s < 2^E: below
// 2^(kTau + kWShift) = 2^15, inside fp16 range, and far above fp16's
// subnormal floor, whose one-sided rounding error the z-term cancellation
// would otherwise amplify.
constexpr int kWShift = 7;

__device__ __forceinline__ f4_t mfma(const Frag &a, const Frag &b, f4_t c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a.h, b.h, c, 0, 0, 0);
}

// fp32 pair -> (hi, lo) fp16 pairs with x ~= hi + lo
__device__ __forceinline__ void split_pair(float x0, float x1, uint32_t &hi, uint32_t &lo)
{
    const auto h = __builtin_amdgcn_cvt_pkrtz(x0, x1);
    const float r0 = x0 - static_cast<float>(h[0]);
    const float r1 = x1 - static_cast<float>(h[1]);
    const auto l = __builtin_amdgcn_cvt_pkrtz(r0, r1);
    hi = __builtin_bit_cast(uint32_t, h);
    lo = __builtin_bit_cast(uint32_t, l);
}

template <int N>
__device__ __forceinline__ void load_words(const uint32_t *p, uint32_t (&r)[N])
{
    if constexpr (N % 4 == 0) {
#pragma unroll
        for (int i = 0; i < N; i += 4) {
            const uint4 v = *reinterpret_cast<const uint4 *>(p + i);
            r[i] = v.x;
            r[i + 1] = v.y;
            r[i + 2] = v.z;
            r[i + 3] = v.w;
        }
    } else if constexpr (N == 2) {
        const uint2 v = *reinterpret_cast<const uint2 *>(p);
        r[0] = v.x;
        r[1] = v.y;
    } else {
#pragma unroll
        for (int i = 0; i < N; ++i)
            r[i] = p[i];
    }
}

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

// Register R of an unpacked code run: codes of 2 channels (or slots) as fp16
// integers in the two halves.
template <int B, int N>
__device__ __forceinline__ uint32_t code_reg(const uint32_t (&w)[N], int R)
{
    constexpr int P = 16 / B;
    constexpr uint32_t M = ((1u << B) - 1u) * 0x00010001u;
    const uint32_t biased = ((w[R / P] >> (B * (R % P))) & M) | 0x64006400u;  // 1024 + k
    const half2_t k = __builtin_bit_cast(half2_t, biased) - half2_t{1024.0f16, 1024.0f16};
    return __builtin_bit_cast(uint32_t, k);
}

__device__ __forceinline__ float xor_sum(float v)
{
    v += __shfl_xor(v, 16, 64);
    v += __shfl_xor(v, 32, 64);
    return v;
}

__device__ __forceinline__ float xor_max(float v)
{
    v = fmaxf(v, __shfl_xor(v, 16, 64));
    v = fmaxf(v, __shfl_xor(v, 32, 64));
    return v;
}

template <int KB, int VB, int D>
__device__ void mfma_unit(const AttnArgs &a, int bh, int unit, int lane)
{
    constexpr int NC = D / 32;          // 32-channel chunks of q.K
    constexpr int QC = D / 4;           // channels owned by one lane quad
    constexpr int KW = D * KB / 128;    // K words per lane per token
    constexpr int PK = 16 / KB;         // K code pairs per word
    constexpr int CW = 32 / KB;         // K channels per word
    constexpr int FW = D * VB / 64;     // V words per lane per 32-token block
    constexpr int MT = D / 16;          // 16-channel tiles of P.V

    const LayerDev &L = a.L;
    const int G = L.G, g = a.g;
    const int col = lane & 15, q = lane >> 4;
    const int NG = 16 / g;
    const bool used = col < NG * g;
    const int h = used ? col % g : 0;
    const int jslot = used ? col / g : NG;
    const int b = bh / a.Hkv, kvh = bh % a.Hkv;
    const int n_groups = a.Tq / G;
    const int g_beg = unit * a.unit_groups;
    const int g_end = min(g_beg + a.unit_groups, n_groups);
    const int t_unit = g_beg * G;
    const int nblk = (g_end - g_beg) * G / 32;
    const int win_tokens = NG * G;

    const size_t q_base = (static_cast<size_t>(b) * a.Hkv * g + kvh * g + h) * D + q * QC;
    const uint32_t *kw_base = L.k_words + static_cast<size_t>(bh) * L.capq * L.wk + q * KW;
    const float *km_base = L.k_meta + static_cast<size_t>(bh) * (L.capq / G) * 2 * D + q * QC;
    const uint32_t *vw_base = L.v_words + static_cast<size_t>(bh) * L.capq * L.wv + lane * FW;
    const float *vm_base = L.v_meta + static_cast<size_t>(bh) * L.capq * 2;

    // block data: K rows of both 16-token tiles, V fragment, V meta of 8 tokens
    uint32_t kr0[KW], kr1[KW], vf[FW];
    float4 vm[4];
    auto load_block = [&](int t0) {
        load_words(kw_base + static_cast<size_t>(t0 + col) * L.wk, kr0);
        load_words(kw_base + static_cast<size_t>(t0 + 16 + col) * L.wk, kr1);
        load_words(vw_base + static_cast<size_t>(t0) * L.wv, vf);
        const float4 *m0 = reinterpret_cast<const float4 *>(vm_base + static_cast<size_t>(t0 + 4 * q) * 2);
        const float4 *m1 = reinterpret_cast<const float4 *>(vm_base + static_cast<size_t>(t0 + 16 + 4 * q) * 2);
        vm[0] = m0[0];
        vm[1] = m0[1];
        vm[2] = m1[0];
        vm[3] = m1[1];
    };
    load_block(t_unit);

    float m_run = -INFINITY, l_run = 0.0f, zb_run = 0.0f;
    int E = -1000;  // running V-scale exponent: all weights are scaled by 2^-E
    f4_t O[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m)
        O[m] = f4_t{0.0f, 0.0f, 0.0f, 0.0f};

    Frag bhi[NC], blo[NC];
    float bias = 0.0f;
    int kexp = 0;
    int w_first = t_unit;  // first token of the current window
    bool act_win = false;

    for (int bi = 0; bi < nblk; ++bi) {
        const int t0 = t_unit + bi * 32;
        if ((t0 - t_unit) % win_tokens == 0) {
            // ---- new window: B operand of q.K for this lane's column, q * s as hi/lo fp16 ----
            w_first = t0;
            const int w0 = t0 / G;
            const int nwin = min(NG, g_end - w0);
            act_win = jslot < nwin;
            const int gi = w0 + (act_win ? jslot : 0);
            const float *sp = km_base + static_cast<size_t>(gi) * 2 * D;
            const float *zp = sp + D;
            float qs[QC];
            float amax = 0.0f;
            bias = 0.0f;
#pragma unroll
            for (int i = 0; i < QC; i += 4) {
                const float4 s4 = *reinterpret_cast<const float4 *>(sp + i);
                const float4 z4 = *reinterpret_cast<const float4 *>(zp + i);
                const float sv[4] = {s4.x, s4.y, s4.z, s4.w};
                const float zv[4] = {z4.x, z4.y, z4.z, z4.w};
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const float qq = act_win ? load_q(a.q, a.q_dtype, q_base + i + k) * a.scale_log2 : 0.0f;
                    qs[i + k] = qq * sv[k];
                    bias = __builtin_fmaf(qq, zv[k], bias);
                    amax = fmaxf(amax, fabsf(qs[i + k]));
                }
            }
            bias = xor_sum(bias);
            amax = xor_max(amax);
            const int sexp = amax > 0.0f ? __builtin_amdgcn_frexp_expf(amax) : 0;
            const int sh = 14 - sexp;  // |q s| * 2^sh < 2^14
#pragma unroll
            for (int k = 0; k < NC; ++k) {
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    const int R = 4 * k + p;
                    const int clo = (R / PK) * CW + (R % PK), chi = clo + PK;
                    split_pair(ldexpf(qs[clo], sh), ldexpf(qs[chi], sh), bhi[k].u[p], blo[k].u[p]);
                }
            }
            kexp = -sh;  // acc * 2^-sh
        }
        const int slot = (t0 - w_first) / G;
        const bool act = act_win && jslot == slot;

        // take this block's data, then start loading the next block
        uint32_t k0[KW], k1[KW], v[FW];
#pragma unroll
        for (int i = 0; i < KW; ++i) {
            k0[i] = kr0[i];
            k1[i] = kr1[i];
        }
#pragma unroll
        for (int i = 0; i < FW; ++i)
            v[i] = vf[i];
        const float vs[8] = {vm[0].x, vm[0].z, vm[1].x, vm[1].z, vm[2].x, vm[2].z, vm[3].x, vm[3].z};
        const float vz[8] = {vm[0].y, vm[0].w, vm[1].y, vm[1].w, vm[2].y, vm[2].w, vm[3].y, vm[3].w};
        if (bi + 1 < nblk)
            load_block(t0 + 32);

        // q.K for tokens t0 + 4q + j (acc0) and t0 + 16 + 4q + j (acc1)
        f4_t acc0 = {0.0f, 0.0f, 0.0f, 0.0f}, acc1 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int k = 0; k < NC; ++k) {
            Frag a0, a1;
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                a0.u[p] = code_reg<KB>(k0, 4 * k + p);
                a1.u[p] = code_reg<KB>(k1, 4 * k + p);
            }
            acc0 = mfma(a0, bhi[k], acc0);
            acc0 = mfma(a0, blo[k], acc0);
            acc1 = mfma(a1, bhi[k], acc1);
            acc1 = mfma(a1, blo[k], acc1);
        }
        float sc[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            sc[j] = ldexpf(acc0[j], kexp) + bias;
            sc[4 + j] = ldexpf(acc1[j], kexp) + bias;
        }
        float tmax = sc[0];
#pragma unroll
        for (int j = 1; j < 8; ++j)
            tmax = fmaxf(tmax, sc[j]);
        tmax = xor_max(tmax);
        int eb = -1000;
#pragma unroll
        for (int j = 0; j < 8; ++j)
            if (vs[j] > 0.0f)
                eb = max(eb, __builtin_amdgcn_frexp_expf(vs[j]));
        eb = max(eb, __shfl_xor(eb, 16, 64));
        eb = max(eb, __shfl_xor(eb, 32, 64));
        eb = __builtin_amdgcn_readfirstlane(eb);
        const bool need = act && (tmax > m_run + kTau);
        if (__builtin_amdgcn_ballot_w64(need) != 0 || eb > E) {
            const float m_new = need ? tmax : m_run;
            const int E_new = max(E, eb);
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
        float p[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            p[j] = act ? exp2f(sc[j] - m_run) : 0.0f;
            l_run += p[j];
            zb_run = __builtin_fmaf(p[j], vz[j], zb_run);
        }
        // B operand of P.V: weights p s 2^(kWShift - E), k-slot pairs (0,1) (2,3) (4,5) (6,7)
        Frag whi, wlo;
        const int wsh = kWShift - E;
#pragma unroll
        for (int r = 0; r < 4; ++r)
            split_pair(ldexpf(p[2 * r] * vs[2 * r], wsh), ldexpf(p[2 * r + 1] * vs[2 * r + 1], wsh),
                       whi.u[r], wlo.u[r]);
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            Frag av;
#pragma unroll
            for (int r = 0; r < 4; ++r)
                av.u[r] = code_reg<VB>(v, 4 * m + r);
            O[m] = mfma(av, whi, O[m]);
            O[m] = mfma(av, wlo, O[m]);
        }
    }

    // ---- finish: per column totals, then merge the NG columns of each head ----
    // this lane's column: l, z-term and o (weights carry 2^(kWShift - E))
    const float Lcol = xor_sum(l_run);
    const float ZB = xor_sum(zb_run);
    float ocol[MT][4];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            ocol[m][j] = ldexpf(O[m][j], E - kWShift) + ZB;
    // head h = col (col < g) gathers the unmerged columns j*g + h, j = 1..NG-1
    float M = m_run, Lc = Lcol;
    float oc[MT][4];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            oc[m][j] = ocol[m][j];
    for (int jn = 1; jn < NG; ++jn) {
        const int src = ((col + jn * g) & 15) + 16 * q;
        const float m2 = __shfl(m_run, src, 64);
        const float L2 = __shfl(Lcol, src, 64);
        const float Mn = fmaxf(M, m2);
        const float a1 = (M == Mn) ? 1.0f : exp2f(M - Mn);
        const float a2 = (m2 == Mn) ? 1.0f : exp2f(m2 - Mn);
        Lc = Lc * a1 + L2 * a2;
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float o2 = __shfl(ocol[m][j], src, 64);
                oc[m][j] = oc[m][j] * a1 + o2 * a2;
            }
        M = Mn;
    }
    if (col < g) {
        const int ps = part_stride(D);
        float *part = a.part + ((static_cast<size_t>(bh) * a.n_part + unit) * g + col) * ps;
#pragma unroll
        for (int m = 0; m < MT; ++m)
            *reinterpret_cast<float4 *>(part + 16 * m + 4 * q) =
                make_float4(oc[m][0], oc[m][1], oc[m][2], oc[m][3]);
        if (q == 0) {
            part[D] = M;
            part[D + 1] = Lc;
        }
    }
}

template <int KB, int VB, int D>
__global__ __launch_bounds__(kAttnThreads) void attn_mfma_kernel(AttnArgs a)
{
    const int bh = blockIdx.y, wg = blockIdx.x;
    if (wg < a.mfma_wgs) {
        const int unit = wg * 4 + (threadIdx.x >> 6);
        if (unit < a.units_q)
            mfma_unit<KB, VB, D>(a, bh, unit, threadIdx.x & 63);
    } else {
        const int r = wg - a.mfma_wgs;
        const int t_beg = a.valu_beg + r * a.valu_tps;
        const int t_end = min(a.N, t_beg + a.valu_tps);
        extern __shared__ float smem[];
        if (a.g <= 4)
            valu_range<D, 4>(a, bh, t_beg, t_end, a.units_q + r, smem);
        else if (a.g <= 8)
            valu_range<D, 8>(a, bh, t_beg, t_end, a.units_q + r, smem);
        else
            valu_range<D, 16>(a, bh, t_beg, t_end, a.units_q + r, smem);
    }
    arrive_and_merge(a, bh, gridDim.x);
}

template <int KB, int VB>
hipError_t launch_pair(const AttnArgs &a, hipStream_t st)
{
    dim3 grid(a.mfma_wgs + a.valu_wgs, a.BH);
    const size_t lds = a.valu_wgs > 0 ? valu_lds_bytes(a.g, a.D) : 0;
    hipLaunchKernelGGL((attn_mfma_kernel<KB, VB, KVQ_D>), grid, dim3(kAttnThreads), lds, st, a);
    return hipGetLastError();
}

}  // namespace

#define KVQ_CAT2(x, y) x##y
#define KVQ_CAT(x, y) KVQ_CAT2(x, y)

hipError_t KVQ_CAT(launch_mfma_d, KVQ_D)(const AttnArgs &a, hipStream_t st)
{
    const int kb = a.L.kb, vb = a.L.vb;
#define KVQ_PAIR(K, V)                 \
    if (kb == K && vb == V)            \
        return launch_pair<K, V>(a, st);
    KVQ_PAIR(2, 2) KVQ_PAIR(2, 4) KVQ_PAIR(2, 8)
    KVQ_PAIR(4, 2) KVQ_PAIR(4, 4) KVQ_PAIR(4, 8)
    KVQ_PAIR(8, 2) KVQ_PAIR(8, 4) KVQ_PAIR(8, 8)
#undef KVQ_PAIR
    return hipErrorInvalidValue;
}

}  // namespace kvq
