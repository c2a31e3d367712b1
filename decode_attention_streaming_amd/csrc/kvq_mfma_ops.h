// kvq_mfma_ops.h -- operand building blocks of the matrix-core attention
// kernels (decode and prefill): v_mfma_f32_16x16x32_f16 / _bf16 wrappers,
// fp32 -> fp16 hi/lo (or three-part bfloat16) splits of the fp32 factors,
// code unpacking into exact fp16 integers (KVmix notes, key design 4:
// dequantization folded into the products), the 3-bit Key register map
// (KVmix notes, key design 2), q loads, and row-rotation reductions.
#pragma once

#include "kvq_attn_common.h"

namespace kvq {
namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
union Frag {
    uint32_t u[4];
    half8_t h;
    bf16x8_t b;
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

__device__ __forceinline__ f4_t mfma_bf16(const Frag &a, const Frag &b, f4_t c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.b, b.b, c, 0, 0, 0);
}

// Softmax weight 2^x for x <= kTau: the hardware exp2, without the library's
// rescaling for subnormal results (weights below 2^-126 of the running
// maximum become 0, a relative change far below fp32 rounding of the sums).
__device__ __forceinline__ float weight_exp2(float x)
{
    return __builtin_amdgcn_exp2f(x);
}

// fp32 pair -> three bfloat16 pairs with x ~= p1 + p2 + p3 (truncations; about
// 24 significant bits)
__device__ __forceinline__ void split3_bf16(float x0, float x1, uint32_t &p1, uint32_t &p2, uint32_t &p3)
{
    const uint32_t u0 = __float_as_uint(x0) & 0xFFFF0000u, u1 = __float_as_uint(x1) & 0xFFFF0000u;
    const float r0 = x0 - __uint_as_float(u0), r1 = x1 - __uint_as_float(u1);
    const uint32_t v0 = __float_as_uint(r0) & 0xFFFF0000u, v1 = __float_as_uint(r1) & 0xFFFF0000u;
    const float s0 = r0 - __uint_as_float(v0), s1 = r1 - __uint_as_float(v1);
    p1 = (u0 >> 16) | u1;
    p2 = (v0 >> 16) | v1;
    p3 = (__float_as_uint(s0) >> 16) | (__float_as_uint(s1) & 0xFFFF0000u);
}

// x - (the low / high fp16 half of h2, widened): one mixed-precision FMA
// (exact: h2's half is x rounded toward zero to fp16, so the difference is an
// fp32 number), instead of a conversion and a subtraction
__device__ __forceinline__ float minus_f16_lo(uint32_t h2, float x)
{
    float r;
    asm("v_fma_mix_f32 %0, -%1, 1.0, %2 op_sel_hi:[1,0,0]" : "=v"(r) : "v"(h2), "v"(x));
    return r;
}
__device__ __forceinline__ float minus_f16_hi(uint32_t h2, float x)
{
    float r;
    asm("v_fma_mix_f32 %0, -%1, 1.0, %2 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(r) : "v"(h2), "v"(x));
    return r;
}

// fp32 pair -> (hi, lo) fp16 pairs with x ~= hi + lo
__device__ __forceinline__ void split_pair(float x0, float x1, uint32_t &hi, uint32_t &lo)
{
    const auto h = __builtin_amdgcn_cvt_pkrtz(x0, x1);
    hi = __builtin_bit_cast(uint32_t, h);
    const float r0 = minus_f16_lo(hi, x0);
    const float r1 = minus_f16_hi(hi, x1);
    const auto l = __builtin_amdgcn_cvt_pkrtz(r0, r1);
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

__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t m, uint32_t c)
{
    uint32_t r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "v"(m), "s"(c));
    return r;
}

// Operand register R of a run of b-bit codes (P = 16 / b registers per word):
// the codes in bits b*j and 16 + b*j of word R / P, j = R % P.  A code sitting
// at bit offset e = (b * j) % 8 of its 16-bit half (after a shift by 8 when
// b * j >= 8) is masked into the mantissa of 1024.0 and 1024 is subtracted, both
// exact, leaving the fp16 integer code * 2^e.  The matching factor 2^-e is
// applied to the other operand (class_exp()).
template <int B>
__device__ __forceinline__ constexpr int class_exp(int R)
{
    return (B * (R % (16 / B))) % 8;
}

template <int B, int N>
__device__ __forceinline__ uint32_t code_reg(const uint32_t (&w)[N], const uint32_t (&w8)[N], int R)
{
    constexpr int P = 16 / B;
    const int j = R % P;
    const uint32_t src = (B * j >= 8) ? w8[R / P] : w[R / P];
    const uint32_t mask = (((1u << B) - 1u) << class_exp<B>(R)) * 0x00010001u;
    const uint32_t biased = and_or(src, mask, 0x64006400u);  // 1024 + code * 2^e
    const half2_t k = __builtin_bit_cast(half2_t, biased) - half2_t{1024.0f16, 1024.0f16};
    return __builtin_bit_cast(uint32_t, k);
}

template <int N>
__device__ __forceinline__ void shift8(const uint32_t (&w)[N], uint32_t (&w8)[N])
{
#pragma unroll
    for (int i = 0; i < N; ++i)
        w8[i] = w[i] >> 8;
}

// 3-bit K rows (KVmix notes, key design 2): each word holds channels 11w + j,
// j < 10 as 3-bit codes at bits 3j, and j = 10 as a 2-bit code at bits 30-31.
// Six operand registers per word, each taking one code from each 16-bit half
// at bit offset e <= 7 of that half (registers 3-5 read the word shifted right
// by 8, so that slots 3-5 and 8-10 sit low enough):
//   register  source  lo half (slot, e)  hi half (slot, e)
//   0         w       (0, 0)             (6, 2)
//   1         w       (1, 3)             (7, 5)
//   2         w       (2, 6)             none
//   3         w >> 8  (3, 1)             (8, 0)
//   4         w >> 8  (4, 4)             (9, 3)
//   5         w >> 8  (5, 7)             (10, 6), two bits
__host__ __device__ constexpr int k3_lo_e(int r)
{
    return r == 0 ? 0 : r == 1 ? 3 : r == 2 ? 6 : r == 3 ? 1 : r == 4 ? 4 : 7;
}
__host__ __device__ constexpr int k3_hi_slot(int r)
{
    return r == 0 ? 6 : r == 1 ? 7 : r == 2 ? -1 : r == 3 ? 8 : r == 4 ? 9 : 10;
}
__host__ __device__ constexpr int k3_hi_e(int r)
{
    return r == 0 ? 2 : r == 1 ? 5 : r == 2 ? 0 : r == 3 ? 0 : r == 4 ? 3 : 6;
}
__host__ __device__ constexpr uint32_t k3_mask(int r)
{
    return (7u << k3_lo_e(r)) |
           (k3_hi_slot(r) < 0 ? 0u : ((k3_hi_slot(r) == 10 ? 3u : 7u) << (16 + k3_hi_e(r))));
}

// Operand register R (word R / 6, register R % 6 of the table above) of a
// run of 3-bit K words: fp16 integers code * 2^e in both halves.
template <int N>
__device__ __forceinline__ uint32_t code_reg3(const uint32_t (&w)[N], const uint32_t (&w8)[N], int R)
{
    const int r = R % 6;
    const uint32_t src = r >= 3 ? w8[R / 6] : w[R / 6];
    const uint32_t biased = and_or(src, k3_mask(r), 0x64006400u);
    const half2_t k = __builtin_bit_cast(half2_t, biased) - half2_t{1024.0f16, 1024.0f16};
    return __builtin_bit_cast(uint32_t, k);
}

// The two 16-bit values of a word, widened to fp32: bfloat16 (a shift or a
// mask) or IEEE fp16 (instantiated per format: no per-element select).
template <bool BF>
__device__ __forceinline__ void widen_pair(uint32_t w, float &lo, float &hi)
{
    if constexpr (BF) {
        lo = __uint_as_float(w << 16);
        hi = __uint_as_float(w & 0xFFFF0000u);
    } else {
        lo = __half2float(__ushort_as_half(static_cast<uint16_t>(w & 0xFFFFu)));
        hi = __half2float(__ushort_as_half(static_cast<uint16_t>(w >> 16)));
    }
}

// q values of runs i0 + stride * k, k < K, of 8 consecutive elements (fp32,
// fp16 or bf16; 16-byte aligned): every load is issued before any is used.
template <int K>
__device__ __forceinline__ void load_q_runs(const void *q, int dtype, size_t i0, int stride, float (&r)[K][8])
{
    if (dtype == 0) {
        float4 v[K][2];
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const float4 *p = reinterpret_cast<const float4 *>(static_cast<const float *>(q) + i0 + stride * k);
            v[k][0] = p[0];
            v[k][1] = p[1];
        }
#pragma unroll
        for (int k = 0; k < K; ++k) {
            r[k][0] = v[k][0].x; r[k][1] = v[k][0].y; r[k][2] = v[k][0].z; r[k][3] = v[k][0].w;
            r[k][4] = v[k][1].x; r[k][5] = v[k][1].y; r[k][6] = v[k][1].z; r[k][7] = v[k][1].w;
        }
    } else {
        uint4 v[K];
#pragma unroll
        for (int k = 0; k < K; ++k)
            v[k] = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(q) + i0 + stride * k);
        if (dtype == 2) {
#pragma unroll
            for (int k = 0; k < K; ++k) {
                const uint32_t w[4] = {v[k].x, v[k].y, v[k].z, v[k].w};
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    widen_pair<true>(w[j], r[k][2 * j], r[k][2 * j + 1]);
            }
        } else {
#pragma unroll
            for (int k = 0; k < K; ++k) {
                const uint32_t w[4] = {v[k].x, v[k].y, v[k].z, v[k].w};
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    widen_pair<false>(w[j], r[k][2 * j], r[k][2 * j + 1]);
            }
        }
    }
}

// v of the lane R columns away in the same 16-lane row (row rotation)
template <int R>
__device__ __forceinline__ float row_ror(float v)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x120 + R, 0xF, 0xF, true));
}

// Sum (or max) over the columns h, h + S, h + 2S, ... of each row, left in
// every one of them (S a compile-time power of two: no branches).
template <int S>
__device__ __forceinline__ float coset_sum(float v)
{
    if constexpr (S <= 8)
        v += row_ror<8>(v);
    if constexpr (S <= 4)
        v += row_ror<4>(v);
    if constexpr (S <= 2)
        v += row_ror<2>(v);
    if constexpr (S <= 1)
        v += row_ror<1>(v);
    return v;
}

template <int S>
__device__ __forceinline__ float coset_max(float v)
{
    if constexpr (S <= 8)
        v = fmaxf(v, row_ror<8>(v));
    if constexpr (S <= 4)
        v = fmaxf(v, row_ror<4>(v));
    if constexpr (S <= 2)
        v = fmaxf(v, row_ror<2>(v));
    if constexpr (S <= 1)
        v = fmaxf(v, row_ror<1>(v));
    return v;
}

}  // namespace
}  // namespace kvq
