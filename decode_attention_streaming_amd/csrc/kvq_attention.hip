// kvq_attention.hip -- split-sequence decode attention over the quantized
// cache, vector-ALU variant, plus the log-sum-exp merge of split partials.
//
// o = softmax(q K^T / sqrt(D)) V for one query token per sequence (KVTuner
// summary, A3 attention equation), K and V dequantized on the fly inside the
// dot products (KVmix notes, key design 4), the query heads of one GQA group
// sharing each K/V read (KIVI notes, section 7.2).  Quantized tokens are
// x^ = code * s + z; recent tokens are read in their 16-bit format.
//
// The vector-ALU kernel serves every bit width, including the 11-per-word
// 3-bit Key layout.  One workgroup handles one split of one (sequence, kv-head)
// stream, 256 tokens per tile: one thread per token for the scores, then one
// thread per (channel, head slot) for P.V with the value scale folded into the
// probability (sum_t p_t (c_t s_t + z_t) = sum_t (p_t s_t) c_t + sum_t p_t z_t).
#include "kvq_internal.h"

#include <hip/hip_bf16.h>
#include <hip/hip_fp16.h>

namespace kvq {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxG = 16;

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

// Code of channel c in a packed row.
__device__ __forceinline__ uint32_t code_at(const uint32_t *row, int bits, int c)
{
    if (bits == 3) {
        const int sl = c % 11;
        return (row[c / 11] >> (3 * sl)) & (sl == 10 ? 3u : 7u);
    }
    const int bitpos = c * bits;
    return (row[bitpos >> 5] >> (bitpos & 31)) & ((1u << bits) - 1u);
}

template <int GM>
__global__ __launch_bounds__(kThreads) void attn_valu_kernel(AttnArgs a)
{
    const int split = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int D = a.D, g = a.g;
    const int b = bh / a.Hkv, kvh = bh % a.Hkv;
    const int t_beg = split * a.tps;
    const int t_end = min(a.N, t_beg + a.tps);
    const LayerDev &L = a.L;

    __shared__ float q_l[kMaxG][256];
    __shared__ float p_l[kMaxG][kThreads];
    __shared__ float red[3][4][kMaxG];

    for (int i = tid; i < g * D; i += kThreads) {
        const int h = i / D, c = i % D;
        const size_t qi = (static_cast<size_t>(b) * a.Hkv * g + kvh * g + h) * D + c;
        q_l[h][c] = load_q(a.q, a.q_dtype, qi) * a.scale_log2;
    }
    __syncthreads();

    // Output slots of this thread: channel oc, heads oh0, oh0 + hstep, ...
    const int oc = tid % D, oh0 = tid / D, hstep = kThreads / D;
    float o[GM], m[GM], l[GM];
#pragma unroll
    for (int k = 0; k < GM; ++k) {
        o[k] = 0.0f;
        m[k] = -INFINITY;
        l[k] = 0.0f;
    }

    const int ngcap = L.capq / L.G;
    for (int tile = t_beg; tile < t_end; tile += kThreads) {
        const int t = tile + tid;
        const bool valid = t < t_end;
        float sc[GM];
#pragma unroll
        for (int h = 0; h < GM; ++h)
            sc[h] = 0.0f;
        float vs = 1.0f, vz = 0.0f;
        if (valid) {
            if (t < a.Tq) {
                const float *ks = L.k_meta + (static_cast<size_t>(bh) * ngcap + t / L.G) * 2 * D;
                const float *kz = ks + D;
                const uint32_t *row = L.k_words + (static_cast<size_t>(bh) * L.capq + t) * L.wk;
                for (int c = 0; c < D; ++c) {
                    const float x = __builtin_fmaf(static_cast<float>(code_at(row, L.kb, c)), ks[c], kz[c]);
#pragma unroll
                    for (int h = 0; h < GM; ++h)
                        if (h < g)
                            sc[h] = __builtin_fmaf(q_l[h][c], x, sc[h]);
                }
                const float *vm = L.v_meta + (static_cast<size_t>(bh) * L.capq + t) * 2;
                vs = vm[0];
                vz = vm[1];
            } else {
                const uint16_t *row = L.ring_k + (static_cast<size_t>(bh) * L.R + t % L.R) * D;
                for (int c = 0; c < D; ++c) {
                    const float x = widen16(row[c], a.kv_bf16);
#pragma unroll
                    for (int h = 0; h < GM; ++h)
                        if (h < g)
                            sc[h] = __builtin_fmaf(q_l[h][c], x, sc[h]);
                }
            }
        }
        // tile maximum per head
#pragma unroll
        for (int h = 0; h < GM; ++h) {
            if (h < g) {
                const float w = wave_max(valid ? sc[h] : -INFINITY);
                if (lane == 0)
                    red[0][wave][h] = w;
            }
        }
        __syncthreads();
        float alpha[GM], mnew[GM];
#pragma unroll
        for (int h = 0; h < GM; ++h) {
            if (h < g) {
                const float tm = fmaxf(fmaxf(red[0][0][h], red[0][1][h]), fmaxf(red[0][2][h], red[0][3][h]));
                mnew[h] = fmaxf(m[h], tm);
                alpha[h] = exp2f(m[h] - mnew[h]);
                const float p = valid ? exp2f(sc[h] - mnew[h]) : 0.0f;
                p_l[h][tid] = p * vs;
                const float ps = wave_sum(p), pz = wave_sum(p * vz);
                if (lane == 0) {
                    red[1][wave][h] = ps;
                    red[2][wave][h] = pz;
                }
            }
        }
        __syncthreads();
#pragma unroll
        for (int h = 0; h < GM; ++h) {
            if (h < g) {
                l[h] = l[h] * alpha[h] + (red[1][0][h] + red[1][1][h] + red[1][2][h] + red[1][3][h]);
                m[h] = mnew[h];
            }
        }
        // P.V: this thread's channel for each of its head slots
        float zb[GM];
#pragma unroll
        for (int k = 0; k < GM; ++k) {
            const int h = oh0 + k * hstep;
            if (h < g) {
                zb[k] = red[2][0][h] + red[2][1][h] + red[2][2][h] + red[2][3][h];
                o[k] = o[k] * alpha[h] + zb[k];
            }
        }
        const int ntile = min(kThreads, t_end - tile);
        for (int i = 0; i < ntile; ++i) {
            const int tt = tile + i;
            float x;
            if (tt < a.Tq)
                x = static_cast<float>(
                    code_at(L.v_words + (static_cast<size_t>(bh) * L.capq + tt) * L.wv, L.vb, oc));
            else
                x = widen16(L.ring_v[(static_cast<size_t>(bh) * L.R + tt % L.R) * D + oc], a.kv_bf16);
#pragma unroll
            for (int k = 0; k < GM; ++k) {
                const int h = oh0 + k * hstep;
                if (h < g)
                    o[k] = __builtin_fmaf(p_l[h][i], x, o[k]);
            }
        }
        __syncthreads();
    }

    // partials: o[D], m, l per (split, head)
    float *part = a.part + (static_cast<size_t>(bh) * a.n_splits + split) * g * (D + 2);
#pragma unroll
    for (int k = 0; k < GM; ++k) {
        const int h = oh0 + k * hstep;
        if (h < g) {
            part[h * (D + 2) + oc] = o[k];
            if (oc == 0) {
                part[h * (D + 2) + D] = m[h];
                part[h * (D + 2) + D + 1] = l[h];
            }
        }
    }
}

// out[b, hq, :] = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s, M = max_s m_s.
__global__ __launch_bounds__(kThreads) void merge_kernel(AttnArgs a)
{
    const int bh = blockIdx.x;
    const int D = a.D, g = a.g, S = a.n_splits;
    const int b = bh / a.Hkv, kvh = bh % a.Hkv;
    const float *part = a.part + static_cast<size_t>(bh) * S * g * (D + 2);
    for (int i = threadIdx.x; i < g * D; i += kThreads) {
        const int h = i / D, c = i % D;
        float M = -INFINITY;
        for (int s = 0; s < S; ++s)
            M = fmaxf(M, part[(s * g + h) * (D + 2) + D]);
        float num = 0.0f, den = 0.0f;
        for (int s = 0; s < S; ++s) {
            const float *ps = part + (s * g + h) * (D + 2);
            const float w = exp2f(ps[D] - M);
            num = __builtin_fmaf(w, ps[c], num);
            den = __builtin_fmaf(w, ps[D + 1], den);
        }
        a.out[(static_cast<size_t>(b) * a.Hkv * g + kvh * g + h) * D + c] = num / den;
    }
}

}  // namespace

hipError_t launch_attention_valu(const AttnArgs &a, hipStream_t st)
{
    dim3 grid(a.n_splits, a.BH);
    if (a.g <= 1)
        hipLaunchKernelGGL(attn_valu_kernel<1>, grid, dim3(kThreads), 0, st, a);
    else if (a.g <= 2)
        hipLaunchKernelGGL(attn_valu_kernel<2>, grid, dim3(kThreads), 0, st, a);
    else if (a.g <= 4)
        hipLaunchKernelGGL(attn_valu_kernel<4>, grid, dim3(kThreads), 0, st, a);
    else if (a.g <= 8)
        hipLaunchKernelGGL(attn_valu_kernel<8>, grid, dim3(kThreads), 0, st, a);
    else
        hipLaunchKernelGGL(attn_valu_kernel<16>, grid, dim3(kThreads), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_merge(const AttnArgs &a, hipStream_t st)
{
    hipLaunchKernelGGL(merge_kernel, dim3(a.BH), dim3(kThreads), 0, st, a);
    return hipGetLastError();
}

}  // namespace kvq
