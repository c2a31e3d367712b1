// kvq_append.hip -- streaming quantize-and-append kernels for gfx950.
//
// Key is quantized per channel over a group of G tokens, Value per token, each
// with an fp32 scale s = (max - min) / qmax and zero z = min, codes
// round-half-even((x - z) / s) clamped to [0, qmax] (KVTuner summary, A3 "KV
// cache quantization basics"; KVmix notes, key design 2; KIVI notes, sections
// 6.1-6.2).  Codes are packed into 32-bit words, least significant bits first;
// the 3-bit Key layout puts eleven channels in a word, slot 10 at 2 bits
// (KVmix notes, key design 2).  Quantizing straight into the packed history
// follows KVmix key design 4.
//
// One workgroup quantizes the K half, another the V half of one group of one
// stream.  The group's 16-bit tile is staged in LDS with 16-byte loads; K is
// reduced per channel (min/max over the G tokens), or per token in the
// per-token-asym Key mode (KVTuner summary: the KIVI and per-token-asym
// modes), V per token (min/max over head_dim, a few threads per token); then
// the codes are packed.
//
// Bit-exactness with a serial CPU evaluation: min/max are exact in any order;
// the subtraction and the IEEE fp32 division are correctly rounded (no fast
// math, no contraction); rintf is round-half-even; zero scales and zero points
// are stored as +0.
#include <hip/hip_fp16.h>

#include "kvq_internal.h"
#include "kvq_layout.h"

namespace kvq {
namespace {

constexpr int kThreads = 256;
constexpr int kTileElems = 16384;  // 16-bit elements of one staged G x D tile

__device__ __forceinline__ float widen16(uint16_t x, int bf16)
{
    if (bf16)
        return __uint_as_float(static_cast<uint32_t>(x) << 16);
    return __half2float(__ushort_as_half(x));
}

__device__ __forceinline__ int qmax_of(int bits, int c)
{
    if (bits == 3)
        return (c % 11 == 10) ? 3 : 7;
    return (1 << bits) - 1;
}

// Code of x for a group with minimum mn and scale s.
__device__ __forceinline__ uint32_t code_of(float x, float mn, float s, int qmax)
{
#pragma clang fp contract(off)
    if (s == 0.0f)
        return 0u;
    float r = rintf((x - mn) / s);
    r = fminf(fmaxf(r, 0.0f), static_cast<float>(qmax));
    return static_cast<uint32_t>(r);
}

__device__ __forceinline__ const uint16_t *src_row(const FlushArgs &a, const uint16_t *ring,
                                                   const uint16_t *fresh, int bh, int t)
{
    if (t < a.N0)
        return ring + (static_cast<size_t>(bh) * a.L.R + (t % a.L.R)) * a.D;
    return fresh + (static_cast<size_t>(bh) * a.n_new + (t - a.N0)) * a.D;
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Copy the G x D tile of tokens [t0, t0 + G) into LDS, in passes of two
// 16-byte chunks per thread: a pass issues both loads before storing either
// (one memory round trip per pass; one pass covers G x D = 4096).  The chunks
// are native vectors, so they stay in registers (an array of the struct-based
// vector type was kept in scratch memory, which made each load wait for the
// one before).  D is a power of two: row and chunk by shifts.
__device__ __forceinline__ void stage(const FlushArgs &a, const uint16_t *ring, const uint16_t *fresh,
                                      int bh, int t0, uint16_t *tile)
{
    const int D = a.D, cs = __builtin_ctz(static_cast<unsigned>(D / 8)), n = a.L.G << cs;
    const int cmask = (1 << cs) - 1;
    for (int base = 0; base < n; base += 2 * kThreads) {
        const int i0 = base + threadIdx.x, i1 = i0 + kThreads;
        u32x4 v0 = u32x4{0u, 0u, 0u, 0u}, v1 = v0;
        if (i0 < n)
            v0 = *reinterpret_cast<const u32x4 *>(src_row(a, ring, fresh, bh, t0 + (i0 >> cs)) + (i0 & cmask) * 8);
        if (i1 < n)
            v1 = *reinterpret_cast<const u32x4 *>(src_row(a, ring, fresh, bh, t0 + (i1 >> cs)) + (i1 & cmask) * 8);
        if (i0 < n)
            *reinterpret_cast<u32x4 *>(tile + (i0 >> cs) * D + (i0 & cmask) * 8) = v0;
        if (i1 < n)
            *reinterpret_cast<u32x4 *>(tile + (i1 >> cs) * D + (i1 & cmask) * 8) = v1;
    }
}

// Per-token min / max over the D channels of the G staged tokens, tpt threads
// per token; scale s = (max - min) / qmax and minimum of token i go to s_c[i]
// and mn_c[i] (G <= 256) and, as the pair (scale, zero), to meta[2 i].
__device__ __forceinline__ void token_scales(const uint16_t *tile, int G, int D, int bf, int qmax, float *meta,
                                             float *s_c, float *mn_c, float *red_mn, float *red_mx)
{
#pragma clang fp contract(off)
    const int tid = threadIdx.x;
    const int tpt = G <= kThreads ? kThreads / G : 1;  // threads per token
    for (int i0 = 0; i0 < G; i0 += kThreads / tpt) {
        const int i = i0 + tid / tpt, sub = tid % tpt;
        float vmn = INFINITY, vmx = -INFINITY;
        if (i < G && tid / tpt < kThreads / tpt) {
            for (int cc = sub; cc < D; cc += tpt) {
                const float x = widen16(tile[i * D + cc], bf);
                vmn = fminf(vmn, x);
                vmx = fmaxf(vmx, x);
            }
        }
        __syncthreads();  // red_* of the previous pass are consumed
        red_mn[tid] = vmn;
        red_mx[tid] = vmx;
        __syncthreads();
        if (i < G && sub == 0 && tid / tpt < kThreads / tpt) {
            for (int r = 1; r < tpt; ++r) {
                vmn = fminf(vmn, red_mn[tid + r]);
                vmx = fmaxf(vmx, red_mx[tid + r]);
            }
            const float s = (vmx - vmn) / static_cast<float>(qmax);
            s_c[i % 256] = s;
            mn_c[i % 256] = vmn;
            meta[2 * i] = (s == 0.0f) ? 0.0f : s;
            meta[2 * i + 1] = (vmn == 0.0f) ? 0.0f : vmn;
        }
    }
    __syncthreads();
}

// One workgroup per (group, stream, K or V): the K and V halves of a group
// are independent and run side by side.
__global__ __launch_bounds__(kThreads) void flush_kernel(FlushArgs a)
{
#pragma clang fp contract(off)
    const int j = blockIdx.x, bh = blockIdx.y, is_v = blockIdx.z, tid = threadIdx.x;
    const int D = a.D, G = a.L.G;
    const int t0 = a.Tq0 + j * G;
    const int gi = t0 / G;
    const int bf = a.kv_bf16;
    const QAddr qa(a.L, bh);  // rows of the group's tokens (one page when paged)
    const size_t row0 = qa.row(t0);

    __shared__ uint16_t tile[kTileElems];
    __shared__ float red_mn[kThreads], red_mx[kThreads];
    __shared__ float s_c[256], mn_c[256];

    if (!is_v && a.L.k_tok) {
        // ---- Key, per-token asymmetric: one scale and zero per token ----
        stage(a, a.L.ring_k, a.k_new, bh, t0, tile);
        __syncthreads();
        const int kb = a.L.kb, kq = (1 << kb) - 1, wk = a.L.wk;
        token_scales(tile, G, D, bf, kq, a.L.k_meta + row0 * 2, s_c, mn_c,
                     red_mn, red_mx);
        const int epw = 32 / kb;
        for (int it = tid; it < G * wk; it += kThreads) {
            const int i = it / wk, w = it % wk;
            uint32_t word = 0;
            for (int sl = 0; sl < epw; ++sl) {
                const int cc = w * epw + sl;
                word |= code_of(widen16(tile[i * D + cc], bf), mn_c[i], s_c[i], kq) << (kb * sl);
            }
            a.L.k_words[(row0 + i) * wk + w] = word;
        }
    } else if (!is_v) {
        // ---- Key: min / max per channel over the G tokens ----
        stage(a, a.L.ring_k, a.k_new, bh, t0, tile);
        __syncthreads();
        const int parts = kThreads / D;  // threads per channel (D divides 256)
        const int c = tid % D, p = tid / D;
        float mn = INFINITY, mx = -INFINITY;
        for (int i = p; i < G; i += parts) {
            const float x = widen16(tile[i * D + c], bf);
            mn = fminf(mn, x);
            mx = fmaxf(mx, x);
        }
        red_mn[tid] = mn;
        red_mx[tid] = mx;
        __syncthreads();
        if (p == 0) {
            for (int r = 1; r < parts; ++r) {
                mn = fminf(mn, red_mn[r * D + c]);
                mx = fmaxf(mx, red_mx[r * D + c]);
            }
            const float s = (mx - mn) / static_cast<float>(qmax_of(a.L.kb, c));
            s_c[c] = s;
            mn_c[c] = mn;
            float *meta = a.L.k_meta + qa.grp(gi) * 2 * D;
            meta[c] = (s == 0.0f) ? 0.0f : s;
            meta[D + c] = (mn == 0.0f) ? 0.0f : mn;
        }
        __syncthreads();

        // ---- Key codes: one packed word per work item (token i, word w) ----
        const int wk = a.L.wk, kb = a.L.kb;
        for (int it = tid; it < G * wk; it += kThreads) {
            const int i = it / wk, w = it % wk;
            const uint16_t *row = tile + i * D;
            uint32_t word = 0;
            if (kb == 3) {
                for (int sl = 0; sl < 11; ++sl) {
                    const int cc = w * 11 + sl;
                    if (cc < D)
                        word |= code_of(widen16(row[cc], bf), mn_c[cc], s_c[cc], qmax_of(3, cc)) << (3 * sl);
                }
            } else {
                const int epw = 32 / kb, qm = (1 << kb) - 1;
                for (int sl = 0; sl < epw; ++sl) {
                    const int cc = w * epw + sl;
                    word |= code_of(widen16(row[cc], bf), mn_c[cc], s_c[cc], qm) << (kb * sl);
                }
            }
            a.L.k_words[(row0 + i) * wk + w] = word;
        }
    } else {
        // ---- Value: min / max per token over the D channels, tpt threads per token ----
        stage(a, a.L.ring_v, a.v_new, bh, t0, tile);
        __syncthreads();
        const int vb = a.L.vb, vq = (1 << vb) - 1;
        token_scales(tile, G, D, bf, vq, a.L.v_meta + row0 * 2, s_c, mn_c,
                     red_mn, red_mx);

        const int wv = a.L.wv;
        uint32_t *vrow0 = a.L.v_words + row0 * wv;
        if (a.L.v_tiled) {
            // 32-token blocks of operand fragments (layout in kvq_layout.h)
            const int fw = D * vb / 64, P = 16 / vb, blk_words = D * vb;
            for (int it = tid; it < G * wv; it += kThreads) {
                const int blk = it / blk_words, wi = it % blk_words;
                const int frag = wi / fw, u = wi % fw;
                const int q = frag >> 4, c16 = frag & 15;
                uint32_t word = 0;
                for (int jj = 0; jj < P; ++jj) {
                    const int R = u * P + jj, m = R >> 2;
                    for (int half = 0; half < 2; ++half) {
                        const int s = 2 * (R & 3) + half;
                        const int tb = (s >> 2) * 16 + 4 * q + (s & 3);
                        const int i = blk * 32 + tb, cc = 16 * m + c16;
                        word |= code_of(widen16(tile[i * D + cc], bf), mn_c[i], s_c[i], vq) << (vb * jj + 16 * half);
                    }
                }
                vrow0[it] = word;
            }
        } else {
            const int epw = 32 / vb;
            for (int it = tid; it < G * wv; it += kThreads) {
                const int i = it / wv, w = it % wv;
                uint32_t word = 0;
                for (int sl = 0; sl < epw; ++sl) {
                    const int cc = w * epw + sl;
                    word |= code_of(widen16(tile[i * D + cc], bf), mn_c[i], s_c[i], vq) << (vb * sl);
                }
                vrow0[it] = word;
            }
        }
    }

    if (a.ring_after && j == 0) {
        // single-token append: the new token takes the slot of the oldest
        // flushed token, which was staged above (K by the K workgroup, V by the V one)
        __syncthreads();
        const size_t dst = (static_cast<size_t>(bh) * a.L.R + (a.N0 % a.L.R)) * D;
        const size_t src = static_cast<size_t>(bh) * D;
        uint16_t *ring = is_v ? a.L.ring_v : a.L.ring_k;
        const uint16_t *fresh = is_v ? a.v_new : a.k_new;
        for (int ch = tid; ch < D / 8; ch += kThreads)
            *reinterpret_cast<uint4 *>(ring + dst + ch * 8) = *reinterpret_cast<const uint4 *>(fresh + src + ch * 8);
    }
}

__global__ __launch_bounds__(kThreads) void ring_write_kernel(RingArgs a)
{
    const int chunks = a.D / 8;  // 8 16-bit values per 16-byte chunk
    const int ntok = a.t_last - a.t_first;
    const long total = static_cast<long>(a.BH) * ntok * chunks;
    for (long it = static_cast<long>(blockIdx.x) * kThreads + threadIdx.x; it < total;
         it += static_cast<long>(gridDim.x) * kThreads) {
        const int ch = static_cast<int>(it % chunks);
        const long rest = it / chunks;
        const int t = a.t_first + static_cast<int>(rest % ntok);
        const int bh = static_cast<int>(rest / ntok);
        const size_t src = (static_cast<size_t>(bh) * a.n_new + (t - a.N0)) * a.D + ch * 8;
        const size_t dst = (static_cast<size_t>(bh) * a.L.R + (t % a.L.R)) * a.D + ch * 8;
        *reinterpret_cast<uint4 *>(a.L.ring_k + dst) = *reinterpret_cast<const uint4 *>(a.k_new + src);
        *reinterpret_cast<uint4 *>(a.L.ring_v + dst) = *reinterpret_cast<const uint4 *>(a.v_new + src);
    }
}

__global__ void zero_kernel(unsigned *p, int n)
{
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n)
        p[i] = 0u;
}

}  // namespace

hipError_t launch_flush(const FlushArgs &a, hipStream_t st)
{
    dim3 grid(a.n_groups, a.BH, 2);
    hipLaunchKernelGGL(flush_kernel, grid, dim3(kThreads), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_ring_write(const RingArgs &a, hipStream_t st)
{
    const long total = static_cast<long>(a.BH) * (a.t_last - a.t_first) * (a.D / 8);
    long blocks = (total + kThreads - 1) / kThreads;
    if (blocks > 65536)
        blocks = 65536;
    hipLaunchKernelGGL(ring_write_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0, st,
                       a);
    return hipGetLastError();
}

hipError_t launch_zero(unsigned *p, int n, hipStream_t st)
{
    hipLaunchKernelGGL(zero_kernel, dim3((n + 255) / 256), dim3(256), 0, st, p, n);
    return hipGetLastError();
}

}  // namespace kvq
