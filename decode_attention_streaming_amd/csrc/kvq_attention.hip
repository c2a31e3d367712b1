// kvq_attention.hip -- vector-ALU split-sequence decode attention (every bit
// width, including the 3-bit Key layout, and 16-bit layers) and the dispatch
// between it and the matrix-core kernel.  Device code shared with the
// matrix-core kernel is in kvq_attn_common.h.
#include "kvq_attn_common.h"

namespace kvq {

hipError_t launch_mfma_d64(const AttnArgs &a, const RaggedTables *rt, hipStream_t st);
hipError_t launch_mfma_d128(const AttnArgs &a, const RaggedTables *rt, hipStream_t st);
hipError_t launch_mfma_d256(const AttnArgs &a, const RaggedTables *rt, hipStream_t st);
hipError_t launch_prefill_d64(const PrefillArgs &a, hipStream_t st);
hipError_t launch_prefill_d128(const PrefillArgs &a, hipStream_t st);
hipError_t launch_prefill_d256(const PrefillArgs &a, hipStream_t st);

namespace {

template <int D, int GM>
__device__ __forceinline__ void attn_valu_body(const AttnArgs &a, const RaggedTables *rt)
{
    const int split = blockIdx.x, bh = blockIdx.y;
    const int t_beg = a.valu_beg + split * a.valu_tps;
    const int t_end = min(stream_dims(a, rt, bh).N, t_beg + a.valu_tps);
    extern __shared__ float smem[];
    // heads h0 .. h0 + GM - 1 at a time (two passes over the range for more
    // than eight heads per kv head: their per-head state would not fit the
    // registers at once)
    for (int h0 = 0; h0 < a.g; h0 += GM)
        valu_range<D, GM>(a, rt, bh, t_beg, t_end, split, smem, h0);
    arrive_and_merge<D>(a, bh, gridDim.x);
}

template <int D, int GM>
__global__ __launch_bounds__(kAttnThreads) void attn_valu_kernel(AttnArgs a)
{
    attn_valu_body<D, GM>(a, nullptr);
}

template <int D, int GM>
__global__ __launch_bounds__(kAttnThreads) void attn_valu_kernel_rg(RaggedAttnArgs r)
{
    attn_valu_body<D, GM>(r.a, &r.t);
}

template <int D, int GM>
void launch_valu_g(const AttnArgs &a, const RaggedTables *rt, dim3 grid, size_t lds, hipStream_t st)
{
    if (rt) {
        const RaggedAttnArgs r{a, *rt};
        hipLaunchKernelGGL((attn_valu_kernel_rg<D, GM>), grid, dim3(kAttnThreads), lds, st, r);
    } else {
        hipLaunchKernelGGL((attn_valu_kernel<D, GM>), grid, dim3(kAttnThreads), lds, st, a);
    }
}

template <int D>
void launch_valu(const AttnArgs &a, const RaggedTables *rt, dim3 grid, size_t lds, hipStream_t st)
{
    if (a.g <= 1)
        launch_valu_g<D, 1>(a, rt, grid, lds, st);
    else if (a.g <= 2)
        launch_valu_g<D, 2>(a, rt, grid, lds, st);
    else if (a.g <= 4)
        launch_valu_g<D, 4>(a, rt, grid, lds, st);
    else
        launch_valu_g<D, 8>(a, rt, grid, lds, st);  // g > 8: two passes of eight heads
}

}  // namespace

bool mfma_supported(int kb, int vb, int D)
{
    const bool vbits = vb == 2 || vb == 4 || vb == 8;
    if (kb == 3)  // twelve words per row, three per lane quad
        return vbits && D == 128;
    return vbits && (kb == 2 || kb == 4 || kb == 8) && (D == 64 || D == 128 || D == 256);
}

bool prefill_supported(int kb, int vb, int D, int v_tiled)
{
    if (D != 64 && D != 128 && D != 256)
        return false;
    if (kb == 16)
        return vb == 16;
    const bool vbits = vb == 2 || vb == 4 || vb == 8;
    const bool kbits = kb == 2 || kb == 4 || kb == 8 || (kb == 3 && D == 128);  // 3 bits: twelve words a row
    return kbits && vbits && v_tiled;  // V codes in the matrix-core tile layout (G a multiple of 32)
}

hipError_t launch_prefill(const PrefillArgs &a, hipStream_t st)
{
    if (a.D == 64)
        return launch_prefill_d64(a, st);
    if (a.D == 128)
        return launch_prefill_d128(a, st);
    return launch_prefill_d256(a, st);
}

// a 16-bit layer runs only recent-token units: any instantiation serves
static AttnArgs as_plain(const AttnArgs &a)
{
    AttnArgs b = a;
    if (b.L.kb == 16) {
        b.L.kb = 2;
        b.L.vb = 2;
    }
    return b;
}

hipError_t launch_attention(const AttnArgs &a, const RaggedTables *rt, bool use_mfma, hipStream_t st)
{
    if (use_mfma) {
        const AttnArgs b = as_plain(a);
        if (a.D == 64)
            return launch_mfma_d64(b, rt, st);
        if (a.D == 128)
            return launch_mfma_d128(b, rt, st);
        return launch_mfma_d256(b, rt, st);
    }
    dim3 grid(a.valu_wgs, a.BH);
    const size_t lds = valu_lds_bytes(a.g, a.D);
    if (a.D == 64)
        launch_valu<64>(a, rt, grid, lds, st);
    else if (a.D == 128)
        launch_valu<128>(a, rt, grid, lds, st);
    else
        launch_valu<256>(a, rt, grid, lds, st);
    return hipGetLastError();
}

}  // namespace kvq
