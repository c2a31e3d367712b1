// kvq_internal.h -- device-side layout descriptors and kernel launchers shared
// by the host runtime (kvq_runtime.cpp) and the HIP kernels (*.hip).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace kvq {

// Physical layout of one layer in the workspace.  BH = batch * n_kv_heads
// streams, each with its own rows; capq = quantized-token capacity per stream.
//
// K codes are token-major rows of wk words (channels along the row, least
// significant bits first; 3-bit: eleven channels per word).
//
// V codes are either token-major rows (v_tiled == 0) or, for the matrix-core
// path, 32-token blocks laid out as that kernel's operand fragments
// (v_tiled == 1): inside a block, 64 fragments of D*vb/64 words, fragment
// f = 16*q + c16 holding channels c16, c16+16, ... for the eight tokens
// {4q..4q+3, 16+4q..16+4q+3}; see v_tile_bit() in kvq_layout.h.
struct LayerDev {
    uint32_t *k_words;  // [BH][capq][wk]
    float *k_meta;      // [BH][capq / G][2][D]   per group: D scales, then D zeros
                        // (per-token Key: [BH][capq][2], scale and zero per token)
    uint32_t *v_words;  // [BH][capq][wv] (row-major or 32-token tiles, same size)
    float *v_meta;      // [BH][capq][2]          per token: scale, zero
    uint16_t *ring_k;   // [BH][R][D]             recent tokens, slot = t % R
    uint16_t *ring_v;   // [BH][R][D]
    int kb, vb;         // bits: 2, 3 (K), 4, 8; 16 = layer not quantized
    int wk, wv;         // 32-bit words per packed row
    int R;              // recent-token capacity (max_context for a 16-bit layer)
    int G;              // tokens per K group
    int capq;           // quantized-token capacity per stream (multiple of G and 32)
    int ngq;            // capq / G: K groups per stream
    int v_tiled;        // V code layout, see above
    int k_tok;          // 1: Key quantized per token (k_meta per token), 0: per channel
    // Paging (table != nullptr): the quantized state lives in a pool of
    // n_pages pages (plus one spare page that out-of-range page ids fall on),
    // each holding 2^P_log2 consecutive tokens of one sequence for all Hkv
    // heads; token t of sequence b is in page table[b * tstride + (t >>
    // P_log2)].  The arrays above are then [n_pages + 1][Hkv][P][...] instead
    // of [BH][capq][...].  bh0 is added to a stream index before the table is
    // read (a view of streams bh0.. of the layer).  Unpaged: table == nullptr.
    const int32_t *table;
    int P_log2, Hkv, tstride, n_pages, bh0;
    int gpp;            // 2^P_log2 / G: K groups per page
};

// Addressing of one stream's quantized state: row(t) indexes the rows of
// k_words (wk words), v_words (wv words), v_meta (2 floats) and the per-token
// k_meta (2 floats) of token t; grp(gi) the [2][D] per-channel k_meta block of
// group gi.  A 32-token block (t a multiple of 32) and a whole group stay in
// one page, so their rows are consecutive.
struct QAddr {
    const int32_t *trow;  // the sequence's page ids (paged), or nullptr
    size_t base, gbase;   // unpaged: the stream's first row and first group
    int h, P_log2, n_pages, Hkv, gpp, G;

    __host__ __device__ QAddr(const LayerDev &L, int bh)
        : trow(nullptr), base(static_cast<size_t>(bh) * L.capq), gbase(static_cast<size_t>(bh) * L.ngq), h(0),
          P_log2(L.P_log2), n_pages(L.n_pages), Hkv(L.Hkv), gpp(L.gpp), G(L.G)
    {
        if (L.table) {
            const int gbh = bh + L.bh0, b = gbh / L.Hkv;
            trow = L.table + static_cast<size_t>(b) * L.tstride;
            h = gbh - b * L.Hkv;
        }
    }
    // first row of token t's page, in pages of one kv head (page * Hkv + h)
    __host__ __device__ size_t page_slot(int t) const
    {
        int page = trow[t >> P_log2];
        if (static_cast<unsigned>(page) >= static_cast<unsigned>(n_pages))
            page = n_pages;  // the spare page: memory-safe, contents undefined
        return static_cast<size_t>(page) * Hkv + h;
    }
    __host__ __device__ size_t row(int t) const
    {
        if (!trow)
            return base + t;
        return (page_slot(t) << P_log2) + (t & ((1 << P_log2) - 1));
    }
    __host__ __device__ size_t grp(int gi) const
    {
        if (!trow)
            return gbase + gi;
        const int t = gi * G, pi = t >> P_log2;
        return page_slot(t) * gpp + (gi - pi * gpp);
    }
    // the same with token t's (or group gi's) page id already read
    // (clamped into the pool)
    __host__ __device__ size_t page_row(int page, int t) const
    {
        return ((static_cast<size_t>(page) * Hkv + h) << P_log2) + (t & ((1 << P_log2) - 1));
    }
    __host__ __device__ size_t page_grp(int page, int gi) const
    {
        const int pi = (gi * G) >> P_log2;
        return (static_cast<size_t>(page) * Hkv + h) * gpp + (gi - pi * gpp);
    }
    __host__ __device__ int clamp_page(int page) const
    {
        return static_cast<unsigned>(page) >= static_cast<unsigned>(n_pages) ? n_pages : page;
    }
};

// Quantize and pack groups [Tq0 + j*G, Tq0 + (j+1)*G), j < n_groups, for every
// stream.  Token t comes from the ring (t < N0) or from the new tokens (t >= N0).
// When ring_after != 0 (single-token append), the same workgroup afterwards
// stores new token N0 into ring slot N0 % R.
struct FlushArgs {
    LayerDev L;
    const uint16_t *k_new, *v_new;  // [BH][n_new][D]
    int D, n_new, N0, Tq0, n_groups, BH, kv_bf16;
    int ring_after;
};

// Copy new tokens t in [t_first, t_last) (t >= N0) into ring slot t % R.
struct RingArgs {
    LayerDev L;
    const uint16_t *k_new, *v_new;
    int D, n_new, N0, t_first, t_last, BH;
};

// Arrival counters of the attention launches: one per stream, each on a
// 128-byte line of its own, so that the device-scope atomics of different
// streams do not queue on one line.
constexpr int kCounterStride = 32;  // u32 words between consecutive streams' counters

// Floats of one workgroup's partial entry (g heads of o[D], m, l and two
// unused floats), rounded up to whole 128-byte lines so that the entries of
// different workgroups share no line.
__host__ __device__ inline int part_entry_floats(int g, int D)
{
    return (g * (D + 4) + 31) & ~31;
}

// The statically allocated scratch of kvq_decode_attention_noalloc(): the
// arrival counters of up to kStaticScratchStreams streams (one 128-byte line
// each), then the partial entries of one call (a stream's entries contiguous,
// as in a workspace).  Between two calls every counter is zero: the merging
// workgroup of each stream re-arms its counter, and the partial entries need
// no initial value (each call writes the entries it reads).
constexpr size_t kStaticScratchBytes = size_t(16) << 20;
constexpr int kStaticScratchStreams = 4096;
constexpr size_t kStaticScratchWordsBytes = size_t(kStaticScratchStreams) * kCounterStride * 4;

// Device address of this GPU's static scratch (set up on first use: its
// counters are zeroed on stream st).
hipError_t static_scratch(int device, hipStream_t st, void **out);

// Sequences one attention launch can take with lengths of their own.
constexpr int kMaxRaggedSeqs = 64;

struct AttnArgs {
    LayerDev L;
    const void *q;        // [B][Hq][D] in q_dtype
    float *out;           // [B][Hq][D]
    float *part;          // [BH][n_part] entries of part_entry_floats(g, D): [g][D + 4] o[D], m (log2 domain), l, 2 unused
    unsigned *counters;   // arrival counter of stream bh at bh * kCounterStride, zero between calls
    int q_dtype, kv_bf16;
    int D, g, Hkv, N, Tq, BH;
    int n_part;           // partial entries per stream (one per workgroup)
    // vector-ALU ranges: wg_valu workgroups per stream cover tokens [valu_beg, N)
    int valu_beg, valu_wgs, valu_tps;
    // matrix-core units: units_q waves per stream cover groups [0, Tq / G),
    // unit u taking unit_groups groups, plus one more for u < unit_extra
    // (the remainder); then units_r waves cover the recent tokens
    // [Tq, N), res_tokens each (a multiple of 32); mfma_wgs = ceil((units_q +
    // units_r) / 4) workgroups
    int units_q, unit_groups, unit_extra, units_r, res_tokens, mfma_wgs;
    // matrix-core grid numbering: 0 = 2D (x: workgroup of the stream, y:
    // stream); s > 0 = 1D, workgroup i serving stream (i % 8) + 8 * ((i / 8) >> s)
    // as its workgroup (i / 8) & (2^s - 1), mfma_wgs = 2^s: workgroups are dealt
    // to the eight XCDs in turn, so each stream's workgroups share one XCD and
    // its L2 (the hand-off then reads the partials from that L2)
    int xcd_shift;
    // Tq / G, capq / G, and log2 of the columns per group slot of the
    // matrix-core products (S = 16 / NG, NG the largest power of two with
    // NG * g <= 16)
    int n_groups, ngcap, s_log2;
    // 1: units whose windows hold at most two groups walk their rounds
    // double-buffered where the type allows (next round's loads in flight
    // during this one); 0: one round at a time
    int pipe;
    float scale_log2;     // log2(e) / sqrt(D)
    // token new_t (>= 0) has just been appended and is not in the ring yet: it
    // is read from new_k / new_v ([BH][D]) and written to its ring slot by the
    // workgroup that attends to it; new_t = -1 when there is none
    const uint16_t *new_k, *new_v;
    int new_t;
};

// Ragged batches (sequences of different lengths): the streams of sequence b
// (bh / Hkv == b) take N, Tq, new_t and their split of the quantized groups
// over the launch's units_q units (unit_groups, unit_extra) from entry b; the
// launch's own fields hold the sizes it is shaped for.  Passed by value to
// separate kernel instantiations, so that uniform launches keep their small
// argument block.
struct RaggedTables {
    int N[kMaxRaggedSeqs], Tq[kMaxRaggedSeqs], unit_groups[kMaxRaggedSeqs], unit_extra[kMaxRaggedSeqs],
        new_t[kMaxRaggedSeqs];
};

struct RaggedAttnArgs {
    AttnArgs a;
    RaggedTables t;
};

// Causal attention of the queries of the last n_q appended tokens (a prefill
// chunk): query j (position N - n_q + j) attends to tokens 0 .. N - n_q + j.
// Tiles of QT = 16 / g queries of one stream, tw per wave (two up to head_dim
// 128 when that still gives a workgroup per compute unit, else one);
// workgroups of eight waves of one stream, wg_per_stream of them per stream,
// n_wg in all.
struct PrefillArgs {
    LayerDev L;
    const void *q;   // [B][Hq][n_q][D] in q_dtype
    float *out;      // [B][Hq][n_q][D]
    int q_dtype, kv_bf16;
    int D, g, BH, N, Tq, n_q;
    int QT, n_tiles, n_wg, wg_per_stream;
    int tw;          // query tiles per wave: 2 (head_dim <= 128, enough workgroups) or 1
    int ngcap;       // capq / G
    float scale_log2;  // log2(e) / sqrt(D)
    // ragged layer: sequence b = bh / Hkv holds seqN[b] tokens, seqTq[b] of
    // them quantized (N and Tq unused)
    int ragged, Hkv;
    int seqN[kMaxRaggedSeqs], seqTq[kMaxRaggedSeqs];
};

// LDS floats per wave of the matrix-core kernel, one region used three ways:
// a quantized unit's K scales and zeros of one window (ng groups of [2][D]
// floats, ng = the largest power of two with ng * g <= 16) followed by the
// stream's q; a recent-token unit's V tile (32 x D 16-bit values); and, at the
// end of either, the wave's results o[g][D].
__host__ __device__ inline int mfma_wave_region(int D, int g, bool has_q_units, bool has_r_units)
{
    int ng = 16;
    while (ng * g > 16)
        ng >>= 1;
    const int vt = has_r_units ? 16 * D : 0;
    const int meta = has_q_units ? ng * 2 * D + g * D : 0;  // + q (up to fp32)
    int r = g * D;
    r = vt > r ? vt : r;
    return meta > r ? meta : r;
}

// 32-token blocks (one per group slot) the matrix-core kernel processes
// together in one round: four, or fewer when a block's operands take many
// registers (K rows of two 16-token tiles + the V fragment, + the 3-bit
// path's extra q.K operand chunk).
__host__ __device__ constexpr int mfma_round_blocks(int kb, int vb, int D)
{
    const int regs = 2 * (D * kb / 128) + D * vb / 64 + (kb == 3 ? 4 : 0);
    return regs >= 48 ? 1 : (regs >= 24 ? 2 : 4);
}

hipError_t launch_flush(const FlushArgs &a, hipStream_t st);
hipError_t launch_ring_write(const RingArgs &a, hipStream_t st);
// True when the matrix-core kernel is built for this (k_bits, v_bits, D).
bool mfma_supported(int kb, int vb, int D);
// rt: per-sequence lengths of a ragged batch, or nullptr
hipError_t launch_attention(const AttnArgs &a, const RaggedTables *rt, bool use_mfma, hipStream_t st);
hipError_t launch_zero(unsigned *p, int n, hipStream_t st);
// True when the prefill kernel is built for this layer format.
bool prefill_supported(int kb, int vb, int D, int v_tiled);
hipError_t launch_prefill(const PrefillArgs &a, hipStream_t st);

}  // namespace kvq
