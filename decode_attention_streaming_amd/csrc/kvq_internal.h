// kvq_internal.h -- device-side layout descriptors and kernel launchers shared
// by the host runtime (kvq_runtime.cpp) and the HIP kernels (*.hip).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace kvq {

// Physical layout of one layer in the workspace.  BH = batch * n_kv_heads
// streams, each with its own rows; capq = quantized-token capacity per stream.
struct LayerDev {
    uint32_t *k_words;  // [BH][capq][wk]         packed K rows, token-major
    float *k_meta;      // [BH][capq / G][2][D]   per group: D scales, then D zeros
    uint32_t *v_words;  // [BH][capq][wv]         packed V rows, token-major
    float *v_meta;      // [BH][capq][2]          per token: scale, zero
    uint16_t *ring_k;   // [BH][R][D]             recent tokens, slot = t % R
    uint16_t *ring_v;   // [BH][R][D]
    int kb, vb;         // bits: 2, 3 (K), 4, 8; 16 = layer not quantized
    int wk, wv;         // 32-bit words per packed row
    int R;              // recent-token capacity (max_context for a 16-bit layer)
    int G;              // tokens per K group
    int capq;           // quantized-token capacity per stream (multiple of G)
};

// Quantize and pack groups [Tq0 + j*G, Tq0 + (j+1)*G), j < n_groups, for every
// stream.  Token t comes from the ring (t < N0) or from the new tokens (t >= N0).
struct FlushArgs {
    LayerDev L;
    const uint16_t *k_new, *v_new;  // [BH][n_new][D]
    int D, n_new, N0, Tq0, n_groups, BH, kv_bf16;
};

// Copy new tokens t in [t_first, t_last) (t >= N0) into ring slot t % R.
struct RingArgs {
    LayerDev L;
    const uint16_t *k_new, *v_new;
    int D, n_new, N0, t_first, t_last, BH;
};

struct AttnArgs {
    LayerDev L;
    const void *q;      // [B][Hq][D] in q_dtype
    float *out;         // [B][Hq][D]
    float *part;        // [BH][n_splits][g][D + 2]: o[D], m (log2 domain), l
    int q_dtype, kv_bf16;
    int D, g, Hkv, N, Tq, BH;
    int n_splits, tps;  // splits per stream, tokens per split
    float scale_log2;   // log2(e) / sqrt(D)
};

hipError_t launch_flush(const FlushArgs &a, hipStream_t st);
hipError_t launch_ring_write(const RingArgs &a, hipStream_t st);
hipError_t launch_attention_valu(const AttnArgs &a, hipStream_t st);
hipError_t launch_merge(const AttnArgs &a, hipStream_t st);

}  // namespace kvq
