/*
 * kvq_oracle.c -- plain, slow CPU oracle for quantized-KV streaming decode
 * attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link,
 * load or call this file; only the tests, the smoke check and the CPU-baseline
 * leg of the benchmark use it.  It shares no code, header, table or helper with
 * the HIP library.
 *
 * Build:  gcc -std=c99 -O2 -fno-fast-math -ffp-contract=off -fPIC -shared
 * (no FMA contraction, no flush-to-zero, default round-to-nearest-even mode).
 *
 * Sources (web pages, cited by title and section):
 *   [KVTuner]  "KVTuner: Sensitivity-Aware Layer-Wise Mixed-Precision KV Cache
 *              Quantization ..." (papercache.org summary), section A3:
 *              "Transformer and KV cache" (attention equation a = softmax(qK^T/sqrt D),
 *              o = aV, K = concat(K_{:i-1}, k_i)) and "KV cache quantization
 *              basics" (Q(X) = round((X - z)/s), X^ = Q(X)s + z, z = min X,
 *              s = (max X - min X)/(2^B - 1)).
 *   [KVmix]    "KVmix: Gradient-Based Layer Importance-Aware Mixed-Precision
 *              Quantization for KV Cache" (paper notes), key design 2
 *              (Key per channel, Value per token, q = round((x - min)/s),
 *              s = (max - min)/q_max, results packed into int32; the 3-bit
 *              layout of eleven elements per word: ten at 3 bits, one at 2).
 *   [KVTuner]  also: the two Key quantization modes it evaluates, KIVI
 *              (per-channel Key) and per-token-asym (each token's Key
 *              quantized over its channels, like Value).
 *   [KIVI]     "LLM quantization notes 08: KV cache quantization and KIVI",
 *              section 6.1 (one scale + zero-point per head per channel for K,
 *              per token for V), section 6.2 (streaming: recent tokens kept in
 *              a 16-bit buffer, K quantized one small token segment at a time),
 *              section 2.1 (KV memory formula).
 *
 * Readings where the pages are silent (each listed in the design notes):
 *   - round() is round-half-to-even, evaluated in fp32: codes are
 *     rint((x - mn) / s) with an IEEE correctly-rounded fp32 division, then
 *     clamped to [0, qmax].
 *   - a group whose max equals its min gets s = 0, all codes 0, z = min.
 *   - a zero z or s is stored as +0.0.
 *   - scale and zero-point are fp32; z is the float minimum itself.
 *   - codes are packed along head_dim, one token row after another, least
 *     significant bits first; a 3-bit word holds channels 11w .. 11w+10 with
 *     slot 10 at 2 bits; that channel's own min/max is quantized with qmax 3.
 *   - K and V share one recent-token buffer of R tokens; when an append finds
 *     it full, the oldest G tokens are quantized (flushed) first.
 *   - [KVmix] key design 3 (dynamic RPC ratio r per layer, num_RPC =
 *     floor(r * current_RPC)): with r > 0, an append that finds the buffer full
 *     keeps floor(r * current) of its current tokens in 16 bits and quantizes
 *     the older rest, rounded down to whole groups of G (at least one group).
 *     r is given in parts per thousand so that the rule is integer arithmetic.
 *   - the softmax scale is 1/sqrt(head_dim).
 *   - a (16,16) layer keeps every token in its 16-bit input format.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include "kvq_oracle.h"

/* ---------------------------------------------------------------------------
 * 16-bit storage formats, widened exactly.
 * ------------------------------------------------------------------------- */

/* IEEE binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
float kvqo_f16_to_f32(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int m = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24); /* zero or subnormal: m * 2^-24 */
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(m + 1024), e - 25); /* (1024 + m) * 2^(e - 15 - 10) */
    return (float)(sign ? -v : v);
}

/* bfloat16 is the upper half of an IEEE binary32. */
float kvqo_bf16_to_f32(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

static float widen(uint16_t x, int is_bf16)
{
    return is_bf16 ? kvqo_bf16_to_f32(x) : kvqo_f16_to_f32(x);
}

/* ---------------------------------------------------------------------------
 * Packing into 32-bit words.
 * ------------------------------------------------------------------------- */

int kvqo_words_per_row(int d, int bits)
{
    if (bits == 3)
        return (d + 10) / 11; /* eleven channels per word */
    return d * bits / 32;
}

/* Largest code of channel c in a row quantized at `bits`. */
int kvqo_qmax(int bits, int c)
{
    if (bits == 3)
        return (c % 11 == 10) ? 3 : 7; /* slot 10 of a 3-bit word has 2 bits */
    return (1 << bits) - 1;
}

static void slot_of(int bits, int c, int *word, int *shift)
{
    if (bits == 3) {
        *word = c / 11;
        *shift = 3 * (c % 11);
    } else {
        int per_word = 32 / bits;
        *word = c / per_word;
        *shift = bits * (c % per_word);
    }
}

void kvqo_pack_row(const uint8_t *codes, int d, int bits, uint32_t *words)
{
    int nw = kvqo_words_per_row(d, bits);
    for (int w = 0; w < nw; ++w)
        words[w] = 0;
    for (int c = 0; c < d; ++c) {
        int w, sh;
        slot_of(bits, c, &w, &sh);
        words[w] |= (uint32_t)codes[c] << sh;
    }
}

void kvqo_unpack_row(const uint32_t *words, int d, int bits, uint8_t *codes)
{
    for (int c = 0; c < d; ++c) {
        int w, sh;
        slot_of(bits, c, &w, &sh);
        codes[c] = (uint8_t)((words[w] >> sh) & (uint32_t)kvqo_qmax(bits, c));
    }
}

/* ---------------------------------------------------------------------------
 * Asymmetric uniform quantization of one group of n fp32 values.
 * [KVTuner] A3 quantization basics; [KVmix] key design 2.
 * x[i * stride], i = 0..n-1.  Writes codes[i * cstride], *s_out, *z_out.
 * ------------------------------------------------------------------------- */
void kvqo_quantize(const float *x, int n, long stride, int qmax,
                   uint8_t *codes, long cstride, float *s_out, float *z_out)
{
    float mn = x[0], mx = x[0];
    for (int i = 1; i < n; ++i) {
        float v = x[(long)i * stride];
        if (v < mn)
            mn = v;
        if (v > mx)
            mx = v;
    }
    float s = (mx - mn) / (float)qmax; /* fp32 subtraction, then fp32 division */
    for (int i = 0; i < n; ++i) {
        uint8_t q = 0;
        if (s != 0.0f) {
            float t = (x[(long)i * stride] - mn) / s;
            float r = rintf(t); /* default mode: round half to even */
            if (r < 0.0f)
                r = 0.0f;
            if (r > (float)qmax)
                r = (float)qmax;
            q = (uint8_t)r;
        }
        codes[(long)i * cstride] = q;
    }
    if (s == 0.0f)
        s = 0.0f; /* store +0.0 */
    if (mn == 0.0f)
        mn = 0.0f;
    *s_out = s;
    *z_out = mn;
}

/* ---------------------------------------------------------------------------
 * Streaming layer state.  Arrays are owned by the caller (see the header).
 * ------------------------------------------------------------------------- */

static int is_plain(const kvqo_layer *L) { return L->k_bits == 16; }

/* Quantize tokens [Tq, Tq + G) of every stream and advance Tq.
 * [KIVI] 6.2: K per channel over a token segment, V per token. */
static void flush_group(kvqo_layer *L)
{
    const int d = L->d, G = L->G, t0 = L->Tq, gi = L->Tq / L->G;
    const int wk = kvqo_words_per_row(d, L->k_bits);
    const int wv = kvqo_words_per_row(d, L->v_bits);
    float *x = (float *)malloc(sizeof(float) * (size_t)G * (size_t)(d > G ? d : G) * 2);
    uint8_t *codes = (uint8_t *)malloc((size_t)G * (size_t)d);
    for (int s = 0; s < L->n_streams; ++s) {
        const uint16_t *hk = L->hist_k + ((size_t)s * L->cap + t0) * d;
        const uint16_t *hv = L->hist_v + ((size_t)s * L->cap + t0) * d;
        if (L->k_tok) {
            /* Key, per-token-asym mode: one (scale, zero) per token over its
             * d channels, as for Value. */
            for (int i = 0; i < G; ++i) {
                for (int c = 0; c < d; ++c)
                    x[c] = widen(hk[(size_t)i * d + c], L->is_bf16);
                size_t t = (size_t)s * L->cap + t0 + i;
                kvqo_quantize(x, d, 1, (1 << L->k_bits) - 1, codes, 1,
                              &L->k_scale[t], &L->k_zero[t]);
                kvqo_pack_row(codes, d, L->k_bits, L->k_words + t * wk);
            }
        } else {
            /* Key: one (scale, zero) per channel over the G tokens of the group. */
            for (int i = 0; i < G; ++i)
                for (int c = 0; c < d; ++c)
                    x[(size_t)i * d + c] = widen(hk[(size_t)i * d + c], L->is_bf16);
            float *ks = L->k_scale + ((size_t)s * (L->cap / G) + gi) * d;
            float *kz = L->k_zero + ((size_t)s * (L->cap / G) + gi) * d;
            for (int c = 0; c < d; ++c)
                kvqo_quantize(x + c, G, d, kvqo_qmax(L->k_bits, c), codes + c, d,
                              &ks[c], &kz[c]);
            for (int i = 0; i < G; ++i)
                kvqo_pack_row(codes + (size_t)i * d, d, L->k_bits,
                              L->k_words + ((size_t)s * L->cap + t0 + i) * wk);
        }
        /* Value: one (scale, zero) per token over its d channels. */
        for (int i = 0; i < G; ++i) {
            for (int c = 0; c < d; ++c)
                x[c] = widen(hv[(size_t)i * d + c], L->is_bf16);
            size_t t = (size_t)s * L->cap + t0 + i;
            kvqo_quantize(x, d, 1, (1 << L->v_bits) - 1, codes, 1,
                          &L->v_scale[t], &L->v_zero[t]);
            kvqo_pack_row(codes, d, L->v_bits, L->v_words + t * wv);
        }
    }
    free(codes);
    free(x);
    L->Tq += G;
}

int kvqo_append(kvqo_layer *L, const uint16_t *k_new, const uint16_t *v_new, int n)
{
    const int d = L->d;
    if (n < 0 || L->N + n > L->cap)
        return -1;
    for (int i = 0; i < n; ++i) {
        /* A full recent-token buffer is flushed before the new token enters:
         * its oldest G tokens, or with a ratio r all but floor(r * current)
         * of its tokens, in whole groups. */
        if (!is_plain(L) && L->N - L->Tq == L->R) {
            const int current = L->N - L->Tq;
            int n_flush = L->G;
            if (L->rpc_permille > 0) {
                const int keep = (int)(((long long)current * L->rpc_permille) / 1000);
                n_flush = (current - keep) / L->G * L->G;
                if (n_flush < L->G)
                    n_flush = L->G;
            }
            for (int f = 0; f < n_flush; f += L->G)
                flush_group(L);
        }
        for (int s = 0; s < L->n_streams; ++s) {
            memcpy(L->hist_k + ((size_t)s * L->cap + L->N) * d,
                   k_new + ((size_t)s * n + i) * d, sizeof(uint16_t) * d);
            memcpy(L->hist_v + ((size_t)s * L->cap + L->N) * d,
                   v_new + ((size_t)s * n + i) * d, sizeof(uint16_t) * d);
        }
        L->N += 1;
    }
    return 0;
}

/* Dequantized Key of token t of stream s, channel c, in fp64. */
static double key_hat(const kvqo_layer *L, int s, int t, int c, const uint8_t *row_codes)
{
    if (t < L->Tq && L->k_tok) {
        size_t tt = (size_t)s * L->cap + t;
        return (double)row_codes[c] * (double)L->k_scale[tt] + (double)L->k_zero[tt];
    }
    if (t < L->Tq) {
        size_t g = (size_t)s * (L->cap / L->G) + t / L->G;
        return (double)row_codes[c] * (double)L->k_scale[g * L->d + c] +
               (double)L->k_zero[g * L->d + c];
    }
    return (double)widen(L->hist_k[((size_t)s * L->cap + t) * L->d + c], L->is_bf16);
}

static double value_hat(const kvqo_layer *L, int s, int t, int c, const uint8_t *row_codes)
{
    if (t < L->Tq) {
        size_t tt = (size_t)s * L->cap + t;
        return (double)row_codes[c] * (double)L->v_scale[tt] + (double)L->v_zero[tt];
    }
    return (double)widen(L->hist_v[((size_t)s * L->cap + t) * L->d + c], L->is_bf16);
}

/* Decode attention over every token appended so far, in fp64.
 * [KVTuner] A3: a = softmax(q K^T / sqrt(D)), o = a V; D read as head_dim.
 * q and out: [n_streams][g][d]; query head h of stream s attends to stream s. */
void kvqo_attention(const kvqo_layer *L, const double *q, double *out)
{
    const int d = L->d, N = L->N, g = L->g;
    const int wk = kvqo_words_per_row(d, L->k_bits);
    const int wv = kvqo_words_per_row(d, L->v_bits);
    double *e = (double *)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
    double *kh = (double *)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1) * d);
    double *vh = (double *)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1) * d);
    uint8_t *codes = (uint8_t *)malloc((size_t)d);
    const double scale = 1.0 / sqrt((double)d);
    for (int s = 0; s < L->n_streams; ++s) {
        /* dequantize the whole history of this stream once */
        for (int t = 0; t < N; ++t) {
            if (t < L->Tq)
                kvqo_unpack_row(L->k_words + ((size_t)s * L->cap + t) * wk, d, L->k_bits, codes);
            for (int c = 0; c < d; ++c)
                kh[(size_t)t * d + c] = key_hat(L, s, t, c, codes);
            if (t < L->Tq)
                kvqo_unpack_row(L->v_words + ((size_t)s * L->cap + t) * wv, d, L->v_bits, codes);
            for (int c = 0; c < d; ++c)
                vh[(size_t)t * d + c] = value_hat(L, s, t, c, codes);
        }
        for (int h = 0; h < g; ++h) {
            const double *qv = q + ((size_t)s * g + h) * d;
            double *o = out + ((size_t)s * g + h) * d;
            double m = -INFINITY;
            for (int t = 0; t < N; ++t) {
                double acc = 0.0;
                for (int c = 0; c < d; ++c)
                    acc += qv[c] * kh[(size_t)t * d + c];
                e[t] = acc * scale;
                if (e[t] > m)
                    m = e[t];
            }
            double l = 0.0;
            for (int t = 0; t < N; ++t) {
                e[t] = exp(e[t] - m);
                l += e[t];
            }
            for (int c = 0; c < d; ++c) {
                double acc = 0.0;
                for (int t = 0; t < N; ++t)
                    acc += e[t] * vh[(size_t)t * d + c];
                o[c] = N > 0 ? acc / l : 0.0;
            }
        }
    }
    free(codes);
    free(vh);
    free(kh);
    free(e);
}

/* Attention of the last n_q appended tokens' queries over the cache, in fp64:
 * the prefill form of the same equation.  [KVTuner] A3: the query of step i
 * attends to the keys and values of steps up to and including i
 * (K = concat(K_{:i-1}, k_i)); [KVTuner] A2 (calibration): prefill attention
 * runs on the dequantized cache.  Query j (0 <= j < n_q) sits at position
 * p = N - n_q + j and attends to tokens 0..p as the cache holds them (codes
 * dequantized for t < Tq, the 16-bit values for the recent tokens).
 * q and out: [n_streams][g][n_q][d]. */
void kvqo_prefill_attention(const kvqo_layer *L, const double *q, int n_q, double *out)
{
    const int d = L->d, N = L->N, g = L->g;
    const int wk = kvqo_words_per_row(d, L->k_bits);
    const int wv = kvqo_words_per_row(d, L->v_bits);
    const size_t n1 = (size_t)(N > 0 ? N : 1);
    double *e = (double *)malloc(sizeof(double) * n1);
    double *kh = (double *)malloc(sizeof(double) * n1 * d);
    double *vh = (double *)malloc(sizeof(double) * n1 * d);
    uint8_t *codes = (uint8_t *)malloc((size_t)d);
    const double scale = 1.0 / sqrt((double)d);
    for (int s = 0; s < L->n_streams; ++s) {
        for (int t = 0; t < N; ++t) {
            if (t < L->Tq)
                kvqo_unpack_row(L->k_words + ((size_t)s * L->cap + t) * wk, d, L->k_bits, codes);
            for (int c = 0; c < d; ++c)
                kh[(size_t)t * d + c] = key_hat(L, s, t, c, codes);
            if (t < L->Tq)
                kvqo_unpack_row(L->v_words + ((size_t)s * L->cap + t) * wv, d, L->v_bits, codes);
            for (int c = 0; c < d; ++c)
                vh[(size_t)t * d + c] = value_hat(L, s, t, c, codes);
        }
        for (int h = 0; h < g; ++h) {
            for (int j = 0; j < n_q; ++j) {
                const int p = N - n_q + j; /* this query's position: keys 0..p */
                const double *qv = q + (((size_t)s * g + h) * n_q + j) * d;
                double *o = out + (((size_t)s * g + h) * n_q + j) * d;
                double m = -INFINITY;
                for (int t = 0; t <= p; ++t) {
                    double acc = 0.0;
                    for (int c = 0; c < d; ++c)
                        acc += qv[c] * kh[(size_t)t * d + c];
                    e[t] = acc * scale;
                    if (e[t] > m)
                        m = e[t];
                }
                double l = 0.0;
                for (int t = 0; t <= p; ++t) {
                    e[t] = exp(e[t] - m);
                    l += e[t];
                }
                for (int c = 0; c < d; ++c) {
                    double acc = 0.0;
                    for (int t = 0; t <= p; ++t)
                        acc += e[t] * vh[(size_t)t * d + c];
                    o[c] = acc / l;
                }
            }
        }
    }
    free(codes);
    free(vh);
    free(kh);
    free(e);
}

/* Live bytes of one stream with N tokens of which Tq are quantized.
 * Codes: Tq rows of K words and V words (4 bytes each).  K metadata: one fp32
 * scale and zero per channel per group.  V metadata: one fp32 scale and zero
 * per token.  Recent tokens: K and V at 2 bytes per element.  A (16,16) layer
 * holds N tokens at 2 bytes per element for K and V.
 * [KIVI] 2.1: the 16-bit case is 2 * head_dim * 2 bytes per token per head. */
long long kvqo_stream_bytes(int d, int k_bits, int v_bits, int G, long long N, long long Tq, int k_tok)
{
    if (k_bits == 16)
        return N * 4LL * d;
    long long Tr = N - Tq;
    long long code_bytes = Tq * 4LL * (kvqo_words_per_row(d, k_bits) + kvqo_words_per_row(d, v_bits));
    long long kmeta = k_tok ? Tq * 8LL : (Tq / G) * 8LL * d; /* per token or per group and channel */
    long long vmeta = Tq * 8LL;
    return code_bytes + kmeta + vmeta + Tr * 4LL * d;
}
