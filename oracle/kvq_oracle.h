/*
 * kvq_oracle.h -- interface of the CPU oracle (test infrastructure only).
 *
 * The oracle keeps, per layer, n_streams independent (batch, kv-head) streams.
 * Every array is allocated and owned by the caller; the oracle only reads and
 * writes through the pointers.  Shapes (cap = token capacity, a multiple of G):
 *   hist_k, hist_v   uint16 [n_streams][cap][d]   every appended token, raw
 *   k_words          uint32 [n_streams][cap][W(k_bits)]   rows 0..Tq-1 valid
 *   k_scale, k_zero  float  [n_streams][cap/G][d]         groups 0..Tq/G-1
 *                    (per-token Key, k_tok = 1: float [n_streams][cap])
 *   v_words          uint32 [n_streams][cap][W(v_bits)]
 *   v_scale, v_zero  float  [n_streams][cap]
 * Tokens [0, Tq) are quantized; tokens [Tq, N) are the recent 16-bit tokens.
 */
#ifndef KVQ_ORACLE_H
#define KVQ_ORACLE_H
#include <stdint.h>

typedef struct kvqo_layer {
    int n_streams, g, d;
    int k_bits, v_bits;   /* 2, 3 (K only), 4, 8; or 16 for both = not quantized */
    int G, R;             /* group size, recent-token capacity */
    int cap;              /* token capacity */
    int is_bf16;          /* 16-bit inputs: 0 = IEEE binary16, 1 = bfloat16 */
    int N, Tq;            /* tokens appended, tokens quantized */
    int k_tok;            /* 1: Key per token (like Value), 0: per channel over G tokens */
    int rpc_permille;     /* 0: a full recent buffer gives up its oldest G tokens;
                             r > 0: it keeps floor(r * current / 1000) of its current
                             tokens and gives up the rest, in whole groups (>= one) */
    uint16_t *hist_k, *hist_v;
    uint32_t *k_words;
    float *k_scale, *k_zero;
    uint32_t *v_words;
    float *v_scale, *v_zero;
} kvqo_layer;

float kvqo_f16_to_f32(uint16_t h);
float kvqo_bf16_to_f32(uint16_t b);
int kvqo_words_per_row(int d, int bits);
int kvqo_qmax(int bits, int c);
void kvqo_pack_row(const uint8_t *codes, int d, int bits, uint32_t *words);
void kvqo_unpack_row(const uint32_t *words, int d, int bits, uint8_t *codes);
void kvqo_quantize(const float *x, int n, long stride, int qmax,
                   uint8_t *codes, long cstride, float *s_out, float *z_out);
/* k_new, v_new: uint16 [n_streams][n][d].  Returns 0, or -1 past capacity. */
int kvqo_append(kvqo_layer *L, const uint16_t *k_new, const uint16_t *v_new, int n);
/* q, out: double [n_streams][g][d]. */
void kvqo_attention(const kvqo_layer *L, const double *q, double *out);
/* Causal attention of the queries of the last n_q appended tokens (1 <= n_q <= N):
 * q, out: double [n_streams][g][n_q][d]; query j attends to tokens 0..N-n_q+j. */
void kvqo_prefill_attention(const kvqo_layer *L, const double *q, int n_q, double *out);
long long kvqo_stream_bytes(int d, int k_bits, int v_bits, int G, long long N, long long Tq, int k_tok);

#endif
