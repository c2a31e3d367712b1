/*
 * kvq.h -- C ABI of libkvq: layer-wise mixed-precision quantized KV cache with
 * streaming quantize-and-append and decode attention, for AMD MI355X (gfx950).
 *
 * What the library computes (cited by page title and section):
 *   - Asymmetric uniform quantization Q(x) = round((x - z) / s), x^ = Q(x) s + z,
 *     z = min, s = (max - min) / qmax.  (KVTuner summary, A3 "KV cache
 *     quantization basics"; KVmix notes, key design 2.)  round() is
 *     round-half-to-even of the IEEE fp32 quotient; s and z are fp32.
 *   - Key quantized per channel over a group of G tokens (one fp32 scale and
 *     zero per kv-head per channel per group); Value quantized per token (one
 *     scale and zero per token).  (KIVI notes, sections 6.1-6.2; KVmix notes,
 *     key design 2.)
 *   - Codes packed into 32-bit words at 2, 4 or 8 bits, and for Key also the
 *     3-bit layout of eleven codes per word, ten at 3 bits and the eleventh at
 *     2 bits.  (KVmix notes, key design 2.)
 *   - Streaming: the newest tokens stay in their 16-bit input format in a
 *     recent-token buffer of R_l tokens shared by K and V; when an append finds
 *     the buffer full, its oldest G tokens are quantized first.  (KIVI notes,
 *     section 6.2; KVmix notes, key design 3 for a per-layer buffer length.)
 *   - A static per-layer (k_bits, v_bits) table such as K8V4 or K4V2, fixed at
 *     creation; no decision is taken online.  (KVTuner summary, A1 and A2.)
 *   - Decode attention o = softmax(q K^T / sqrt(head_dim)) V over every token
 *     appended so far, K and V dequantized on the fly, query heads of a GQA
 *     group sharing one K/V read.  (KVTuner summary, A3 attention equation;
 *     KIVI notes, sections 2.2 and 7.2 for GQA; KVmix notes, key design 4 for
 *     dequantizing inside the matrix-vector product.)
 *
 * Conventions
 *   - All device work is enqueued on the handle's HIP stream; calls return
 *     without waiting unless documented otherwise.  Inputs must stay valid until
 *     the stream has passed the call.  A handle is not thread-safe.
 *   - Every argument is validated on the host before any device work.  On error
 *     the call returns a negative KVQ_E* code, enqueues nothing, leaves the
 *     handle's state unchanged and records a message for kvq_last_error().
 *   - The caller owns every buffer, including the device workspace that holds
 *     the whole cache state; the library allocates no device memory.
 *   - Query head hq reads kv-head hq / g, g = n_q_heads / n_kv_heads.
 *   - Sequences of the batch hold the same number of tokens unless appended
 *     with kvq_append_ragged(); then each sequence keeps its own count, applies
 *     the streaming rule to its own recent tokens and attends to its own
 *     tokens only.
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define KVQ_OK 0
#define KVQ_EINVAL (-1)       /* bad argument (null pointer, range, shape) */
#define KVQ_ENOMEM (-2)       /* workspace missing, misaligned or too small */
#define KVQ_ECAPACITY (-3)    /* append would exceed max_context */
#define KVQ_EUNSUPPORTED (-4) /* valid request outside what the kernels support */
#define KVQ_EDEVICE (-5)      /* a HIP call failed */

/* Element formats. */
#define KVQ_F32 0
#define KVQ_F16 1  /* IEEE binary16 */
#define KVQ_BF16 2 /* bfloat16 */

/* Required alignment of the device workspace, in bytes. */
#define KVQ_WORKSPACE_ALIGN 256

/* Key quantization modes (KVTuner summary, A3 and the evaluation of the
 * KIVI and per-token-asym modes): KIVI's per-channel Key (one scale and zero
 * per channel over a group of G tokens) or per-token asymmetric Key (one scale
 * and zero per token over its head_dim channels, like Value). */
#define KVQ_K_PER_CHANNEL 0
#define KVQ_K_PER_TOKEN 1

/* The recent-token buffer of a layer gives up, when an append finds it full,
 * either its oldest G tokens (KIVI notes, section 6.2: rpc_permille = 0), or,
 * with KVmix's dynamic ratio r (KVmix notes, key design 3: num_RPC =
 * floor(r x current_RPC), 20 % for high-precision layers, 10 % for the rest),
 * all but floor(r * current / 1000) of its current tokens, rounded down to whole
 * groups of G and at least one group: r = rpc_permille in parts per thousand.
 * Either way the tokens given up are quantized exactly as a G-token flush. */

/* One row of the per-layer precision table.
 *   k_bits in {2, 3, 4, 8, 16}; v_bits in {2, 4, 8, 16}; 16 means the layer is
 *   not quantized and must be given as the pair (16, 16).
 *   residual_len: recent-token buffer length R_l for this layer; 0 selects the
 *   config's residual_len.  Must be >= group_size.  Ignored for (16, 16).
 *   k_mode: KVQ_K_PER_CHANNEL (0) or KVQ_K_PER_TOKEN (1); per-token Key needs
 *   k_bits in {2, 4, 8} (the 3-bit layout's 2-bit slot is a per-channel
 *   format).  Ignored for (16, 16).  Both modes keep the same recent-token
 *   buffer and flush G tokens at a time.
 *   rpc_permille: 0 (flush G tokens at a time) or a recent-token ratio in
 *   (0, 1000) parts per thousand, see above.  Ignored for (16, 16). */
typedef struct kvq_layer_cfg {
    int32_t k_bits;
    int32_t v_bits;
    int32_t residual_len;
    int32_t k_mode;
    int32_t rpc_permille;
} kvq_layer_cfg;

/* Cache geometry.  All counts are >= 1.
 *   n_q_heads must be a multiple of n_kv_heads, with n_q_heads / n_kv_heads
 *   <= 16; head_dim in {64, 128, 256}; kv_dtype in {KVQ_F16, KVQ_BF16};
 *   q_dtype in {KVQ_F32, KVQ_F16, KVQ_BF16}; group_size G >= 1;
 *   residual_len R >= G; layers points to n_layers rows (copied at create);
 *   stream is a hipStream_t (NULL selects the null stream).
 *
 * Paging (KIVI notes, section 8: a block-table cache manager combines with the
 * quantized cache; KVTuner summary: compatible with serving engines' paged
 * attention).  page_tokens = 0: every (sequence, kv-head) stream keeps its
 * quantized tokens in a region of its own sized for max_context.  Otherwise the
 * quantized state (codes, scales and zeros) of each quantized layer lives in a
 * pool of n_pages pages, one page holding page_tokens consecutive tokens of one
 * sequence for all its kv heads, and block_table gives the pages:
 *   page_tokens  P: a power of two, >= 128 and a multiple of group_size;
 *   n_pages      pages in each quantized layer's pool (every layer has a pool
 *                of its own, indexed by the same page ids);
 *   block_table  device memory owned by the caller, int32 [batch][table_stride],
 *                shared by all layers: entry j of row b is the page holding
 *                tokens [j P, (j + 1) P) of sequence b;
 *   table_stride entries per row, table_stride * P >= max_context.
 * The kernels read the table when they run, in stream order: before any call
 * that makes sequence b hold Tq quantized tokens in some layer (an append that
 * flushes), entries [0, ceil(Tq / P)) of row b must name pages in
 * [0, n_pages), and the pages named for different (sequence, entry) pairs must
 * differ; between calls the caller may rewrite entries of pages no longer held
 * (after kvq_reset_sequence).  An entry outside [0, n_pages) sends the kernels
 * to a spare page: memory stays safe, that sequence's results are undefined.
 * Appends check on the host that every layer's sequences fit the pool (sum over
 * b of ceil(Tq_b / P) <= n_pages; KVQ_ECAPACITY otherwise).  The recent-token
 * buffers and (16, 16) layers are not paged. */
typedef struct kvq_config {
    int32_t n_layers;
    int32_t batch;
    int32_t n_q_heads;
    int32_t n_kv_heads;
    int32_t head_dim;
    int32_t max_context;
    int32_t kv_dtype;
    int32_t q_dtype;
    int32_t group_size;
    int32_t residual_len;
    const kvq_layer_cfg *layers;
    void *stream;
    int32_t page_tokens;
    int32_t n_pages;
    const int32_t *block_table;
    int32_t table_stride;
} kvq_config;

typedef struct kvq_handle kvq_handle;

/* Bytes of device workspace kvq_create() needs for cfg (the cache at
 * max_context for every layer plus scratch for split partials).  Returns 0 if
 * cfg is invalid or unsupported; kvq_last_error(NULL) then says why. */
size_t kvq_workspace_bytes(const kvq_config *cfg);

/* Create a cache in a caller-owned device workspace of ws_bytes bytes, aligned
 * to KVQ_WORKSPACE_ALIGN, that must outlive the handle.  Every layer starts
 * empty.  Does no device work.  On success *out receives the handle.
 * Errors: KVQ_EINVAL, KVQ_EUNSUPPORTED, KVQ_ENOMEM (see kvq_last_error(NULL)). */
int kvq_create(const kvq_config *cfg, void *workspace, size_t ws_bytes, kvq_handle **out);

/* Append n_new tokens to one layer, as if appended one at a time: before each
 * token enters, a full recent-token buffer has its oldest G tokens quantized
 * (K per channel over the group, V per token) and packed.
 *   k_new, v_new: device pointers, [batch][n_kv_heads][n_new][head_dim] in
 *   kv_dtype, contiguous.  n_new == 0 is a no-op.
 * Errors: KVQ_EINVAL (bad layer, null pointer, n_new < 0), KVQ_ECAPACITY (the
 * layer would hold more than max_context tokens), KVQ_EDEVICE. */
int kvq_append(kvq_handle *h, int layer, const void *k_new, const void *v_new, int n_new);

/* Append n_new[b] tokens to sequence b of one layer (b < batch), each sequence
 * on its own as in kvq_append().  Serving batches hold sequences of different
 * lengths (KIVI notes, section 8: paging and other cache managers combine with
 * the quantized cache).
 *   k_new, v_new: device pointers, [batch][n_kv_heads][n_max][head_dim] in
 *   kv_dtype, 16-byte aligned; sequence b uses rows [0, n_new[b]).
 *   n_new: host array of batch counts, 0 <= n_new[b] <= n_max.
 * After appends of different counts the layer is ragged: decode and prefill
 * attention then take each sequence's own tokens, for batch <= 64
 * (KVQ_EUNSUPPORTED above); kvq_export_layer() refuses it (use
 * kvq_export_sequence()).
 * Errors: KVQ_EINVAL, KVQ_ECAPACITY (a sequence would exceed max_context; no
 * sequence is changed), KVQ_EDEVICE. */
int kvq_append_ragged(kvq_handle *h, int layer, const void *k_new, const void *v_new, const int32_t *n_new,
                      int n_max);

/* Tokens held (n_tokens) and quantized (n_quantized) by each sequence of a
 * layer: host arrays of batch entries; either pointer may be NULL. */
int kvq_sequence_lengths(const kvq_handle *h, int layer, int32_t *n_tokens, int32_t *n_quantized);

/* Empty sequence b in every layer (host bookkeeping only; no device work): its
 * next append starts a new sequence in that batch slot, and with paging the
 * pages it held may be named for other sequences.  Calls enqueued before still
 * see the old contents.  Errors: KVQ_EINVAL (b out of range). */
int kvq_reset_sequence(kvq_handle *h, int b);

/* Decode attention of one query token per sequence over every token of `layer`
 * (quantized tokens dequantized on the fly, recent tokens in 16 bits), scale
 * 1/sqrt(head_dim).
 *   q:   device pointer, [batch][n_q_heads][head_dim] in q_dtype, 16-byte aligned.
 *   out: device pointer, [batch][n_q_heads][head_dim] fp32, 16-byte aligned.
 * Errors: KVQ_EINVAL (bad layer, null or misaligned pointer, empty layer),
 * KVQ_EDEVICE. */
int kvq_decode_attention(kvq_handle *h, int layer, const void *q, float *out);

/* kvq_decode_attention() for callers that cannot allocate device memory or
 * must not (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation): the same kernels and the same result, bit for bit, but
 * the hand-off between the workgroups of each (sequence, kv-head) stream --
 * per-stream hand-off words and the partial results of the call's workgroups
 * -- lives in the library's static device buffer instead of the handle's
 * workspace.  That buffer is 16 MiB per GPU, allocated when the library's code
 * is loaded and held until the process ends; on each GPU it is set up (its
 * address looked up and its hand-off state initialised by one small kernel on
 * the handle's stream) by the first call made there.  This call allocates
 * nothing: no hipMalloc, no hipFree.
 * Every call on one GPU, from any handle, shares that GPU's buffer, and each
 * call leaves it in its initial state when it completes: calls that overlap in
 * time on one GPU (different streams, different threads) race and give wrong
 * results; order them on one stream or with events.
 * Errors: those of kvq_decode_attention(), and KVQ_ENOMEM when the call would
 * need more than 4096 streams (batch x n_kv_heads) or more than 16 MiB - 512
 * KiB of partial results (batch x n_kv_heads x workgroups per stream x
 * (n_q_heads / n_kv_heads) x (head_dim + 2) x 8 bytes, each stream's entries
 * rounded up to 128 bytes); nothing is enqueued then. */
int kvq_decode_attention_noalloc(kvq_handle *h, int layer, const void *q, float *out);

/* One decode step of one layer: kvq_append of one token per sequence
 * (k_new, v_new: [batch][n_kv_heads][1][head_dim]) followed by
 * kvq_decode_attention, with results identical to those two calls (state,
 * export and output).  When the append needs no flush, the new token reaches
 * the recent-token buffer inside the attention launch (one launch instead of
 * two); the streaming rule is the one of the KIVI notes, section 6.2.
 * Errors: those of the two calls; on error the layer is unchanged. */
int kvq_append_decode_attention(kvq_handle *h, int layer, const void *k_new, const void *v_new, const void *q,
                                float *out);

/* Causal attention of a prefill chunk over the cache as stored: the queries of
 * the last n_q tokens appended to `layer` (append the chunk's K and V first),
 * query j (0 <= j < n_q, position p = N - n_q + j) attending to tokens 0..p
 * (on a ragged layer N is each sequence's own length),
 * quantized tokens dequantized on the fly and recent tokens in 16 bits, scale
 * 1/sqrt(head_dim).  (KVTuner summary, A3 attention equation: the query of step
 * i attends to the keys of steps up to i; A2: calibration runs prefill attention
 * on the dequantized cache.)
 *   q:   device pointer, [batch][n_q_heads][n_q][head_dim] in q_dtype,
 *        16-byte aligned.
 *   out: device pointer, [batch][n_q_heads][n_q][head_dim] fp32, 16-byte aligned.
 *   1 <= n_q <= tokens in the layer (in its shortest sequence when ragged).
 * Supported layers: k_bits in {2, 4, 8} (either Key mode) or 3 (head_dim 128),
 * v_bits in {2, 4, 8}, with group_size a multiple of 32; or (16, 16) layers.
 * Errors: KVQ_EINVAL (bad layer, pointer or n_q), KVQ_EUNSUPPORTED (layer
 * format; a ragged layer of more than 64 sequences), KVQ_EDEVICE. */
int kvq_prefill_attention(kvq_handle *h, int layer, const void *q, int n_q, float *out);

/* Live bytes of the cache state over all layers, host arithmetic only: per
 * (sequence, kv-head): Tq rows of packed K and V codes (4 bytes per word), one
 * fp32 scale and zero per channel per K group (per-token Key: per K token),
 * one fp32 scale and zero per V token, and 2 bytes per element for the recent
 * K and V tokens; a (16, 16)
 * layer counts all its tokens at 2 bytes per element.  (KIVI notes, section 2.1
 * for the 16-bit case.)  Returns -1 for a NULL handle. */
int64_t kvq_bytes(const kvq_handle *h);

typedef struct kvq_bytes_info {
    int64_t k_codes, k_meta, v_codes, v_meta, residual, total;
    int32_t n_tokens;     /* N: tokens appended (-1: sequences differ, see
                             kvq_sequence_lengths) */
    int32_t n_quantized;  /* Tq: tokens held as codes (-1 likewise) */
    int32_t n_residual;   /* Tr = N - Tq: tokens held in 16 bits (-1 likewise) */
    int32_t k_words;      /* 32-bit words per packed K row */
    int32_t v_words;      /* 32-bit words per packed V row */
    int32_t k_bits, v_bits, residual_len;
    int32_t k_mode;       /* KVQ_K_PER_CHANNEL or KVQ_K_PER_TOKEN */
    int32_t rpc_permille; /* recent-token ratio, 0 = G tokens per flush */
} kvq_bytes_info;

/* Byte breakdown and token counts of one layer (host only). */
int kvq_bytes_layer(const kvq_handle *h, int layer, kvq_bytes_info *info);

/* Synchronously copy one layer's state to host memory in canonical order
 * (waits for the stream).  Any pointer may be NULL to skip that part.  With
 * B = batch, H = n_kv_heads, d = head_dim, Tq, Tr and words from
 * kvq_bytes_layer():
 *   k_words  uint32 [B][H][Tq][k_words]   row t = channels 0..d-1 of token t,
 *            codes least-significant bits first (3-bit: channel c in word c/11,
 *            bits 3(c%11), 2 bits wide in slot 10; unused slots 0)
 *   k_scale, k_zero  float [B][H][Tq/G][d] (per-channel Key) or
 *            float [B][H][Tq] (per-token Key)
 *   v_words  uint32 [B][H][Tq][v_words]
 *   v_scale, v_zero  float [B][H][Tq]
 *   res_k, res_v     kv_dtype [B][H][Tr][d], oldest token first
 * For a (16, 16) layer Tq = 0 and res_* hold all N tokens. */
int kvq_export_layer(kvq_handle *h, int layer, uint32_t *k_words, float *k_scale, float *k_zero,
                     uint32_t *v_words, float *v_scale, float *v_zero, void *res_k, void *res_v);

/* kvq_export_layer() for sequence b alone: the same arrays with B = 1 and
 * that sequence's Tq and Tr (kvq_sequence_lengths). */
int kvq_export_sequence(kvq_handle *h, int layer, int b, uint32_t *k_words, float *k_scale, float *k_zero,
                        uint32_t *v_words, float *v_scale, float *v_zero, void *res_k, void *res_v);

/* Wait for all work enqueued by the handle.  KVQ_EDEVICE reports an error the
 * stream raised. */
int kvq_sync(kvq_handle *h);

/* Replace the handle's stream (for calls made after this one).  All calls on
 * one handle share its cache state and its attention hand-off words and
 * partial results, so its device work must stay ordered: before switching,
 * the caller makes the new stream wait for the old one (an event, or a
 * synchronize); attention calls of one handle in flight on two streams at once
 * would mix each other's partial results. */
int kvq_set_stream(kvq_handle *h, void *stream);

/* Message of the last failed call on h; with h == NULL, of the last failed
 * kvq_workspace_bytes / kvq_create on this thread.  Never NULL. */
const char *kvq_last_error(const kvq_handle *h);

/* Release the handle (not the workspace).  Waits for the stream.  NULL is a no-op. */
void kvq_destroy(kvq_handle *h);

/* Launch configuration of the last kvq_decode_attention on h, for measurement:
 * splits per (sequence, kv-head) and kernel variant (0 = vector ALU,
 * 1 = matrix-core).  Either pointer may be NULL. */
int kvq_last_launch(const kvq_handle *h, int *splits, int *variant);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H */
