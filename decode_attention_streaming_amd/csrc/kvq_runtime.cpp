// kvq_runtime.cpp -- host side of libkvq: validation, workspace planning,
// streaming counters, kernel dispatch, byte accounting and state export.
// The C ABI is declared in include/kvq.h.
#include "kvq.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "kvq_internal.h"
#include "kvq_layout.h"

namespace {

thread_local std::string g_create_error = "no error";

constexpr int kMaxPart = 128;  // partial entries per stream (one per workgroup), as the merge supports
constexpr int kMaxUnits = 4 * kMaxPart;  // matrix-core units per stream (four per workgroup)
constexpr int kMaxG = 16;
constexpr int kMaxTileElems = 16384;  // group_size * head_dim staged by the flush kernel

struct LayerState {
    kvq::LayerDev dev;
    size_t off_kw = 0, off_km = 0, off_vw = 0, off_vm = 0, off_rk = 0, off_rv = 0;
    int N = 0, Tq = 0;     // tokens appended and quantized, when every sequence has as many
    int rpc_permille = 0;  // recent-token ratio (0: G tokens per flush)
    // per sequence: tokens appended and quantized; ragged when they differ
    // (N and Tq above are then those of the longest sequence)
    std::vector<int> seqN, seqTq;
    bool ragged = false;
};

// Tokens quantized after n appends to a stream holding N0 tokens, Tq0 of them
// quantized: before each token enters, a full recent buffer (R tokens) gives
// up its oldest G tokens, or, with a recent-token ratio r, all but
// floor(r * R) of them in whole groups (at least one group).
int tq_after(const kvq::LayerDev &d, int rpc_permille, int N0, int Tq0, int n)
{
    int Tq1 = Tq0;
    if (d.kb == 16 || N0 + n <= d.R)
        return Tq1;
    if (rpc_permille == 0) {
        Tq1 = (N0 + n - d.R + d.G - 1) / d.G * d.G;
        return Tq1 < Tq0 ? Tq0 : Tq1;
    }
    int n_flush = d.G;
    const int keep = static_cast<int>(static_cast<long>(d.R) * rpc_permille / 1000);
    if ((d.R - keep) / d.G * d.G > n_flush)
        n_flush = (d.R - keep) / d.G * d.G;
    for (int N = N0; N < N0 + n; ++N)
        if (N - Tq1 == d.R)
            Tq1 += n_flush;
    return Tq1;
}

// View of streams [s0, ...) of a layer as a layer of its own.
kvq::LayerDev sub_layer(const kvq::LayerDev &d, int s0, int D)
{
    kvq::LayerDev v = d;
    const size_t S = static_cast<size_t>(s0);
    if (d.table) {
        v.bh0 = d.bh0 + s0;  // pooled pages: the streams' rows come from the table
    } else if (d.kb != 16) {
        v.k_words += S * d.capq * d.wk;
        v.k_meta += d.k_tok ? S * d.capq * 2 : S * (d.capq / d.G) * 2 * D;
        v.v_words += S * d.capq * d.wv;
        v.v_meta += S * d.capq * 2;
    }
    v.ring_k += S * d.R * D;
    v.ring_v += S * d.R * D;
    return v;
}

struct Plan {
    std::vector<LayerState> layers;
    size_t off_part = 0;
    size_t off_cnt = 0;
    size_t total = 0;
    int v_tiled = 0;
};

int words_per_row(int d, int bits)
{
    if (bits == 3)
        return (d + 10) / 11;
    return d * bits / 32;
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

bool valid_pair(int kb, int vb)
{
    if (kb == 16 || vb == 16)
        return kb == 16 && vb == 16;
    return (kb == 2 || kb == 3 || kb == 4 || kb == 8) && (vb == 2 || vb == 4 || vb == 8);
}

// Validates cfg and lays the workspace out.  Returns KVQ_OK or an error code
// with a message in err.
int plan_layout(const kvq_config *cfg, Plan *plan, std::string *err)
{
    char buf[256];
    auto fail = [&](int code, const char *fmt, ...) {
        va_list ap;
        va_start(ap, fmt);
        vsnprintf(buf, sizeof buf, fmt, ap);
        va_end(ap);
        *err = buf;
        return code;
    };
    if (!cfg)
        return fail(KVQ_EINVAL, "config is NULL");
    if (cfg->n_layers < 1 || cfg->batch < 1 || cfg->n_q_heads < 1 || cfg->n_kv_heads < 1 ||
        cfg->head_dim < 1 || cfg->max_context < 1 || cfg->group_size < 1)
        return fail(KVQ_EINVAL, "n_layers, batch, heads, head_dim, max_context and group_size must be >= 1");
    if (!cfg->layers)
        return fail(KVQ_EINVAL, "layer table is NULL");
    if (cfg->n_q_heads % cfg->n_kv_heads != 0)
        return fail(KVQ_EINVAL, "n_q_heads (%d) is not a multiple of n_kv_heads (%d)", cfg->n_q_heads,
                    cfg->n_kv_heads);
    if (cfg->n_q_heads / cfg->n_kv_heads > kMaxG)
        return fail(KVQ_EUNSUPPORTED, "more than %d query heads per kv-head", kMaxG);
    if (cfg->head_dim != 64 && cfg->head_dim != 128 && cfg->head_dim != 256)
        return fail(KVQ_EUNSUPPORTED, "head_dim %d not in {64, 128, 256}", cfg->head_dim);
    if (cfg->kv_dtype != KVQ_F16 && cfg->kv_dtype != KVQ_BF16)
        return fail(KVQ_EINVAL, "kv_dtype must be KVQ_F16 or KVQ_BF16");
    if (cfg->q_dtype != KVQ_F32 && cfg->q_dtype != KVQ_F16 && cfg->q_dtype != KVQ_BF16)
        return fail(KVQ_EINVAL, "q_dtype must be KVQ_F32, KVQ_F16 or KVQ_BF16");
    if (cfg->residual_len < cfg->group_size)
        return fail(KVQ_EINVAL, "residual_len (%d) < group_size (%d)", cfg->residual_len, cfg->group_size);
    if (static_cast<long>(cfg->group_size) * cfg->head_dim > kMaxTileElems)
        return fail(KVQ_EUNSUPPORTED, "group_size * head_dim = %ld exceeds %d", 
                    static_cast<long>(cfg->group_size) * cfg->head_dim, kMaxTileElems);

    const size_t BH = static_cast<size_t>(cfg->batch) * cfg->n_kv_heads;
    const int D = cfg->head_dim, G = cfg->group_size;
    const size_t A = KVQ_WORKSPACE_ALIGN;
    const int P = cfg->page_tokens;
    int P_log2 = 0;
    if (P != 0) {
        if (P < 128 || (P & (P - 1)) != 0 || P % G != 0)
            return fail(KVQ_EINVAL, "page_tokens %d must be 0, or a power of two >= 128 and a multiple of group_size %d",
                        P, G);
        while ((1 << P_log2) < P)
            ++P_log2;
        if (cfg->n_pages < 1)
            return fail(KVQ_EINVAL, "n_pages must be >= 1 with page_tokens %d", P);
        if (!cfg->block_table)
            return fail(KVQ_EINVAL, "block_table is NULL with page_tokens %d", P);
        if (static_cast<long>(cfg->table_stride) * P < cfg->max_context)
            return fail(KVQ_EINVAL, "table_stride %d x page_tokens %d < max_context %d", cfg->table_stride, P,
                        cfg->max_context);
    }
    size_t off = 0;
    plan->layers.assign(cfg->n_layers, LayerState());
    // V codes use the matrix-core tile layout when groups are whole 32-token blocks
    plan->v_tiled = (G % 32 == 0) ? 1 : 0;
    const int cap_unit = G;
    for (int l = 0; l < cfg->n_layers; ++l) {
        const kvq_layer_cfg &lc = cfg->layers[l];
        if (!valid_pair(lc.k_bits, lc.v_bits))
            return fail(KVQ_EINVAL, "layer %d: (k_bits, v_bits) = (%d, %d) not supported", l, lc.k_bits,
                        lc.v_bits);
        if (lc.k_mode != KVQ_K_PER_CHANNEL && lc.k_mode != KVQ_K_PER_TOKEN)
            return fail(KVQ_EINVAL, "layer %d: k_mode %d is neither per-channel (0) nor per-token (1)", l,
                        lc.k_mode);
        if (lc.rpc_permille < 0 || lc.rpc_permille >= 1000)
            return fail(KVQ_EINVAL, "layer %d: rpc_permille %d outside [0, 1000)", l, lc.rpc_permille);
        if (lc.k_mode == KVQ_K_PER_TOKEN && lc.k_bits == 3)
            return fail(KVQ_EUNSUPPORTED, "layer %d: per-token Key needs k_bits 2, 4 or 8", l);
        LayerState &s = plan->layers[l];
        s.seqN.assign(cfg->batch, 0);
        s.seqTq.assign(cfg->batch, 0);
        kvq::LayerDev &d = s.dev;
        d.kb = lc.k_bits;
        d.vb = lc.v_bits;
        d.G = G;
        d.v_tiled = plan->v_tiled;
        d.k_tok = (lc.k_mode == KVQ_K_PER_TOKEN && lc.k_bits != 16) ? 1 : 0;
        s.rpc_permille = lc.k_bits != 16 ? lc.rpc_permille : 0;
        d.table = nullptr;  // set at create for paged quantized layers
        d.P_log2 = P_log2;
        d.Hkv = cfg->n_kv_heads;
        d.tstride = cfg->table_stride;
        d.n_pages = cfg->n_pages;
        d.bh0 = 0;
        d.gpp = P != 0 ? P / G : 0;
        if (d.kb == 16) {
            d.R = cfg->max_context;
            d.capq = G;  // unused
            d.ngq = 1;
            d.wk = d.wv = 0;
        } else {
            d.R = lc.residual_len == 0 ? cfg->residual_len : lc.residual_len;
            if (d.R < G)
                return fail(KVQ_EINVAL, "layer %d: residual_len (%d) < group_size (%d)", l, d.R, G);
            if (d.R < 0 || d.R > cfg->max_context + G)
                return fail(KVQ_EINVAL, "layer %d: residual_len %d out of range", l, d.R);
            d.capq = (cfg->max_context + cap_unit - 1) / cap_unit * cap_unit;
            d.ngq = d.capq / G;
            d.wk = words_per_row(D, d.kb);
            d.wv = words_per_row(D, d.vb);
        }
        if (d.kb != 16 && P != 0) {
            // a pool of n_pages pages (+ the spare page) of P tokens for all kv heads
            const size_t rows = (static_cast<size_t>(cfg->n_pages) + 1) * cfg->n_kv_heads * P;
            s.off_kw = off;
            off = align_up(off + rows * d.wk * 4, A);
            s.off_km = off;
            off = align_up(off + (d.k_tok ? rows * 2 * 4 : rows / G * 2 * D * 4), A);
            s.off_vw = off;
            off = align_up(off + rows * d.wv * 4, A);
            s.off_vm = off;
            off = align_up(off + rows * 2 * 4, A);
        } else if (d.kb != 16) {
            s.off_kw = off;
            off = align_up(off + BH * d.capq * d.wk * 4, A);
            s.off_km = off;
            off = align_up(off + (d.k_tok ? BH * d.capq * 2 * 4 : BH * (d.capq / G) * 2 * D * 4), A);
            s.off_vw = off;
            off = align_up(off + BH * d.capq * d.wv * 4, A);
            s.off_vm = off;
            off = align_up(off + BH * d.capq * 2 * 4, A);
        }
        s.off_rk = off;
        off = align_up(off + BH * static_cast<size_t>(d.R) * D * 2, A);
        s.off_rv = off;
        off = align_up(off + BH * static_cast<size_t>(d.R) * D * 2, A);
    }
    plan->off_part = off;
    off = align_up(off + BH * kMaxPart * static_cast<size_t>(kvq::part_entry_floats(cfg->n_q_heads / cfg->n_kv_heads, D)) * 4,
                   A);
    plan->off_cnt = off;
    off = align_up(off + BH * 4 * kvq::kCounterStride, A);
    plan->total = off;
    return KVQ_OK;
}

}  // namespace

struct kvq_handle {
    kvq_config cfg;
    std::vector<kvq_layer_cfg> table;
    Plan plan;
    char *ws = nullptr;
    size_t ws_bytes = 0;
    hipStream_t stream = nullptr;
    int cu_count = 0;
    int last_splits = 0, last_variant = -1;
    // launch-shape overrides for tests and tuning, read once at create from
    // KVQ_FORCE_VALU, KVQ_UNIT_GROUPS, KVQ_UNITS_Q, KVQ_RES_TOKENS, KVQ_SPLITS,
    // KVQ_NO_PIPE (0 = not set)
    int env_force_valu = 0, env_unit_groups = 0, env_units_q = 0, env_res_tokens = 0, env_splits = 0,
        env_no_pipe = 0;
    bool touched = false;  // device work was enqueued
    bool counters_ready = false;
    std::string err = "no error";

    int fail(int code, const char *fmt, ...)
    {
        char buf[256];
        va_list ap;
        va_start(ap, fmt);
        vsnprintf(buf, sizeof buf, fmt, ap);
        va_end(ap);
        err = buf;
        return code;
    }
    int dev_fail(hipError_t e, const char *what)
    {
        return fail(KVQ_EDEVICE, "%s: %s", what, hipGetErrorString(e));
    }
    int BH() const { return cfg.batch * cfg.n_kv_heads; }
};

extern "C" {

size_t kvq_workspace_bytes(const kvq_config *cfg)
{
    Plan p;
    std::string err;
    if (plan_layout(cfg, &p, &err) != KVQ_OK) {
        g_create_error = err;
        return 0;
    }
    return p.total;
}

int kvq_create(const kvq_config *cfg, void *workspace, size_t ws_bytes, kvq_handle **out)
{
    if (!out) {
        g_create_error = "out is NULL";
        return KVQ_EINVAL;
    }
    *out = nullptr;
    Plan p;
    std::string err;
    int rc = plan_layout(cfg, &p, &err);
    if (rc != KVQ_OK) {
        g_create_error = err;
        return rc;
    }
    if (!workspace) {
        g_create_error = "workspace is NULL";
        return KVQ_ENOMEM;
    }
    if (reinterpret_cast<uintptr_t>(workspace) % KVQ_WORKSPACE_ALIGN != 0) {
        g_create_error = "workspace is not 256-byte aligned";
        return KVQ_ENOMEM;
    }
    if (ws_bytes < p.total) {
        char buf[160];
        snprintf(buf, sizeof buf, "workspace too small: %zu bytes given, %zu needed", ws_bytes, p.total);
        g_create_error = buf;
        return KVQ_ENOMEM;
    }
    kvq_handle *h = new kvq_handle();
    h->cfg = *cfg;
    h->table.assign(cfg->layers, cfg->layers + cfg->n_layers);
    h->cfg.layers = h->table.data();
    h->plan = std::move(p);
    h->ws = static_cast<char *>(workspace);
    h->ws_bytes = ws_bytes;
    h->stream = static_cast<hipStream_t>(cfg->stream);
    auto env_int = [](const char *name) {
        const char *v = getenv(name);
        const int x = v ? atoi(v) : 0;
        return x > 0 ? x : 0;
    };
    h->env_force_valu = env_int("KVQ_FORCE_VALU");
    h->env_unit_groups = env_int("KVQ_UNIT_GROUPS");
    h->env_units_q = env_int("KVQ_UNITS_Q");
    h->env_res_tokens = env_int("KVQ_RES_TOKENS");
    h->env_splits = env_int("KVQ_SPLITS");
    h->env_no_pipe = env_int("KVQ_NO_PIPE");
    const size_t BH = static_cast<size_t>(h->BH());
    for (LayerState &s : h->plan.layers) {
        kvq::LayerDev &d = s.dev;
        if (d.kb != 16) {
            d.k_words = reinterpret_cast<uint32_t *>(h->ws + s.off_kw);
            d.k_meta = reinterpret_cast<float *>(h->ws + s.off_km);
            d.v_words = reinterpret_cast<uint32_t *>(h->ws + s.off_vw);
            d.v_meta = reinterpret_cast<float *>(h->ws + s.off_vm);
        }
        d.ring_k = reinterpret_cast<uint16_t *>(h->ws + s.off_rk);
        d.ring_v = reinterpret_cast<uint16_t *>(h->ws + s.off_rv);
        if (cfg->page_tokens != 0 && d.kb != 16)
            d.table = cfg->block_table;
        (void)BH;
    }
    *out = h;
    return KVQ_OK;
}

static int append_streams(kvq_handle *h, const kvq::LayerDev &dl, int s0, int nbh, const void *k_new,
                          const void *v_new, int stride, int n, int N0, int Tq0, int rpc_permille, int *Tq_out);
static int append_sequences(kvq_handle *h, int layer, const void *k_new, const void *v_new, const int32_t *n_new,
                            int n_max);
static void refresh_lengths(LayerState &s);

// Paged layers: pages the layer's sequences occupy when sequence b holds tq[b]
// quantized tokens must fit its pool.
static int check_pages(kvq_handle *h, int layer, const std::vector<int> &tq)
{
    const int P = h->cfg.page_tokens;
    const LayerState &s = h->plan.layers[layer];
    if (P == 0 || s.dev.kb == 16)
        return KVQ_OK;
    long pages = 0;
    for (int t : tq)
        pages += (t + P - 1) / P;
    if (pages > h->cfg.n_pages)
        return h->fail(KVQ_ECAPACITY, "layer %d: its sequences would occupy %ld pages of %d tokens; the pool has %d",
                       layer, pages, P, h->cfg.n_pages);
    return KVQ_OK;
}

int kvq_append(kvq_handle *h, int layer, const void *k_new, const void *v_new, int n_new)
{
    if (!h)
        return KVQ_EINVAL;
    if (layer < 0 || layer >= h->cfg.n_layers)
        return h->fail(KVQ_EINVAL, "layer %d out of range [0, %d)", layer, h->cfg.n_layers);
    if (n_new < 0)
        return h->fail(KVQ_EINVAL, "n_new = %d < 0", n_new);
    if (n_new == 0)
        return KVQ_OK;
    if (!k_new || !v_new)
        return h->fail(KVQ_EINVAL, "k_new or v_new is NULL");
    if (reinterpret_cast<uintptr_t>(k_new) % 16 || reinterpret_cast<uintptr_t>(v_new) % 16)
        return h->fail(KVQ_EINVAL, "k_new and v_new must be 16-byte aligned");
    LayerState &s = h->plan.layers[layer];
    const kvq::LayerDev &d = s.dev;
    if (static_cast<long>(s.N) + n_new > h->cfg.max_context)
        return h->fail(KVQ_ECAPACITY, "layer %d: %d + %d tokens exceed max_context %d", layer, s.N, n_new,
                       h->cfg.max_context);

    if (!s.ragged) {
        int Tq1 = 0;
        int rc = check_pages(h, layer, std::vector<int>(h->cfg.batch, tq_after(d, s.rpc_permille, s.N, s.Tq, n_new)));
        if (rc != KVQ_OK)
            return rc;
        rc = append_streams(h, d, 0, h->BH(), k_new, v_new, n_new, n_new, s.N, s.Tq, s.rpc_permille, &Tq1);
        if (rc != KVQ_OK)
            return rc;
        s.N += n_new;
        s.Tq = Tq1;
        s.seqN.assign(h->cfg.batch, s.N);
        s.seqTq.assign(h->cfg.batch, s.Tq);
        return KVQ_OK;
    }
    std::vector<int> n(h->cfg.batch, n_new);
    return append_sequences(h, layer, k_new, v_new, n.data(), n_new);
}

// Append n tokens to streams [s0, s0 + nbh) of a layer, all holding N0 tokens
// of which Tq0 are quantized: one flush launch for every group the appends
// give up, then the ring write of the tokens that stay recent.  New tokens of
// stream i are rows [i][0 .. n) of [nbh][stride][D].
static int append_streams(kvq_handle *h, const kvq::LayerDev &dl, int s0, int nbh, const void *k_new,
                          const void *v_new, int stride, int n, int N0, int Tq0, int rpc_permille, int *Tq_out)
{
    const int D = h->cfg.head_dim;
    const kvq::LayerDev d = s0 == 0 ? dl : sub_layer(dl, s0, D);
    const int N1 = N0 + n;
    const int Tq1 = tq_after(d, rpc_permille, N0, Tq0, n);
    const int bf16 = h->cfg.kv_dtype == KVQ_BF16;
    hipError_t e;
    const int t_first = Tq1 > N0 ? Tq1 : N0;
    const bool fuse_ring = Tq1 > Tq0 && n == 1 && N1 > t_first;
    if (Tq1 > Tq0) {
        kvq::FlushArgs fa;
        fa.L = d;
        fa.k_new = static_cast<const uint16_t *>(k_new);
        fa.v_new = static_cast<const uint16_t *>(v_new);
        fa.D = D;
        fa.n_new = stride;
        fa.N0 = N0;
        fa.Tq0 = Tq0;
        fa.n_groups = (Tq1 - Tq0) / d.G;
        fa.BH = nbh;
        fa.kv_bf16 = bf16;
        fa.ring_after = fuse_ring ? 1 : 0;
        e = kvq::launch_flush(fa, h->stream);
        if (e != hipSuccess)
            return h->dev_fail(e, "flush launch");
    }
    if (N1 > t_first && !fuse_ring) {
        kvq::RingArgs ra;
        ra.L = d;
        ra.k_new = static_cast<const uint16_t *>(k_new);
        ra.v_new = static_cast<const uint16_t *>(v_new);
        ra.D = D;
        ra.n_new = stride;
        ra.N0 = N0;
        ra.t_first = t_first;
        ra.t_last = N1;
        ra.BH = nbh;
        e = kvq::launch_ring_write(ra, h->stream);
        if (e != hipSuccess)
            return h->dev_fail(e, "ring write launch");
    }
    *Tq_out = Tq1;
    h->touched = true;
    return KVQ_OK;
}

// Sequence b appends n_new[b] tokens, rows [b][h][0 .. n_new[b]) of
// [batch][n_kv_heads][n_max][D]; one flush / ring launch per sequence that
// appends.  Arguments are already checked.
static int append_sequences(kvq_handle *h, int layer, const void *k_new, const void *v_new, const int32_t *n_new,
                            int n_max)
{
    LayerState &s = h->plan.layers[layer];
    const int Hkv = h->cfg.n_kv_heads, D = h->cfg.head_dim;
    const size_t seq_elems = static_cast<size_t>(Hkv) * n_max * D;
    std::vector<int> tq1(h->cfg.batch);
    for (int b = 0; b < h->cfg.batch; ++b)
        tq1[b] = tq_after(s.dev, s.rpc_permille, s.seqN[b], s.seqTq[b], n_new[b]);
    const int rc0 = check_pages(h, layer, tq1);
    if (rc0 != KVQ_OK)
        return rc0;
    for (int b = 0; b < h->cfg.batch; ++b) {
        if (n_new[b] == 0)
            continue;
        int Tq1 = 0;
        const int rc = append_streams(h, s.dev, b * Hkv, Hkv, static_cast<const uint16_t *>(k_new) + b * seq_elems,
                                      static_cast<const uint16_t *>(v_new) + b * seq_elems, n_max, n_new[b], s.seqN[b],
                                      s.seqTq[b], s.rpc_permille, &Tq1);
        if (rc != KVQ_OK)
            return rc;
        s.seqN[b] += n_new[b];
        s.seqTq[b] = Tq1;
    }
    refresh_lengths(s);
    return KVQ_OK;
}

// Uniform view of the per-sequence lengths: ragged when they differ; N and Tq
// are those of the longest sequence.
static void refresh_lengths(LayerState &s)
{
    int b_max = 0;
    s.ragged = false;
    for (size_t b = 0; b < s.seqN.size(); ++b) {
        if (s.seqN[b] != s.seqN[0])
            s.ragged = true;
        if (s.seqN[b] > s.seqN[b_max])
            b_max = static_cast<int>(b);
    }
    s.N = s.seqN[b_max];
    s.Tq = s.seqTq[b_max];
}

int kvq_append_ragged(kvq_handle *h, int layer, const void *k_new, const void *v_new, const int32_t *n_new,
                      int n_max)
{
    if (!h)
        return KVQ_EINVAL;
    if (layer < 0 || layer >= h->cfg.n_layers)
        return h->fail(KVQ_EINVAL, "layer %d out of range [0, %d)", layer, h->cfg.n_layers);
    if (!n_new)
        return h->fail(KVQ_EINVAL, "n_new is NULL");
    if (n_max < 0)
        return h->fail(KVQ_EINVAL, "n_max = %d < 0", n_max);
    LayerState &s = h->plan.layers[layer];
    bool any = false, equal = true;
    for (int b = 0; b < h->cfg.batch; ++b) {
        if (n_new[b] < 0 || n_new[b] > n_max)
            return h->fail(KVQ_EINVAL, "n_new[%d] = %d outside [0, n_max = %d]", b, n_new[b], n_max);
        if (static_cast<long>(s.seqN[b]) + n_new[b] > h->cfg.max_context)
            return h->fail(KVQ_ECAPACITY, "layer %d, sequence %d: %d + %d tokens exceed max_context %d", layer, b,
                           s.seqN[b], n_new[b], h->cfg.max_context);
        any = any || n_new[b] > 0;
        equal = equal && n_new[b] == n_max;
    }
    if (!any)
        return KVQ_OK;
    if (!k_new || !v_new)
        return h->fail(KVQ_EINVAL, "k_new or v_new is NULL");
    if (reinterpret_cast<uintptr_t>(k_new) % 16 || reinterpret_cast<uintptr_t>(v_new) % 16)
        return h->fail(KVQ_EINVAL, "k_new and v_new must be 16-byte aligned");
    if (equal && !s.ragged)
        return kvq_append(h, layer, k_new, v_new, n_max);
    return append_sequences(h, layer, k_new, v_new, n_new, n_max);
}

int kvq_reset_sequence(kvq_handle *h, int b)
{
    if (!h)
        return KVQ_EINVAL;
    if (b < 0 || b >= h->cfg.batch)
        return h->fail(KVQ_EINVAL, "sequence %d out of range [0, %d)", b, h->cfg.batch);
    for (LayerState &s : h->plan.layers) {
        s.seqN[b] = 0;
        s.seqTq[b] = 0;
        refresh_lengths(s);
    }
    return KVQ_OK;
}

int kvq_sequence_lengths(const kvq_handle *h, int layer, int32_t *n_tokens, int32_t *n_quantized)
{
    if (!h)
        return KVQ_EINVAL;
    if (layer < 0 || layer >= h->cfg.n_layers)
        return const_cast<kvq_handle *>(h)->fail(KVQ_EINVAL, "layer %d out of range", layer);
    const LayerState &s = h->plan.layers[layer];
    for (int b = 0; b < h->cfg.batch; ++b) {
        if (n_tokens)
            n_tokens[b] = s.seqN[b];
        if (n_quantized)
            n_quantized[b] = s.seqTq[b];
    }
    return KVQ_OK;
}


// Arguments of a decode-attention call, checked before any state changes.
static int check_attention_args(kvq_handle *h, int layer, const void *q, const float *out)
{
    if (layer < 0 || layer >= h->cfg.n_layers)
        return h->fail(KVQ_EINVAL, "layer %d out of range [0, %d)", layer, h->cfg.n_layers);
    if (!q || !out)
        return h->fail(KVQ_EINVAL, "q or out is NULL");
    if (reinterpret_cast<uintptr_t>(q) % 16 || reinterpret_cast<uintptr_t>(out) % 16)
        return h->fail(KVQ_EINVAL, "q and out must be 16-byte aligned");
    return KVQ_OK;
}

// One attention launch over the layer's current state.  new_t >= 0: token
// new_t was appended but is not in the ring yet (its rows are new_k / new_v);
// the launch also stores it there.
static int attention_launch(kvq_handle *h, int layer, const void *q, float *out, const void *new_k,
                            const void *new_v, int new_t, const int *seq_new_t = nullptr,
                            bool static_scratch = false);

int kvq_decode_attention(kvq_handle *h, int layer, const void *q, float *out)
{
    if (!h)
        return KVQ_EINVAL;
    const int rc = check_attention_args(h, layer, q, out);
    if (rc != KVQ_OK)
        return rc;
    const LayerState &s = h->plan.layers[layer];
    for (int b = 0; b < h->cfg.batch; ++b)
        if (s.seqN[b] == 0)
            return h->fail(KVQ_EINVAL, "layer %d holds no tokens for sequence %d", layer, b);
    return attention_launch(h, layer, q, out, nullptr, nullptr, -1);
}

int kvq_decode_attention_noalloc(kvq_handle *h, int layer, const void *q, float *out)
{
    if (!h)
        return KVQ_EINVAL;
    const int rc = check_attention_args(h, layer, q, out);
    if (rc != KVQ_OK)
        return rc;
    const LayerState &s = h->plan.layers[layer];
    for (int b = 0; b < h->cfg.batch; ++b)
        if (s.seqN[b] == 0)
            return h->fail(KVQ_EINVAL, "layer %d holds no tokens for sequence %d", layer, b);
    return attention_launch(h, layer, q, out, nullptr, nullptr, -1, nullptr, true);
}

int kvq_append_decode_attention(kvq_handle *h, int layer, const void *k_new, const void *v_new, const void *q,
                                float *out)
{
    if (!h)
        return KVQ_EINVAL;
    int rc = check_attention_args(h, layer, q, out);
    if (rc != KVQ_OK)
        return rc;
    if (!k_new || !v_new)
        return h->fail(KVQ_EINVAL, "k_new or v_new is NULL");
    if (reinterpret_cast<uintptr_t>(k_new) % 16 || reinterpret_cast<uintptr_t>(v_new) % 16)
        return h->fail(KVQ_EINVAL, "k_new and v_new must be 16-byte aligned");
    LayerState &s = h->plan.layers[layer];
    const kvq::LayerDev &d = s.dev;
    if (static_cast<long>(s.N) + 1 > h->cfg.max_context)
        return h->fail(KVQ_ECAPACITY, "layer %d: %d + 1 tokens exceed max_context %d", layer, s.N,
                       h->cfg.max_context);
    if (s.ragged) {
        // per sequence: a full recent buffer is flushed first (its flush launch
        // also stores the new token); otherwise the attention launch stores it
        if (h->cfg.batch > kvq::kMaxRaggedSeqs)
            return h->fail(KVQ_EUNSUPPORTED, "sequences of different lengths: batch %d exceeds %d",
                           h->cfg.batch, kvq::kMaxRaggedSeqs);
        const int Hkv = h->cfg.n_kv_heads, D = h->cfg.head_dim;
        std::vector<int> tq1(h->cfg.batch);
        for (int b = 0; b < h->cfg.batch; ++b)
            tq1[b] = tq_after(d, s.rpc_permille, s.seqN[b], s.seqTq[b], 1);
        rc = check_pages(h, layer, tq1);
        if (rc != KVQ_OK)
            return rc;
        std::vector<int> nt(h->cfg.batch, -1);
        for (int b = 0; b < h->cfg.batch; ++b) {
            const size_t off = static_cast<size_t>(b) * Hkv * D;
            if (d.kb != 16 && s.seqN[b] - s.seqTq[b] == d.R) {
                int Tq1 = 0;
                rc = append_streams(h, d, b * Hkv, Hkv, static_cast<const uint16_t *>(k_new) + off,
                                    static_cast<const uint16_t *>(v_new) + off, 1, 1, s.seqN[b], s.seqTq[b],
                                    s.rpc_permille, &Tq1);
                if (rc != KVQ_OK)
                    return rc;
                s.seqTq[b] = Tq1;
            } else {
                nt[b] = s.seqN[b];
            }
            s.seqN[b] += 1;
        }
        refresh_lengths(s);
        return attention_launch(h, layer, q, out, k_new, v_new, -1, nt.data());
    }
    const bool flush = d.kb != 16 && s.N - s.Tq == d.R;  // the recent buffer is full
    if (flush) {
        rc = kvq_append(h, layer, k_new, v_new, 1);
        if (rc != KVQ_OK)
            return rc;
        return attention_launch(h, layer, q, out, nullptr, nullptr, -1);
    }
    const int t = s.N;
    s.N = t + 1;
    rc = attention_launch(h, layer, q, out, k_new, v_new, t);
    if (rc != KVQ_OK)
        s.N = t;
    s.seqN.assign(h->cfg.batch, s.N);
    return rc;
}

// Compute units of device dev, read once per handle (launch shapes depend on it).
static hipError_t ensure_cu_count(kvq_handle *h, int dev)
{
    if (h->cu_count == 0) {
        int n = 0;
        const hipError_t e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess)
            return e;
        h->cu_count = n > 0 ? n : 256;
    }
    return hipSuccess;
}

int kvq_prefill_attention(kvq_handle *h, int layer, const void *q, int n_q, float *out)
{
    if (!h)
        return KVQ_EINVAL;
    const int rc = check_attention_args(h, layer, q, out);
    if (rc != KVQ_OK)
        return rc;
    const LayerState &s = h->plan.layers[layer];
    const kvq::LayerDev &d = s.dev;
    int n_min = s.N;
    if (s.ragged) {
        if (h->cfg.batch > kvq::kMaxRaggedSeqs)
            return h->fail(KVQ_EUNSUPPORTED, "a ragged layer's prefill attention takes at most %d sequences",
                           kvq::kMaxRaggedSeqs);
        n_min = *std::min_element(s.seqN.begin(), s.seqN.end());
    }
    if (n_q < 1 || n_q > n_min)
        return h->fail(KVQ_EINVAL, "n_q = %d outside [1, %d] (tokens in the shortest sequence of layer %d)", n_q,
                       n_min, layer);
    const int D = h->cfg.head_dim;
    if (!kvq::prefill_supported(d.kb, d.vb, D, d.v_tiled))
        return h->fail(KVQ_EUNSUPPORTED,
                       "layer %d: prefill attention needs k_bits in {2, 3 (head_dim 128), 4, 8} and v_bits in "
                       "{2, 4, 8} with group_size a multiple of 32, or a (16, 16) layer (layer is K%dV%d, "
                       "group_size %d)",
                       layer, d.kb, d.vb, d.G);
    const int g = h->cfg.n_q_heads / h->cfg.n_kv_heads;
    kvq::PrefillArgs a;
    a.L = d;
    a.q = q;
    a.out = out;
    a.q_dtype = h->cfg.q_dtype;
    a.kv_bf16 = h->cfg.kv_dtype == KVQ_BF16;
    a.D = D;
    a.g = g;
    a.BH = h->BH();
    a.N = s.N;
    a.Tq = s.Tq;
    a.n_q = n_q;
    a.ragged = s.ragged ? 1 : 0;
    a.Hkv = h->cfg.n_kv_heads;
    for (int b = 0; b < kvq::kMaxRaggedSeqs; ++b) {
        a.seqN[b] = s.ragged && b < h->cfg.batch ? s.seqN[b] : 0;
        a.seqTq[b] = s.ragged && b < h->cfg.batch ? s.seqTq[b] : 0;
    }
    a.QT = 16 / g;
    a.n_tiles = (n_q + a.QT - 1) / a.QT;
    // workgroups of eight waves, each on one stream: two query tiles per wave
    // (up to head_dim 128) when that still leaves a workgroup for every
    // compute unit, else one
    int dev = 0;
    hipError_t e0 = hipGetDevice(&dev);
    if (e0 == hipSuccess)
        e0 = ensure_cu_count(h, dev);
    if (e0 != hipSuccess)
        return h->dev_fail(e0, "device query");
    a.tw = 1;
    if (D <= 128 && static_cast<long>(a.BH) * ((a.n_tiles + 15) / 16) >= h->cu_count)
        a.tw = 2;
    const int tiles_wg = 8 * a.tw;
    a.wg_per_stream = (a.n_tiles + tiles_wg - 1) / tiles_wg;
    const long wgs = static_cast<long>(a.BH) * a.wg_per_stream;
    if (wgs > INT32_MAX / 2)
        return h->fail(KVQ_EUNSUPPORTED, "%ld prefill workgroups exceed one launch", wgs);
    a.n_wg = static_cast<int>(wgs);
    a.ngcap = d.capq / d.G;
    a.scale_log2 = static_cast<float>(1.4426950408889634 / std::sqrt(static_cast<double>(D)));
    const hipError_t e = kvq::launch_prefill(a, h->stream);
    if (e != hipSuccess)
        return h->dev_fail(e, "prefill attention launch");
    h->touched = true;
    return KVQ_OK;
}

static int attention_launch(kvq_handle *h, int layer, const void *q, float *out, const void *new_k,
                            const void *new_v, int new_t, const int *seq_new_t, bool static_scratch)
{
    LayerState &s = h->plan.layers[layer];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return h->dev_fail(e, "device query");
    e = ensure_cu_count(h, dev);
    if (e != hipSuccess)
        return h->dev_fail(e, "device query");
    const int D = h->cfg.head_dim, BH = h->BH();
    const kvq::LayerDev &d = s.dev;
    kvq::AttnArgs a;
    a.L = d;
    a.q = q;
    a.out = out;
    a.q_dtype = h->cfg.q_dtype;
    a.kv_bf16 = h->cfg.kv_dtype == KVQ_BF16;
    a.D = D;
    a.g = h->cfg.n_q_heads / h->cfg.n_kv_heads;
    a.Hkv = h->cfg.n_kv_heads;
    a.N = s.N;
    a.Tq = s.Tq;
    a.BH = BH;
    a.scale_log2 = static_cast<float>(1.4426950408889634 / std::sqrt(static_cast<double>(D)));
    a.new_t = new_t;
    // launch shape: sized for the most quantized groups and the most recent
    // tokens any sequence holds
    int n_groups_sz = s.Tq / d.G, Tr_sz = s.N - s.Tq;
    if (s.ragged) {
        if (h->cfg.batch > kvq::kMaxRaggedSeqs)
            return h->fail(KVQ_EUNSUPPORTED, "sequences of different lengths: batch %d exceeds %d", h->cfg.batch,
                           kvq::kMaxRaggedSeqs);
        n_groups_sz = Tr_sz = 0;
        for (int b = 0; b < h->cfg.batch; ++b) {
            n_groups_sz = std::max(n_groups_sz, s.seqTq[b] / d.G);
            Tr_sz = std::max(Tr_sz, s.seqN[b] - s.seqTq[b]);
        }
    }
    const bool has_new = new_t >= 0 || seq_new_t != nullptr;
    a.new_k = has_new ? static_cast<const uint16_t *>(new_k) : d.ring_k;
    a.new_v = has_new ? static_cast<const uint16_t *>(new_v) : d.ring_v;
    const bool use_mfma = (d.kb == 16 || (d.v_tiled && kvq::mfma_supported(d.kb, d.vb, D))) &&
                          h->env_force_valu == 0;
    int S = 0;
    if (use_mfma) {
        // matrix-core units over whole groups, then over the recent tokens
        const int n_groups = n_groups_sz;
        const int Tr = Tr_sz;
        // recent tokens: 32-token blocks, about as many per unit as a quantized unit holds
        auto res_len = [&](long ug_) {
            int r = static_cast<int>(ug_ * d.G);
            r = (r + 31) / 32 * 32;
            return r < 64 ? 64 : r;
        };
        const int g = h->cfg.n_q_heads / h->cfg.n_kv_heads;
        // workgroups resident at once: two per CU by the register allocation
        // (two waves per SIMD), fewer when the LDS of four wave regions and the
        // merge's own arrays do not fit twice in a CU's 160 KiB
        const long wg_lds = 4L * kvq::mfma_wave_region(D, g, n_groups > 0, Tr > 0) * 4 + 8192;
        const long per_cu = std::max(1L, std::min(2L, (160L * 1024) / wg_lds));
        const long res_wgs = per_cu * h->cu_count;
        // quantized units: uq per stream, groups split as evenly as possible;
        // recent-token units: ceil(Tr / rt) per stream, rt tokens each
        long uq = 0;
        int rt = 0;
        const int env_ug = h->env_unit_groups;
        if (BH * 2 > res_wgs && env_ug == 0) {
            // Many streams: each stream's work splits into U units (U a
            // multiple of four: whole workgroups), the recent tokens into as
            // many units as their share of the work, chosen to minimise
            // (workgroup generations) x (unit duration) under a rough cost
            // model in microseconds: per unit 5, per quantized 32-token block
            // 0.8 (1.3 for K8V8/K8V4-wide rounds), per recent block 2.5.
            const double c_blk = (d.kb + d.vb > 12) ? 1.3 : 0.8;
            const double wq = static_cast<double>(n_groups) * (d.G / 32) * c_blk;
            const double wr = ((Tr + 31) / 32) * 2.5;
            int best_u = 4;
            double best = 1e300;
            for (int U = 4; U <= 64; U += 4) {
                const double gens = std::ceil(static_cast<double>(BH) * (U / 4) / res_wgs);
                const double cost = gens * (5.0 + (wq + wr) / U);
                if (cost < best * 0.999) {
                    best = cost;
                    best_u = U;
                }
            }
            int ur = Tr > 0 ? static_cast<int>(std::lround(best_u * wr / (wq + wr))) : 0;
            if (Tr > 0 && ur < 1)
                ur = 1;
            if (n_groups > 0 && ur > best_u - 1)
                ur = best_u - 1;
            uq = best_u - ur;
            if (ur > 0)
                rt = ((Tr + ur - 1) / ur + 31) / 32 * 32;
        } else if (n_groups > 0) {
            // units of whole windows (the kernel's ng groups, one per column slot
            // of the matrix products), as many units (waves) as stay resident at
            // once: no second, partly filled generation of waves
            long ng = 16;
            while (ng * g > 16)
                ng >>= 1;
            const long cap = 4 * res_wgs;
            long ug = (static_cast<long>(n_groups) * BH + cap - 1) / cap;
            ug = (ug + ng - 1) / ng * ng;
            while (ug < n_groups &&
                   BH * ((n_groups + ug - 1) / ug + (Tr + res_len(ug) - 1) / res_len(ug)) > cap)
                ug += ng;
            if (env_ug > 0)
                ug = env_ug;
            if (ug > n_groups)
                ug = n_groups;
            uq = (n_groups + ug - 1) / ug;
            rt = res_len(ug);
            // whole workgroups: when the units leave the last workgroup of each
            // stream partly idle, more (smaller) quantized units fill it if that
            // takes a group off the longest unit
            const long ur = (Tr + rt - 1) / rt;
            const long U4 = (uq + ur + 3) / 4 * 4, uq4 = U4 - ur;
            if (env_ug == 0 && BH * U4 <= cap && uq4 <= n_groups &&
                (n_groups + uq4 - 1) / uq4 < (n_groups + uq - 1) / uq)
                uq = uq4;
            // few streams: while there are more SIMDs than waves, shorter units
            // (one wave per SIMD, whole workgroups) shorten the critical path;
            // when such a unit would still walk eight or more 32-token blocks
            // (several dependent load rounds), twice as many units, two waves
            // per SIMD, hide each other's load latency, provided they fit one
            // generation of resident workgroups (Llama-2-70B shape: 39.9 ->
            // 35.2 us per call; the Qwen2.5-7B shape would need a second
            // generation and keeps its units).  All units, the recent-token
            // ones included, stay one workgroup per stream short of that
            // generation's slots: a launch that fills them exactly ran slower
            // than one that leaves a few free, and one whose recent-token
            // workgroups spill past them slower still (Llama-2-70B shape: 128
            // quantized + 1 recent units per stream 34.4 us, 127 + 1 37.3 us,
            // 123 + 1 33.5 us)
            const long u_simd = (4L * h->cu_count / BH) / 4 * 4;
            if (env_ug == 0) {
                const long base = std::max<long>(uq, u_simd - ur);
                const bool walks = base > 0 && (n_groups + base - 1) / base * (d.G / 32) >= 8;
                const long wgs2 = static_cast<long>(BH) * ((2 * base + ur + 3) / 4);
                const long fit = 4 * (res_wgs / BH) - 4 - ur;  // quantized unit slots, one workgroup spare
                if (walks && wgs2 * 20 <= res_wgs * 21)
                    uq = std::min<long>(n_groups, std::min<long>(2 * base, std::max<long>(base, fit)));
                else if (u_simd > uq + ur)
                    uq = std::min<long>(n_groups, u_simd - ur);
            }
        }
        if (rt == 0)
            rt = res_len(uq > 0 ? (n_groups + uq - 1) / uq : 1);
        if (h->env_res_tokens > 0)
            rt = (h->env_res_tokens + 31) / 32 * 32;
        if (h->env_units_q > 0)
            uq = h->env_units_q;
        if (uq > n_groups)
            uq = n_groups;
        // the merge takes at most kMaxUnits / 4 workgroups per stream
        while (uq + (Tr + rt - 1) / rt > kMaxUnits) {
            if (uq > (Tr + rt - 1) / rt)
                --uq;
            else
                rt += 32;
        }
        a.units_q = static_cast<int>(uq);
        a.n_groups = n_groups;
        a.pipe = h->env_no_pipe ? 0 : 1;
        a.ngcap = d.capq / d.G;
        a.s_log2 = 0;
        while ((16 >> a.s_log2) * g > 16)
            ++a.s_log2;
        a.unit_groups = uq > 0 ? static_cast<int>(n_groups / uq) : 0;
        a.unit_extra = uq > 0 ? static_cast<int>(n_groups % uq) : 0;
        a.res_tokens = rt;
        a.units_r = (Tr + rt - 1) / rt;
        a.mfma_wgs = (a.units_q + a.units_r + 3) / 4;
        // one XCD per stream when the streams fill the eight XCDs evenly and
        // each has at most eight workgroups (a power of two)
        a.xcd_shift = 0;
        if (BH % 8 == 0 && a.mfma_wgs >= 2 && a.mfma_wgs <= 8 && (a.mfma_wgs & (a.mfma_wgs - 1)) == 0)
            while ((1 << a.xcd_shift) < a.mfma_wgs)
                ++a.xcd_shift;
        a.valu_beg = a.valu_tps = a.valu_wgs = 0;
        S = a.units_q + a.units_r;
    } else {
        // splits: about two workgroups per compute unit, >= 64 tokens each
        S = (2 * h->cu_count + BH - 1) / BH;
        if (h->env_splits > 0)
            S = h->env_splits;
        const int max_by_len = (s.N + 63) / 64;
        if (S > max_by_len)
            S = max_by_len;
        if (S > kMaxPart)
            S = kMaxPart;
        if (S < 1)
            S = 1;
        int tps = (s.N + S - 1) / S;
        tps = (tps + 127) / 128 * 128;  // whole LDS tiles and 32-token V blocks
        S = (s.N + tps - 1) / tps;
        a.valu_beg = 0;
        a.valu_tps = tps;
        a.valu_wgs = S;
        a.units_q = a.unit_groups = a.unit_extra = a.units_r = a.res_tokens = a.mfma_wgs = a.pipe = 0;
        a.xcd_shift = 0;
        a.n_groups = a.ngcap = a.s_log2 = 0;
    }
    kvq::RaggedTables rt;
    if (s.ragged) {
        // each sequence's own lengths, and its groups split over the units_q units
        for (int b = 0; b < h->cfg.batch; ++b) {
            const int ng = s.seqTq[b] / d.G;
            rt.N[b] = s.seqN[b];
            rt.Tq[b] = s.seqTq[b];
            rt.unit_groups[b] = a.units_q > 0 ? ng / a.units_q : 0;
            rt.unit_extra[b] = a.units_q > 0 ? ng % a.units_q : 0;
            rt.new_t[b] = seq_new_t ? seq_new_t[b] : -1;
        }
    }
    // one partial entry per workgroup
    a.n_part = use_mfma ? a.mfma_wgs : a.valu_wgs;
    if (a.n_part < 1 || a.n_part > kMaxPart)
        return h->fail(KVQ_EINVAL, "internal: %d partial entries per stream", a.n_part);
    const int g = h->cfg.n_q_heads / h->cfg.n_kv_heads;
    if (static_scratch) {
        // hand-off words and this call's partial entries in the library's
        // static scratch, left in their initial state by the call itself
        const size_t need = static_cast<size_t>(BH) * a.n_part * kvq::part_entry_floats(g, D) * 4;
        if (BH > kvq::kStaticScratchStreams || need > kvq::kStaticScratchBytes - kvq::kStaticScratchWordsBytes)
            return h->fail(KVQ_ENOMEM,
                           "layer %d: %d streams x %d partial entries need %zu bytes of static scratch; at most %d "
                           "streams and %zu bytes are available",
                           layer, BH, a.n_part, need, kvq::kStaticScratchStreams,
                           kvq::kStaticScratchBytes - kvq::kStaticScratchWordsBytes);
        void *p = nullptr;
        e = kvq::static_scratch(dev, h->stream, &p);
        if (e != hipSuccess)
            return h->dev_fail(e, "static scratch set-up");
        a.counters = static_cast<unsigned *>(p);
        a.part = reinterpret_cast<float *>(static_cast<char *>(p) + kvq::kStaticScratchWordsBytes);
    } else {
        a.counters = reinterpret_cast<unsigned *>(h->ws + h->plan.off_cnt);
        a.part = reinterpret_cast<float *>(h->ws + h->plan.off_part);
        if (!h->counters_ready) {
            e = kvq::launch_zero(a.counters, BH * kvq::kCounterStride, h->stream);
            if (e != hipSuccess)
                return h->dev_fail(e, "counter init");
            h->counters_ready = true;
        }
    }
    e = kvq::launch_attention(a, s.ragged ? &rt : nullptr, use_mfma, h->stream);
    if (e != hipSuccess)
        return h->dev_fail(e, "attention launch");
    h->last_splits = S;
    h->last_variant = use_mfma ? 1 : 0;
    h->touched = true;
    return KVQ_OK;
}

static void layer_bytes(const kvq_handle *h, const LayerState &s, kvq_bytes_info *info)
{
    const int64_t Hkv = h->cfg.n_kv_heads, D = h->cfg.head_dim;
    const kvq::LayerDev &d = s.dev;
    memset(info, 0, sizeof *info);
    // token counts: those of every sequence, or -1 when they differ
    info->n_tokens = s.ragged ? -1 : s.N;
    info->n_quantized = s.ragged ? -1 : s.Tq;
    info->n_residual = s.ragged ? -1 : s.N - s.Tq;
    info->k_bits = d.kb;
    info->v_bits = d.vb;
    info->residual_len = d.R;
    info->k_mode = d.k_tok ? KVQ_K_PER_TOKEN : KVQ_K_PER_CHANNEL;
    info->rpc_permille = s.rpc_permille;
    if (d.kb != 16) {
        info->k_words = d.wk;
        info->v_words = d.wv;
    }
    for (size_t b = 0; b < s.seqN.size(); ++b) {
        const int64_t N = s.seqN[b], Tq = s.seqTq[b];
        if (d.kb == 16) {
            info->residual += Hkv * N * 4 * D;
            continue;
        }
        info->k_codes += Hkv * Tq * 4 * d.wk;
        info->v_codes += Hkv * Tq * 4 * d.wv;
        info->k_meta += d.k_tok ? Hkv * Tq * 8 : Hkv * (Tq / d.G) * 8 * D;
        info->v_meta += Hkv * Tq * 8;
        info->residual += Hkv * (N - Tq) * 4 * D;
    }
    info->total = info->k_codes + info->v_codes + info->k_meta + info->v_meta + info->residual;
}

int64_t kvq_bytes(const kvq_handle *h)
{
    if (!h)
        return -1;
    int64_t total = 0;
    kvq_bytes_info info;
    for (const LayerState &s : h->plan.layers) {
        layer_bytes(h, s, &info);
        total += info.total;
    }
    return total;
}

int kvq_bytes_layer(const kvq_handle *h, int layer, kvq_bytes_info *info)
{
    if (!h || !info)
        return KVQ_EINVAL;
    if (layer < 0 || layer >= h->cfg.n_layers)
        return const_cast<kvq_handle *>(h)->fail(KVQ_EINVAL, "layer %d out of range", layer);
    layer_bytes(h, h->plan.layers[layer], info);
    return KVQ_OK;
}

// Canonical copy of streams [s0, s0 + BH) holding N tokens, Tq quantized;
// output arrays are indexed by the stream's position in the range.
static int export_streams(kvq_handle *h, const kvq::LayerDev &dl, int s0, int BH, int N, int Tq, uint32_t *k_words,
                          float *k_scale, float *k_zero, uint32_t *v_words, float *v_scale, float *v_zero,
                          void *res_k, void *res_v)
{
    const int D = h->cfg.head_dim, Tr = N - Tq;
    const kvq::LayerDev d = s0 == 0 ? dl : sub_layer(dl, s0, D);
    hipError_t e = hipStreamSynchronize(h->stream);
    if (e != hipSuccess)
        return h->dev_fail(e, "stream synchronize");
    if (d.kb != 16 && Tq > 0) {
        const int ng = Tq / d.G;
        // rows are addressed as the kernels address them; with paging through
        // a host copy of the page table (its rows of this view's sequences)
        kvq::LayerDev dh = d;
        std::vector<int32_t> tab;
        if (d.table) {
            tab.assign(static_cast<size_t>(h->cfg.batch) * d.tstride, 0);
            if ((e = hipMemcpy(tab.data(), d.table, tab.size() * 4, hipMemcpyDeviceToHost)) != hipSuccess)
                return h->dev_fail(e, "export block table");
            dh.table = tab.data();
        }
        // copy rows [first, first + count) of stream bh (unit 1: token rows of
        // row_bytes; unit G: group rows) to dst, one piece per page
        auto gather = [&](const void *dev, size_t row_bytes, int bh, int first, int count, bool groups,
                          void *dst) -> hipError_t {
            const kvq::QAddr qa(dh, bh);
            const int per_page = groups ? (1 << d.P_log2) / d.G : (1 << d.P_log2);
            for (int i = 0; i < count;) {
                const int r = first + i;
                const size_t row = groups ? qa.grp(r) : qa.row(r);
                int n = count - i;
                if (d.table)
                    n = std::min(n, per_page - r % per_page);
                const hipError_t er =
                    hipMemcpy(static_cast<char *>(dst) + static_cast<size_t>(i) * row_bytes,
                              static_cast<const char *>(dev) + row * row_bytes, static_cast<size_t>(n) * row_bytes,
                              hipMemcpyDeviceToHost);
                if (er != hipSuccess)
                    return er;
                i += n;
            }
            return hipSuccess;
        };
        for (int bh = 0; bh < BH; ++bh) {
            if (k_words && (e = gather(d.k_words, d.wk * 4, bh, 0, Tq, false,
                                       k_words + static_cast<size_t>(bh) * Tq * d.wk)) != hipSuccess)
                return h->dev_fail(e, "export k_words");
            if (v_words) {
                uint32_t *dst = v_words + static_cast<size_t>(bh) * Tq * d.wv;
                if (d.v_tiled) {
                    // 32-token operand tiles -> token-major rows
                    std::vector<uint32_t> tiles(static_cast<size_t>(Tq) * d.wv);
                    if ((e = gather(d.v_words, d.wv * 4, bh, 0, Tq, false, tiles.data())) != hipSuccess)
                        return h->dev_fail(e, "export v_words");
                    memset(dst, 0, tiles.size() * 4);
                    const int epw = 32 / d.vb;
                    const uint32_t mask = (1u << d.vb) - 1u;
                    for (int t = 0; t < Tq; ++t)
                        for (int c = 0; c < D; ++c) {
                            int word, bit;
                            kvq::v_tile_pos(t & 31, c, d.vb, D, &word, &bit);
                            const uint32_t code =
                                (tiles[static_cast<size_t>(t & ~31) * d.wv + word] >> bit) & mask;
                            dst[static_cast<size_t>(t) * d.wv + c / epw] |= code << (d.vb * (c % epw));
                        }
                } else if ((e = gather(d.v_words, d.wv * 4, bh, 0, Tq, false, dst)) != hipSuccess) {
                    return h->dev_fail(e, "export v_words");
                }
            }
            if ((k_scale || k_zero) && d.k_tok) {
                std::vector<float> m(static_cast<size_t>(Tq) * 2);
                if ((e = gather(d.k_meta, 8, bh, 0, Tq, false, m.data())) != hipSuccess)
                    return h->dev_fail(e, "export k_meta");
                for (int t = 0; t < Tq; ++t) {
                    if (k_scale)
                        k_scale[static_cast<size_t>(bh) * Tq + t] = m[2 * t];
                    if (k_zero)
                        k_zero[static_cast<size_t>(bh) * Tq + t] = m[2 * t + 1];
                }
            } else if (k_scale || k_zero) {
                std::vector<float> m(static_cast<size_t>(ng) * 2 * D);
                if ((e = gather(d.k_meta, static_cast<size_t>(2) * D * 4, bh, 0, ng, true, m.data())) != hipSuccess)
                    return h->dev_fail(e, "export k_meta");
                for (int gi = 0; gi < ng; ++gi)
                    for (int c = 0; c < D; ++c) {
                        const size_t o = (static_cast<size_t>(bh) * ng + gi) * D + c;
                        if (k_scale)
                            k_scale[o] = m[static_cast<size_t>(gi) * 2 * D + c];
                        if (k_zero)
                            k_zero[o] = m[static_cast<size_t>(gi) * 2 * D + D + c];
                    }
            }
            if (v_scale || v_zero) {
                std::vector<float> m(static_cast<size_t>(Tq) * 2);
                if ((e = gather(d.v_meta, 8, bh, 0, Tq, false, m.data())) != hipSuccess)
                    return h->dev_fail(e, "export v_meta");
                for (int t = 0; t < Tq; ++t) {
                    if (v_scale)
                        v_scale[static_cast<size_t>(bh) * Tq + t] = m[2 * t];
                    if (v_zero)
                        v_zero[static_cast<size_t>(bh) * Tq + t] = m[2 * t + 1];
                }
            }
        }
    }
    if ((res_k || res_v) && Tr > 0) {
        std::vector<uint16_t> ring(static_cast<size_t>(d.R) * D);
        for (int which = 0; which < 2; ++which) {
            uint16_t *dst = static_cast<uint16_t *>(which ? res_v : res_k);
            const uint16_t *src = which ? d.ring_v : d.ring_k;
            if (!dst)
                continue;
            for (int bh = 0; bh < BH; ++bh) {
                if ((e = hipMemcpy(ring.data(), src + static_cast<size_t>(bh) * d.R * D, ring.size() * 2,
                                   hipMemcpyDeviceToHost)) != hipSuccess)
                    return h->dev_fail(e, "export ring");
                for (int i = 0; i < Tr; ++i) {
                    const int t = Tq + i;
                    memcpy(dst + (static_cast<size_t>(bh) * Tr + i) * D,
                           ring.data() + static_cast<size_t>(t % d.R) * D, static_cast<size_t>(D) * 2);
                }
            }
        }
    }
    return KVQ_OK;
}

int kvq_export_layer(kvq_handle *h, int layer, uint32_t *k_words, float *k_scale, float *k_zero,
                     uint32_t *v_words, float *v_scale, float *v_zero, void *res_k, void *res_v)
{
    if (!h)
        return KVQ_EINVAL;
    if (layer < 0 || layer >= h->cfg.n_layers)
        return h->fail(KVQ_EINVAL, "layer %d out of range", layer);
    const LayerState &s = h->plan.layers[layer];
    if (s.ragged)
        return h->fail(KVQ_EINVAL, "layer %d holds sequences of different lengths: export them one by one", layer);
    return export_streams(h, s.dev, 0, h->BH(), s.N, s.Tq, k_words, k_scale, k_zero, v_words, v_scale, v_zero,
                          res_k, res_v);
}

int kvq_export_sequence(kvq_handle *h, int layer, int b, uint32_t *k_words, float *k_scale, float *k_zero,
                        uint32_t *v_words, float *v_scale, float *v_zero, void *res_k, void *res_v)
{
    if (!h)
        return KVQ_EINVAL;
    if (layer < 0 || layer >= h->cfg.n_layers)
        return h->fail(KVQ_EINVAL, "layer %d out of range", layer);
    if (b < 0 || b >= h->cfg.batch)
        return h->fail(KVQ_EINVAL, "sequence %d out of range [0, %d)", b, h->cfg.batch);
    const LayerState &s = h->plan.layers[layer];
    const int Hkv = h->cfg.n_kv_heads;
    return export_streams(h, s.dev, b * Hkv, Hkv, s.seqN[b], s.seqTq[b], k_words, k_scale, k_zero, v_words, v_scale,
                          v_zero, res_k, res_v);
}

int kvq_sync(kvq_handle *h)
{
    if (!h)
        return KVQ_EINVAL;
    hipError_t e = hipStreamSynchronize(h->stream);
    if (e != hipSuccess)
        return h->dev_fail(e, "stream synchronize");
    return KVQ_OK;
}

int kvq_set_stream(kvq_handle *h, void *stream)
{
    if (!h)
        return KVQ_EINVAL;
    h->stream = static_cast<hipStream_t>(stream);
    return KVQ_OK;
}

const char *kvq_last_error(const kvq_handle *h)
{
    if (!h)
        return g_create_error.c_str();
    return h->err.c_str();
}

void kvq_destroy(kvq_handle *h)
{
    if (!h)
        return;
    if (h->touched)
        (void)hipStreamSynchronize(h->stream);
    delete h;
}

int kvq_last_launch(const kvq_handle *h, int *splits, int *variant)
{
    if (!h)
        return KVQ_EINVAL;
    if (splits)
        *splits = h->last_splits;
    if (variant)
        *variant = h->last_variant;
    return KVQ_OK;
}

}  // extern "C"
