"""Helpers shared by the GPU parity tests: run the HIP path through the C ABI
and the CPU oracle on the same seeded inputs, and compare."""
import numpy as np
import torch

from decode_attention_streaming_amd import kvq, synth
from oracle import oracle as ora

# Attention tolerance: relative L2 over a layer's whole output and max-abs
# per element, against the fp64 oracle.
REL_L2 = 1e-3
MAX_ABS = 5e-3
# Regression guard beside the acceptance bound: the kernels' products carry
# about 22 significant bits (fp32 factors as two fp16 halves, fp32
# accumulation) and reach ~1e-6 relative L2; a loss of precision by an order of
# magnitude or more fails here long before it reaches the acceptance bound.
GUARD_REL_L2 = 2e-5


def ad_hoc_workload(cid, B, Hq, Hkv, d, kb, vb, G, R, ctx, kv="bf16", q="f32",
                    k_outliers=(2, 10.0), v_kind="normal", k_mode=0):
    """k_mode 1: per-token Key (the layer row gets a fourth element)."""
    lc = (kb, vb, R, k_mode) if k_mode else (kb, vb, R)
    w = synth.Workload(cid, "case%d" % cid, 1, B, Hq, Hkv, d, ctx, kv, q, G, R,
                       layers=[lc], k_outliers=k_outliers, v_kind=v_kind)
    return w


def make_cache(w, layers=None, max_context=None):
    return kvq.Cache(len(layers or w.layers), w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim,
                     max_context or w.context, w.kv_dtype, w.q_dtype, w.G, w.R,
                     layers or w.layers)


def make_oracle(w, layer_cfg, cap, streams=None):
    kb, vb, R = layer_cfg[:3]
    k_tok = len(layer_cfg) > 3 and layer_cfg[3] == 1
    rpc = layer_cfg[4] if len(layer_cfg) > 4 else 0
    S = w.batch * w.n_kv_heads if streams is None else len(streams)
    return ora.Layer(S, w.g, w.head_dim, kb, vb, w.G, R if R else w.R, cap, w.kv_dtype == "bf16",
                     k_tok=k_tok, rpc_permille=rpc)


def stream_view(t, streams=None):
    """[B, H, n, d] device tensor -> uint16 [S, n, d] host bits (all or selected streams)."""
    B, H, n, d = t.shape
    flat = t.reshape(B * H, n, d)
    if streams is not None:
        flat = flat[torch.as_tensor(streams, device=t.device)]
    return synth.bits16(flat)


def q_streams(q, g, streams=None):
    """[B, Hq, d] -> float64 [S, g, d] (query heads of each kv stream)."""
    B, Hq, d = q.shape
    x = q.reshape(B * (Hq // g), g, d)
    if streams is not None:
        x = x[torch.as_tensor(streams, device=q.device)]
    return synth.as_f64(x)


def compare_export(ex, ref, streams=None):
    """Bit-exact comparison of the canonical export with the oracle's state."""
    assert ex["N"] == ref["N"] and ex["Tq"] == ref["Tq"], (ex["N"], ex["Tq"], ref["N"], ref["Tq"])
    for key in ("k_words", "k_scale", "k_zero", "v_words", "v_scale", "v_zero", "res_k", "res_v"):
        a = np.asarray(ex[key])
        if streams is not None:
            a = a[np.asarray(streams)]
        b = np.asarray(ref[key])
        if key in ("k_words", "v_words") and b.size == 0 and a.size == 0:
            continue
        assert a.shape == b.shape, (key, a.shape, b.shape)
        if a.dtype == np.float32:
            a, b = a.view(np.uint32), b.view(np.uint32)
        bad = np.nonzero(a != b)
        assert bad[0].size == 0, "%s differs at %d places, first %s: %r vs %r" % (
            key, bad[0].size, tuple(int(x[0]) for x in bad), a[tuple(x[0] for x in bad)],
            b[tuple(x[0] for x in bad)])


def attention_error(out, ref, g, streams=None):
    """(relative L2, max abs, worst per-head relative L2) of out vs fp64 ref."""
    B, Hq, d = out.shape
    o = out.reshape(B * (Hq // g), g, d)
    if streams is not None:
        o = o[torch.as_tensor(streams, device=out.device)]
    o = synth.as_f64(o)
    diff = o - ref
    rel = np.linalg.norm(diff) / np.linalg.norm(ref)
    per = np.linalg.norm(diff, axis=-1) / np.maximum(np.linalg.norm(ref, axis=-1), 1e-30)
    return float(rel), float(np.abs(diff).max()), float(per.max())


def check_attention(out, ref, g, streams=None, what="", guard=GUARD_REL_L2):
    rel, mx, worst = attention_error(out, ref, g, streams)
    assert np.isfinite(rel) and rel <= REL_L2 and mx <= MAX_ABS, (
        "%s rel-L2 %.3e max-abs %.3e worst-head %.3e" % (what, rel, mx, worst))
    assert guard is None or rel <= guard, (
        "%s: rel-L2 %.3e is within the acceptance bound but above the precision guard %.1e" % (what, rel, guard))
    return rel, mx, worst
