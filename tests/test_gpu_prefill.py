"""GPU parity of chunked-prefill attention: the queries of the last n_q
appended tokens attend causally (query j sees tokens 0 .. N - n_q + j) over
the cache as stored, through the C ABI, against the CPU oracle's fp64 causal
attention on the same seeded inputs.  Tolerance: relative L2 1e-3 over the
whole output and max-abs 5e-3 per element."""
import numpy as np
import pytest
import torch

from decode_attention_streaming_amd import kvq, synth
from gpu_common import (GUARD_REL_L2, MAX_ABS, REL_L2, ad_hoc_workload, compare_export, make_cache, make_oracle,
                        stream_view)

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _prefill_queries(w, n_q, seed=0):
    """[B, Hq, n_q, d] queries of the chunk's tokens (q_dtype)."""
    return synth.queries(w, 0, n_q, DEV, seed=seed).permute(1, 2, 0, 3).contiguous()


def _q_streams(q, g, streams=None):
    B, Hq, n_q, d = q.shape
    x = q.reshape(B * (Hq // g), g, n_q, d)
    if streams is not None:
        x = x[torch.as_tensor(streams, device=q.device)]
    return synth.as_f64(x)


def _check(out, ref, g, streams=None, what=""):
    B, Hq, n_q, d = out.shape
    o = out.reshape(B * (Hq // g), g, n_q, d)
    if streams is not None:
        o = o[torch.as_tensor(streams, device=out.device)]
    o = synth.as_f64(o)
    diff = o - ref
    rel = np.linalg.norm(diff) / np.linalg.norm(ref)
    mx = np.abs(diff).max()
    assert np.isfinite(rel) and rel <= REL_L2 and mx <= MAX_ABS, "%s rel-L2 %.3e max-abs %.3e" % (what, rel, mx)
    assert rel <= GUARD_REL_L2, "%s: rel-L2 %.3e above the precision guard" % (what, rel)
    return rel, mx


def _run(w, n0, n_q, streams=None, seed=0):
    """Append n0 tokens, then the n_q-token chunk, on both sides; compare the
    state bit for bit and the chunk's causal attention."""
    lc = w.layers[0]
    cache = make_cache(w, layers=[lc])
    orc = make_oracle(w, lc, w.context, streams=streams)
    st = synth.LayerStats(w, 0, seed)
    t0 = 0
    for n in (n0, n_q):
        if n == 0:
            continue
        k, v = synth.layer_tokens(w, 0, t0, n, DEV, stats=st, seed=seed)
        cache.append(0, k, v)
        orc.append(stream_view(k, streams), stream_view(v, streams))
        t0 += n
    q = _prefill_queries(w, n_q, seed)
    out = cache.prefill_attention(0, q)
    torch.cuda.synchronize()
    compare_export(cache.export(0), orc.export(), streams)
    ref = orc.prefill_attention(_q_streams(q, w.g, streams))
    res = _check(out, ref, w.g, streams, what="N=%d n_q=%d" % (t0, n_q))
    cache.close()
    return res, cache


CASES = {
    # name: (B, Hq, Hkv, d, kb, vb, G, R, kv, q, n0, n_q, k_mode)
    "k4v2_g4_chunk_near_recent": (2, 8, 2, 128, 4, 2, 32, 64, "bf16", "bf16", 300, 40, 0),
    "k8v4_g4_chunk_spans_groups": (2, 8, 2, 128, 8, 4, 32, 32, "bf16", "bf16", 200, 150, 0),
    "k2v2_mha_whole_sequence": (1, 4, 4, 64, 2, 2, 32, 32, "f16", "f32", 0, 200, 0),
    "k4v4_g7_d64_ragged_tiles": (2, 14, 2, 64, 4, 4, 64, 64, "bf16", "bf16", 500, 77, 0),
    "k2v8_g16_d256": (1, 16, 1, 256, 2, 8, 32, 32, "bf16", "f32", 130, 9, 0),
    "k8v8_g8_G128": (2, 16, 2, 128, 8, 8, 128, 128, "bf16", "bf16", 700, 100, 0),
    "k4v8_mha_f16": (2, 4, 4, 128, 4, 8, 32, 48, "f16", "f16", 333, 45, 0),
    "k4v2_per_token_key": (2, 8, 2, 128, 4, 2, 32, 32, "bf16", "bf16", 300, 60, 1),
    "k8v4_per_token_key_d64": (1, 4, 1, 64, 8, 4, 64, 80, "f16", "f32", 250, 111, 1),
    "plain16_g4_bf16": (2, 8, 2, 128, 16, 16, 32, 32, "bf16", "f32", 100, 50, 0),
    "plain16_f16_whole": (1, 2, 1, 64, 16, 16, 32, 32, "f16", "f16", 0, 70, 0),
    "k2v4_single_query": (2, 8, 2, 128, 2, 4, 32, 32, "bf16", "bf16", 400, 1, 0),
    "k4v2_one_token_cache": (1, 4, 2, 128, 4, 2, 32, 32, "bf16", "f32", 0, 1, 0),
    "k3v4_mha_R819_chunk": (2, 2, 2, 128, 3, 4, 32, 819, "f16", "f16", 3000, 200, 0),
    "k3v2_g4_bf16_spans_groups": (2, 8, 2, 128, 3, 2, 32, 32, "bf16", "bf16", 300, 90, 0),
    "k3v8_g2_G64_whole": (1, 4, 2, 128, 3, 8, 64, 64, "f16", "f32", 0, 250, 0),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_prefill_parity(name):
    B, Hq, Hkv, d, kb, vb, G, R, kv, qd, n0, n_q, km = CASES[name]
    w = ad_hoc_workload(sorted(CASES).index(name) + 3000, B, Hq, Hkv, d, kb, vb, G, R, n0 + n_q, kv, qd, k_mode=km)
    print("prefill case", name, flush=True)
    _run(w, n0, n_q)


def test_prefill_single_query_matches_decode():
    """n_q = 1 is decode attention: both library calls agree closely."""
    w = ad_hoc_workload(3901, 2, 8, 2, 128, 4, 2, 32, 32, 420, "bf16", "f32")
    cache = make_cache(w)
    k, v = synth.layer_tokens(w, 0, 0, 420, DEV)
    cache.append(0, k, v)
    q = synth.query(w, 0, 0, DEV)
    a = cache.decode_attention(0, q)
    b = cache.prefill_attention(0, q.unsqueeze(2).contiguous())
    torch.cuda.synchronize()
    diff = (a - b[:, :, 0]).abs().max().item()
    assert diff <= 1e-4 * a.abs().max().item(), diff
    cache.close()


def test_prefill_llama31_shape_sampled_streams():
    """Llama-3.1-8B-shaped layer (B8, 32/8 heads, d128, K4V2, G = R = 32):
    1024 cached tokens then a 256-token chunk, in the launch configuration of a
    full layer; three streams checked against the oracle."""
    w = ad_hoc_workload(3902, 8, 32, 8, 128, 4, 2, 32, 32, 1280, "bf16", "bf16")
    print("prefill llama31-shaped", flush=True)
    _run(w, 1024, 256, streams=[0, 37, 63])


def test_prefill_unsupported_formats():
    w = ad_hoc_workload(3903, 1, 4, 1, 64, 3, 4, 32, 32, 64, "f16", "f32")  # 3-bit Key at head_dim 64
    cache = make_cache(w)
    k, v = synth.layer_tokens(w, 0, 0, 40, DEV)
    cache.append(0, k, v)
    q = _prefill_queries(w, 4)
    with pytest.raises(kvq.KvqError) as e:
        cache.prefill_attention(0, q)
    assert e.value.code == kvq.KVQ_EUNSUPPORTED
    with pytest.raises(kvq.KvqError) as e:
        cache.prefill_attention(0, _prefill_queries(w, 41))
    assert e.value.code == kvq.KVQ_EINVAL
    cache.close()
    w = ad_hoc_workload(3904, 1, 4, 1, 64, 4, 2, 16, 16, 64, "f16", "f32")
    cache = make_cache(w)
    k, v = synth.layer_tokens(w, 0, 0, 40, DEV)
    cache.append(0, k, v)
    with pytest.raises(kvq.KvqError) as e:
        cache.prefill_attention(0, _prefill_queries(w, 4))
    assert e.value.code == kvq.KVQ_EUNSUPPORTED
    cache.close()
