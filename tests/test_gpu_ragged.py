"""GPU parity of ragged batches: sequences of one batch hold different numbers
of tokens (kvq_append_ragged), each applying the streaming rule to its own
recent tokens and attending to its own tokens only.  Each sequence is checked
against an oracle layer of its own (the oracle's streams are independent):
state bit for bit through kvq_export_sequence, attention within relative L2
1e-3 / max-abs 5e-3, after a ragged prefill and across one-call decode steps
that flush different sequences at different steps."""
import numpy as np
import pytest
import torch

from decode_attention_streaming_amd import kvq, synth
from gpu_common import (GUARD_REL_L2, MAX_ABS, REL_L2, ad_hoc_workload, check_attention, compare_export, make_cache,
                        make_oracle, stream_view)

pytestmark = pytest.mark.gpu

DEV = "cuda"

CASES = {
    # name: (B, Hq, Hkv, d, kb, vb, G, R, k_mode, rpc, kv, q, prefill lengths, decode steps)
    "k4v2_g4_matrix_core": (4, 8, 2, 128, 4, 2, 32, 32, 0, 0, "bf16", "bf16", [300, 37, 129, 1], 40),
    "k3v4_mha_d64_vector_alu": (3, 2, 2, 64, 3, 4, 32, 40, 0, 0, "f16", "f16", [100, 250, 5], 30),
    "k8v4_recent_ratio": (3, 4, 1, 128, 8, 4, 32, 96, 0, 200, "bf16", "f32", [500, 90, 200], 70),
    "plain16": (2, 4, 2, 128, 16, 16, 32, 32, 0, 0, "bf16", "f32", [70, 3], 10),
    "k2v2_G16_vector_alu": (3, 6, 3, 128, 2, 2, 16, 20, 0, 0, "f16", "f32", [60, 17, 33], 25),
    "k4v4_per_token_key": (2, 8, 2, 128, 4, 4, 64, 64, 1, 0, "bf16", "bf16", [257, 64], 70),
    "k3v2_d128_matrix_core": (2, 8, 2, 128, 3, 2, 32, 50, 0, 0, "f16", "f16", [400, 51], 40),
}


def _oracles(w, lc, B):
    return [make_oracle(w, lc, w.context, streams=list(range(w.n_kv_heads))) for _ in range(B)]


def _check_state(cache, orcs):
    for b, o in enumerate(orcs):
        compare_export(cache.export(0, seq=b), o.export())
    ns, tqs = cache.sequence_lengths(0)
    assert ns == [o.N for o in orcs] and tqs == [o.Tq for o in orcs]
    assert cache.bytes_layer(0).total == sum(o.bytes() for o in orcs)


def _check_out(out, q, orcs, g, what):
    B, Hq, d = out.shape
    for b, o in enumerate(orcs):
        qb = synth.as_f64(q[b].reshape(Hq // g, g, d))
        check_attention(out[b:b + 1], o.attention(qb), g, what="%s seq %d" % (what, b))


@pytest.mark.parametrize("name", sorted(CASES))
def test_ragged_parity(name):
    B, Hq, Hkv, d, kb, vb, G, R, km, rpc, kv, qd, lens, steps = CASES[name]
    lc = (kb, vb, R, km, rpc)
    n_max = max(lens)
    w = ad_hoc_workload(sorted(CASES).index(name) + 8000, B, Hq, Hkv, d, kb, vb, G, R, n_max + steps + 8, kv, qd)
    w.layers = [lc]
    print("ragged case", name, flush=True)
    cache = make_cache(w, layers=[lc])
    orcs = _oracles(w, lc, B)
    st = synth.LayerStats(w, 0, 0)
    k, v = synth.layer_tokens(w, 0, 0, n_max, DEV, stats=st)
    cache.append_ragged(0, k, v, lens)
    for b in range(B):
        orcs[b].append(stream_view(k[b:b + 1, :, :lens[b]].contiguous()),
                       stream_view(v[b:b + 1, :, :lens[b]].contiguous()))
    torch.cuda.synchronize()
    _check_state(cache, orcs)
    info = cache.bytes_layer(0)
    assert (info.n_tokens == -1) == (len(set(lens)) > 1)
    q = synth.query(w, 0, 0, DEV)
    out = cache.decode_attention(0, q)
    torch.cuda.synchronize()
    _check_out(out, q, orcs, w.g, "after prefill")
    # a uniform append on a ragged layer appends to every sequence
    k, v = synth.layer_tokens(w, 0, n_max, 3, DEV, stats=st)
    cache.append(0, k, v)
    for b in range(B):
        orcs[b].append(stream_view(k[b:b + 1]), stream_view(v[b:b + 1]))
    flushes = 0
    for s in range(steps):
        k, v = synth.layer_tokens(w, 0, n_max + 3 + s, 1, DEV, stats=st)
        q = synth.query(w, 0, s + 1, DEV)
        tq = [o.Tq for o in orcs]
        out = cache.append_decode_attention(0, k, v, q)
        for b in range(B):
            orcs[b].append(stream_view(k[b:b + 1]), stream_view(v[b:b + 1]))
        torch.cuda.synchronize()
        _check_out(out, q, orcs, w.g, "step %d" % s)
        changed = [b for b in range(B) if orcs[b].Tq != tq[b]]
        flushes += len(changed)
        if changed or s == steps - 1:
            _check_state(cache, orcs)
    if kb != 16:
        assert flushes >= 1
    cache.close()


def test_ragged_refusals_and_uniform_again():
    w = ad_hoc_workload(8900, 2, 4, 1, 128, 4, 2, 32, 32, 200, "bf16", "f32")
    cache = make_cache(w)
    k, v = synth.layer_tokens(w, 0, 0, 60, DEV)
    cache.append_ragged(0, k, v, [60, 20])
    q = synth.queries(w, 0, 4, DEV).permute(1, 2, 0, 3).contiguous()
    q21 = synth.queries(w, 0, 21, DEV).permute(1, 2, 0, 3).contiguous()
    with pytest.raises(kvq.KvqError) as e:
        cache.prefill_attention(0, q21)  # more queries than the shorter sequence holds
    assert e.value.code == kvq.KVQ_EINVAL
    with pytest.raises(kvq.KvqError) as e:
        cache.export(0)
    assert e.value.code == kvq.KVQ_EINVAL
    with pytest.raises(kvq.KvqError) as e:
        cache.append_ragged(0, k, v, [0, 61])  # more than n_max rows
    assert e.value.code == kvq.KVQ_EINVAL
    # the shorter sequence catches up: the layer is uniform again
    cache.append_ragged(0, k, v, [0, 40])
    info = cache.bytes_layer(0)
    assert (info.n_tokens, info.n_quantized) == (60, 32)
    cache.prefill_attention(0, q)
    cache.export(0)
    torch.cuda.synchronize()
    cache.close()


PREFILL_CASES = {
    # name: (B, Hq, Hkv, d, kb, vb, G, R, k_mode, rpc, kv, q, lengths before the chunk, n_q)
    "k4v2_g4": (4, 8, 2, 128, 4, 2, 32, 32, 0, 0, "bf16", "bf16", [300, 37, 129, 1], 24),
    "k3v4_d128_recent_ratio": (3, 8, 2, 128, 3, 4, 32, 64, 0, 250, "f16", "f16", [400, 61, 200], 40),
    "k8v8_per_token_key_g8": (2, 16, 2, 128, 8, 8, 64, 64, 1, 0, "bf16", "f32", [257, 64], 33),
    "plain16_d64": (3, 4, 2, 64, 16, 16, 32, 32, 0, 0, "f16", "f32", [70, 3, 33], 5),
}


@pytest.mark.parametrize("name", sorted(PREFILL_CASES))
def test_ragged_prefill_parity(name):
    """Prefill attention on a ragged layer: after a ragged fill, one uniform
    append of an n_q-token chunk, whose queries then attend causally over each
    sequence's own tokens (query j of sequence b at position N_b - n_q + j)."""
    B, Hq, Hkv, d, kb, vb, G, R, km, rpc, kv, qd, lens, n_q = PREFILL_CASES[name]
    lc = (kb, vb, R, km, rpc)
    n_max = max(lens)
    w = ad_hoc_workload(sorted(PREFILL_CASES).index(name) + 8100, B, Hq, Hkv, d, kb, vb, G, R,
                        n_max + n_q + 8, kv, qd)
    w.layers = [lc]
    print("ragged prefill case", name, flush=True)
    cache = make_cache(w, layers=[lc])
    orcs = _oracles(w, lc, B)
    st = synth.LayerStats(w, 0, 0)
    k, v = synth.layer_tokens(w, 0, 0, n_max, DEV, stats=st)
    cache.append_ragged(0, k, v, lens)
    for b in range(B):
        orcs[b].append(stream_view(k[b:b + 1, :, :lens[b]].contiguous()),
                       stream_view(v[b:b + 1, :, :lens[b]].contiguous()))
    k, v = synth.layer_tokens(w, 0, n_max, n_q, DEV, stats=st)
    cache.append(0, k, v)
    for b in range(B):
        orcs[b].append(stream_view(k[b:b + 1]), stream_view(v[b:b + 1]))
    q = synth.queries(w, 0, n_q, DEV, seed=3).permute(1, 2, 0, 3).contiguous()
    out = cache.prefill_attention(0, q)
    torch.cuda.synchronize()
    _check_state(cache, orcs)
    g = Hq // Hkv
    for b in range(B):
        qb = synth.as_f64(q[b].reshape(Hkv, g, n_q, d))
        ref = orcs[b].prefill_attention(qb)
        ob = synth.as_f64(out[b].reshape(Hkv, g, n_q, d))
        diff = ob - ref
        rel = np.linalg.norm(diff) / np.linalg.norm(ref)
        mx = np.abs(diff).max()
        print("  seq %d N=%d Tq=%d rel-L2 %.2e max-abs %.2e" % (b, orcs[b].N, orcs[b].Tq, rel, mx), flush=True)
        assert np.isfinite(rel) and rel <= REL_L2 and mx <= MAX_ABS, (name, b, rel, mx)
        assert rel <= GUARD_REL_L2, (name, b, rel)
    cache.close()
