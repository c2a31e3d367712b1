"""GPU parity of the dynamic recent-token ratio (KVmix notes, key design 3):
a layer with ratio r keeps floor(r * current) of a full recent buffer and
quantizes the rest in whole groups.  Prefill appends that cross several such
compressions, then one-call decode steps (append + attention) across more of
them; the state is compared bit for bit with the oracle and every attention
output within relative L2 1e-3 / max-abs 5e-3."""
import numpy as np
import pytest
import torch

from decode_attention_streaming_amd import synth
from gpu_common import (ad_hoc_workload, check_attention, compare_export, make_cache, make_oracle, q_streams,
                        stream_view)

pytestmark = pytest.mark.gpu

DEV = "cuda"

CASES = {
    # name: (B, Hq, Hkv, d, kb, vb, G, R, rpc, kv, q, n_prefill, n_steps)
    "k4v2_g4_R96_r200": (2, 8, 2, 128, 4, 2, 32, 96, 200, "bf16", "bf16", 100, 150),
    "k3v4_mha_R100_r100": (2, 2, 2, 128, 3, 4, 32, 100, 100, "f16", "f16", 150, 120),
    "k2v2_valu_G16_R48_r200": (1, 2, 2, 64, 2, 2, 16, 48, 200, "f16", "f32", 60, 80),
    "k8v8_prefill_many_events": (1, 4, 1, 128, 8, 8, 32, 96, 150, "bf16", "f32", 700, 40),
    "k4v4_per_token_key_r200": (1, 8, 2, 128, 4, 4, 64, 200, 200, "bf16", "bf16", 450, 70),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_rpc_parity(name):
    B, Hq, Hkv, d, kb, vb, G, R, rpc, kv, qd, n0, steps = CASES[name]
    km = 1 if "per_token" in name else 0
    lc = (kb, vb, R, km, rpc)
    w = ad_hoc_workload(sorted(CASES).index(name) + 7000, B, Hq, Hkv, d, kb, vb, G, R, n0 + steps, kv, qd)
    w.layers = [lc]
    print("rpc case", name, flush=True)
    cache = make_cache(w, layers=[lc])
    orc = make_oracle(w, lc, w.context)
    st = synth.LayerStats(w, 0, 0)
    k, v = synth.layer_tokens(w, 0, 0, n0, DEV, stats=st)
    cache.append(0, k, v)
    orc.append(stream_view(k), stream_view(v))
    torch.cuda.synchronize()
    compare_export(cache.export(0), orc.export())
    events = 0
    for s in range(steps):
        k, v = synth.layer_tokens(w, 0, n0 + s, 1, DEV, stats=st)
        q = synth.query(w, 0, s, DEV)
        tq = orc.Tq
        out = cache.append_decode_attention(0, k, v, q)
        orc.append(stream_view(k), stream_view(v))
        events += orc.Tq > tq
        torch.cuda.synchronize()
        check_attention(out, orc.attention(q_streams(q, w.g)), w.g, what="%s step %d" % (name, s))
        if orc.Tq != tq or s == steps - 1:
            compare_export(cache.export(0), orc.export())
        info = cache.bytes_layer(0)
        assert (info.n_tokens, info.n_quantized, info.rpc_permille) == (orc.N, orc.Tq, rpc)
        assert info.total == orc.bytes()
    assert events >= 1  # at least one compression during the one-call decode steps
    cache.close()
