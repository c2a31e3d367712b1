"""GPU parity of the decode hand-off when a stream's workgroups share one XCD
(batch x kv-heads a multiple of 8, 2 / 4 / 8 workgroups per stream): the last
workgroup then reads the others' partial results through that XCD's L2.  Many
one-call decode steps in a row, each with new tokens and a new query, so a
stale partial from an earlier call would show; every output is checked
against the oracle."""
import pytest
import torch

from decode_attention_streaming_amd import kvq, synth
from gpu_common import ad_hoc_workload, check_attention, compare_export, make_cache, make_oracle, q_streams, stream_view

pytestmark = pytest.mark.gpu

DEV = "cuda"

CASES = {
    # name: (B, Hq, Hkv, d, kb, vb, G, R, kv, q, n0, steps, workgroups per stream while stepping)
    "four_wgs_g4": (8, 32, 8, 128, 4, 2, 32, 32, "bf16", "bf16", 490, 22, 4),
    "two_wgs_g4": (8, 4, 1, 128, 2, 2, 32, 32, "bf16", "f32", 240, 16, 2),
    "four_wgs_mha_d64": (16, 16, 1, 64, 8, 4, 32, 32, "f16", "f16", 490, 20, 4),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_xcd_local_handoff(name):
    B, Hq, Hkv, d, kb, vb, G, R, kv, qd, n0, steps, wgs = CASES[name]
    w = ad_hoc_workload(sorted(CASES).index(name) + 9100, B, Hq, Hkv, d, kb, vb, G, R, n0 + steps, kv, qd)
    assert (B * Hkv) % 8 == 0
    print("xcd case", name, flush=True)
    cache = make_cache(w)
    orc = make_oracle(w, w.layers[0], w.context)
    st = synth.LayerStats(w, 0, 0)
    k, v = synth.layer_tokens(w, 0, 0, n0, DEV, stats=st)
    cache.append(0, k, v)
    orc.append(stream_view(k), stream_view(v))
    seen = set()
    for s in range(steps):
        k, v = synth.layer_tokens(w, 0, n0 + s, 1, DEV, stats=st)
        q = synth.query(w, 0, s, DEV)
        out = cache.append_decode_attention(0, k, v, q)
        orc.append(stream_view(k), stream_view(v))
        torch.cuda.synchronize()
        units, variant = kvq.kvq_last_launch(cache.h)
        seen.add((units + 3) // 4)
        check_attention(out, orc.attention(q_streams(q, w.g)), w.g, what="%s step %d" % (name, s))
    assert wgs in seen, seen  # the shape ran with the intended number of workgroups per stream
    compare_export(cache.export(0), orc.export())
    cache.close()


def test_handoff_interleaved_launch_shapes():
    """One handle, layers whose calls use very different numbers of workgroups
    per stream (a long layer, a short one, a medium one), called in turn for
    several decode steps: each stream's partial entries are rewritten by calls
    of every size, so an entry left by an earlier, wider call must never be
    taken for the current call's.  Every output is checked against the
    oracle."""
    layers = [(4, 2, 32), (2, 2, 32), (8, 4, 32)]
    lens = [1900, 40, 330]
    steps = 5
    w = synth.Workload(9200, "interleaved", len(layers), 2, 8, 2, 128, max(lens) + 2 * steps, "bf16", "bf16",
                       32, 32, layers=layers)
    cache = make_cache(w)
    orcs, stats = [], []
    for l, lc in enumerate(layers):
        orc = make_oracle(w, lc, lens[l] + 2 * steps)
        st = synth.LayerStats(w, l)
        k, v = synth.layer_tokens(w, l, 0, lens[l], DEV, stats=st)
        cache.append(l, k, v)
        orc.append(stream_view(k), stream_view(v))
        orcs.append(orc)
        stats.append(st)
    wgs = set()
    for s in range(steps):
        for l in (0, 1, 2, 1, 0):
            k, v = synth.layer_tokens(w, l, orcs[l].N, 1, DEV, stats=stats[l])
            q = synth.query(w, l, 10 * s + l, DEV)
            out = cache.append_decode_attention(l, k, v, q)
            orcs[l].append(stream_view(k), stream_view(v))
            torch.cuda.synchronize()
            units, variant = kvq.kvq_last_launch(cache.h)
            wgs.add((units + 3) // 4)
            check_attention(out, orcs[l].attention(q_streams(q, w.g)), w.g, what="layer %d step %d" % (l, s))
    assert len(wgs) >= 3 and max(wgs) >= 8, wgs
    cache.close()
