"""Parity at the full workload sizes, in the launch configuration the benchmark
times: every layer type of each workload is prefilled over all streams, one
decode step is appended and attended, and a sample of streams is checked
against the oracle (codes bit-exact, attention within tolerance)."""
import numpy as np
import pytest
import torch

from decode_attention_streaming_amd import kvq, synth
from gpu_common import check_attention, compare_export, make_oracle, q_streams, stream_view

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _layer_sample(w):
    """First layer of each distinct (k_bits, v_bits) pair."""
    seen, out = set(), []
    for i, lc in enumerate(w.layers):
        if lc[:2] not in seen:
            seen.add(lc[:2])
            out.append(i)
    return out


@pytest.mark.parametrize("cid", [2, 3, 4, 5])
def test_workload_full_size(cid):
    w = synth.workload(cid)
    layers = _layer_sample(w)
    BH = w.batch * w.n_kv_heads
    rng = np.random.default_rng(cid)
    streams = sorted(set([0, BH - 1] + rng.choice(BH, size=min(4, BH), replace=False).tolist()))
    print("workload", cid, "layers", layers, "streams", streams, flush=True)
    sub = [w.layers[i] for i in layers]
    cache = kvq.Cache(len(sub), w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.context + 8,
                      w.kv_dtype, w.q_dtype, w.G, w.R, sub)
    for j, l in enumerate(layers):
        st = synth.LayerStats(w, l)
        orc = make_oracle(w, w.layers[l], w.context + 8, streams=streams)
        k, v = synth.layer_tokens(w, l, 0, w.context, DEV, stats=st)
        cache.append(j, k, v)
        orc.append(stream_view(k, streams), stream_view(v, streams))
        del k, v
        k, v = synth.layer_tokens(w, l, w.context, 1, DEV, stats=st)
        cache.append(j, k, v)
        orc.append(stream_view(k, streams), stream_view(v, streams))
        q = synth.query(w, l, 0, DEV)
        out = cache.decode_attention(j, q)
        torch.cuda.synchronize()
        ex = cache.export(j)
        compare_export(ex, orc.export(), streams=streams)
        ref = orc.attention(q_streams(q, w.g, streams))
        rel, mx, worst = check_attention(out, ref, w.g, streams=streams,
                                         what="workload %d layer %d" % (cid, l))
        print("  layer %d pair %s: N=%d Tq=%d rel-L2 %.2e max-abs %.2e worst-head %.2e splits %s"
              % (l, w.layers[l][:2], ex["N"], ex["Tq"], rel, mx, worst,
                 kvq.kvq_last_launch(cache.h)), flush=True)
        del ex
    cache.close()
