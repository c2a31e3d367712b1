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


@pytest.mark.parametrize("cid", [2, 3, 4])
def test_workload_fused_decode_steps(cid):
    """Full-size workloads through the one-call decode step the benchmark
    times: after the prefill, G + 8 steps of one appended token per sequence
    plus attention (so that every layer's recent buffer fills and flushes at
    least once), each step's outputs checked on a sample of streams, and the
    final state bit-exact."""
    w = synth.workload(cid)
    layers = _layer_sample(w)[:3]
    BH = w.batch * w.n_kv_heads
    rng = np.random.default_rng(100 + cid)
    streams = sorted(set([0, BH - 1] + rng.choice(BH, size=min(3, BH), replace=False).tolist()))
    S = w.G + 8
    print("workload", cid, "layers", layers, "streams", streams, "steps", S, flush=True)
    sub = [w.layers[i] for i in layers]
    cache = kvq.Cache(len(sub), w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.context + S + 8,
                      w.kv_dtype, w.q_dtype, w.G, w.R, sub)
    for j, l in enumerate(layers):
        st = synth.LayerStats(w, l)
        orc = make_oracle(w, w.layers[l], w.context + S + 8, streams=streams)
        k, v = synth.layer_tokens(w, l, 0, w.context, DEV, stats=st)
        cache.append(j, k, v)
        orc.append(stream_view(k, streams), stream_view(v, streams))
        del k, v
        k, v = synth.layer_tokens(w, l, w.context, S, DEV, stats=st)
        qs = synth.queries(w, l, S, DEV)
        worst = 0.0
        n0, tq0 = cache.sequence_lengths(j)[0][0], cache.sequence_lengths(j)[1][0]
        for s in range(S):
            k1 = k[:, :, s:s + 1, :].contiguous()
            v1 = v[:, :, s:s + 1, :].contiguous()
            out = cache.append_decode_attention(j, k1, v1, qs[s])
            orc.append(stream_view(k1, streams), stream_view(v1, streams))
            torch.cuda.synchronize()
            ref = orc.attention(q_streams(qs[s], w.g, streams))
            rel, mx, _ = check_attention(out, ref, w.g, streams=streams,
                                         what="workload %d layer %d step %d" % (cid, l, s))
            worst = max(worst, rel)
        ex = cache.export(j)
        compare_export(ex, orc.export(), streams=streams)
        assert ex["N"] == n0 + S
        assert ex["Tq"] > tq0, "no flush inside the fused steps"
        print("  layer %d pair %s: %d fused steps from N=%d, final Tq=%d, worst rel-L2 %.2e"
              % (l, w.layers[l][:2], S, n0, ex["Tq"], worst), flush=True)
        del ex, k, v
    cache.close()
