"""GPU checks of kvq_decode_attention_noalloc, the decode-attention entry point
whose workgroup hand-off lives in the library's static device scratch instead
of the handle's workspace: through the C ABI its output equals
kvq_decode_attention's bit for bit (and the oracle's to the attention
tolerance), on calls in a row of decreasing size, across handles, with a
ragged batch and on the vector-ALU kernel; oversized requests are refused."""
import pytest
import torch

from decode_attention_streaming_amd import kvq, synth
from gpu_common import ad_hoc_workload, check_attention, make_cache, make_oracle, q_streams, stream_view

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _filled(w, n, seed_layer=0):
    cache = make_cache(w, max_context=n + 4)
    orc = make_oracle(w, w.layers[0], n + 4)
    k, v = synth.layer_tokens(w, seed_layer, 0, n, DEV)
    cache.append(0, k, v)
    orc.append(stream_view(k), stream_view(v))
    return cache, orc


def _both(cache, q):
    ref = cache.decode_attention(0, q)
    out = cache.decode_attention_noalloc(0, q)
    torch.cuda.synchronize()
    return ref, out


def test_noalloc_equals_workspace_call_decreasing_sizes():
    """Two calls in a row, the second on a smaller cache (fewer streams, fewer
    tokens, fewer workgroups per stream), then the larger again: each equals
    the workspace entry point bit for bit and the oracle within tolerance."""
    big = ad_hoc_workload(9300, 4, 16, 4, 128, 4, 2, 32, 32, 1500, "bf16", "bf16")
    small = ad_hoc_workload(9301, 1, 4, 1, 128, 8, 4, 32, 32, 70, "bf16", "f32")
    cb, ob = _filled(big, 1400)
    cs, os_ = _filled(small, 60)
    print("noalloc: big then small then big", flush=True)
    for cache, orc, w in ((cb, ob, big), (cs, os_, small), (cb, ob, big)):
        q = synth.query(w, 0, 3, DEV)
        ref, out = _both(cache, q)
        assert torch.equal(out, ref), (out - ref).abs().max()
        check_attention(out, orc.attention(q_streams(q, w.g)), w.g, what="noalloc")
        units, _ = kvq.kvq_last_launch(cache.h)
        print("  streams %d units per stream %d" % (w.batch * w.n_kv_heads, units), flush=True)
    cb.close()
    cs.close()


def test_noalloc_ragged_and_vector_alu(monkeypatch):
    """A ragged batch (each sequence its own length) on the matrix-core kernel,
    then a layer on the vector-ALU kernel (group size 16): the same outputs as
    the workspace entry point."""
    w = ad_hoc_workload(9302, 3, 8, 2, 64, 2, 2, 32, 32, 700, "f16", "f16")
    cache = make_cache(w, max_context=720)
    k, v = synth.layer_tokens(w, 0, 0, 700, DEV)
    cache.append_ragged(0, k, v, [700, 35, 300])
    q = synth.query(w, 0, 1, DEV)
    ref, out = _both(cache, q)
    assert torch.equal(out, ref)
    cache.close()
    w2 = ad_hoc_workload(9303, 2, 4, 2, 128, 4, 4, 16, 16, 400, "bf16", "bf16")
    c2, o2 = _filled(w2, 390)
    q = synth.query(w2, 0, 2, DEV)
    ref, out = _both(c2, q)
    assert kvq.kvq_last_launch(c2.h)[1] == 0  # the vector-ALU kernel ran
    assert torch.equal(out, ref)
    check_attention(out, o2.attention(q_streams(q, w2.g)), w2.g, what="noalloc valu")
    c2.close()


def test_noalloc_refuses_more_streams_than_the_scratch_holds():
    """4100 (sequence, kv-head) streams exceed the static scratch's 4096
    hand-off words: KVQ_ENOMEM, nothing enqueued, and the workspace entry
    point still serves the same cache."""
    w = ad_hoc_workload(9304, 4100, 1, 1, 64, 4, 2, 32, 32, 40, "f16", "f32")
    cache, orc = _filled(w, 33)
    q = synth.query(w, 0, 0, DEV)
    with pytest.raises(kvq.KvqError) as e:
        cache.decode_attention_noalloc(0, q)
    assert e.value.code == kvq.KVQ_ENOMEM and "static scratch" in str(e.value)
    out = cache.decode_attention(0, q)
    torch.cuda.synchronize()
    check_attention(out, orc.attention(q_streams(q, w.g)), w.g, what="workspace after refusal")
    cache.close()
