"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs.  Codes, scales, zeros and recent tokens bit-exact;
attention within relative-L2 1e-3 and max-abs 5e-3 of the fp64 oracle."""
import numpy as np
import pytest
import torch

from decode_attention_streaming_amd import kvq, synth
from gpu_common import (ad_hoc_workload, attention_error, check_attention, compare_export,
                        make_cache, make_oracle, q_streams, stream_view)

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _run_case(w, chunks, decode_checks=(), layer_cfg=None, seed=0):
    """Append `chunks` (token counts) to one layer on both sides; compare the
    state after every chunk listed in decode_checks (and at the end) and the
    attention output."""
    lc = layer_cfg or w.layers[0]
    cache = make_cache(w, layers=[lc])
    orc = make_oracle(w, lc, w.context)
    st = synth.LayerStats(w, 0, seed)
    t0 = 0
    results = []
    for i, n in enumerate(chunks):
        k, v = synth.layer_tokens(w, 0, t0, n, DEV, stats=st, seed=seed)
        cache.append(0, k, v)
        orc.append(stream_view(k), stream_view(v))
        t0 += n
        if i in decode_checks or i == len(chunks) - 1:
            q = synth.query(w, 0, i, DEV, seed=seed)
            out = cache.decode_attention(0, q)
            torch.cuda.synchronize()
            compare_export(cache.export(0), orc.export())
            ref = orc.attention(q_streams(q, w.g))
            results.append(check_attention(out, ref, w.g, what="chunk %d N=%d" % (i, t0)))
            info = cache.bytes_layer(0)
            assert info.total == orc.bytes()
    cache.close()
    return results


CASES = {
    # name: (B, Hq, Hkv, d, kb, vb, G, R, ctx, kv, q, chunks)
    "cfg1_k4v2_d64": (1, 1, 1, 64, 4, 2, 32, 32, 288, "f16", "f32", [288]),
    "k8v4_g4_ragged": (2, 8, 2, 128, 8, 4, 32, 40, 320, "bf16", "bf16", [300, 1, 1, 7]),
    "k3v4_mha_R50": (2, 2, 2, 128, 3, 4, 32, 50, 400, "f16", "f16", [333, 2]),
    "k3v2_g4_bf16": (2, 8, 2, 128, 3, 2, 32, 32, 700, "bf16", "bf16", [650, 1, 20]),
    "k3v8_g2_G64": (1, 4, 2, 128, 3, 8, 64, 70, 600, "f16", "f32", [520, 3]),
    # 3-bit K outside the matrix-core path: head_dim 64, groups of 16
    "valu_k3v4_d64": (2, 4, 2, 64, 3, 4, 32, 40, 300, "f16", "f16", [260, 1]),
    "valu_k3v2_G16": (1, 2, 1, 128, 3, 2, 16, 20, 200, "bf16", "f32", [150, 2]),
    "k2v2_d256_g16": (1, 16, 1, 256, 2, 2, 16, 16, 300, "bf16", "f32", [250, 3]),
    "k4v4_d64_g7_tiles": (2, 14, 2, 64, 4, 4, 64, 64, 1100, "bf16", "bf16", [1000, 1, 50]),
    "plain16_g4": (2, 8, 2, 128, 16, 16, 32, 32, 600, "bf16", "f32", [513, 1]),
    "k8v8_G1_R1": (1, 4, 1, 128, 8, 8, 1, 1, 80, "f16", "f32", [70, 1]),
    "k4v2_G8_R9_tokenwise": (1, 2, 1, 64, 4, 2, 8, 9, 64, "f16", "f32", [1] * 40),
    "k2v8_g3": (3, 9, 3, 128, 2, 8, 16, 24, 200, "bf16", "f16", [5, 150, 20]),
    # groups of whole 32-token blocks: the matrix-core path
    "mfma_k2v8_g16_d256": (1, 16, 1, 256, 2, 8, 32, 32, 300, "bf16", "f32", [290, 1]),
    "mfma_k8v2_g1": (2, 2, 2, 128, 8, 2, 32, 48, 400, "f16", "f16", [330, 5]),
    "mfma_k4v4_g8_G128": (1, 8, 1, 128, 4, 4, 128, 128, 700, "bf16", "bf16", [600, 3]),
    # g > 4 with four-block round types: the double-buffered round walk
    "mfma_k2v8_g6_G64": (2, 12, 2, 128, 2, 8, 64, 64, 1500, "bf16", "f32", [1400, 37]),
    "mfma_k8v2_g7_d64": (3, 21, 3, 64, 8, 2, 32, 32, 900, "f16", "f16", [871, 1]),
    # and with one-block rounds (eight-bit types)
    "mfma_k8v4_g8_G128": (1, 8, 1, 128, 8, 4, 128, 128, 1000, "bf16", "bf16", [900, 3]),
    "mfma_k4v8_g5_G64": (2, 10, 2, 128, 4, 8, 64, 70, 800, "f16", "f32", [700, 29]),
    "mfma_k2v4_g5_d64": (2, 10, 2, 64, 2, 4, 64, 70, 500, "f16", "f32", [400, 30]),
    "mfma_k8v8_g4_long": (1, 4, 1, 128, 8, 8, 32, 32, 2100, "bf16", "bf16", [2050, 1]),
    # head_dim 256 with windows of 16 (g = 1) and 4 (g = 4) groups: the largest
    # per-wave LDS regions (one workgroup per compute unit at g = 1)
    "mfma_k8v8_g1_d256": (2, 2, 2, 256, 8, 8, 32, 32, 400, "bf16", "f32", [330, 2]),
    "mfma_k2v4_g4_d256": (1, 4, 1, 256, 2, 4, 32, 40, 500, "f16", "f16", [420, 3]),
    # more streams than resident workgroups: units sized per stream, the recent
    # tokens split over several units
    "mfma_k2v2_many_streams": (8, 40, 40, 128, 2, 2, 32, 256, 640, "f16", "f16", [600, 1]),
    "mfma_k8v4_g2_many_streams": (16, 48, 24, 128, 8, 4, 32, 96, 420, "bf16", "bf16", [400, 1]),
    # per-token-asym Key (13th element: k_mode 1)
    "tok_mfma_k4v2_g4": (2, 8, 2, 128, 4, 2, 32, 32, 420, "bf16", "bf16", [350, 1, 30], 1),
    "tok_mfma_k8v4_mha": (2, 2, 2, 128, 8, 4, 32, 48, 400, "f16", "f16", [330, 5], 1),
    "tok_mfma_k2v8_g16_d256": (1, 16, 1, 256, 2, 8, 32, 32, 300, "bf16", "f32", [290, 1], 1),
    "tok_mfma_k2v2_d64_G64": (2, 10, 2, 64, 2, 2, 64, 70, 500, "f16", "f32", [400, 30], 1),
    "tok_mfma_k8v8_long": (1, 4, 1, 128, 8, 8, 32, 32, 2100, "bf16", "bf16", [2050, 1], 1),
    "tok_mfma_k2v2_g8_G64": (2, 16, 2, 128, 2, 2, 64, 64, 1300, "bf16", "f32", [1250, 1], 1),
    "tok_mfma_k8v4_g7": (2, 14, 2, 128, 8, 4, 32, 32, 700, "f16", "f32", [650, 1], 1),
    "tok_mfma_k4v4_many_streams": (8, 40, 40, 128, 4, 4, 32, 256, 640, "f16", "f16", [600, 1], 1),
    "tok_valu_k4v4_G16": (2, 8, 2, 128, 4, 4, 16, 20, 300, "bf16", "f32", [250, 1, 7], 1),
    "tok_valu_k8v2_G8_d64": (1, 4, 1, 64, 8, 2, 8, 9, 120, "f16", "f16", [1] * 40, 1),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_small_parity(name):
    B, Hq, Hkv, d, kb, vb, G, R, ctx, kv, q, chunks = CASES[name][:12]
    k_mode = CASES[name][12] if len(CASES[name]) > 12 else 0
    w = ad_hoc_workload(200 + sorted(CASES).index(name), B, Hq, Hkv, d, kb, vb, G, R, ctx, kv, q,
                        k_mode=k_mode)
    print("case", name, flush=True)
    _run_case(w, chunks, decode_checks=set(range(len(chunks))))


def test_workload1_exact_state():
    """The single-layer K4V2 workload: 256 quantized tokens + 32 recent."""
    w = synth.workload(1)
    print("workload 1", flush=True)
    res = _run_case(w, [288])
    assert res


def test_prefill_equals_token_by_token_and_deterministic():
    w = ad_hoc_workload(300, 2, 8, 2, 128, 4, 2, 32, 32, 200, "bf16", "bf16")
    st = synth.LayerStats(w, 0)
    k, v = synth.layer_tokens(w, 0, 0, 200, DEV, stats=st)
    a = make_cache(w)
    b = make_cache(w)
    a.append(0, k, v)
    for t in range(200):
        b.append(0, k[:, :, t:t + 1].contiguous(), v[:, :, t:t + 1].contiguous())
    q = synth.query(w, 0, 0, DEV)
    oa1 = a.decode_attention(0, q)
    oa2 = a.decode_attention(0, q)
    ob = b.decode_attention(0, q)
    torch.cuda.synchronize()
    ea, eb = a.export(0), b.export(0)
    compare_export(ea, {k_: (v_ if not isinstance(v_, np.ndarray) else v_) for k_, v_ in eb.items()})
    assert torch.equal(oa1, oa2), "two runs differ"
    assert torch.equal(oa1, ob), "prefill and token-by-token states attend differently"


def test_degenerate_and_tiny_values():
    """Constant channels (s = 0), constant tokens, signed zeros and values in
    the fp16 subnormal range."""
    w = ad_hoc_workload(301, 1, 4, 1, 128, 4, 4, 32, 32, 128, "f16", "f32")
    gen = torch.Generator(device=DEV)
    gen.manual_seed(7)
    k = torch.randn((1, 1, 100, 128), generator=gen, device=DEV)
    v = torch.randn((1, 1, 100, 128), generator=gen, device=DEV)
    k[..., :40, 3] = 1.5            # constant channel within the first groups
    k[..., 5] = 0.0
    k[..., 0:32, 6] = -0.0          # signed zeros
    k[..., 7] *= 2.0 ** -17         # fp16 subnormals
    v[..., 10, :] = -2.25           # constant token
    v[..., 11, ::2] = 0.0
    v[..., 11, 1::2] = -0.0
    v[..., 12, :] *= 2.0 ** -18
    k, v = k.half().contiguous(), v.half().contiguous()
    cache = make_cache(w)
    orc = make_oracle(w, w.layers[0], w.context)
    cache.append(0, k, v)
    orc.append(stream_view(k), stream_view(v))
    q = torch.randn((1, 4, 128), generator=gen, device=DEV)
    out = cache.decode_attention(0, q)
    torch.cuda.synchronize()
    compare_export(cache.export(0), orc.export())
    check_attention(out, orc.attention(q_streams(q, 4)), 4)
    ex = cache.export(0)
    assert (ex["v_scale"][0, 10] == 0.0) and ex["v_zero"][0, 10] == np.float32(-2.25)


def test_bf16_tiny_values():
    """bf16 values far below the fp32 normal range of the scale."""
    w = ad_hoc_workload(302, 1, 2, 1, 64, 8, 4, 16, 16, 64, "bf16", "f32")
    gen = torch.Generator(device=DEV)
    gen.manual_seed(8)
    k = (torch.randn((1, 1, 48, 64), generator=gen, device=DEV) * 1e-37).to(torch.bfloat16)
    v = (torch.randn((1, 1, 48, 64), generator=gen, device=DEV) * 1e-36).to(torch.bfloat16)
    cache = make_cache(w)
    orc = make_oracle(w, w.layers[0], w.context)
    cache.append(0, k.contiguous(), v.contiguous())
    orc.append(stream_view(k), stream_view(v))
    torch.cuda.synchronize()
    compare_export(cache.export(0), orc.export())


def test_capacity_and_empty_append():
    w = ad_hoc_workload(303, 1, 2, 1, 64, 4, 2, 16, 16, 96, "f16", "f32")
    cache = make_cache(w)
    orc = make_oracle(w, w.layers[0], w.context)
    k, v = synth.layer_tokens(w, 0, 0, 96, DEV)
    cache.append(0, k, v)
    orc.append(stream_view(k), stream_view(v))
    e = torch.empty((1, 1, 0, 64), dtype=torch.float16, device=DEV)
    cache.append(0, e, e)
    k1, v1 = synth.layer_tokens(w, 0, 96, 1, DEV)
    with pytest.raises(kvq.KvqError) as err:
        cache.append(0, k1, v1)
    assert err.value.code == kvq.KVQ_ECAPACITY
    torch.cuda.synchronize()
    compare_export(cache.export(0), orc.export())
    q = synth.query(w, 0, 0, DEV)
    check_attention(cache.decode_attention(0, q), orc.attention(q_streams(q, w.g)), w.g)


def test_multi_layer_table():
    """Several layers with different pairs in one cache; each attends to its own state."""
    layers = [(8, 8, 0), (4, 2, 48), (16, 16, 0), (3, 4, 40), (2, 2, 0)]
    w = synth.Workload(304, "multi", len(layers), 2, 8, 2, 128, 260, "bf16", "bf16", 32, 32,
                       layers=layers)
    cache = make_cache(w)
    for l, lc in enumerate(layers):
        orc = make_oracle(w, lc, w.context)
        st = synth.LayerStats(w, l)
        k, v = synth.layer_tokens(w, l, 0, 257, DEV, stats=st)
        cache.append(l, k, v)
        orc.append(stream_view(k), stream_view(v))
        q = synth.query(w, l, 0, DEV)
        out = cache.decode_attention(l, q)
        torch.cuda.synchronize()
        compare_export(cache.export(l), orc.export())
        check_attention(out, orc.attention(q_streams(q, w.g)), w.g, what="layer %d" % l)


@pytest.mark.parametrize("ug", ["1", "3", "40"])
def test_unit_sizes_and_column_merge(ug, monkeypatch):
    """Matrix-core units of 1, 3 and 40 groups: windows holding up to 16 / g
    groups per column set, merged per head at the end of each unit (g 8 and 7:
    the double-buffered walk over windows of two groups, one odd, in rounds of
    two blocks, or of one for K8V4 and K4V8)."""
    monkeypatch.setenv("KVQ_UNIT_GROUPS", ug)
    for (Hq, Hkv, kb, vb, G) in [(2, 2, 2, 2, 32), (16, 4, 4, 2, 32), (16, 2, 8, 4, 64), (2, 2, 3, 4, 32),
                                 (16, 2, 4, 4, 64), (14, 2, 2, 2, 32), (16, 2, 4, 8, 32)]:
        w = ad_hoc_workload(400 + Hq + kb, 2, Hq, Hkv, 128, kb, vb, G, G, 1700, "bf16", "bf16")
        print("unit groups", ug, "g", Hq // Hkv, "pair", (kb, vb), flush=True)
        _run_case(w, [1650, 1])


FUSED_KINDS = ["mfma_k4v2", "mfma_k3v4", "valu_k3v4", "plain16", "valu_g16", "tok_mfma_k4v4", "tok_valu_k2v4"]


@pytest.mark.parametrize("kind", FUSED_KINDS)
def test_append_decode_attention_equals_two_calls(kind):
    """The one-call decode step (append one token, then attend) gives the same
    outputs, bit for bit, and the same state as kvq_append + kvq_decode_attention,
    across flushes of the recent-token buffer."""
    spec = {  # (B, Hq, Hkv, d, kb, vb, G, R, ctx, kv, q)
        "mfma_k4v2": (2, 8, 2, 128, 4, 2, 32, 32, 200, "bf16", "bf16"),
        "mfma_k3v4": (2, 2, 2, 128, 3, 4, 32, 50, 200, "f16", "f32"),
        "valu_k3v4": (2, 2, 2, 128, 3, 4, 16, 50, 200, "f16", "f32"),
        "plain16": (1, 4, 1, 128, 16, 16, 32, 32, 160, "bf16", "bf16"),
        "valu_g16": (1, 8, 2, 64, 8, 4, 16, 24, 160, "f16", "f16"),
        "tok_mfma_k4v4": (2, 8, 2, 128, 4, 4, 32, 32, 200, "bf16", "bf16"),
        "tok_valu_k2v4": (1, 4, 1, 128, 2, 4, 16, 20, 200, "f16", "f32"),
    }[kind]
    w = ad_hoc_workload(500 + sorted(FUSED_KINDS).index(kind), *spec, k_mode=1 if kind.startswith("tok") else 0)
    print("fused step", kind, flush=True)
    st = synth.LayerStats(w, 0)
    n0 = 70
    k, v = synth.layer_tokens(w, 0, 0, n0 + 80, DEV, stats=st)
    two, one = make_cache(w), make_cache(w)
    two.append(0, k[:, :, :n0].contiguous(), v[:, :, :n0].contiguous())
    one.append(0, k[:, :, :n0].contiguous(), v[:, :, :n0].contiguous())
    for i in range(80):
        kt = k[:, :, n0 + i:n0 + i + 1].contiguous()
        vt = v[:, :, n0 + i:n0 + i + 1].contiguous()
        q = synth.query(w, 0, i, DEV)
        two.append(0, kt, vt)
        oa = two.decode_attention(0, q)
        ob = one.append_decode_attention(0, kt, vt, q)
        torch.cuda.synchronize()
        assert torch.equal(oa, ob), "step %d: outputs differ" % i
    compare_export(one.export(0), two.export(0))
    orc = make_oracle(w, w.layers[0], w.context)
    orc.append(stream_view(k), stream_view(v))
    compare_export(one.export(0), orc.export())


@pytest.mark.parametrize("d,G,kb,k_mode,variant", [(128, 32, 3, 0, 1), (64, 32, 3, 0, 0), (128, 16, 3, 0, 0),
                                                  (64, 32, 4, 1, 1), (128, 16, 4, 1, 0)])
def test_path_choice(d, G, kb, k_mode, variant):
    """3-bit K layers run on the matrix core at head_dim 128 with 32-token
    multiples for G (variant 1), on the vector ALU otherwise (variant 0);
    per-token Key takes the matrix core whenever G is a multiple of 32."""
    w = ad_hoc_workload(600 + d + G + kb, 1, 2, 1, d, kb, 4, G, G, 200, "f16", "f32", k_mode=k_mode)
    cache = make_cache(w)
    orc = make_oracle(w, w.layers[0], w.context)
    k, v = synth.layer_tokens(w, 0, 0, 150, DEV)
    cache.append(0, k, v)
    orc.append(stream_view(k), stream_view(v))
    q = synth.query(w, 0, 0, DEV)
    out = cache.decode_attention(0, q)
    torch.cuda.synchronize()
    assert kvq.kvq_last_launch(cache.h)[1] == variant
    check_attention(out, orc.attention(q_streams(q, w.g)), w.g)
    cache.close()


def test_graph_replay_matches_eager():
    """Decode attention calls captured in a HIP graph (no allocation, no
    memset, counters re-armed by the kernel itself) give the eager outputs,
    bit for bit, on every replay, with eager work between the replays."""
    layers = [(4, 2, 0), (8, 8, 0), (16, 16, 0), (2, 2, 0, 1)]
    w = synth.Workload(700, "graph", len(layers), 2, 8, 2, 128, 400, "bf16", "bf16", 32, 32,
                       layers=layers)
    cache = make_cache(w)
    qs, eager = [], []
    for l in range(len(layers)):
        k, v = synth.layer_tokens(w, l, 0, 300, DEV)
        cache.append(l, k, v)
        qs.append(synth.query(w, l, 0, DEV))
        eager.append(cache.decode_attention(l, qs[l]))
    torch.cuda.synchronize()
    outs = [torch.zeros_like(e) for e in eager]
    side = torch.cuda.Stream()
    main = cache.stream
    side.wait_stream(torch.cuda.current_stream())
    cache.set_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        for l in range(len(layers)):
            cache.decode_attention(l, qs[l], outs[l])
    cache.set_stream(main)
    torch.cuda.synchronize()
    for rep in range(3):
        for o in outs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for l in range(len(layers)):
            assert torch.equal(outs[l], eager[l]), "replay %d layer %d" % (rep, l)
        # eager work between replays, on the library's own stream
        again = cache.decode_attention(0, qs[0])
        torch.cuda.synchronize()
        assert torch.equal(again, eager[0])
    cache.close()
