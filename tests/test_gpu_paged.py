"""GPU parity of paged layers: the quantized state of every layer lives in a
pool of pages named by a caller-owned block table (KIVI notes, section 8:
block-table cache managers combine with the quantized cache).  Tables are
shuffled and non-contiguous (pages of one sequence scattered over a pool with
unused pages in between).  Each case runs a paged cache and an unpaged one on
the same inputs: the exported state (read back through the table) is bit-exact
against the oracle, every attention output is within tolerance of the oracle
and equal, bit for bit, to the unpaged cache's."""
import numpy as np
import pytest
import torch

from decode_attention_streaming_amd import kvq, synth
from gpu_common import (GUARD_REL_L2, MAX_ABS, REL_L2, ad_hoc_workload, check_attention, compare_export, make_oracle,
                        q_streams, stream_view)

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _table(B, stride, n_pages, seed):
    """Every (sequence, page) entry a distinct page of a pool of n_pages, in a
    random order."""
    rng = np.random.default_rng(seed)
    perm = rng.permutation(n_pages)[:B * stride].astype(np.int32)
    return torch.from_numpy(perm.reshape(B, stride)).to(DEV)


def _pair(w, P, cap, seed, spare=5):
    stride = -(-cap // P)
    n_pages = w.batch * stride + spare
    table = _table(w.batch, stride, n_pages, seed)
    args = (len(w.layers), w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, cap, w.kv_dtype, w.q_dtype,
            w.G, w.R, w.layers)
    flat = kvq.Cache(*args)
    paged = kvq.Cache(*args, page_tokens=P, n_pages=n_pages, block_table=table)
    return flat, paged


CASES = {
    # name: (B, Hq, Hkv, d, kb, vb, G, R, kv, q, P, prefill, steps, k_mode, rpc)
    "mfma_k4v2_g4": (3, 8, 2, 128, 4, 2, 32, 32, "bf16", "bf16", 128, 700, 40, 0, 0),
    "mfma_k3v4_mha": (2, 2, 2, 128, 3, 4, 32, 40, "f16", "f32", 256, 600, 45, 0, 0),
    "mfma_k8v8_tok_g64": (2, 8, 2, 64, 8, 8, 64, 64, "bf16", "f16", 128, 500, 70, 1, 0),
    "mfma_k2v2_rpc": (2, 8, 1, 128, 2, 2, 32, 160, "bf16", "bf16", 128, 900, 60, 0, 200),
    "mfma_k4v4_g7_G64": (2, 14, 2, 128, 4, 4, 64, 64, "bf16", "f32", 128, 1500, 40, 0, 0),
    "mfma_k4v8_g6_G64": (2, 12, 2, 128, 4, 8, 64, 64, "bf16", "bf16", 128, 1200, 40, 0, 0),
    "valu_k2v4_g16": (2, 4, 2, 64, 2, 4, 16, 16, "f16", "f32", 128, 350, 35, 0, 0),
    "mfma_k4v4_d256": (2, 4, 2, 256, 4, 4, 32, 32, "bf16", "bf16", 128, 300, 33, 0, 0),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_paged_decode_parity(name):
    B, Hq, Hkv, d, kb, vb, G, R, kv, qd, P, n0, steps, km, rpc = CASES[name]
    print("paged case", name, flush=True)
    w = ad_hoc_workload(9400 + sorted(CASES).index(name), B, Hq, Hkv, d, kb, vb, G, R, n0 + steps, kv, qd,
                        k_mode=km)
    if rpc:
        w.layers = [(kb, vb, R, km, rpc)]
    flat, paged = _pair(w, P, n0 + steps, seed=len(name))
    orc = make_oracle(w, w.layers[0], n0 + steps)
    st = synth.LayerStats(w, 0)
    k, v = synth.layer_tokens(w, 0, 0, n0, DEV, stats=st)
    flat.append(0, k, v)
    paged.append(0, k, v)
    orc.append(stream_view(k), stream_view(v))
    for s in range(steps):
        k, v = synth.layer_tokens(w, 0, n0 + s, 1, DEV, stats=st)
        q = synth.query(w, 0, s, DEV)
        o_flat = flat.append_decode_attention(0, k, v, q)
        o_paged = paged.append_decode_attention(0, k, v, q)
        orc.append(stream_view(k), stream_view(v))
        torch.cuda.synchronize()
        assert torch.equal(o_paged, o_flat), "%s step %d: paged output differs" % (name, s)
        if s % 7 == 0 or s == steps - 1:
            check_attention(o_paged, orc.attention(q_streams(q, w.g)), w.g, what="%s step %d" % (name, s))
    compare_export(paged.export(0), orc.export())
    assert paged.bytes() == flat.bytes() == orc.bytes()
    flat.close()
    paged.close()


def test_paged_ragged_reset_and_page_reuse():
    """Sequences of different lengths in one paged layer (their own pages),
    decode steps that flush them at different times; then one sequence is
    reset, its pages are named again (in another order) for a new sequence in
    its slot, which is prefilled and decoded: every sequence checked against an
    oracle layer of its own, every output equal to the unpaged cache's."""
    B, Hq, Hkv, d, G, P = 3, 8, 2, 128, 32, 128
    lens = [620, 90, 300]
    cap = 800
    w = ad_hoc_workload(9450, B, Hq, Hkv, d, 4, 2, G, 32, cap, "bf16", "bf16")
    stride = cap // P + 1
    n_pages = B * stride
    table = _table(B, stride, n_pages, 77)
    args = (1, B, Hq, Hkv, d, cap, "bf16", "bf16", G, 32, w.layers)
    flat = kvq.Cache(*args)
    paged = kvq.Cache(*args, page_tokens=P, n_pages=n_pages, block_table=table)
    st = synth.LayerStats(w, 0)
    k, v = synth.layer_tokens(w, 0, 0, max(lens), DEV, stats=st)
    for c in (flat, paged):
        c.append_ragged(0, k, v, lens)
    orcs = []
    for b in range(B):
        o = make_oracle(w, w.layers[0], cap, streams=list(range(b * Hkv, (b + 1) * Hkv)))
        sel = list(range(b * Hkv, (b + 1) * Hkv))
        o.append(stream_view(k[:, :, :lens[b]], sel), stream_view(v[:, :, :lens[b]], sel))
        orcs.append(o)

    def step(tag, s):
        k1, v1 = synth.layer_tokens(w, 0, 5000 + s, 1, DEV, stats=st)
        q = synth.query(w, 0, 100 + s, DEV)
        of = flat.append_decode_attention(0, k1, v1, q)
        op = paged.append_decode_attention(0, k1, v1, q)
        torch.cuda.synchronize()
        assert torch.equal(op, of), "%s step %d" % (tag, s)
        for b in range(B):
            sel = list(range(b * Hkv, (b + 1) * Hkv))
            orcs[b].append(stream_view(k1, sel), stream_view(v1, sel))
            ref = orcs[b].attention(q_streams(q, w.g, sel))
            check_attention(op, ref, w.g, streams=sel, what="%s step %d seq %d" % (tag, s, b))

    for s in range(36):
        step("ragged", s)
    for b in range(B):
        sel = list(range(b * Hkv, (b + 1) * Hkv))
        compare_export(paged.export(0, seq=b), orcs[b].export(), streams=None)
    # reset sequence 1 and give its slot a new sequence on its old pages, reordered
    for c in (flat, paged):
        c.reset_sequence(1)
    table[1] = table[1].flip(0).contiguous()
    n_new = 260
    k, v = synth.layer_tokens(w, 0, 9000, n_new, DEV, stats=st)
    counts = [0, n_new, 0]
    for c in (flat, paged):
        c.append_ragged(0, k, v, counts)
    orcs[1] = make_oracle(w, w.layers[0], cap, streams=[2, 3])
    orcs[1].append(stream_view(k, [2, 3]), stream_view(v, [2, 3]))
    for s in range(36, 60):
        step("after reset", s)
    for b in range(B):
        compare_export(paged.export(0, seq=b), orcs[b].export())
    flat.close()
    paged.close()


def test_paged_prefill_attention():
    """Chunked-prefill attention over a paged layer equals the unpaged
    layer's, bit for bit, and the oracle's causal attention within tolerance."""
    B, Hq, Hkv, d, G, P, n0, C = 2, 8, 2, 128, 32, 256, 700, 100
    w = ad_hoc_workload(9460, B, Hq, Hkv, d, 8, 4, G, 32, n0 + C, "bf16", "bf16")
    flat, paged = _pair(w, P, n0 + C, seed=5)
    orc = make_oracle(w, w.layers[0], n0 + C)
    k, v = synth.layer_tokens(w, 0, 0, n0 + C, DEV)
    for c in (flat, paged):
        c.append(0, k, v)
    orc.append(stream_view(k), stream_view(v))
    q = synth.queries(w, 0, C, DEV).permute(1, 2, 0, 3).contiguous()  # [B, Hq, C, d]
    of = flat.prefill_attention(0, q)
    op = paged.prefill_attention(0, q)
    torch.cuda.synchronize()
    assert torch.equal(op, of)
    ref = orc.prefill_attention(synth.as_f64(q.reshape(B * Hkv, w.g, C, d)))
    o = synth.as_f64(op.reshape(B * Hkv, w.g, C, d))
    rel = np.linalg.norm(o - ref) / np.linalg.norm(ref)
    assert rel <= REL_L2 and np.abs(o - ref).max() <= MAX_ABS and rel <= GUARD_REL_L2, rel
    flat.close()
    paged.close()


def test_paged_pool_capacity():
    """An append whose quantized tokens would need more pages than the pool
    holds is refused (KVQ_ECAPACITY) before any device work; the layer keeps
    its state and serves attention."""
    B, Hq, Hkv, d, G, P = 2, 4, 2, 128, 32, 128
    w = ad_hoc_workload(9470, B, Hq, Hkv, d, 4, 2, G, 32, 1024, "bf16", "bf16")
    # 8 pages for 2 sequences: 512 quantized tokens each at most; entries past
    # those a sequence holds are never read (0 here)
    perm = np.random.default_rng(3).permutation(8).astype(np.int32).reshape(2, 4)
    table = torch.zeros((B, 8), dtype=torch.int32)
    table[:, :4] = torch.from_numpy(perm)
    table = table.to(DEV)
    cache = kvq.Cache(1, B, Hq, Hkv, d, 1024, "bf16", "bf16", G, 32, w.layers, page_tokens=P, n_pages=8,
                      block_table=table)
    orc = make_oracle(w, w.layers[0], 1024)
    k, v = synth.layer_tokens(w, 0, 0, 500, DEV)
    cache.append(0, k, v)  # 480 quantized: 4 pages per sequence
    orc.append(stream_view(k), stream_view(v))
    k2, v2 = synth.layer_tokens(w, 0, 500, 100, DEV)
    with pytest.raises(kvq.KvqError) as e:
        cache.append(0, k2, v2)
    assert e.value.code == kvq.KVQ_ECAPACITY and "pool" in str(e.value)
    assert cache.sequence_lengths(0) == ([500, 500], [orc.Tq, orc.Tq]) and orc.Tq == 480
    q = synth.query(w, 0, 0, DEV)
    out = cache.decode_attention(0, q)
    torch.cuda.synchronize()
    check_attention(out, orc.attention(q_streams(q, w.g)), w.g, what="after refusal")
    compare_export(cache.export(0), orc.export())
    cache.close()
