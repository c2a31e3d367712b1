"""Decode-step benchmark of the quantized-KV cache on one MI355X.

One step = for every layer: append one token per sequence (K and V, with a
group flush whenever the recent-token buffer is full), then decode attention
of one query token per sequence over the layer's whole cache, issued as one
kvq_append_decode_attention call (one launch when no flush is due).  Inputs are
seeded synthetic tensors already resident in HBM.

Default workload: Llama-3.1-8B-shaped decode (32 layers, 32 query / 8 KV heads,
head_dim 128, batch 8, context 1024, bf16 K/V and q, a per-layer K/V bit table
averaging 3.25 equivalent bits, G = R = 32).

Prints one JSON line.  `value` is the whole-job effective bandwidth: the
algorithmic bytes of every step (cache state read by attention + q + out, and
the append/flush traffic) over the wall time of the timed steps.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0


def stream_state_bytes(d, kb, vb, G, N, Tq, k_tok=False):
    """Live bytes of one (sequence, kv-head) stream, as kvq_bytes documents
    (k_tok: per-token Key, one scale and zero per Key token)."""
    if kb == 16:
        return N * 4 * d
    wk = (d + 10) // 11 if kb == 3 else d * kb // 32
    wv = d * vb // 32
    kmeta = Tq * 8 if k_tok else (Tq // G) * 8 * d
    return Tq * 4 * (wk + wv) + kmeta + Tq * 8 + (N - Tq) * 4 * d


def layer_row(lc):
    """(kb, vb, R, per-token Key, recent-token ratio in parts per thousand) of a
    layer-table row (kb, vb, R[, k_mode[, rpc_permille]])."""
    return lc[0], lc[1], lc[2], len(lc) > 3 and lc[3] == 1, lc[4] if len(lc) > 4 else 0


def quantized_count(N, R, G, kb, rpc=0):
    """Tokens held as codes after N appends: a full buffer (N - Tq = R before an
    append) gives up f tokens, f = G, or with a recent-token ratio the whole
    groups beyond floor(R * rpc / 1000); this happens before the appends of
    tokens R, R + f, R + 2f, ..."""
    if kb == 16 or N <= R:
        return 0
    f = G if rpc == 0 else max(G, (R - R * rpc // 1000) // G * G)
    return f * ((N - 1 - R) // f + 1)


def step_bytes(w, N_before, qbytes):
    """Algorithmic bytes of one decode step over all layers, and of attention
    only; N_before: tokens held by each sequence before the step (a list, or
    one count for every sequence)."""
    B, Hkv, Hq, d, G = w.batch, w.n_kv_heads, w.n_q_heads, w.head_dim, w.G
    Ns = N_before if isinstance(N_before, (list, tuple)) else [N_before] * B
    att = app = 0
    for lc in w.layers:
        kb, vb, R, kt, rpc = layer_row(lc)
        att += B * Hq * d * (qbytes + 4)
        for N0 in Ns:
            N1 = N0 + 1
            Tq0 = quantized_count(N0, R, G, kb, rpc)
            Tq1 = quantized_count(N1, R, G, kb, rpc)
            att += Hkv * stream_state_bytes(d, kb, vb, G, N1, Tq1, kt)
            app += Hkv * 2 * d * 2 * 2  # read new K and V, write them to the ring
            if Tq1 > Tq0:  # flush: read the given-up 16-bit K/V rows, write codes and metadata
                wk = (d + 10) // 11 if kb == 3 else d * kb // 32
                nf = Tq1 - Tq0
                app += Hkv * (nf * 4 * d + nf * 4 * (wk + d * vb // 32) + (8 * nf if kt else 8 * d * nf // G)
                              + 8 * nf)
    return att, app


def ragged_contexts(context, B):
    """Sequence b starts with context * (0.25 + 1.5 b / (B - 1)) tokens: lengths
    spread evenly from a quarter to 1.75 times the workload's context (mean
    about the context)."""
    if B == 1:
        return [context]
    return [max(1, int(round(context * (0.25 + 1.5 * b / (B - 1))))) for b in range(B)]


def kernel_source_digest():
    """Digest of the HIP sources: a stored counter measurement applies only to
    the kernels it was taken on."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "decode_attention_streaming_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def stored_traffic(workload, table, kind="attention"):
    """HBM bytes per launch (kind: "attention" for decode, "prefill") from the
    stored FETCH_SIZE / WRITE_SIZE measurement of this workload, or None when
    the kernels have changed since."""
    path = os.path.join(ROOT, "profiles", "%s_traffic_workload%d_%s.json" % (kind, workload, table))
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_digest") != kernel_source_digest():
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(w, seconds, layers_sample):
    """Time the CPU oracle (single thread) on a sample of the same workload:
    prefill the sampled layers (untimed), then repeat decode steps (append one
    token + attention) until `seconds` have passed; scale to all layers."""
    import numpy as np
    import torch

    from decode_attention_streaming_amd import synth
    from oracle import oracle as ora

    B, Hkv, g, d = w.batch, w.n_kv_heads, w.g, w.head_dim
    BH = B * Hkv
    qb = 2 if w.q_dtype != "f32" else 4
    cap = w.context + 4096
    layers = []
    for l in layers_sample:
        kb, vb, R, kt, rpc = layer_row(w.layers[l])
        o = ora.Layer(BH, g, d, kb, vb, w.G, R, cap, w.kv_dtype == "bf16", k_tok=kt, rpc_permille=rpc)
        k, v = synth.layer_tokens(w, l, 0, w.context, "cpu")
        o.append(synth.bits16(k.reshape(BH, w.context, d)), synth.bits16(v.reshape(BH, w.context, d)))
        layers.append((l, o))
    steps = 0
    nbytes = 0
    el = 0.0  # oracle time only; input generation is excluded
    while el < seconds:
        for l, o in layers:
            k, v = synth.layer_tokens(w, l, o.N, 1, "cpu")
            q = synth.as_f64(synth.query(w, l, steps, "cpu").reshape(BH, g, d))
            kb16 = synth.bits16(k.reshape(BH, 1, d))
            vb16 = synth.bits16(v.reshape(BH, 1, d))
            t0 = time.perf_counter()
            o.append(kb16, vb16)
            o.attention(q)
            el += time.perf_counter() - t0
            nbytes += BH * stream_state_bytes(d, o.k_bits, o.v_bits, o.G, o.N, o.Tq, o.k_tok) + \
                B * w.n_q_heads * d * (qb + 4) + BH * 2 * d * 2 * 2
        steps += 1
    layer_steps = steps * len(layers)
    step_time = el / layer_steps * len(w.layers)  # one full step over all layers
    return {
        "value": round(nbytes / el / 1e9, 4),
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "tok_per_s": round(B / step_time, 3),
        "sample": "%d decode steps (append 1 token + fp64 attention) on layers %s of %d, all %d "
                  "streams, %.1f s of oracle time; tok/s scaled to all layers"
                  % (steps, list(layers_sample), len(w.layers), BH, el),
    }


MFMA_F16_PEAK_TFLOPS = 2500.0


def prefill_leg(cache, w, C, ends, qbytes, rounds, stream, dev):
    """Causal attention of the last C tokens' queries over every layer's cache
    (the chunk is already appended; sequence b holds ends[b] tokens), timed
    with HIP events on the library's stream over back-to-back calls.
    Algorithmic flops: 2 d per visible (query head, token) pair for q.K and
    2 d for P.V; algorithmic bytes: the layer's cache state once, q and out."""
    import torch

    from decode_attention_streaming_amd import synth

    B, Hq, Hkv, d, L = w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.n_layers
    qs = [synth.queries(w, l, C, dev, seed=7).permute(1, 2, 0, 3).contiguous() for l in range(L)]
    outs = [torch.empty((B, Hq, C, d), dtype=torch.float32, device=dev) for _ in range(L)]
    for l in range(L):
        cache.prefill_attention(l, qs[l], outs[l])
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for r in range(rounds):
        for l in range(L):
            cache.prefill_attention(l, qs[l], outs[l])
    ev1.record(stream)
    torch.cuda.synchronize()
    call_us = ev0.elapsed_time(ev1) * 1e3 / (rounds * L)
    visible = sum(C * (n - C) + C * (C + 1) // 2 for n in ends)  # (query, token) pairs per head
    flops = 4.0 * d * visible * Hq
    nbytes = 0
    for lc in w.layers:
        kb, vb, R, kt, rpc = layer_row(lc)
        nbytes += Hkv * sum(stream_state_bytes(d, kb, vb, w.G, n, quantized_count(n, R, w.G, kb, rpc), kt)
                            for n in ends)
    nbytes = nbytes / L + B * Hq * C * d * (qbytes + 4)
    tflops = flops / (call_us * 1e-6) / 1e12
    return {
        "chunk": C, "context": ends[0] if len(set(ends)) == 1 else ends, "avg_call_us": round(call_us, 3),
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": MFMA_F16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / MFMA_F16_PEAK_TFLOPS, 4)},
        "gbs": round(nbytes / (call_us * 1e-6) / 1e9, 1),
        "flops_per_call": flops, "bytes_per_call": int(nbytes),
        "tok_per_s": round(B * C / (call_us * 1e-6 * L), 1),
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=128)
    ap.add_argument("--warmup", type=int, default=32)
    ap.add_argument("--workload", type=int, default=2)
    ap.add_argument("--table", default="default", choices=["default", "k8v8", "k4v4"],
                    help="layer table: the workload's mixed table, or uniform KV8 / KV4 baselines")
    ap.add_argument("--k-mode", default="per-channel", choices=["per-channel", "per-token"],
                    help="Key quantization: per channel over G tokens (KIVI) or per token")
    ap.add_argument("--rpc", action="store_true",
                    help="KVmix dynamic recent-token ratio: 20 %% on the table's higher-precision "
                         "layers, 10 %% on the lowest-precision ones")
    ap.add_argument("--ragged", action="store_true",
                    help="sequences of different lengths: sequence b starts with context x "
                         "(0.25 + 1.5 b / (B - 1)) tokens")
    ap.add_argument("--kernel-rounds", type=int, default=20)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--prefill-chunk", type=int, default=256,
                    help="also time causal prefill attention of the last C tokens of every layer "
                         "(0 = skip)")
    ap.add_argument("--copy-mb", type=int, default=0,
                    help="also run a plain device copy of this size (counter scaling)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this build measures one GPU only; --gpus %d is not supported "
              "(the sharded path is described in the design notes, not built)" % args.gpus,
              file=sys.stderr)
        sys.exit(2)

    import torch

    from decode_attention_streaming_amd import kvq, synth

    dev = "cuda"
    w = synth.workload(args.workload)
    if args.table in ("k8v8", "k4v4"):
        b = int(args.table[1])
        w.layers = [(b, b, r) for (_, _, r) in w.layers]
    if args.k_mode == "per-token":
        if any(lc[0] == 3 for lc in w.layers):
            print("per-token Key needs 2, 4 or 8 Key bits; this table has 3-bit layers", file=sys.stderr)
            sys.exit(2)
        w.layers = [(kb, vb, r, 1) for (kb, vb, r) in w.layers]
    if args.rpc:
        low = min(lc[0] + lc[1] for lc in w.layers)
        w.layers = [(lc[0], lc[1], lc[2], lc[3] if len(lc) > 3 else 0, 200 if lc[0] + lc[1] > low else 100)
                    for lc in w.layers]
    L, B, Hq, Hkv, d = w.n_layers, w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim
    total = args.warmup + args.steps
    qbytes = 4 if w.q_dtype == "f32" else 2
    ctx = ragged_contexts(w.context, B) if args.ragged else [w.context] * B
    cache = kvq.Cache(L, B, Hq, Hkv, d, max(ctx) + total, w.kv_dtype, w.q_dtype, w.G, w.R, w.layers)
    stream = cache.stream

    # prefill every layer, then stage all decode inputs in HBM
    knew, vnew, qs = [], [], []
    for l in range(L):
        st = synth.LayerStats(w, l)
        k, v = synth.layer_tokens(w, l, 0, max(ctx), dev, stats=st)
        if args.ragged:
            cache.append_ragged(l, k, v, ctx)
        else:
            cache.append(l, k, v)
        del k, v
        k, v = synth.layer_tokens(w, l, max(ctx), total, dev, stats=st)
        knew.append(k.permute(2, 0, 1, 3).contiguous().unsqueeze(3))  # [total, B, Hkv, 1, d]
        vnew.append(v.permute(2, 0, 1, 3).contiguous().unsqueeze(3))
        qs.append(synth.queries(w, l, total, dev))
    outs = [torch.empty((B, Hq, d), dtype=torch.float32, device=dev) for _ in range(L)]
    torch.cuda.synchronize()

    def step(s):
        # one call per layer: append one token per sequence, then attend
        for l in range(L):
            cache.append_decode_attention(l, knew[l][s], vnew[l][s], qs[l][s], outs[l])

    for s in range(args.warmup):
        step(s)
    torch.cuda.synchronize()

    att_bytes = app_bytes = 0
    for s in range(args.warmup, total):
        a, p = step_bytes(w, [c + s for c in ctx], qbytes)
        att_bytes += a
        app_bytes += p

    t0 = time.perf_counter()
    for s in range(args.warmup, total):
        step(s)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall / args.steps * 1e3

    # the state the library reports agrees with the byte model used above
    ends = [c + total for c in ctx]
    for l, lc in enumerate(w.layers):
        kb, vb, R, kt, rpc = layer_row(lc)
        info = cache.bytes_layer(l)
        assert cache.sequence_lengths(l)[0] == ends
        assert info.total == sum(Hkv * stream_state_bytes(d, kb, vb, w.G, n, quantized_count(n, R, w.G, kb, rpc), kt)
                                 for n in ends)

    # dominant kernel: decode attention (one launch per call).  HIP events on
    # the stream the library launches on bracket back-to-back calls over every
    # layer (state fixed), several rounds; average = elapsed / calls.
    rounds = args.kernel_rounds
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for l in range(L):  # warm
        cache.decode_attention(l, qs[l][total - 1], outs[l])
    ev0.record(stream)
    for r in range(rounds):
        for l in range(L):
            cache.decode_attention(l, qs[l][total - 1], outs[l])
    ev1.record(stream)
    torch.cuda.synchronize()
    avg_call_us = ev0.elapsed_time(ev1) * 1e3 / (rounds * L)

    # the same calls captured once in a HIP graph and replayed: no host work
    # between the launches (the library allocates nothing and sets no memory
    # from the host, so the calls are capturable); outputs checked against eager
    ref = [o.clone() for o in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    cache.set_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        for l in range(L):
            cache.decode_attention(l, qs[l][total - 1], outs[l])
    cache.set_stream(stream)
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    assert all(torch.equal(o, r) for o, r in zip(outs, ref)), "graph replay differs from eager calls"
    gev0, gev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    gev0.record()
    for r in range(rounds):
        graph.replay()
    gev1.record()
    torch.cuda.synchronize()
    graph_call_us = gev0.elapsed_time(gev1) * 1e3 / (rounds * L)
    del graph
    att_per_layer = []
    for l, lc in enumerate(w.layers):
        kb, vb, R, kt, rpc = layer_row(lc)
        att_per_layer.append(sum(Hkv * stream_state_bytes(d, kb, vb, w.G, n, quantized_count(n, R, w.G, kb, rpc), kt)
                                 for n in ends) + B * Hq * d * (qbytes + 4))
    avg_att_bytes = sum(att_per_layer) / L
    achieved = avg_att_bytes / (avg_call_us * 1e-6) / 1e9
    splits, variant = kvq.kvq_last_launch(cache.h)
    traffic = stored_traffic(args.workload, args.table) if args.k_mode == "per-channel" and not (
        args.ragged or args.rpc) else None

    prefill = None
    C = min(args.prefill_chunk, min(ends))
    if C > 0 and (w.head_dim == 128 or all(lc[0] != 3 for lc in w.layers)) and w.G % 32 == 0:
        prefill = prefill_leg(cache, w, C, ends, qbytes, rounds, stream, dev)
        if C == 256 and args.k_mode == "per-channel" and not (args.ragged or args.rpc):
            prefill["roofline"]["traffic"] = stored_traffic(args.workload, args.table, "prefill")

    if args.copy_mb > 0:  # a plain copy of known size, for scaling memory counters
        n = args.copy_mb * (1 << 20)
        src = torch.ones(n // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()

    value = (att_bytes + app_bytes) / wall / 1e9
    res = {
        "metric": "quantized-KV decode attention: effective HBM GB/s (% of peak), decode tok/s",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "pct_of_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "tok_per_s": round(B * args.steps / wall, 1),
        "attention_gbs_wall": round(att_bytes / wall / 1e9, 2),
        "config": {
            "workload": w.name,
            "layers": L, "batch": B, "n_q_heads": Hq, "n_kv_heads": Hkv, "head_dim": d,
            "context_start": w.context if not args.ragged else ctx, "G": w.G, "R": w.R,
            "kv_dtype": w.kv_dtype, "q_dtype": w.q_dtype,
            "table": "".join("K%dV%d " % tuple(lc[:2]) for lc in w.layers).strip(),
            "k_mode": args.k_mode,
            "equiv_bits": w.equiv_bits()["kv"],
            "parallelism": "single GPU",
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "kernel": "decode attention (one launch per call: split units + in-kernel merge), "
                      "variant %d (1 = matrix core), %d work units per stream" % (variant, splits),
            "avg_call_us": round(avg_call_us, 3),
            "graph_avg_call_us": round(graph_call_us, 3),
            "bytes_per_call": int(avg_att_bytes),
        },
    }
    if prefill is not None:
        res["prefill"] = prefill
    if not args.no_cpu_baseline and not args.ragged:
        sample = [0, 1] if L >= 2 else [0]
        res["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds, sample)
    cache.close()
    print(json.dumps(res))


if __name__ == "__main__":
    main()
