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
    """The stored HBM-traffic measurement of this workload (L2-to-fabric read
    and write requests by size; decode: the record, with the state it was
    taken at; prefill: HBM bytes per launch), or None when the kernels have
    changed since."""
    path = os.path.join(ROOT, "profiles", "%s_traffic_workload%d_%s.json" % (kind, workload, table))
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_digest") != kernel_source_digest():
        return None
    return rec if kind == "attention" else rec.get("hbm_bytes_per_launch")


def host_cores():
    """CPUs this process may run on (read at run time), and the host's model name."""
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return n, model


def _oracle_decode_run(w, layers_sample, threads, seconds):
    """The oracle as it stands on a sample of the workload: the sampled layers'
    streams are split into `threads` independent oracle layers (disjoint
    (sequence, kv-head) streams, so the results do not change), prefilled
    untimed; then decode steps (append one token + fp64 attention on every
    stream) run until `seconds` of wall time have passed, each step's oracle
    calls spread over a pool of `threads` threads (the oracle's C calls release
    the interpreter lock).  Returns (steps, bytes, elapsed seconds)."""
    from concurrent.futures import ThreadPoolExecutor

    from decode_attention_streaming_amd import synth
    from oracle import oracle as ora

    B, Hkv, g, d = w.batch, w.n_kv_heads, w.g, w.head_dim
    BH = B * Hkv
    qb = 2 if w.q_dtype != "f32" else 4
    cap = w.context + 2048
    bounds = [(BH * i // threads, BH * (i + 1) // threads) for i in range(threads)]
    parts = []  # (layer index, [(s0, s1, oracle layer)])
    for l in layers_sample:
        kb, vb, R, kt, rpc = layer_row(w.layers[l])
        k, v = synth.layer_tokens(w, l, 0, w.context, "cpu")
        k16 = synth.bits16(k.reshape(BH, w.context, d))
        v16 = synth.bits16(v.reshape(BH, w.context, d))
        subs = []
        for s0, s1 in bounds:
            o = ora.Layer(s1 - s0, g, d, kb, vb, w.G, R, cap, w.kv_dtype == "bf16", k_tok=kt, rpc_permille=rpc)
            o.append(k16[s0:s1], v16[s0:s1])
            subs.append((s0, s1, o))
        parts.append((l, subs))
    steps = nbytes = 0
    el = 0.0  # oracle time only; input generation is excluded
    with ThreadPoolExecutor(max_workers=threads) as pool:
        while el < seconds:
            work = []
            for l, subs in parts:
                k, v = synth.layer_tokens(w, l, subs[0][2].N, 1, "cpu")
                q = synth.as_f64(synth.query(w, l, steps, "cpu").reshape(BH, g, d))
                kb16 = synth.bits16(k.reshape(BH, 1, d))
                vb16 = synth.bits16(v.reshape(BH, 1, d))
                for s0, s1, o in subs:
                    work.append((o, kb16[s0:s1], vb16[s0:s1], q[s0:s1]))

            def run(item):
                o, kk, vv, qq = item
                o.append(kk, vv)
                o.attention(qq)

            t0 = time.perf_counter()
            list(pool.map(run, work))
            el += time.perf_counter() - t0
            for l, subs in parts:
                o0 = subs[0][2]
                nbytes += BH * stream_state_bytes(d, o0.k_bits, o0.v_bits, o0.G, o0.N, o0.Tq, o0.k_tok) + \
                    B * w.n_q_heads * d * (qb + 4) + BH * 2 * d * 2 * 2
            steps += 1
    return steps, nbytes, el


def cpu_baseline(w, seconds, layers_sample):
    """Time the CPU oracle on a sample of the same workload, on one core and
    on every host core this process may use (core count read at run time), and
    scale tok/s to all layers."""
    n_cores, model = host_cores()
    B, BH = w.batch, w.batch * w.n_kv_heads
    threads = max(1, min(n_cores, BH))
    res = {}
    for key, t, sec in (("one", 1, seconds / 2), ("all", threads, seconds / 2)):
        steps, nbytes, el = _oracle_decode_run(w, layers_sample, t, sec)
        step_time = el / steps * len(w.layers) / len(layers_sample)  # one full step over all layers
        res[key] = dict(value=round(nbytes / el / 1e9, 4), tok_per_s=round(B / step_time, 3), steps=steps,
                        seconds=round(el, 2), threads=t)
    one, allc = res["one"], res["all"]
    return {
        "value": allc["value"],
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "tok_per_s": allc["tok_per_s"],
        "one_core": {"value": one["value"], "unit": "GB/s", "tok_per_s": one["tok_per_s"]},
        "host": {"cpus_available": n_cores, "model": model},
        "sample": "decode steps (append 1 token + fp64 attention, all %d streams) on layers %s of %d: "
                  "%d steps in %.1f s on 1 thread, %d steps in %.1f s of wall time on %d threads "
                  "(streams split into %d independent oracle layers); tok/s scaled to all layers"
                  % (BH, list(layers_sample), len(w.layers), one["steps"], one["seconds"], allc["steps"],
                     allc["seconds"], threads, threads),
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


def page_table(B, cap_tokens, P, seed, dev):
    """A block table for B sequences of up to cap_tokens tokens in pages of P:
    every (sequence, page) entry a distinct page of a pool with a few unused
    pages, in a seeded random order (non-contiguous).  Returns (table, n_pages)."""
    import numpy as np
    import torch
    stride = -(-cap_tokens // P)
    n_pages = B * stride + 8
    perm = np.random.default_rng(seed).permutation(n_pages)[:B * stride].astype(np.int32)
    return torch.from_numpy(perm.reshape(B, stride)).to(dev), n_pages


def build_cache(kvq, synth, w, ctx, cap_tokens, dev, ragged, paged=0, seed=0):
    """A cache of workload w holding ctx[b] prefilled tokens per sequence
    (paged > 0: its quantized state in pages of that many tokens)."""
    L, B, Hq, Hkv, d = w.n_layers, w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim
    kw = {}
    if paged:
        table, n_pages = page_table(B, cap_tokens, paged, seed, dev)
        kw = dict(page_tokens=paged, n_pages=n_pages, block_table=table)
    cache = kvq.Cache(L, B, Hq, Hkv, d, cap_tokens, w.kv_dtype, w.q_dtype, w.G, w.R, w.layers, **kw)
    for l in range(L):
        k, v = synth.layer_tokens(w, l, 0, max(ctx), dev, stats=synth.LayerStats(w, l))
        if ragged:
            cache.append_ragged(l, k, v, ctx)
        else:
            cache.append(l, k, v)
        del k, v
    return cache


def decode_inputs(synth, w, t0, n_steps, dev):
    """Per layer: K and V of the next n_steps tokens ([n_steps, B, Hkv, 1, d])
    and n_steps queries ([n_steps, B, Hq, d])."""
    knew, vnew, qs = [], [], []
    for l in range(w.n_layers):
        k, v = synth.layer_tokens(w, l, t0, n_steps, dev, stats=synth.LayerStats(w, l))
        knew.append(k.permute(2, 0, 1, 3).contiguous().unsqueeze(3))
        vnew.append(v.permute(2, 0, 1, 3).contiguous().unsqueeze(3))
        qs.append(synth.queries(w, l, n_steps, dev))
    return knew, vnew, qs


def timed_calls(torch, stream, fn, rounds):
    """Average time of fn() (one round of back-to-back calls) from HIP events
    on `stream` around `rounds` rounds."""
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    fn()
    ev0.record(stream)
    for _ in range(rounds):
        fn()
    ev1.record(stream)
    torch.cuda.synchronize()
    return ev0.elapsed_time(ev1) * 1e-3 / rounds


def copy_ceiling(torch, stream, nbytes, L, rounds, dev):
    """Plain device copies timed like the attention calls: L buffers of nbytes
    (read + write = nbytes per call), cycled back to back; a sum over L buffers
    of nbytes (a read-only pass); one 256 MiB copy (the box's streaming rate,
    partly from the last-level cache) and a sum over 1 GiB (the streaming read
    rate from HBM).  GB/s of bytes moved."""
    nbytes = int(nbytes)
    half = max(16, nbytes // 2 // 16 * 16)
    src = [torch.ones(half // 4, dtype=torch.float32, device=dev) for _ in range(L)]
    dst = [torch.empty_like(x) for x in src]
    t_copy = timed_calls(torch, stream, lambda: [b.copy_(a) for a, b in zip(src, dst)], rounds) / L
    del src, dst
    full = max(16, nbytes // 16 * 16)
    bufs = [torch.ones(full // 4, dtype=torch.float32, device=dev) for _ in range(L)]
    sink = torch.empty(L, dtype=torch.float32, device=dev)
    t_sum = timed_calls(torch, stream, lambda: [torch.sum(b, dim=0, out=sink[i]) for i, b in enumerate(bufs)],
                        rounds) / L
    del bufs
    big = 256 << 20
    a = torch.ones(big // 4, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    t_big = timed_calls(torch, stream, lambda: b.copy_(a), 5)
    del a, b
    # a read-only pass over 1 GiB (4x the last-level cache): the streaming read
    # rate from HBM of a plain reduction
    huge = 1 << 30
    a = torch.ones(huge // 4, dtype=torch.float32, device=dev)
    s1 = torch.empty((), dtype=torch.float32, device=dev)
    t_read = timed_calls(torch, stream, lambda: torch.sum(a, dim=0, out=s1), 5)
    del a, s1
    res = {
        "bytes_per_call": int(nbytes),
        "copy_gbs": round(2 * half / t_copy / 1e9, 1),
        "copy_us": round(t_copy * 1e6, 3),
        "read_sum_gbs": round(full / t_sum / 1e9, 1),
        "read_sum_us": round(t_sum * 1e6, 3),
        "stream_copy_256mib_gbs": round(2 * big / t_big / 1e9, 1),
        "stream_read_1gib_gbs": round(huge / t_read / 1e9, 1),
    }
    res["ceiling_gbs"] = max(res["copy_gbs"], res["read_sum_gbs"])
    return res


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
    ap.add_argument("--paged", type=int, default=0, metavar="P",
                    help="keep each quantized layer's state in pages of P tokens named by a shuffled "
                         "block table (0: a region per stream)")
    ap.add_argument("--kernel-rounds", type=int, default=20)
    ap.add_argument("--cpu-seconds", type=float, default=20.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--prefill-chunk", type=int, default=256,
                    help="also time causal prefill attention of the last C tokens of every layer "
                         "(0 = skip)")
    ap.add_argument("--copy-mb", type=int, default=0,
                    help="also run a plain device copy of this size (counter scaling)")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the second cache instance, the flush probe, the copy ceiling and the "
                         "KV8 comparison (shorter runs under a profiler)")
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
    probe = 0 if args.no_extras else 2 * w.G  # flush probe: steps after the timed ones
    qbytes = 4 if w.q_dtype == "f32" else 2
    ctx = ragged_contexts(w.context, B) if args.ragged else [w.context] * B
    cap_tokens = max(ctx) + total + probe + 1
    cache = build_cache(kvq, synth, w, ctx, cap_tokens, dev, args.ragged, args.paged, seed=1)
    stream = cache.stream
    knew, vnew, qs = decode_inputs(synth, w, max(ctx), total + probe, dev)
    outs = [torch.empty((B, Hq, d), dtype=torch.float32, device=dev) for _ in range(L)]
    torch.cuda.synchronize()

    def step(c, s):
        # one call per layer: append one token per sequence, then attend
        for l in range(L):
            c.append_decode_attention(l, knew[l][s], vnew[l][s], qs[l][s], outs[l])

    for s in range(args.warmup):
        step(cache, s)
    torch.cuda.synchronize()

    att_bytes = app_bytes = 0
    for s in range(args.warmup, total):
        a, p = step_bytes(w, [c + s for c in ctx], qbytes)
        att_bytes += a
        app_bytes += p

    t0 = time.perf_counter()
    for s in range(args.warmup, total):
        step(cache, s)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall / args.steps * 1e3
    # flush launches inside the timed steps (a layer whose recent buffer is full)
    timed_flushes = 0
    for s in range(args.warmup, total):
        for lc in w.layers:
            kb, vb, R, kt, rpc = layer_row(lc)
            due = [quantized_count(c + s + 1, R, w.G, kb, rpc) > quantized_count(c + s, R, w.G, kb, rpc)
                   for c in ctx]
            timed_flushes += sum(due) if args.ragged else int(any(due))

    # the state the library reports agrees with the byte model used above
    ends = [c + total for c in ctx]
    for l, lc in enumerate(w.layers):
        kb, vb, R, kt, rpc = layer_row(lc)
        info = cache.bytes_layer(l)
        assert cache.sequence_lengths(l)[0] == ends
        assert info.total == sum(Hkv * stream_state_bytes(d, kb, vb, w.G, n, quantized_count(n, R, w.G, kb, rpc), kt)
                                 for n in ends)
    att_per_layer = []
    for l, lc in enumerate(w.layers):
        kb, vb, R, kt, rpc = layer_row(lc)
        att_per_layer.append(sum(Hkv * stream_state_bytes(d, kb, vb, w.G, n, quantized_count(n, R, w.G, kb, rpc), kt)
                                 for n in ends) + B * Hq * d * (qbytes + 4))
    avg_att_bytes = sum(att_per_layer) / L

    # dominant kernel: decode attention (one launch per call).  HIP events on
    # the stream the library launches on bracket back-to-back calls over every
    # layer (state fixed), several rounds; average = elapsed / calls.
    rounds = args.kernel_rounds
    qlast = [qs[l][total - 1] for l in range(L)]

    def one_round(c):
        for l in range(L):
            c.decode_attention(l, qlast[l], outs[l])

    avg_call_us = timed_calls(torch, stream, lambda: one_round(cache), rounds) * 1e6 / L

    # the same calls captured once in a HIP graph and replayed: no host work
    # between the launches (the library allocates nothing and sets no memory
    # from the host, so the calls are capturable); outputs checked against eager
    ref = [o.clone() for o in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    cache.set_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        one_round(cache)
    cache.set_stream(stream)
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    assert all(torch.equal(o, r) for o, r in zip(outs, ref)), "graph replay differs from eager calls"
    graph_call_us = timed_calls(torch, torch.cuda.current_stream(), graph.replay, rounds) * 1e6 / L
    del graph

    # a second cache instance with the same state: calls alternate between the
    # two, so that the working set (2 x all layers) is well beyond the 256 MB
    # last-level cache and every call reads its state from HBM
    two_call_us = None
    if not args.no_extras:
        cache2 = build_cache(kvq, synth, w, ctx, cap_tokens, dev, args.ragged, args.paged, seed=2)
        for s in range(total):
            step(cache2, s)
        outs2 = [torch.empty_like(o) for o in outs]

        def two_rounds():
            for l in range(L):
                cache.decode_attention(l, qlast[l], outs[l])
                cache2.decode_attention(l, qlast[l], outs2[l])

        two_call_us = timed_calls(torch, stream, two_rounds, rounds) * 1e6 / (2 * L)
        assert all(torch.equal(a, b) for a, b in zip(outs, outs2)), "second instance differs"
        cache2.close()
        del cache2, outs2
        torch.cuda.empty_cache()

    splits, variant = kvq.kvq_last_launch(cache.h)
    call_us = two_call_us if two_call_us is not None else avg_call_us
    achieved = avg_att_bytes / (call_us * 1e-6) / 1e9
    traffic = None
    if args.k_mode == "per-channel" and not (args.ragged or args.rpc or args.paged):
        traffic = stored_traffic(args.workload, args.table)

    # flush probe: 2G more steps timed one by one with events; the steps in
    # which some layer's recent buffer is full carry a flush launch
    flush = None
    if probe > 0:
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(probe + 1)]
        evs[0].record(stream)
        for i in range(probe):
            step(cache, total + i)
            evs[i + 1].record(stream)
        torch.cuda.synchronize()
        times = [evs[i].elapsed_time(evs[i + 1]) for i in range(probe)]
        nfl = []  # flush launches per step: one per layer, or one per sequence of a ragged batch
        for i in range(probe):
            n = 0
            for lc in w.layers:
                kb, vb, R, kt, rpc = layer_row(lc)
                due = [quantized_count(c + total + i + 1, R, w.G, kb, rpc) >
                       quantized_count(c + total + i, R, w.G, kb, rpc) for c in ctx]
                n += sum(due) if args.ragged else int(any(due))
            nfl.append(n)
        fl = [t for t, n in zip(times, nfl) if n > 0]
        plain = [t for t, n in zip(times, nfl) if n == 0]
        flush = {"probe_steps": probe, "flush_steps": len(fl), "flush_launches": sum(nfl),
                 "plain_step_ms": round(sum(plain) / len(plain), 4) if plain else None,
                 "flush_step_ms": round(sum(fl) / len(fl), 4) if fl else None,
                 "timed_window_flush_launches": timed_flushes}
        if fl and plain:
            extra = sum(fl) / len(fl) - sum(plain) / len(plain)
            flush["extra_ms_per_flush_step"] = round(extra, 4)
            flush["amortized_ms_per_step"] = round(extra * len(fl) / probe, 4)
            flush["per_flush_launch_us"] = round(1e3 * extra * len(fl) / sum(nfl), 3)
        ends = [c + total + probe for c in ctx]

    ceiling = None
    if not args.no_extras:
        ceiling = copy_ceiling(torch, stream, avg_att_bytes, L, rounds, dev)

    prefill = None
    C = min(args.prefill_chunk, min(ends))
    if C > 0 and (w.head_dim == 128 or all(lc[0] != 3 for lc in w.layers)) and w.G % 32 == 0:
        prefill = prefill_leg(cache, w, C, ends, qbytes, rounds, stream, dev)
        if C == 256 and args.k_mode == "per-channel" and not (args.ragged or args.rpc or args.paged):
            prefill["roofline"]["traffic"] = stored_traffic(args.workload, args.table, "prefill")
    cache.close()
    del cache
    torch.cuda.empty_cache()

    # KIVI-KV8 analogue: the same shape with every layer K8V8, same steps
    kv8 = None
    if not args.no_extras and args.table == "default" and args.k_mode == "per-channel" and not (
            args.ragged or args.rpc or args.paged) and all(lc[0] != 3 for lc in w.layers):
        w8 = synth.workload(args.workload)
        w8.layers = [(8, 8, r) for (_, _, r) in w8.layers]
        c8 = build_cache(kvq, synth, w8, ctx, cap_tokens, dev, False)
        for s in range(args.warmup):
            step(c8, s)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for s in range(args.warmup, total):
            step(c8, s)
        torch.cuda.synchronize()
        wall8 = time.perf_counter() - t0
        a8 = p8 = 0
        for s in range(args.warmup, total):
            a, p = step_bytes(w8, [c + s for c in ctx], qbytes)
            a8 += a
            p8 += p
        c8.close()
        del c8
        kv8 = {"table": "K8V8 on every layer", "ms_per_step": round(wall8 / args.steps * 1e3, 4),
               "tok_per_s": round(B * args.steps / wall8, 1), "gbs": round((a8 + p8) / wall8 / 1e9, 2),
               "bytes_ratio_vs_table": round((a8 + p8) / (att_bytes + app_bytes), 3),
               "table_speedup_vs_kv8": round(wall8 / wall, 3)}

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
        "dtype": "f16/bf16 matrix-core products (fp32 factors as hi+lo fp16 pairs), fp32 accumulation",
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
            "paged": ({"page_tokens": args.paged, "table": "shuffled, non-contiguous"} if args.paged
                      else None),
            "parallelism": "single GPU",
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic["hbm_bytes_per_launch"] if traffic else None,
            "kernel": "decode attention (one launch per call: split units + in-kernel merge), "
                      "variant %d (1 = matrix core), %d work units per stream" % (variant, splits),
            "avg_call_us": round(call_us, 3),
            "timing": ("two cache instances with the same state, calls alternating (working set %.0f MB)"
                       % (2 * sum(att_per_layer) / 1e6)) if two_call_us is not None else
                      "one cache instance, calls over every layer",
            "single_instance_avg_call_us": round(avg_call_us, 3),
            "graph_avg_call_us": round(graph_call_us, 3),
            "bytes_per_call": int(avg_att_bytes),
            "state_tokens": max(c + total for c in ctx),
        },
    }
    if traffic:
        res["roofline"]["traffic_measured"] = {
            k: traffic.get(k) for k in ("state_tokens", "algorithmic_bytes_per_launch", "ratio")}
    if ceiling is not None:
        ceiling["frac_of_ceiling"] = round(achieved / ceiling["ceiling_gbs"], 4)
        res["roofline"]["copy_ceiling"] = ceiling
    if flush is not None:
        res["flush"] = flush
    if prefill is not None:
        res["prefill"] = prefill
    if kv8 is not None:
        res["kv8_comparison"] = kv8
    if not args.no_cpu_baseline and not args.ragged:
        sample = [0, 1] if L >= 2 else [0]
        res["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds, sample)
    print(json.dumps(res))


if __name__ == "__main__":
    main()
