"""Pins of the CPU oracle against what the pages and mathematics fix.

Each test checks the oracle against something other than itself: a printed
worked example, a closed form, an invariant, a special case that reduces to a
library routine (numpy/torch conversions, torch's fp64 scaled-dot-product
attention), or brute force on tiny inputs.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import oracle as ora

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------------------
# KV memory formula (KIVI notes, sections 2.1-2.2 and exercise 1)
# ---------------------------------------------------------------------------

def test_kv_bytes_worked_examples():
    for ex in _gold("kv_bytes_examples.json")["examples"]:
        L, H, d = ex["n_layers"], ex["n_kv_heads"], ex["head_dim"]
        per_tok = L * H * ora.stream_bytes(d, 16, 16, 32, 1, 0)
        assert per_tok == ex["per_token_bytes_printed"]
        if "per_token_MB_approx" in ex:
            assert round(per_tok / 2 ** 20, 2) == ex["per_token_MB_approx"]
        if "per_token_KB_printed" in ex:
            assert per_tok / 1024 == ex["per_token_KB_printed"]
        for c in ex["contexts"]:
            total = L * H * ora.stream_bytes(d, 16, 16, 32, c["tokens"], 0)
            digits = 2 if c["GB_approx"] < 10 else (1 if c["GB_approx"] != int(c["GB_approx"]) else 0)
            assert round(total / 1e9, digits) == c["GB_approx"]


def test_kv_bytes_two_bit_exercise_reading():
    """Exercise 1 prints '2-bit ~ 2.15 GB (4x saving)' for 64 L x 4 H x 128 at
    64K tokens.  The codes alone at 2 bits come to 1,073,741,824 B (8x less than
    fp16); 2.15 GB is exactly the 4-bit code size.  The test fixes the
    arithmetic and records the page's figure as the 4-bit one."""
    ex = _gold("kv_bytes_examples.json")["examples"][1]
    L, H, d, S = 64, 4, 128, 65536
    fp16 = L * H * ora.stream_bytes(d, 16, 16, 32, S, 0)

    def codes_only(bits):
        return L * H * S * 4 * (ora.words_per_row(d, bits) * 2)

    assert codes_only(2) == 1073741824 and fp16 // codes_only(2) == 8
    assert codes_only(4) == 2147483648
    assert round(codes_only(4) / 1e9, 2) == ex["two_bit_GB_approx_printed"]
    assert fp16 // codes_only(4) == ex["two_bit_saving_printed"]


def test_stream_bytes_closed_form():
    # per stream: codes + K meta per group + V meta per token + 16-bit recent tokens
    d, G = 128, 32
    for kb, vb in [(8, 8), (8, 4), (4, 4), (4, 2), (2, 2), (3, 4)]:
        N, Tq = 1024, 992
        wk = {2: 8, 3: 12, 4: 16, 8: 32}[kb]
        wv = {2: 8, 4: 16, 8: 32}[vb]
        expect = Tq * 4 * (wk + wv) + (Tq // G) * 2 * 4 * d + Tq * 2 * 4 + (N - Tq) * 2 * 2 * d
        assert ora.stream_bytes(d, kb, vb, G, N, Tq) == expect


# ---------------------------------------------------------------------------
# Packing (KVmix notes, key design 2)
# ---------------------------------------------------------------------------

def test_packing_printed_words():
    gold = _gold("packing_examples.json")
    for w in gold["words"]:
        codes = np.array(w["codes"], np.uint8)
        d = len(codes) if w["bits"] != 3 else 11
        words = ora.pack_row(codes, w["bits"])
        assert words[0] == int(w["word"], 16), w
        assert np.array_equal(ora.unpack_row(words, d, w["bits"]), codes)


def test_three_bit_layout_d128():
    gold = _gold("packing_examples.json")["k3_d128"]
    assert ora.words_per_row(128, 3) == gold["words_per_row"]
    two_bit = [c for c in range(128) if ora.qmax(3, c) == 3]
    assert two_bit == gold["two_bit_channels"]
    assert all(ora.qmax(3, c) == 7 for c in range(128) if c not in two_bit)
    # eleven codes per word against ten for a uniform 3-bit packing: 10% denser
    assert 11 / (32 // 3) == pytest.approx(1.1)
    # all-max row: the last word holds channels 121..127 in slots 0..6, pads 0
    codes = np.array([ora.qmax(3, c) for c in range(128)], np.uint8)
    words = ora.pack_row(codes, 3)
    assert all(words[i] == 0xFFFFFFFF for i in range(11))
    assert words[11] == (1 << 21) - 1


@pytest.mark.parametrize("bits,d", [(2, 16), (2, 128), (4, 64), (4, 128), (8, 128),
                                    (8, 256), (3, 128), (3, 64), (3, 33)])
def test_pack_roundtrip(bits, d):
    rng = np.random.default_rng(bits * 1000 + d)
    for _ in range(50):
        codes = np.array([rng.integers(0, ora.qmax(bits, c) + 1) for c in range(d)], np.uint8)
        words = ora.pack_row(codes, bits)
        assert words.shape[0] == ora.words_per_row(d, bits)
        assert np.array_equal(ora.unpack_row(words, d, bits), codes)
        # every bit of the row is accounted for: the number of set bits equals
        # the popcount of the codes (no overlaps, no stray bits in padding)
        assert sum(bin(int(x)).count("1") for x in words) == sum(bin(int(c)).count("1") for c in codes)


# ---------------------------------------------------------------------------
# 16-bit formats widen exactly (library routines decide)
# ---------------------------------------------------------------------------

def test_f16_widening_all_patterns():
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = pats.view(np.float16).astype(np.float32)
    got = np.array([ora.f16_to_f32(p) for p in pats[::7]], np.float32)
    r = ref[::7]
    nan = np.isnan(r)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), r[~nan].view(np.uint32))


def test_bf16_widening_patterns():
    pats = np.arange(0, 65536, 5, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(pats.view(np.int16)).view(torch.bfloat16).to(torch.float32).numpy()
    got = np.array([ora.bf16_to_f32(p) for p in pats], np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


# ---------------------------------------------------------------------------
# Quantizer (KVTuner summary A3; KVmix notes key design 2)
# ---------------------------------------------------------------------------

def test_quantizer_ties_round_half_even():
    for c in _gold("quantizer_ties.json")["cases"]:
        codes, s, z = ora.quantize(np.array(c["x"], np.float32), (1 << c["bits"]) - 1)
        assert codes.tolist() == c["codes"]
        assert s == c["s"] and z == c["z"]


@pytest.mark.parametrize("qm", [3, 7, 15, 255])
def test_quantizer_ends_and_error_bound(qm):
    rng = np.random.default_rng(qm)
    worst = 0.0
    for trial in range(1500):
        n = int(rng.integers(2, 160))
        scale = float(np.exp(rng.normal(0, 3)))
        x = (rng.standard_normal(n) * scale + rng.normal(0, 5) * scale).astype(np.float32)
        codes, s, z = ora.quantize(x, qm)
        if x.max() == x.min():
            continue
        # the minimum maps to code 0 and the maximum to qmax
        assert codes[np.argmin(x)] == 0 and codes[np.argmax(x)] == qm
        assert z == x.min()
        # z and s are the pages' formulas in fp32
        assert s == np.float32(np.float32(x.max() - x.min()) / np.float32(qm))
        xhat = codes.astype(np.float64) * float(s) + float(z)
        err = np.abs(xhat - x.astype(np.float64)).max()
        # |x - x^| <= s/2 in exact arithmetic; the fp32 subtraction and division
        # can move the rounding point by a few ulps of the quotient (<= qmax)
        assert err <= float(s) / 2 * (1 + qm * 2.0 ** -20), (trial, err, s)
        worst = max(worst, err / (float(s) / 2))
        assert codes.max() <= qm
    assert worst > 0.9  # the bound is tight: errors near s/2 do occur


def test_quantizer_degenerate_and_signed_zero():
    codes, s, z = ora.quantize(np.full(7, 1.25, np.float32), 15)
    assert codes.tolist() == [0] * 7 and s == 0.0 and z == np.float32(1.25)
    codes, s, z = ora.quantize(np.array([-0.0, 0.0, -0.0], np.float32), 3)
    assert codes.tolist() == [0, 0, 0]
    assert np.float32(s).view(np.uint32) == 0 and np.float32(z).view(np.uint32) == 0
    codes, s, z = ora.quantize(np.array([-0.0, 2.0, 3.0], np.float32), 3)
    assert np.float32(z).view(np.uint32) == 0 and codes.tolist() == [0, 2, 3]


def test_quantizer_on_grid_is_lossless():
    rng = np.random.default_rng(5)
    for qm in (3, 7, 15, 255):
        for _ in range(200):
            e = int(rng.integers(-8, 3))
            step = 2.0 ** e
            mn = float(rng.integers(-64, 64)) * step
            k = rng.integers(0, qm + 1, size=40)
            k[int(rng.integers(40))] = 0
            k[int(rng.integers(40))] = qm
            if k.min() != 0 or k.max() != qm:
                continue
            x = (mn + k * step).astype(np.float32)
            assert np.array_equal(x.astype(np.float64), mn + k * step)
            codes, s, z = ora.quantize(x, qm)
            assert np.array_equal(codes, k) and s == step and z == mn


# ---------------------------------------------------------------------------
# Streaming bookkeeping (KIVI notes, section 6.2)
# ---------------------------------------------------------------------------

def _expected_tq(N, R, G):
    return G * max(0, -(-(N - R) // G))


@pytest.mark.parametrize("G,R", [(32, 32), (8, 20), (32, 819), (32, 409), (64, 64), (128, 128),
                                 (1, 1), (4, 7)])
def test_residual_closed_form(G, R):
    lay = ora.Layer(1, 1, 16, 4, 2, G, R, 1200, False)
    rng = np.random.default_rng(G * 7 + R)
    for n in range(1200):
        k = rng.integers(0, 0x3C00, size=(1, 1, 16)).astype(np.uint16)
        lay.append(k, k)
        N = n + 1
        assert lay.N == N and lay.Tq == _expected_tq(N, R, G)
        if N > R:
            assert R - G + 1 <= N - lay.Tq <= R


def test_stated_states():
    # (G, R, N) -> (Tq, Tr) for the five workloads' prefills
    cases = [((32, 32, 288), (256, 32)), ((32, 32, 1024), (992, 32)), ((64, 64, 4096), (4032, 64)),
             ((128, 128, 32768), (32640, 128)), ((32, 819, 4096), (3296, 800)),
             ((32, 409, 4096), (3712, 384))]
    for (G, R, N), (Tq, Tr) in cases:
        assert _expected_tq(N, R, G) == Tq and N - Tq == Tr


def _rand_tokens(rng, S, n, d, bf16):
    x = rng.standard_normal((S, n, d)).astype(np.float32) * 3
    if bf16:
        return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    return x.astype(np.float16).view(np.uint16)


@pytest.mark.parametrize("kb,vb,bf16", [(4, 2, False), (8, 4, True), (3, 4, False), (2, 2, True)])
def test_prefill_equals_token_by_token(kb, vb, bf16):
    rng = np.random.default_rng(kb * 10 + vb)
    S, d, G, R, N = 3, 64, 16, 24, 200
    k = _rand_tokens(rng, S, N, d, bf16)
    v = _rand_tokens(rng, S, N, d, bf16)
    a = ora.Layer(S, 2, d, kb, vb, G, R, N, bf16)
    b = ora.Layer(S, 2, d, kb, vb, G, R, N, bf16)
    a.append(k, v)
    cut = [0, 1, 7, 50, 51, 120, 200]
    for i in range(len(cut) - 1):
        b.append(k[:, cut[i]:cut[i + 1]], v[:, cut[i]:cut[i + 1]])
    ea, eb = a.export(), b.export()
    for key in ea:
        assert np.array_equal(np.asarray(ea[key]), np.asarray(eb[key])), key


def test_group_codes_permutation_invariant_and_value_per_token():
    rng = np.random.default_rng(11)
    S, d, G = 2, 32, 8
    k = _rand_tokens(rng, S, G, d, False)
    v = _rand_tokens(rng, S, G, d, False)
    a = ora.Layer(S, 1, d, 4, 2, G, G, 2 * G, False)
    a.append(k, v)
    a.append(k[:, :1], v[:, :1])  # forces the flush of the first group
    perm = rng.permutation(G)
    b = ora.Layer(S, 1, d, 4, 2, G, G, 2 * G, False)
    b.append(k[:, perm], v[:, perm])
    b.append(k[:, :1], v[:, :1])
    ea, eb = a.export(), b.export()
    assert np.array_equal(ea["k_scale"], eb["k_scale"]) and np.array_equal(ea["k_zero"], eb["k_zero"])
    assert np.array_equal(ea["k_words"][:, perm], eb["k_words"])
    assert np.array_equal(ea["v_words"][:, perm], eb["v_words"])
    # a token's V codes and (s, z) come from that token alone
    for s in range(S):
        for t in range(G):
            x = np.array([ora.f16_to_f32(p) for p in v[s, t]], np.float32)
            lo, hi = x.min(), x.max()
            assert ea["v_zero"][s, t] == lo
            assert ea["v_scale"][s, t] == np.float32(np.float32(hi - lo) / np.float32(3))


# ---------------------------------------------------------------------------
# Attention (KVTuner summary, A3 attention equation; Lemma 1 in A7)
# ---------------------------------------------------------------------------

def _sdpa64(q, K, V):
    """q [S,g,d], K/V [S,N,d] (fp64) -> [S,g,d] via torch's fp64 SDPA on the CPU."""
    qt = torch.from_numpy(q)[:, :, None, :]           # [S, g, 1, d]
    kt = torch.from_numpy(K)[:, None].expand(-1, q.shape[1], -1, -1)
    vt = torch.from_numpy(V)[:, None].expand(-1, q.shape[1], -1, -1)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt.contiguous(), vt.contiguous())
    return o[:, :, 0, :].numpy()


def _widen(bits, bf16):
    if bf16:
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    return bits.view(np.float16).astype(np.float64)


@pytest.mark.parametrize("g,d,N,bf16", [(1, 16, 1, False), (4, 64, 37, True), (7, 32, 100, False)])
def test_attention_unquantized_matches_sdpa(g, d, N, bf16):
    rng = np.random.default_rng(g * 100 + N)
    S = 2
    k = _rand_tokens(rng, S, N, d, bf16)
    v = _rand_tokens(rng, S, N, d, bf16)
    lay = ora.Layer(S, g, d, 16, 16, 8, 8, N, bf16)
    lay.append(k, v)
    q = rng.standard_normal((S, g, d))
    out = lay.attention(q)
    ref = _sdpa64(q, _widen(k, bf16), _widen(v, bf16))
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)


def grid_tokens(rng, S, N, d, G, kb, vb, bf16):
    """K/V whose quantization is lossless: per (group, channel) for K and per
    token for V, the values are z + code * 2^e with both code 0 and code qmax
    present, and every value exact in the 16-bit format."""
    def qmk(c):
        return ora.qmax(kb, c)
    K = np.zeros((S, N, d))
    V = np.zeros((S, N, d))
    for s in range(S):
        for g0 in range(0, N, G):
            n = min(G, N - g0)
            for c in range(d):
                qm = qmk(c)
                e = int(rng.integers(-4, 0)) if qm < 255 else -3
                z = float(rng.integers(-8, 8)) * 2.0 ** e if qm < 255 else 0.0
                codes = rng.integers(0, qm + 1, size=n)
                if n >= 2:
                    i, j = rng.choice(n, 2, replace=False)
                    codes[i], codes[j] = 0, qm
                K[s, g0:g0 + n, c] = z + codes * 2.0 ** e
        for t in range(N):
            qm = (1 << vb) - 1
            e = int(rng.integers(-4, 0)) if qm < 255 else -3
            z = float(rng.integers(-8, 8)) * 2.0 ** e if qm < 255 else 0.0
            codes = rng.integers(0, qm + 1, size=d)
            i, j = rng.choice(d, 2, replace=False)
            codes[i], codes[j] = 0, qm
            V[s, t] = z + codes * 2.0 ** e
    dt = torch.bfloat16 if bf16 else torch.float16
    kb16 = torch.from_numpy(K).to(dt)
    vb16 = torch.from_numpy(V).to(dt)
    assert np.array_equal(kb16.to(torch.float64).numpy(), K)
    assert np.array_equal(vb16.to(torch.float64).numpy(), V)
    return (kb16.view(torch.int16).numpy().view(np.uint16),
            vb16.view(torch.int16).numpy().view(np.uint16), K, V)


@pytest.mark.parametrize("kb,vb,G,R,N,g,bf16", [
    (4, 2, 8, 8, 40, 2, False),
    (2, 2, 4, 6, 33, 1, True),
    (8, 4, 8, 12, 50, 4, False),
    (3, 4, 8, 8, 45, 3, False),
    (8, 8, 16, 16, 64, 1, True),
])
def test_attention_on_grid_matches_sdpa(kb, vb, G, R, N, g, bf16):
    """With lossless quantization, attention over the quantized cache must equal
    plain fp64 attention over the raw tokens: any slip in codes, packing, group
    or token indexing, metadata, the recent-token split or GQA mapping shows."""
    rng = np.random.default_rng(kb * 31 + N)
    S, d = 2, 32 if kb != 3 else 64
    kbits, vbits, K, V = grid_tokens(rng, S, N, d, G, kb, vb, bf16)
    lay = ora.Layer(S, g, d, kb, vb, G, R, N, bf16)
    lay.append(kbits[:, :N - 5], vbits[:, :N - 5])
    for t in range(N - 5, N):
        lay.append(kbits[:, t:t + 1], vbits[:, t:t + 1])
    assert lay.Tq == _expected_tq(N, R, G) and lay.Tq > 0
    q = rng.standard_normal((S, g, d))
    np.testing.assert_allclose(lay.attention(q), _sdpa64(q, K, V), rtol=1e-11, atol=1e-12)
    # q = 0: uniform attention, the output is the mean value row
    np.testing.assert_allclose(lay.attention(np.zeros((S, g, d))),
                               np.repeat(V.mean(axis=1)[:, None], g, axis=1), rtol=1e-12, atol=1e-12)


def test_attention_dominant_key_lemma1():
    """KVTuner summary, A7 Lemma 1: with one dominant key the attention output
    is that token's value; quantization elsewhere does not move it."""
    rng = np.random.default_rng(3)
    S, d, G, N = 1, 32, 8, 48
    kbits, vbits, K, V = grid_tokens(rng, S, N, d, G, 4, 2, False)
    lay = ora.Layer(S, 1, d, 4, 2, G, G, N, False)
    lay.append(kbits, vbits)
    c = 5
    i = int(np.argmax(K[0, :lay.Tq, c]))
    gap = K[0, i, c] - np.sort(K[0, :, c])[-2]
    assert gap > 0
    q = np.zeros((S, 1, d))
    q[0, 0, c] = 60.0 * math.sqrt(d) / gap
    out = lay.attention(q)
    np.testing.assert_allclose(out[0, 0], V[0, i], rtol=0, atol=1e-12)


def test_attention_softmax_shift_invariance():
    """Adding a constant to every key of one channel shifts all scores of a
    head by the same amount; the output must not move."""
    rng = np.random.default_rng(9)
    S, d, G, N = 1, 32, 8, 40
    kbits, vbits, K, V = grid_tokens(rng, S, N, d, G, 4, 4, False)
    a = ora.Layer(S, 2, d, 4, 4, G, G, N, False)
    a.append(kbits, vbits)
    K2 = K.copy()
    K2[:, :, 3] += 2.0
    k2 = torch.from_numpy(K2).to(torch.float16)
    assert np.array_equal(k2.to(torch.float64).numpy(), K2)
    b = ora.Layer(S, 2, d, 4, 4, G, G, N, False)
    b.append(k2.view(torch.int16).numpy().view(np.uint16), vbits)
    q = rng.standard_normal((S, 2, d))
    np.testing.assert_allclose(a.attention(q), b.attention(q), rtol=1e-12, atol=1e-12)
    assert np.array_equal(a.export()["k_words"], b.export()["k_words"])


# ---------------------------------------------------------------------------
# Chunked-prefill attention (KVTuner summary, A3 attention equation: the query
# of step i attends to the keys up to and including step i; A2 calibration:
# prefill attention runs on the dequantized cache)
# ---------------------------------------------------------------------------

def _sdpa64_causal(q, K, V):
    """q [S,g,n_q,d], K/V [S,N,d] (fp64); query j attends to tokens
    0 .. N - n_q + j.  torch's fp64 SDPA with an explicit boolean mask."""
    S, g, n_q, d = q.shape
    N = K.shape[1]
    mask = torch.arange(N)[None, :] <= (N - n_q + torch.arange(n_q))[:, None]  # [n_q, N]
    kt = torch.from_numpy(K)[:, None].expand(-1, g, -1, -1).contiguous()
    vt = torch.from_numpy(V)[:, None].expand(-1, g, -1, -1).contiguous()
    o = torch.nn.functional.scaled_dot_product_attention(torch.from_numpy(q), kt, vt, attn_mask=mask)
    return o.numpy()


@pytest.mark.parametrize("g,d,N,n_q,bf16", [(1, 16, 1, 1, False), (4, 32, 37, 37, True),
                                           (2, 64, 50, 9, False), (7, 32, 70, 1, True)])
def test_prefill_unquantized_matches_causal_sdpa(g, d, N, n_q, bf16):
    rng = np.random.default_rng(g * 1000 + N + n_q)
    S = 2
    k = _rand_tokens(rng, S, N, d, bf16)
    v = _rand_tokens(rng, S, N, d, bf16)
    lay = ora.Layer(S, g, d, 16, 16, 8, 8, N, bf16)
    lay.append(k, v)
    q = rng.standard_normal((S, g, n_q, d))
    ref = _sdpa64_causal(q, _widen(k, bf16), _widen(v, bf16))
    np.testing.assert_allclose(lay.prefill_attention(q), ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("kb,vb,G,R,N,n_q,g,bf16", [
    (4, 2, 8, 8, 40, 40, 2, False),   # whole sequence: the mask cuts through every group
    (2, 4, 4, 6, 33, 20, 1, True),    # chunk longer than the recent buffer
    (8, 8, 16, 16, 64, 5, 4, False),  # chunk inside the recent buffer
    (3, 4, 8, 8, 45, 17, 3, False),
])
def test_prefill_on_grid_matches_causal_sdpa(kb, vb, G, R, N, n_q, g, bf16):
    """Lossless quantization: causal attention over the quantized cache equals
    fp64 causal attention over the raw tokens, whichever tokens the chunk's
    queries see in codes and which in 16 bits."""
    rng = np.random.default_rng(kb * 77 + N + n_q)
    S, d = 2, 32 if kb != 3 else 64
    kbits, vbits, K, V = grid_tokens(rng, S, N, d, G, kb, vb, bf16)
    lay = ora.Layer(S, g, d, kb, vb, G, R, N, bf16)
    lay.append(kbits[:, :N - n_q], vbits[:, :N - n_q])
    lay.append(kbits[:, N - n_q:], vbits[:, N - n_q:])
    assert lay.Tq == _expected_tq(N, R, G) and lay.Tq > 0
    q = rng.standard_normal((S, g, n_q, d))
    np.testing.assert_allclose(lay.prefill_attention(q), _sdpa64_causal(q, K, V), rtol=1e-11, atol=1e-12)


def _np_unpack(words, d, bits):
    """LSB-first codes of 2/4/8-bit rows, written independently of the oracle."""
    per = 32 // bits
    c = np.arange(d)
    return (words[..., c // per] >> np.uint32(bits) * (c % per).astype(np.uint32)) & np.uint32((1 << bits) - 1)


def test_prefill_first_query_and_zero_query_closed_forms():
    """Off-grid data.  With n_q = N the first query sees token 0 alone, so its
    output is that token's dequantized value; a zero query weighs its visible
    tokens equally, so query j's output is the mean of the dequantized values
    of tokens 0 .. N - n_q + j (values rebuilt here from the canonical export)."""
    rng = np.random.default_rng(21)
    S, g, d, G, R, N = 2, 2, 32, 8, 12, 41
    k = _rand_tokens(rng, S, N, d, False)
    v = _rand_tokens(rng, S, N, d, False)
    lay = ora.Layer(S, g, d, 4, 2, G, R, N, False)
    lay.append(k, v)
    ex = lay.export()
    Tq = ex["Tq"]
    vcodes = _np_unpack(ex["v_words"], d, 2).astype(np.float64)
    vhat = np.concatenate([vcodes * ex["v_scale"][..., None].astype(np.float64)
                           + ex["v_zero"][..., None].astype(np.float64),
                           _widen(ex["res_v"], False)], axis=1)  # [S, N, d]
    assert Tq > 0 and vhat.shape == (S, N, d)
    out = lay.prefill_attention(rng.standard_normal((S, g, N, d)))
    np.testing.assert_allclose(out[:, :, 0], np.repeat(vhat[:, None, 0], g, axis=1), rtol=0, atol=1e-12)
    n_q = 30
    out0 = lay.prefill_attention(np.zeros((S, g, n_q, d)))
    for j in range(n_q):
        p = N - n_q + j
        np.testing.assert_allclose(out0[:, :, j], np.repeat(vhat[:, None, :p + 1].mean(axis=2), g, axis=1),
                                   rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------------------
# Dynamic recent-token ratio (KVmix notes, key design 3: num_RPC =
# floor(r x current_RPC), 20 % for high-precision layers, 10 % for the rest).
# Reading: an append that finds the recent buffer full keeps floor(r * current)
# of its tokens in 16 bits and quantizes the older rest in whole groups.
# ---------------------------------------------------------------------------

def _rpc_states(G, R, r, Ns, cap):
    lay = ora.Layer(1, 1, 16, 4, 2, G, R, cap, False, rpc_permille=r)
    seen = {}
    for n in range(1, max(Ns) + 1):
        k = np.full((1, 1, 16), 0x3C00, np.uint16)
        lay.append(k, k)
        assert lay.N - lay.Tq <= R and lay.Tq % G == 0
        if n in Ns:
            seen[n] = (lay.Tq, lay.N - lay.Tq)
    return seen


def test_rpc_worked_examples():
    # G 4, R 20, r 20 %: full at N = 20; the 21st token finds 20 recent tokens,
    # keeps floor(0.2 * 20) = 4, quantizes 16 (four groups) -> Tq 16, Tr 5; full
    # again 15 tokens later (N = 36) -> the 37th gives Tq 32, Tr 5; and so on.
    assert _rpc_states(4, 20, 200, [20, 21, 36, 37, 52, 53], 64) == {
        20: (0, 20), 21: (16, 5), 36: (16, 20), 37: (32, 5), 52: (32, 20), 53: (48, 5)}
    # G 8, R 50, r 10 %: keep floor(5.0) = 5, quantize floor(45 / 8) = 5 groups =
    # 40 -> Tq 40, Tr 11 at N = 51; next at N = 91 -> Tq 80, Tr 11.
    assert _rpc_states(8, 50, 100, [50, 51, 90, 91], 96) == {50: (0, 50), 51: (40, 11), 90: (40, 50),
                                                               91: (80, 11)}
    # Llama-2-7B-shaped MHA layers (G 32): R 819 at 20 % keeps floor(163.8) =
    # 163 and quantizes 20 groups (640 of 656); R 409 at 10 % keeps 40 and
    # quantizes 11 groups (352 of 369).
    assert _rpc_states(32, 819, 200, [819, 820], 832) == {819: (0, 819), 820: (640, 180)}
    assert _rpc_states(32, 409, 100, [409, 410], 416) == {409: (0, 409), 410: (352, 58)}
    # a ratio that keeps more than R - G still gives up one group
    assert _rpc_states(8, 10, 900, [10, 11], 32) == {10: (0, 10), 11: (8, 3)}


@pytest.mark.parametrize("kb,vb,G,R,r,N,g,bf16", [
    (4, 2, 8, 24, 200, 100, 2, False),
    (3, 4, 8, 30, 100, 90, 1, True),
])
def test_rpc_prefill_token_by_token_and_attention_on_grid(kb, vb, G, R, r, N, g, bf16):
    """One call of N tokens equals N single appends (state bit for bit), and on
    lossless data attention over the cache equals fp64 SDPA over the raw tokens."""
    rng = np.random.default_rng(kb * 13 + N + r)
    S, d = 2, 32 if kb != 3 else 64
    kbits, vbits, K, V = grid_tokens(rng, S, N, d, G, kb, vb, bf16)
    a = ora.Layer(S, g, d, kb, vb, G, R, N, bf16, rpc_permille=r)
    b = ora.Layer(S, g, d, kb, vb, G, R, N, bf16, rpc_permille=r)
    a.append(kbits, vbits)
    for t in range(N):
        b.append(kbits[:, t:t + 1], vbits[:, t:t + 1])
    ea, eb = a.export(), b.export()
    assert ea["Tq"] == eb["Tq"] > 0
    for key in ("k_words", "k_scale", "k_zero", "v_words", "v_scale", "v_zero", "res_k", "res_v"):
        assert np.asarray(ea[key]).tobytes() == np.asarray(eb[key]).tobytes(), key
    q = rng.standard_normal((S, g, d))
    np.testing.assert_allclose(a.attention(q), _sdpa64(q, K, V), rtol=1e-11, atol=1e-12)


# ---------------------------------------------------------------------------
# Byte accounting against the stored state (KIVI notes, section 2.1: the KV
# size is what the cache holds; KVTuner summary, A3: codes plus one scale and
# zero per quantization group)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("kb,vb,k_tok,rpc,G,R,N", [
    (2, 2, False, 0, 32, 32, 150), (3, 4, False, 0, 32, 40, 170), (4, 2, False, 0, 16, 16, 75),
    (4, 4, False, 0, 32, 32, 33), (8, 4, False, 0, 8, 24, 61), (8, 8, False, 0, 32, 32, 96),
    (2, 8, True, 0, 16, 16, 90), (4, 2, True, 0, 32, 48, 130), (8, 8, True, 0, 8, 8, 41),
    (4, 4, False, 200, 8, 50, 140), (3, 2, False, 100, 16, 80, 230), (4, 2, True, 150, 8, 40, 111),
    (16, 16, False, 0, 32, 32, 70), (4, 2, False, 0, 32, 32, 20)])
def test_live_bytes_equal_exported_state(kb, vb, k_tok, rpc, G, R, N):
    """The live byte count is the size of the state the layer actually holds:
    Layer.bytes() equals the summed sizes of the arrays its canonical export
    returns (packed K and V words, K and V scales and zeros, 16-bit recent K and
    V), for every bit pair, both Key modes, a recent-token ratio and a layer kept
    in 16 bits, before and after flushes.  The export's array shapes come from
    the stored state (tokens held, words per row, one scale and zero per group
    and channel or per token), not from the byte formula."""
    rng = np.random.default_rng(1000 + kb * 100 + vb * 10 + N)
    S, d, g = 3, 64, 2
    lay = ora.Layer(S, g, d, kb, vb, G, R, N + 8, kb == 4, k_tok=k_tok, rpc_permille=rpc)
    seen = set()
    for n in (N // 3, 1, N - N // 3 - 1):
        if n <= 0:
            continue
        lay.append(_rand_tokens(rng, S, n, d, kb == 4), _rand_tokens(rng, S, n, d, kb == 4))
        ex = lay.export()
        held = sum(ex[k].nbytes for k in ("k_words", "k_scale", "k_zero", "v_words", "v_scale",
                                           "v_zero", "res_k", "res_v"))
        assert lay.bytes() == held, (lay.N, lay.Tq)
        seen.add(lay.Tq > 0)
    if kb != 16 and N > R:
        assert True in seen  # the case crossed at least one flush
