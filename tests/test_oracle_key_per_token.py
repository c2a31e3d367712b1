"""Pins of the oracle's per-token-asym Key mode (KVTuner summary: the KIVI and
per-token-asym quantization modes it evaluates; A3 quantization basics): each
Key token is quantized over its own head_dim channels with one scale and zero,
exactly as a Value token, and the streaming rule (recent-token buffer, flush of
G tokens) is unchanged."""
import numpy as np
import pytest
import torch

from oracle import oracle as ora
from test_oracle_pins import _expected_tq, _sdpa64, _widen


def _rand_rows(rng, S, N, d, bf16, outliers=True):
    """Synthetic K-like rows: channel means and spreads, two outlier channels x10."""
    mu = rng.standard_normal((S, 1, d))
    sig = np.exp(0.5 * rng.standard_normal((S, 1, d)))
    x = mu + sig * rng.standard_normal((S, N, d))
    if outliers:
        for s in range(S):
            x[s, :, rng.choice(d, 2, replace=False)] *= 10.0
    dt = torch.bfloat16 if bf16 else torch.float16
    t = torch.from_numpy(x).to(dt)
    return t.view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("kb,G,R,N,bf16", [(2, 8, 8, 50, False), (4, 32, 40, 140, True),
                                           (8, 16, 16, 70, False)])
def test_per_token_key_scale_zero_and_error_bound(kb, G, R, N, bf16):
    """z_t = min over the token's channels, s_t = fl32(fl32(max - min) / qmax);
    codes in [0, qmax]; every dequantized element within s_t / 2 of its input."""
    rng = np.random.default_rng(kb * 100 + N)
    S, d = 3, 64
    k = _rand_rows(rng, S, N, d, bf16)
    v = _rand_rows(rng, S, N, d, bf16, outliers=False)
    lay = ora.Layer(S, 2, d, kb, 4, G, R, N, bf16, k_tok=True)
    lay.append(k, v)
    Tq = lay.Tq
    assert Tq == _expected_tq(N, R, G) and Tq > 0
    ex = lay.export()
    assert ex["k_scale"].shape == (S, Tq) and ex["k_zero"].shape == (S, Tq)
    x = _widen(k, bf16).astype(np.float32)
    qm = (1 << kb) - 1
    for s in range(S):
        for t in range(Tq):
            row = x[s, t]
            lo, hi = row.min(), row.max()
            assert ex["k_zero"][s, t] == lo
            assert ex["k_scale"][s, t] == np.float32(np.float32(hi - lo) / np.float32(qm))
            codes = ora.unpack_row(ex["k_words"][s, t], d, kb)
            assert codes.min() >= 0 and codes.max() <= qm
            sc = np.float64(ex["k_scale"][s, t])
            deq = codes.astype(np.float64) * sc + np.float64(ex["k_zero"][s, t])
            # s/2 in exact arithmetic; the fp32 subtraction and division can move
            # the rounding point by a few ulps of the quotient (<= qmax)
            assert np.all(np.abs(deq - row.astype(np.float64)) <= sc / 2 * (1 + qm * 2.0 ** -20))
    # the residual part is the raw tail
    assert np.array_equal(ex["res_k"], k[:, Tq:N])


def test_per_token_key_rows_are_independent():
    """Per-token Key codes of a row depend on that row only: permuting the
    tokens of the flushed history permutes the codes and metadata (per-channel
    Key would mix rows through the group's min/max)."""
    rng = np.random.default_rng(11)
    S, d, G, N = 2, 32, 8, 40
    k = _rand_rows(rng, S, N, d, False)
    v = _rand_rows(rng, S, N, d, False, outliers=False)
    perm = np.arange(N)
    perm[:32] = rng.permutation(32)  # tokens 0..31 are flushed below (R = G = 8)
    a = ora.Layer(S, 1, d, 4, 2, G, G, N, False, k_tok=True)
    b = ora.Layer(S, 1, d, 4, 2, G, G, N, False, k_tok=True)
    a.append(k, v)
    b.append(k[:, perm], v[:, perm])
    ea, eb = a.export(), b.export()
    assert ea["Tq"] == eb["Tq"] == 32
    for key in ("k_words", "k_scale", "k_zero"):
        np.testing.assert_array_equal(eb[key], ea[key][:, perm[:32]])
    # per channel, the same permutation does not commute with the groups
    c = ora.Layer(S, 1, d, 4, 2, G, G, N, False)
    e = ora.Layer(S, 1, d, 4, 2, G, G, N, False)
    c.append(k, v)
    e.append(k[:, perm], v[:, perm])
    assert not np.array_equal(e.export()["k_words"], c.export()["k_words"][:, perm[:32]])


def _grid_rows(rng, S, N, d, qm, bf16):
    """Rows z_t + code * 2^e_t with codes 0 and qm present in each row: a row's
    per-token quantization is lossless."""
    X = np.zeros((S, N, d))
    for s in range(S):
        for t in range(N):
            e = int(rng.integers(-4, 0)) if qm < 255 else -3
            z = float(rng.integers(-8, 8)) * 2.0 ** e if qm < 255 else 0.0
            codes = rng.integers(0, qm + 1, size=d)
            i, j = rng.choice(d, 2, replace=False)
            codes[i], codes[j] = 0, qm
            X[s, t] = z + codes * 2.0 ** e
    dt = torch.bfloat16 if bf16 else torch.float16
    xt = torch.from_numpy(X).to(dt)
    assert np.array_equal(xt.to(torch.float64).numpy(), X)
    return xt.view(torch.int16).numpy().view(np.uint16), X


@pytest.mark.parametrize("kb,vb,G,R,N,g,bf16", [(4, 2, 8, 8, 40, 2, False), (2, 4, 4, 6, 33, 1, True),
                                                (8, 8, 16, 16, 64, 4, False)])
def test_per_token_key_on_grid_attention_matches_sdpa(kb, vb, G, R, N, g, bf16):
    """On-grid rows make the quantization lossless: attention over the
    per-token-Key cache equals plain fp64 attention over the raw tokens."""
    rng = np.random.default_rng(kb * 13 + vb + N)
    S, d = 2, 32
    kbits, K = _grid_rows(rng, S, N, d, (1 << kb) - 1, bf16)
    vbits, V = _grid_rows(rng, S, N, d, (1 << vb) - 1, bf16)
    lay = ora.Layer(S, g, d, kb, vb, G, R, N, bf16, k_tok=True)
    lay.append(kbits[:, :N - 3], vbits[:, :N - 3])
    for t in range(N - 3, N):
        lay.append(kbits[:, t:t + 1], vbits[:, t:t + 1])
    assert lay.Tq == _expected_tq(N, R, G) and lay.Tq > 0
    q = rng.standard_normal((S, g, d))
    np.testing.assert_allclose(lay.attention(q), _sdpa64(q, K, V), rtol=1e-11, atol=1e-12)


def test_per_token_key_bytes():
    """One fp32 scale and zero per quantized Key token instead of per (group,
    channel): k_meta = 8 Tq bytes."""
    d, G = 128, 32
    for kb, vb, N, Tq in [(4, 2, 1024, 992), (8, 4, 300, 256), (2, 2, 64, 32)]:
        wk, wv = ora.words_per_row(d, kb), ora.words_per_row(d, vb)
        expect = Tq * 4 * (wk + wv) + Tq * 8 + Tq * 8 + (N - Tq) * 4 * d
        assert ora.stream_bytes(d, kb, vb, G, N, Tq, True) == expect
        assert ora.stream_bytes(d, kb, vb, G, N, Tq, False) - expect == (Tq // G) * 8 * d - Tq * 8
