"""C-ABI checks that need no GPU: the library loads, exports every declared
symbol, and validates arguments on the host before any device work."""
import ctypes
import os
import re

import pytest

from decode_attention_streaming_amd import kvq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "kvq.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(kvq_[a-z_]+)\s*\(", src)))


def test_exports_every_declared_symbol():
    L = kvq.lib()
    names = _declared()
    assert len(names) >= 12
    for n in names:
        assert hasattr(L, n), n
    assert sorted(kvq.EXPORTED) == names


def _cfg(**kw):
    base = dict(n_layers=2, batch=2, n_q_heads=8, n_kv_heads=2, head_dim=128, max_context=256,
                kv_dtype="bf16", q_dtype="f32", group_size=32, residual_len=32,
                layers=[(4, 2, 0), (8, 4, 64)])
    base.update(kw)
    return kvq.make_config(**base)


def test_recent_ratio_validation():
    """rpc_permille must lie in [0, 1000); bytes_layer reports it."""
    for bad in (-1, 1000, 5000):
        assert kvq.kvq_workspace_bytes(_cfg(layers=[(4, 2, 0, 0, bad), (8, 4, 64)])) == 0
        assert "rpc_permille" in kvq.kvq_last_error()
    cfg = _cfg(layers=[(4, 2, 0, 0, 200), (8, 4, 64, 0, 999)])
    n = kvq.kvq_workspace_bytes(cfg)
    assert n > 0
    h = kvq.kvq_create(cfg, ctypes.c_void_p(1 << 20), n)
    try:
        assert kvq.kvq_bytes_layer(h, 0).rpc_permille == 200
        assert kvq.kvq_bytes_layer(h, 1).rpc_permille == 999
    finally:
        kvq.kvq_destroy(h)


def test_ragged_append_validation_without_device_work():
    """kvq_append_ragged checks every count before any device work: counts
    outside [0, n_max], a sequence past max_context, NULL pointers; all-zero
    counts are a no-op; per-sequence lengths start at zero."""
    cfg = _cfg()
    n = kvq.kvq_workspace_bytes(cfg)
    h = kvq.kvq_create(cfg, ctypes.c_void_p(1 << 20), n)
    p = ctypes.c_void_p(1 << 21)
    try:
        cases = [
            (lambda: kvq.kvq_append_ragged(h, 0, p, p, [3, 9], 8), kvq.KVQ_EINVAL, "n_new[1] = 9 outside"),
            (lambda: kvq.kvq_append_ragged(h, 0, p, p, [-1, 0], 8), kvq.KVQ_EINVAL, "n_new[0] = -1 outside"),
            (lambda: kvq.kvq_append_ragged(h, 0, p, p, [0, 257], 300), kvq.KVQ_ECAPACITY, "sequence 1"),
            (lambda: kvq.kvq_append_ragged(h, 0, None, p, [1, 0], 1), kvq.KVQ_EINVAL, "NULL"),
            (lambda: kvq.kvq_append_ragged(h, 2, p, p, [1, 0], 1), kvq.KVQ_EINVAL, "out of range"),
            (lambda: kvq.kvq_append_ragged(h, 0, p, p, [1, 0], -1), kvq.KVQ_EINVAL, "n_max"),
        ]
        for fn, code, msg in cases:
            with pytest.raises(kvq.KvqError) as e:
                fn()
            assert e.value.code == code and msg in str(e.value), str(e.value)
        kvq.kvq_append_ragged(h, 0, p, p, [0, 0], 5)  # no-op: no device work
        assert kvq.kvq_sequence_lengths(h, 0, 2) == ([0, 0], [0, 0])
        assert kvq.kvq_bytes_layer(h, 0).n_tokens == 0
        with pytest.raises(kvq.KvqError) as e:
            kvq.kvq_export_sequence(h, 0, 2)
        assert e.value.code == kvq.KVQ_EINVAL
    finally:
        kvq.kvq_destroy(h)


def test_workspace_bytes_valid_and_invalid():
    n = kvq.kvq_workspace_bytes(_cfg())
    assert n > 0 and n % kvq.KVQ_WORKSPACE_ALIGN == 0
    assert kvq.kvq_workspace_bytes(_cfg(max_context=512)) > n
    bad = [
        (dict(n_q_heads=7), "multiple"),
        (dict(head_dim=96), "head_dim"),
        (dict(layers=[(5, 2, 0), (4, 2, 0)]), "not supported"),
        (dict(layers=[(16, 4, 0), (4, 2, 0)]), "not supported"),
        (dict(layers=[(4, 3, 0), (4, 2, 0)]), "not supported"),
        (dict(residual_len=16), "residual_len"),
        (dict(layers=[(4, 2, 8), (4, 2, 0)]), "residual_len"),
        (dict(kv_dtype="f32"), "kv_dtype"),
        (dict(batch=0), ">= 1"),
        (dict(n_q_heads=64, n_kv_heads=2), "query heads"),
    ]
    for kw, msg in bad:
        assert kvq.kvq_workspace_bytes(_cfg(**kw)) == 0, kw
        assert msg in kvq.kvq_last_error(), (kw, kvq.kvq_last_error())


def test_create_rejects_bad_workspace():
    cfg = _cfg()
    n = kvq.kvq_workspace_bytes(cfg)
    for ptr, size, code in [(None, n, kvq.KVQ_ENOMEM), (ctypes.c_void_p(4096 + 8), n, kvq.KVQ_ENOMEM),
                            (ctypes.c_void_p(4096), n - 1, kvq.KVQ_ENOMEM)]:
        with pytest.raises(kvq.KvqError) as e:
            kvq.kvq_create(cfg, ptr, size)
        assert e.value.code == code
    with pytest.raises(kvq.KvqError) as e:
        kvq.kvq_create(_cfg(head_dim=80), ctypes.c_void_p(4096), n)
    assert e.value.code == kvq.KVQ_EUNSUPPORTED


def test_handle_validation_leaves_state_unchanged():
    # create does no device work, so a host address stands in for the workspace
    cfg = _cfg()
    n = kvq.kvq_workspace_bytes(cfg)
    h = kvq.kvq_create(cfg, ctypes.c_void_p(1 << 20), n)
    try:
        assert kvq.kvq_bytes(h) == 0
        p = ctypes.c_void_p(1 << 21)
        cases = [
            (lambda: kvq.kvq_append(h, 2, p, p, 1), kvq.KVQ_EINVAL, "out of range"),
            (lambda: kvq.kvq_append(h, -1, p, p, 1), kvq.KVQ_EINVAL, "out of range"),
            (lambda: kvq.kvq_append(h, 0, p, p, -3), kvq.KVQ_EINVAL, "< 0"),
            (lambda: kvq.kvq_append(h, 0, None, p, 1), kvq.KVQ_EINVAL, "NULL"),
            (lambda: kvq.kvq_append(h, 0, ctypes.c_void_p((1 << 21) + 2), p, 1), kvq.KVQ_EINVAL,
             "aligned"),
            (lambda: kvq.kvq_append(h, 0, p, p, 257), kvq.KVQ_ECAPACITY, "max_context"),
            (lambda: kvq.kvq_decode_attention(h, 0, p, p), kvq.KVQ_EINVAL, "no tokens"),
            (lambda: kvq.kvq_decode_attention(h, 1, None, p), kvq.KVQ_EINVAL, "NULL"),
            (lambda: kvq.kvq_decode_attention(h, 5, p, p), kvq.KVQ_EINVAL, "out of range"),
            (lambda: kvq.kvq_decode_attention_noalloc(h, 0, p, p), kvq.KVQ_EINVAL, "no tokens"),
            (lambda: kvq.kvq_decode_attention_noalloc(h, 1, None, p), kvq.KVQ_EINVAL, "NULL"),
            (lambda: kvq.kvq_decode_attention_noalloc(h, 5, p, p), kvq.KVQ_EINVAL, "out of range"),
            (lambda: kvq.kvq_bytes_layer(h, 9), kvq.KVQ_EINVAL, "out of range"),
            (lambda: kvq.kvq_prefill_attention(h, 0, p, 1, p), kvq.KVQ_EINVAL, "n_q = 1 outside"),
            (lambda: kvq.kvq_prefill_attention(h, 0, p, 0, p), kvq.KVQ_EINVAL, "n_q = 0 outside"),
            (lambda: kvq.kvq_prefill_attention(h, 2, p, 1, p), kvq.KVQ_EINVAL, "out of range"),
            (lambda: kvq.kvq_prefill_attention(h, 0, p, 1, None), kvq.KVQ_EINVAL, "NULL"),
            (lambda: kvq.kvq_prefill_attention(h, 0, ctypes.c_void_p((1 << 21) + 4), 1, p), kvq.KVQ_EINVAL,
             "aligned"),
        ]
        for fn, code, msg in cases:
            with pytest.raises(kvq.KvqError) as e:
                fn()
            assert e.value.code == code and msg in str(e.value), str(e.value)
            for l in range(2):
                info = kvq.kvq_bytes_layer(h, l)
                assert (info.n_tokens, info.n_quantized, info.total) == (0, 0, 0)
        # an empty append is a no-op
        kvq.kvq_append(h, 0, p, p, 0)
        info = kvq.kvq_bytes_layer(h, 1)
        assert (info.k_bits, info.v_bits, info.residual_len, info.k_words, info.v_words) == (
            8, 4, 64, 32, 16)
        info = kvq.kvq_bytes_layer(h, 0)
        assert (info.residual_len, info.k_words, info.v_words) == (32, 16, 8)
        assert kvq.kvq_last_launch(h) == (0, -1)
    finally:
        kvq.kvq_destroy(h)
    kvq.kvq_destroy(None)
    assert kvq.lib().kvq_bytes(None) == -1


def test_key_mode_validation():
    """k_mode must be 0 (per channel) or 1 (per token); per-token Key needs 2, 4
    or 8 bits; a per-token table is otherwise accepted."""
    assert kvq.kvq_workspace_bytes(_cfg(layers=[(4, 2, 0, 2), (4, 2, 0)])) == 0
    assert "k_mode" in kvq.kvq_last_error()
    assert kvq.kvq_workspace_bytes(_cfg(layers=[(3, 4, 0, 1), (4, 2, 0)])) == 0
    assert "per-token" in kvq.kvq_last_error()
    assert kvq.kvq_workspace_bytes(_cfg(layers=[(4, 2, 0, 1), (8, 8, 0, 1)])) > 0
    assert kvq.kvq_workspace_bytes(_cfg(layers=[(16, 16, 0, 1), (2, 2, 0, 1)])) > 0


def test_paging_config_validation():
    """Paging parameters are checked at create: page length a power of two >=
    128 and a multiple of the group size, a pool of at least one page, a
    table, and rows long enough for max_context; the pooled workspace is
    sized by the pool, not by batch x max_context."""
    T = ctypes.c_void_p(1 << 22)  # create does no device work: any address stands in for the table
    base = dict(n_layers=1, batch=4, n_q_heads=8, n_kv_heads=2, head_dim=128, max_context=4096,
                kv_dtype="bf16", q_dtype="bf16", group_size=32, residual_len=32, layers=[(4, 2, 0)])
    bad = [dict(page_tokens=96, n_pages=8, block_table=T, table_stride=64),
           dict(page_tokens=64, n_pages=8, block_table=T, table_stride=64),
           dict(page_tokens=256, n_pages=0, block_table=T, table_stride=16),
           dict(page_tokens=256, n_pages=8, block_table=None, table_stride=16),
           dict(page_tokens=256, n_pages=8, block_table=T, table_stride=15)]
    for kw in bad:
        cfg = kvq.make_config(**base, **kw)
        assert kvq.kvq_workspace_bytes(cfg) == 0, kw
    g48 = dict(base, group_size=48, residual_len=48)
    assert kvq.kvq_workspace_bytes(kvq.make_config(**g48, page_tokens=256, n_pages=8, block_table=T,
                                                    table_stride=16)) == 0  # 48 does not divide 256
    flat = kvq.kvq_workspace_bytes(kvq.make_config(**base))
    paged = kvq.kvq_workspace_bytes(kvq.make_config(**base, page_tokens=256, n_pages=8, block_table=T,
                                                    table_stride=16))
    assert 0 < paged < flat
    cfg = kvq.make_config(**base, page_tokens=256, n_pages=8, block_table=T, table_stride=16)
    h = kvq.kvq_create(cfg, ctypes.c_void_p(1 << 20), kvq.kvq_workspace_bytes(cfg))
    try:
        with pytest.raises(kvq.KvqError) as e:
            kvq.kvq_reset_sequence(h, 4)
        assert e.value.code == kvq.KVQ_EINVAL
        kvq.kvq_reset_sequence(h, 3)  # host bookkeeping only
        assert kvq.kvq_sequence_lengths(h, 0, 4) == ([0] * 4, [0] * 4)
    finally:
        kvq.kvq_destroy(h)
