"""Thin Python binding of libkvq's C ABI (include/kvq.h), same names.

Argument marshalling only: every step of quantize-append and decode attention
runs in the HIP kernels of libkvq.so.  PyTorch supplies device memory (the
workspace, inputs and outputs) and the HIP stream.  If the library has not been
built this module raises on first use; there is no fallback.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# KVQ_LIB: another build of this same library (the CPU sanitizer tests use one)
LIB_PATH = os.environ.get("KVQ_LIB") or os.path.join(_HERE, "libkvq.so")

KVQ_OK, KVQ_EINVAL, KVQ_ENOMEM, KVQ_ECAPACITY, KVQ_EUNSUPPORTED, KVQ_EDEVICE = 0, -1, -2, -3, -4, -5
KVQ_F32, KVQ_F16, KVQ_BF16 = 0, 1, 2
KVQ_WORKSPACE_ALIGN = 256
_DT = {"f32": KVQ_F32, "f16": KVQ_F16, "bf16": KVQ_BF16}

EXPORTED = ["kvq_workspace_bytes", "kvq_create", "kvq_append", "kvq_decode_attention",
            "kvq_append_decode_attention", "kvq_bytes", "kvq_bytes_layer", "kvq_export_layer", "kvq_sync",
            "kvq_set_stream", "kvq_last_error", "kvq_destroy", "kvq_last_launch", "kvq_prefill_attention",
            "kvq_append_ragged", "kvq_sequence_lengths", "kvq_export_sequence",
            "kvq_decode_attention_noalloc", "kvq_reset_sequence"]


KVQ_K_PER_CHANNEL, KVQ_K_PER_TOKEN = 0, 1


class kvq_layer_cfg(ctypes.Structure):
    _fields_ = [("k_bits", ctypes.c_int32), ("v_bits", ctypes.c_int32),
                ("residual_len", ctypes.c_int32), ("k_mode", ctypes.c_int32),
                ("rpc_permille", ctypes.c_int32)]


class kvq_config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("n_layers", "batch", "n_q_heads", "n_kv_heads", "head_dim", "max_context",
                 "kv_dtype", "q_dtype", "group_size", "residual_len")] + [
        ("layers", ctypes.POINTER(kvq_layer_cfg)), ("stream", ctypes.c_void_p),
        ("page_tokens", ctypes.c_int32), ("n_pages", ctypes.c_int32),
        ("block_table", ctypes.c_void_p), ("table_stride", ctypes.c_int32)]


class kvq_bytes_info(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in
                ("k_codes", "k_meta", "v_codes", "v_meta", "residual", "total")] + [
        (n, ctypes.c_int32) for n in ("n_tokens", "n_quantized", "n_residual", "k_words",
                                      "v_words", "k_bits", "v_bits", "residual_len", "k_mode",
                                      "rpc_permille")]


class KvqError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__("kvq error %d: %s" % (code, msg))
        self.code = code


_lib = None


def lib():
    """Load libkvq.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libkvq.so is not built; run `python -m decode_attention_streaming_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    P, I = ctypes.c_void_p, ctypes.c_int
    sig = {
        "kvq_workspace_bytes": (ctypes.c_size_t, [P]),
        "kvq_create": (I, [P, P, ctypes.c_size_t, P]),
        "kvq_append": (I, [P, I, P, P, I]),
        "kvq_decode_attention": (I, [P, I, P, P]),
        "kvq_append_decode_attention": (I, [P, I, P, P, P, P]),
        "kvq_bytes": (ctypes.c_int64, [P]),
        "kvq_bytes_layer": (I, [P, I, P]),
        "kvq_export_layer": (I, [P, I] + [P] * 8),
        "kvq_sync": (I, [P]),
        "kvq_set_stream": (I, [P, P]),
        "kvq_last_error": (ctypes.c_char_p, [P]),
        "kvq_destroy": (None, [P]),
        "kvq_last_launch": (I, [P, P, P]),
        "kvq_prefill_attention": (I, [P, I, P, I, P]),
        "kvq_append_ragged": (I, [P, I, P, P, P, I]),
        "kvq_sequence_lengths": (I, [P, I, P, P]),
        "kvq_export_sequence": (I, [P, I, I] + [P] * 8),
        "kvq_decode_attention_noalloc": (I, [P, I, P, P]),
        "kvq_reset_sequence": (I, [P, I]),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    _lib = L
    return L


def make_config(n_layers, batch, n_q_heads, n_kv_heads, head_dim, max_context, kv_dtype, q_dtype,
                group_size, residual_len, layers, stream=None, page_tokens=0, n_pages=0, block_table=None,
                table_stride=0):
    """Build a kvq_config; `layers` is a list of (k_bits, v_bits, residual_len[, k_mode[,
    rpc_permille]]); paging: page_tokens, n_pages, block_table (a device address) and
    table_stride."""
    arr = (kvq_layer_cfg * len(layers))(*[kvq_layer_cfg(*l) for l in layers])
    cfg = kvq_config(n_layers, batch, n_q_heads, n_kv_heads, head_dim, max_context,
                     _DT.get(kv_dtype, kv_dtype), _DT.get(q_dtype, q_dtype), group_size,
                     residual_len, ctypes.cast(arr, ctypes.POINTER(kvq_layer_cfg)), stream,
                     page_tokens, n_pages, block_table, table_stride)
    cfg._keep = arr  # keep the table alive as long as the config
    return cfg


def kvq_last_error(h=None):
    return lib().kvq_last_error(h).decode()


def _check(rc, h=None):
    if rc != KVQ_OK:
        raise KvqError(rc, kvq_last_error(h))
    return rc


def kvq_workspace_bytes(cfg):
    return lib().kvq_workspace_bytes(ctypes.byref(cfg))


def kvq_create(cfg, workspace_ptr, ws_bytes):
    h = ctypes.c_void_p()
    _check(lib().kvq_create(ctypes.byref(cfg), workspace_ptr, ws_bytes, ctypes.byref(h)))
    return h


def kvq_append(h, layer, k_ptr, v_ptr, n_new):
    return _check(lib().kvq_append(h, layer, k_ptr, v_ptr, n_new), h)


def kvq_decode_attention(h, layer, q_ptr, out_ptr):
    return _check(lib().kvq_decode_attention(h, layer, q_ptr, out_ptr), h)


def kvq_decode_attention_noalloc(h, layer, q_ptr, out_ptr):
    return _check(lib().kvq_decode_attention_noalloc(h, layer, q_ptr, out_ptr), h)


def kvq_append_decode_attention(h, layer, k_ptr, v_ptr, q_ptr, out_ptr):
    return _check(lib().kvq_append_decode_attention(h, layer, k_ptr, v_ptr, q_ptr, out_ptr), h)


def kvq_prefill_attention(h, layer, q_ptr, n_q, out_ptr):
    return _check(lib().kvq_prefill_attention(h, layer, q_ptr, n_q, out_ptr), h)


def kvq_bytes(h):
    return lib().kvq_bytes(h)


def kvq_bytes_layer(h, layer):
    info = kvq_bytes_info()
    _check(lib().kvq_bytes_layer(h, layer, ctypes.byref(info)), h)
    return info


def kvq_append_ragged(h, layer, k_ptr, v_ptr, n_new, n_max):
    """n_new: sequence of batch token counts (copied to a host int32 array)."""
    arr = (ctypes.c_int32 * len(n_new))(*[int(x) for x in n_new])
    return _check(lib().kvq_append_ragged(h, layer, k_ptr, v_ptr, arr, n_max), h)


def kvq_reset_sequence(h, b):
    return _check(lib().kvq_reset_sequence(h, b), h)


def kvq_sequence_lengths(h, layer, batch):
    n = (ctypes.c_int32 * batch)()
    tq = (ctypes.c_int32 * batch)()
    _check(lib().kvq_sequence_lengths(h, layer, n, tq), h)
    return list(n), list(tq)


def kvq_export_sequence(h, layer, b, k_words=None, k_scale=None, k_zero=None, v_words=None,
                        v_scale=None, v_zero=None, res_k=None, res_v=None):
    return _check(lib().kvq_export_sequence(h, layer, b, k_words, k_scale, k_zero, v_words, v_scale,
                                            v_zero, res_k, res_v), h)


def kvq_export_layer(h, layer, k_words=None, k_scale=None, k_zero=None, v_words=None,
                     v_scale=None, v_zero=None, res_k=None, res_v=None):
    return _check(lib().kvq_export_layer(h, layer, k_words, k_scale, k_zero, v_words, v_scale,
                                         v_zero, res_k, res_v), h)


def kvq_sync(h):
    return _check(lib().kvq_sync(h), h)


def kvq_set_stream(h, stream):
    return _check(lib().kvq_set_stream(h, stream), h)


def kvq_destroy(h):
    lib().kvq_destroy(h)


def kvq_last_launch(h):
    s, v = ctypes.c_int(), ctypes.c_int()
    _check(lib().kvq_last_launch(h, ctypes.byref(s), ctypes.byref(v)), h)
    return s.value, v.value


class Cache:
    """A kvq handle whose workspace, inputs and outputs are torch tensors."""

    def __init__(self, n_layers, batch, n_q_heads, n_kv_heads, head_dim, max_context, kv_dtype,
                 q_dtype, group_size, residual_len, layers, device="cuda", stream=None,
                 page_tokens=0, n_pages=0, block_table=None):
        """Paging: page_tokens > 0, n_pages pages per quantized layer, and block_table a
        contiguous int32 device tensor [batch, table_stride] of page ids (kept alive here; the
        caller may rewrite its entries between calls, in stream order)."""
        import torch
        self.torch = torch
        self.layers = list(layers)
        self.shape = dict(n_layers=n_layers, batch=batch, n_q_heads=n_q_heads,
                          n_kv_heads=n_kv_heads, head_dim=head_dim, max_context=max_context,
                          group_size=group_size)
        self.kv_dtype, self.q_dtype = kv_dtype, q_dtype
        st = stream if stream is not None else torch.cuda.current_stream(device)
        self.stream = st
        self.block_table = block_table
        table_ptr, stride = None, 0
        if page_tokens:
            if block_table is None or block_table.dtype != torch.int32 or not block_table.is_contiguous() \
                    or block_table.dim() != 2 or block_table.shape[0] != batch:
                raise ValueError("block_table must be a contiguous int32 [batch, table_stride] tensor")
            table_ptr, stride = ctypes.c_void_p(block_table.data_ptr()), block_table.shape[1]
        self.cfg = make_config(n_layers, batch, n_q_heads, n_kv_heads, head_dim, max_context,
                               kv_dtype, q_dtype, group_size, residual_len, self.layers,
                               ctypes.c_void_p(st.cuda_stream), page_tokens, n_pages, table_ptr, stride)
        nbytes = kvq_workspace_bytes(self.cfg)
        if nbytes == 0:
            raise KvqError(KVQ_EINVAL, kvq_last_error())
        self.workspace = torch.empty(nbytes + KVQ_WORKSPACE_ALIGN, dtype=torch.uint8, device=device)
        base = self.workspace.data_ptr()
        aligned = (base + KVQ_WORKSPACE_ALIGN - 1) // KVQ_WORKSPACE_ALIGN * KVQ_WORKSPACE_ALIGN
        self.ws_bytes = nbytes
        self.h = kvq_create(self.cfg, ctypes.c_void_p(aligned), nbytes)
        self.device = device

    def set_stream(self, stream):
        """Enqueue later calls on `stream` (a torch stream), e.g. a capturing one."""
        kvq_set_stream(self.h, ctypes.c_void_p(stream.cuda_stream))
        self.stream = stream

    def close(self):
        if self.h is not None:
            kvq_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def _kv_check(self, t):
        s = self.shape
        torch = self.torch
        want = torch.float16 if self.kv_dtype == "f16" else torch.bfloat16
        if t.dtype != want or not t.is_contiguous() or t.dim() != 4:
            raise ValueError("K/V must be contiguous [B, Hkv, n, d] %s" % want)
        if tuple(t.shape[:2]) != (s["batch"], s["n_kv_heads"]) or t.shape[3] != s["head_dim"]:
            raise ValueError("K/V shape %s does not match the cache" % (tuple(t.shape),))

    def append(self, layer, k_new, v_new):
        self._kv_check(k_new)
        self._kv_check(v_new)
        if k_new.shape != v_new.shape:
            raise ValueError("K and V shapes differ")
        kvq_append(self.h, layer, ctypes.c_void_p(k_new.data_ptr()),
                   ctypes.c_void_p(v_new.data_ptr()), k_new.shape[2])

    def append_ragged(self, layer, k_new, v_new, n_new):
        """Sequence b appends rows [b, :, 0:n_new[b]] of k_new / v_new [B, Hkv, n_max, d]."""
        self._kv_check(k_new)
        self._kv_check(v_new)
        if k_new.shape != v_new.shape:
            raise ValueError("K and V shapes differ")
        kvq_append_ragged(self.h, layer, ctypes.c_void_p(k_new.data_ptr()),
                          ctypes.c_void_p(v_new.data_ptr()), n_new, k_new.shape[2])

    def reset_sequence(self, b):
        """Empty sequence b in every layer (its pages may then be named for others)."""
        kvq_reset_sequence(self.h, b)

    def sequence_lengths(self, layer):
        """([N_b], [Tq_b]) per sequence."""
        return kvq_sequence_lengths(self.h, layer, self.shape["batch"])

    def _q_check(self, q, out):
        s = self.shape
        torch = self.torch
        want = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[self.q_dtype]
        if q.dtype != want or not q.is_contiguous() or tuple(q.shape) != (
                s["batch"], s["n_q_heads"], s["head_dim"]):
            raise ValueError("q must be contiguous [B, Hq, d] %s" % want)
        if out is None:
            out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
        return out

    def decode_attention(self, layer, q, out=None):
        out = self._q_check(q, out)
        kvq_decode_attention(self.h, layer, ctypes.c_void_p(q.data_ptr()),
                             ctypes.c_void_p(out.data_ptr()))
        return out

    def decode_attention_noalloc(self, layer, q, out=None):
        """decode_attention() with its hand-off in the library's static scratch
        (no device memory of the handle's workspace is used for it)."""
        out = self._q_check(q, out)
        kvq_decode_attention_noalloc(self.h, layer, ctypes.c_void_p(q.data_ptr()),
                                     ctypes.c_void_p(out.data_ptr()))
        return out

    def append_decode_attention(self, layer, k_new, v_new, q, out=None):
        """One token per sequence appended, then decode attention (one call)."""
        self._kv_check(k_new)
        self._kv_check(v_new)
        if k_new.shape[2] != 1 or v_new.shape[2] != 1:
            raise ValueError("one token per sequence")
        out = self._q_check(q, out)
        kvq_append_decode_attention(self.h, layer, ctypes.c_void_p(k_new.data_ptr()),
                                    ctypes.c_void_p(v_new.data_ptr()), ctypes.c_void_p(q.data_ptr()),
                                    ctypes.c_void_p(out.data_ptr()))
        return out

    def prefill_attention(self, layer, q, out=None):
        """Causal attention of the last n_q appended tokens' queries:
        q [B, Hq, n_q, d] (contiguous, q_dtype); out [B, Hq, n_q, d] fp32."""
        s = self.shape
        torch = self.torch
        want = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[self.q_dtype]
        if q.dtype != want or not q.is_contiguous() or q.dim() != 4 or (
                q.shape[0], q.shape[1], q.shape[3]) != (s["batch"], s["n_q_heads"], s["head_dim"]):
            raise ValueError("q must be contiguous [B, Hq, n_q, d] %s" % want)
        if out is None:
            out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
        kvq_prefill_attention(self.h, layer, ctypes.c_void_p(q.data_ptr()), q.shape[2],
                              ctypes.c_void_p(out.data_ptr()))
        return out

    def bytes(self):
        return kvq_bytes(self.h)

    def bytes_layer(self, layer):
        return kvq_bytes_layer(self.h, layer)

    def export(self, layer, seq=None):
        """Canonical host copy of one layer (numpy arrays); with seq = b, of
        sequence b alone (any layer, ragged or not)."""
        info = self.bytes_layer(layer)
        s = self.shape
        B, H, d, G = s["batch"], s["n_kv_heads"], s["head_dim"], s["group_size"]
        if seq is None:
            if info.n_tokens < 0:  # sequences of different lengths: the library refuses
                kvq_export_layer(self.h, layer)
            Tq, Tr, N = info.n_quantized, info.n_residual, info.n_tokens
        else:
            ns, tqs = self.sequence_lengths(layer)
            B, N, Tq = 1, ns[seq], tqs[seq]
            Tr = N - Tq
        wk, wv = max(info.k_words, 1), max(info.v_words, 1)
        out = dict(
            N=N, Tq=Tq,
            k_words=np.zeros((B * H, Tq, wk), np.uint32),
            k_scale=np.zeros((B * H, Tq) if info.k_mode else (B * H, Tq // G, d), np.float32),
            k_zero=np.zeros((B * H, Tq) if info.k_mode else (B * H, Tq // G, d), np.float32),
            v_words=np.zeros((B * H, Tq, wv), np.uint32),
            v_scale=np.zeros((B * H, Tq), np.float32),
            v_zero=np.zeros((B * H, Tq), np.float32),
            res_k=np.zeros((B * H, Tr, d), np.uint16),
            res_v=np.zeros((B * H, Tr, d), np.uint16),
        )
        p = {k: v.ctypes.data_as(ctypes.c_void_p) for k, v in out.items() if isinstance(v, np.ndarray)}
        args = (p["k_words"], p["k_scale"], p["k_zero"], p["v_words"], p["v_scale"], p["v_zero"],
                p["res_k"], p["res_v"])
        if seq is None:
            kvq_export_layer(self.h, layer, *args)
        else:
            kvq_export_sequence(self.h, layer, seq, *args)
        if info.k_words == 0:
            out["k_words"] = out["k_words"][:, :, :0]
            out["v_words"] = out["v_words"][:, :, :0]
        return out

    def sync(self):
        kvq_sync(self.h)
