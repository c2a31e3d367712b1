"""ctypes wrapper around the plain C oracle (``kvq_oracle.c``).

TEST INFRASTRUCTURE ONLY: imported by the tests, by the smoke check and by the
CPU-baseline leg of the benchmark.  The product path never imports it.

What it computes, with the pages it follows, is documented in ``kvq_oracle.c``:
asymmetric uniform quantization (KVTuner summary, A3 "KV cache quantization
basics"; KVmix notes, key design 2), K per channel over a token group and V per
token with a 16-bit recent-token buffer (KIVI notes, sections 6.1-6.2), int32
packing including the 11-per-word 3-bit layout (KVmix notes, key design 2),
fp64 decode attention (KVTuner summary, A3 attention equation), and fp64 causal
attention of a prefill chunk over the dequantized cache (the same equation;
KVTuner summary, A2 calibration on dequantized KV).
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kvq_oracle.c")
_SO = os.path.join(_HERE, "libkvq_oracle.so")
# A test may point the wrapper at a separately built variant of the oracle.
_SO_OVERRIDE = os.environ.get("KVQ_ORACLE_SO")
_CFLAGS = ["-std=c99", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fPIC", "-shared"]

_lib = None


def build():
    """Compile the oracle with gcc (always recompiles)."""
    tmp = _SO + ".tmp%d" % os.getpid()
    subprocess.check_call(["gcc"] + _CFLAGS + [_SRC, "-o", tmp, "-lm"])
    os.replace(tmp, _SO)


def lib():
    global _lib
    if _lib is not None:
        return _lib
    if _SO_OVERRIDE:
        return _bind(ctypes.CDLL(_SO_OVERRIDE))
    if not os.path.exists(_SO) or os.path.getmtime(_SO) < max(
            os.path.getmtime(_SRC), os.path.getmtime(os.path.join(_HERE, "kvq_oracle.h"))):
        build()
    return _bind(ctypes.CDLL(_SO))


def _bind(L):
    global _lib
    P = ctypes.c_void_p
    L.kvqo_f16_to_f32.restype = ctypes.c_float
    L.kvqo_f16_to_f32.argtypes = [ctypes.c_uint16]
    L.kvqo_bf16_to_f32.restype = ctypes.c_float
    L.kvqo_bf16_to_f32.argtypes = [ctypes.c_uint16]
    L.kvqo_words_per_row.restype = ctypes.c_int
    L.kvqo_words_per_row.argtypes = [ctypes.c_int, ctypes.c_int]
    L.kvqo_qmax.restype = ctypes.c_int
    L.kvqo_qmax.argtypes = [ctypes.c_int, ctypes.c_int]
    L.kvqo_pack_row.restype = None
    L.kvqo_pack_row.argtypes = [P, ctypes.c_int, ctypes.c_int, P]
    L.kvqo_unpack_row.restype = None
    L.kvqo_unpack_row.argtypes = [P, ctypes.c_int, ctypes.c_int, P]
    L.kvqo_quantize.restype = None
    L.kvqo_quantize.argtypes = [P, ctypes.c_int, ctypes.c_long, ctypes.c_int, P,
                                ctypes.c_long, P, P]
    L.kvqo_append.restype = ctypes.c_int
    L.kvqo_append.argtypes = [P, P, P, ctypes.c_int]
    L.kvqo_attention.restype = None
    L.kvqo_attention.argtypes = [P, P, P]
    L.kvqo_prefill_attention.restype = None
    L.kvqo_prefill_attention.argtypes = [P, P, ctypes.c_int, P]
    L.kvqo_stream_bytes.restype = ctypes.c_longlong
    L.kvqo_stream_bytes.argtypes = [ctypes.c_int] * 4 + [ctypes.c_longlong] * 2 + [ctypes.c_int]
    _lib = L
    return L


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


# ---------------------------------------------------------------------------
# Single-row / single-group helpers
# ---------------------------------------------------------------------------

def words_per_row(d, bits):
    return lib().kvqo_words_per_row(d, bits)


def qmax(bits, c):
    return lib().kvqo_qmax(bits, c)


def f16_to_f32(bits16):
    return lib().kvqo_f16_to_f32(int(bits16))


def bf16_to_f32(bits16):
    return lib().kvqo_bf16_to_f32(int(bits16))


def pack_row(codes, bits):
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    d = codes.shape[0]
    out = np.zeros(words_per_row(d, bits), dtype=np.uint32)
    lib().kvqo_pack_row(_ptr(codes), d, bits, _ptr(out))
    return out


def unpack_row(words, d, bits):
    words = np.ascontiguousarray(words, dtype=np.uint32)
    out = np.zeros(d, dtype=np.uint8)
    lib().kvqo_unpack_row(_ptr(words), d, bits, _ptr(out))
    return out


def quantize(x, qmax_):
    """Quantize one group of fp32 values; returns (codes uint8, s, z)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    codes = np.zeros(x.shape[0], dtype=np.uint8)
    s = np.zeros(1, dtype=np.float32)
    z = np.zeros(1, dtype=np.float32)
    lib().kvqo_quantize(_ptr(x), x.shape[0], 1, int(qmax_), _ptr(codes), 1, _ptr(s), _ptr(z))
    return codes, s[0], z[0]


def stream_bytes(d, k_bits, v_bits, G, N, Tq, k_tok=False):
    return lib().kvqo_stream_bytes(d, k_bits, v_bits, G, N, Tq, int(bool(k_tok)))


# ---------------------------------------------------------------------------
# Streaming layer
# ---------------------------------------------------------------------------

class _LayerStruct(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int) for n in
                ("n_streams", "g", "d", "k_bits", "v_bits", "G", "R", "cap", "is_bf16",
                 "N", "Tq", "k_tok", "rpc_permille")] + [(n, ctypes.c_void_p) for n in
                                ("hist_k", "hist_v", "k_words", "k_scale", "k_zero",
                                 "v_words", "v_scale", "v_zero")]


class Layer:
    """One layer of the oracle cache for ``n_streams`` (batch, kv-head) streams.

    k_bits/v_bits in {2,3(K only),4,8}, or 16/16 for a layer kept in 16 bits.
    Inputs are 16-bit bit patterns (numpy uint16), fp16 or bf16 per ``is_bf16``.
    ``k_tok``: Key quantized per token (KVTuner's per-token-asym mode) instead
    of per channel over G tokens (KIVI).  ``rpc_permille``: KVmix's dynamic
    recent-token ratio r (parts per thousand); 0 keeps KIVI's G-at-a-time rule.
    """

    def __init__(self, n_streams, g, d, k_bits, v_bits, G, R, cap, is_bf16, k_tok=False, rpc_permille=0):
        cap = -(-cap // G) * G
        if k_bits == 16 or v_bits == 16:
            assert k_bits == v_bits == 16
            R = cap
        self.n_streams, self.g, self.d = n_streams, g, d
        self.k_bits, self.v_bits, self.G, self.R, self.cap = k_bits, v_bits, G, R, cap
        self.is_bf16 = bool(is_bf16)
        self.k_tok = bool(k_tok) and k_bits != 16
        assert not (self.k_tok and k_bits == 3), "per-token Key: 2, 4 or 8 bits"
        for b in (k_bits, v_bits):
            assert b == 3 or (d * b) % 32 == 0, "a row must fill whole 32-bit words"
        wk, wv = words_per_row(d, k_bits), words_per_row(d, v_bits)
        S = n_streams
        self.hist_k = np.zeros((S, cap, d), np.uint16)
        self.hist_v = np.zeros((S, cap, d), np.uint16)
        self.k_words = np.zeros((S, cap, wk), np.uint32)
        kshape = (S, cap) if self.k_tok else (S, cap // G, d)
        self.k_scale = np.zeros(kshape, np.float32)
        self.k_zero = np.zeros(kshape, np.float32)
        self.v_words = np.zeros((S, cap, wv), np.uint32)
        self.v_scale = np.zeros((S, cap), np.float32)
        self.v_zero = np.zeros((S, cap), np.float32)
        st = _LayerStruct()
        for f in ("n_streams", "g", "d", "k_bits", "v_bits", "G", "R", "cap"):
            setattr(st, f, getattr(self, f))
        st.is_bf16 = int(self.is_bf16)
        st.k_tok = int(self.k_tok)
        self.rpc_permille = int(rpc_permille) if k_bits != 16 else 0
        assert 0 <= self.rpc_permille < 1000
        st.rpc_permille = self.rpc_permille
        st.N = 0
        st.Tq = 0
        for f in ("hist_k", "hist_v", "k_words", "k_scale", "k_zero", "v_words", "v_scale",
                  "v_zero"):
            setattr(st, f, getattr(self, f).ctypes.data)
        self._st = st

    @property
    def N(self):
        return self._st.N

    @property
    def Tq(self):
        return self._st.Tq

    def append(self, k_new, v_new):
        """k_new, v_new: uint16 [n_streams, n, d] (16-bit bit patterns)."""
        k_new = np.ascontiguousarray(k_new, dtype=np.uint16)
        v_new = np.ascontiguousarray(v_new, dtype=np.uint16)
        assert k_new.shape == v_new.shape and k_new.shape[0] == self.n_streams
        assert k_new.shape[2] == self.d
        rc = lib().kvqo_append(ctypes.byref(self._st), _ptr(k_new), _ptr(v_new), k_new.shape[1])
        if rc != 0:
            raise ValueError("oracle: capacity exceeded")

    def attention(self, q):
        """q: float64 [n_streams, g, d]; returns float64 [n_streams, g, d]."""
        q = np.ascontiguousarray(q, dtype=np.float64)
        assert q.shape == (self.n_streams, self.g, self.d)
        out = np.zeros_like(q)
        lib().kvqo_attention(ctypes.byref(self._st), _ptr(q), _ptr(out))
        return out

    def prefill_attention(self, q):
        """Causal attention of the last n_q tokens' queries (chunked prefill):
        q float64 [n_streams, g, n_q, d]; query j attends to tokens
        0 .. N - n_q + j.  Returns float64 [n_streams, g, n_q, d]."""
        q = np.ascontiguousarray(q, dtype=np.float64)
        S, g, n_q, d = q.shape
        assert (S, g, d) == (self.n_streams, self.g, self.d) and 1 <= n_q <= self.N
        out = np.zeros_like(q)
        lib().kvqo_prefill_attention(ctypes.byref(self._st), _ptr(q), n_q, _ptr(out))
        return out

    def export(self):
        """Canonical state: codes/meta for tokens [0, Tq), 16-bit tokens [Tq, N)."""
        Tq, N, G = self.Tq, self.N, self.G
        return dict(
            N=N, Tq=Tq,
            k_words=self.k_words[:, :Tq].copy(),
            k_scale=self.k_scale[:, :(Tq if self.k_tok else Tq // G)].copy(),
            k_zero=self.k_zero[:, :(Tq if self.k_tok else Tq // G)].copy(),
            v_words=self.v_words[:, :Tq].copy(),
            v_scale=self.v_scale[:, :Tq].copy(),
            v_zero=self.v_zero[:, :Tq].copy(),
            res_k=self.hist_k[:, Tq:N].copy(),
            res_v=self.hist_v[:, Tq:N].copy(),
        )

    def bytes(self):
        return self.n_streams * stream_bytes(self.d, self.k_bits, self.v_bits, self.G, self.N,
                                             self.Tq, self.k_tok)
