"""Seeded synthetic workloads: shapes, per-layer K/V bit tables and inputs.

This module only draws random numbers and describes workload shapes; it holds
none of the quantization or attention arithmetic, so the CPU oracle and the HIP
path can both consume what it produces.

Workload shapes follow the models the pages evaluate on: Llama-3.1-8B and
Qwen2.5-7B (KVTuner summary, A4 experimental setup), Llama-2-7B (KVmix notes,
experiments; top-20% layers at high precision, the rest at 2 bits, average
K 2.19 / V 2.38 bits, key designs 2-3), and Llama-2-70B with 8 KV heads and a
32K context (KIVI notes, section 2.2).  Key has per-channel structure with a few
outlier channels (KIVI notes, section 5.1); Value can drift over time (KIVI
notes, section 5.2 and exercise 4).  No dataset item is used: every value is a
seeded draw.

Distributions (sigma always a standard deviation):
  K[b,h,t,c] = mu[h,c] + sig[h,c] * N(0,1); mu ~ N(0,1), sig ~ LogNormal(0, 0.5),
               drawn once per (layer, kv-head, channel) and shared by the batch;
               a seeded set of outlier channels per (layer, kv-head) is scaled by
               a factor (x10 or x20).
  V          : N(0,1); or a per-(layer, b, kv-head) mean that moves by N(0,3)
               every 512 tokens; or N(0,1) then N(10,1) from a given position.
  q          : N(0,1).
Values are drawn in fp32 and rounded to nearest-even into the 16-bit format.
"""
from dataclasses import dataclass, field
from typing import List, Tuple

import numpy as np
import torch

# (k_bits, v_bits) pair names used by the pages (KVTuner summary, A2 intra-layer pruning)
PAIRS = {"K8V8": (8, 8), "K8V4": (8, 4), "K4V4": (4, 4), "K4V2": (4, 2), "K2V2": (2, 2),
         "K3V4": (3, 4), "K16V16": (16, 16)}


@dataclass
class Workload:
    cid: int
    name: str
    n_layers: int
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    context: int
    kv_dtype: str          # "f16" | "bf16"
    q_dtype: str           # "f32" | "f16" | "bf16"
    G: int
    R: int
    layers: List[Tuple[int, ...]] = field(default_factory=list)  # (kb, vb, R_l[, k_mode])
    k_outliers: Tuple[int, float] = (2, 10.0)
    v_kind: str = "normal"  # "normal" | "walk512" | "half_shift"

    @property
    def g(self):
        return self.n_q_heads // self.n_kv_heads

    def equiv_bits(self):
        kb = np.array([l[0] for l in self.layers], float)
        vb = np.array([l[1] for l in self.layers], float)
        return dict(k=float(kb.mean()), v=float(vb.mean()), kv=float(((kb + vb) / 2).mean()))


def _rng(*key):
    return np.random.default_rng(np.random.SeedSequence([abs(hash_key(k)) for k in key]))


def hash_key(k):
    if isinstance(k, int):
        return k
    return int.from_bytes(str(k).encode(), "little") % (2 ** 31)


def _table_llama31(seed=0):
    """Uniform over {K8V8,K8V4,K4V4,K4V2,K2V2} per layer, conditioned on an
    average of 3.25 equivalent bits, (kb + vb) / 2, over 32 layers."""
    names = ["K8V8", "K8V4", "K4V4", "K4V2", "K2V2"]
    eq = np.array([(PAIRS[n][0] + PAIRS[n][1]) / 2 for n in names])
    rng = _rng(seed, "table", 2)
    while True:
        draws = rng.integers(0, 5, size=(200000, 32))
        ok = np.nonzero(eq[draws].sum(axis=1) == 104.0)[0]
        if ok.size:
            return [names[i] for i in draws[ok[0]]]


def _table_qwen25(seed=0):
    """Layers 0,1,25,26,27 K8V8; one seeded middle layer K8V4; the rest K4V4."""
    rng = _rng(seed, "table", 3)
    t = ["K4V4"] * 28
    for i in (0, 1, 25, 26, 27):
        t[i] = "K8V8"
    t[int(rng.integers(2, 25))] = "K8V4"
    return t


def _table_llama2_7b(seed=0):
    """A seeded 20% of the 32 layers (6) K3V4, the rest K2V2."""
    rng = _rng(seed, "table", 4)
    hi = set(rng.choice(32, size=6, replace=False).tolist())
    return ["K3V4" if i in hi else "K2V2" for i in range(32)]


def _table_llama2_70b(seed=0):
    rng = _rng(seed, "table", 5)
    return ["K8V4" if b else "K4V2" for b in rng.integers(0, 2, size=80)]


def workload(cid, seed=0):
    """The five workloads (1: tiny single layer; 2: Llama-3.1-8B-shaped; 3:
    Qwen2.5-7B-shaped; 4: Llama-2-7B-shaped MHA; 5: Llama-2-70B-shaped 32K)."""
    if cid == 1:
        w = Workload(1, "single layer K4V2 d64 ctx288", 1, 1, 1, 1, 64, 288, "f16", "f32", 32, 32)
        names = ["K4V2"]
    elif cid == 2:
        w = Workload(2, "Llama-3.1-8B-shaped decode B8 ctx1024", 32, 8, 32, 8, 128, 1024,
                     "bf16", "bf16", 32, 32)
        names = _table_llama31(seed)
    elif cid == 3:
        w = Workload(3, "Qwen2.5-7B-shaped decode B32 ctx4096", 28, 32, 28, 4, 128, 4096,
                     "bf16", "bf16", 64, 64, k_outliers=(4, 20.0), v_kind="walk512")
        names = _table_qwen25(seed)
    elif cid == 4:
        w = Workload(4, "Llama-2-7B-shaped MHA decode B30 ctx4096", 32, 30, 32, 32, 128, 4096,
                     "f16", "f16", 32, 409)
        names = _table_llama2_7b(seed)
    elif cid == 5:
        w = Workload(5, "Llama-2-70B-shaped decode B2 ctx32768", 80, 2, 64, 8, 128, 32768,
                     "bf16", "bf16", 128, 128, v_kind="half_shift")
        names = _table_llama2_70b(seed)
    else:
        raise ValueError(cid)
    layers = []
    for n in names:
        kb, vb = PAIRS[n]
        r = w.R
        if cid == 4:  # recent-token share: 20% of 4096 for high layers, 10% for the rest
            r = int(0.2 * 4096) if n == "K3V4" else int(0.1 * 4096)
        layers.append((kb, vb, r))
    w.layers = layers
    return w


_TORCH = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}


def torch_dtype(name):
    return _TORCH[name]


def _gen(device, *key):
    seed = int(np.random.SeedSequence([hash_key(k) for k in key]).generate_state(1)[0])
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


class LayerStats:
    """Per-(layer, kv-head, channel) K statistics and per-(layer, b, kv-head) V means."""

    def __init__(self, w: Workload, layer: int, seed=0):
        rng = _rng(seed, "stats", w.cid, layer)
        H, d = w.n_kv_heads, w.head_dim
        self.mu = rng.standard_normal((H, d)).astype(np.float32)
        self.sig = rng.lognormal(0.0, 0.5, (H, d)).astype(np.float32)
        n_out, factor = w.k_outliers
        self.kscale = np.ones((H, d), np.float32)
        for h in range(H):
            self.kscale[h, rng.choice(d, size=n_out, replace=False)] = factor
        self.v_kind = w.v_kind
        if w.v_kind == "walk512":
            nblk = -(-(w.context + 4096) // 512)
            steps = rng.normal(0.0, 3.0, (w.batch, H, nblk)).astype(np.float64)
            steps[:, :, 0] = 0.0
            self.vmean = np.cumsum(steps, axis=2).astype(np.float32)
        self.half = w.context // 2


def layer_tokens(w: Workload, layer: int, t0: int, n: int, device, stats: LayerStats = None,
                 seed=0, batch=None, heads=None):
    """K and V for token positions [t0, t0+n) of one layer: [B, Hkv, n, d] 16-bit."""
    st = stats or LayerStats(w, layer, seed)
    B = w.batch if batch is None else batch
    H, d = w.n_kv_heads, w.head_dim
    dt = _TORCH[w.kv_dtype]
    gk = _gen(device, seed, "K", w.cid, layer, t0, n)
    z = torch.randn((B, H, n, d), generator=gk, device=device, dtype=torch.float32)
    mu = torch.from_numpy(st.mu).to(device)[None, :, None, :]
    sig = torch.from_numpy(st.sig).to(device)[None, :, None, :]
    ks = torch.from_numpy(st.kscale).to(device)[None, :, None, :]
    k = ((mu + sig * z) * ks).to(dt)
    del z
    gv = _gen(device, seed, "V", w.cid, layer, t0, n)
    v = torch.randn((B, H, n, d), generator=gv, device=device, dtype=torch.float32)
    pos = torch.arange(t0, t0 + n, device=device)
    if st.v_kind == "walk512":
        vm = torch.from_numpy(st.vmean[:B]).to(device)  # [B, H, nblk]
        v += vm[:, :, (pos // 512)][..., None]
    elif st.v_kind == "half_shift":
        v += (pos >= st.half).to(torch.float32)[None, None, :, None] * 10.0
    v = v.to(dt)
    return k.contiguous(), v.contiguous()


def query(w: Workload, layer: int, step: int, device, seed=0):
    g = _gen(device, seed, "q", w.cid, layer, step)
    q = torch.randn((w.batch, w.n_q_heads, w.head_dim), generator=g, device=device,
                    dtype=torch.float32)
    return q.to(_TORCH[w.q_dtype]).contiguous()


def bits16(t):
    """16-bit tensor -> numpy uint16 bit patterns on the host."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def as_f64(t):
    return t.detach().to(torch.float64).cpu().numpy()


def queries(w: Workload, layer: int, n_steps: int, device, seed=0):
    """q for n_steps decode steps of one layer: [n_steps, B, Hq, d]."""
    g = _gen(device, seed, "qs", w.cid, layer, n_steps)
    q = torch.randn((n_steps, w.batch, w.n_q_heads, w.head_dim), generator=g, device=device,
                    dtype=torch.float32)
    return q.to(_TORCH[w.q_dtype]).contiguous()
