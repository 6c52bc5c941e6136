"""Seeded synthetic inputs shared by the oracle-side tests, the GPU tests and bench.py.

This module draws random numbers and nothing else: it holds none of the method's
arithmetic (no rotation, no codebook, no quantization). Every array it returns is
an *input* handed identically to the CPU oracle and to the HIP path:

* key/value/query/database tensors follow the workload laws of the pages'
  settings (Llama-3.1-8B-shaped decode layers, a GloVe-like 200-d search set),
  reproduced synthetically because no datasets or weights are available.

The rotation the method draws (the +/-1 diagonal and the Gaussian JL matrix) is not
made here: the library makes it with ``tq_make_rotation`` and the oracle with its own
implementation of the same definition (``oracle.tq_oracle.make_rotation``).  ``rotation``
below only supplies independent random draws of that shape for Monte-Carlo checks of the
oracle's statistics, where thousands of fresh rotations are needed.

All generators are counter-based (numpy Philox) so a (seed, shape) pair gives
the same bytes on any machine.  bf16 tensors are returned as their raw uint16
bit patterns (round-to-nearest-even from fp32); ``bf16_to_f64`` widens them
exactly for the oracle.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "gen", "rotation", "f32_to_bf16_bits", "bf16_to_f32", "bf16_to_f64",
    "c1_inputs", "kv_layer", "kv_layer_device", "decode_queries", "search_set", "data_seed",
    "rotation_seed",
]


def gen(seed: int) -> np.random.Generator:
    """Counter-based generator (Philox 4x64) for one seed."""
    return np.random.Generator(np.random.Philox(int(seed)))


def data_seed(config: int, layer: int = 0) -> int:
    return 1000 * int(config) + int(layer)


def rotation_seed(config: int, layer: int = 0) -> int:
    return data_seed(config, layer) + 500000


def rotation(d: int, seed: int):
    """Random draws of a rotation's shape for Monte-Carlo pins: signs[d] in {+1,-1} (int8)
    and S[d,d] ~ N(0,1) (fp32, drawn in fp64 and rounded once)."""
    g = gen(seed)
    signs = np.where(g.integers(0, 2, size=d) == 0, 1, -1).astype(np.int8)
    S = g.standard_normal((d, d)).astype(np.float32)
    return signs, S


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even); return the uint16 bit patterns."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return bf16_to_f32(bits).astype(np.float64)


def c1_inputs(seed: int = 1000, n: int = 4096, d: int = 128, n_q: int = 64,
              n_outlier: int = 4, outlier_scale: float = 20.0):
    """Single-head setting: K, V [n, d] fp32 N(0,1) with the same `n_outlier` seed-chosen
    channels scaled by `outlier_scale`; queries [n_q, d] fp32 N(0,1)."""
    g = gen(seed)
    ch = np.sort(g.choice(d, size=n_outlier, replace=False))
    k = g.standard_normal((n, d))
    v = g.standard_normal((n, d))
    k[:, ch] *= outlier_scale
    v[:, ch] *= outlier_scale
    q = g.standard_normal((n_q, d))
    return (k.astype(np.float32), v.astype(np.float32), q.astype(np.float32), ch)


def kv_layer(batch: int, hkv: int, ntok: int, d: int, seed: int,
             spike_frac: float = 0.0, spike_scale: float = 10.0):
    """One decode layer's cache contents as bf16 bits, shape [batch, hkv, ntok, d].

    K and V are sigma[h, j] * N(0, 1) with one log-uniform [0.5, 8] draw of sigma per
    (kv head, channel) for K and an independent one for V.  With spike_frac > 0 a
    seed-chosen set of round(spike_frac * ntok) token positions per sequence has its
    keys (all heads) multiplied by spike_scale.
    """
    g = gen(seed)
    sig_k = np.exp(g.uniform(np.log(0.5), np.log(8.0), size=(hkv, d))).astype(np.float32)
    sig_v = np.exp(g.uniform(np.log(0.5), np.log(8.0), size=(hkv, d))).astype(np.float32)
    spikes = []
    n_sp = int(round(spike_frac * ntok))
    for _ in range(batch):
        spikes.append(np.sort(g.choice(ntok, size=n_sp, replace=False)) if n_sp else
                      np.zeros(0, dtype=np.int64))
    k_bits = np.empty((batch, hkv, ntok, d), dtype=np.uint16)
    v_bits = np.empty((batch, hkv, ntok, d), dtype=np.uint16)
    for b in range(batch):
        for h in range(hkv):
            kk = g.standard_normal((ntok, d), dtype=np.float32) * sig_k[h]
            if n_sp:
                kk[spikes[b]] *= np.float32(spike_scale)
            k_bits[b, h] = f32_to_bf16_bits(kk)
            vv = g.standard_normal((ntok, d), dtype=np.float32) * sig_v[h]
            v_bits[b, h] = f32_to_bf16_bits(vv)
    return k_bits, v_bits, spikes


def kv_layer_device(batch: int, hkv: int, ntok: int, d: int, seed: int, device,
                    spike_frac: float = 0.0, spike_scale: float = 10.0):
    """The law of ``kv_layer`` drawn on a GPU with torch's seeded generator (a different
    stream of numbers than the CPU draw): K, V bf16 tensors [batch, hkv, ntok, d] with
    per-(kv head, channel) std log-uniform in [0.5, 8], and round(spike_frac * ntok)
    seed-chosen token positions per sequence whose keys are scaled by spike_scale.  For the
    full-size layers, where a CPU draw of 10^9 values per layer would take minutes."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    lo, hi = float(np.log(0.5)), float(np.log(8.0))
    sig_k = torch.exp(torch.empty((hkv, 1, d), device=device).uniform_(lo, hi, generator=g))
    sig_v = torch.exp(torch.empty((hkv, 1, d), device=device).uniform_(lo, hi, generator=g))
    k = torch.empty((batch, hkv, ntok, d), dtype=torch.bfloat16, device=device)
    v = torch.empty_like(k)
    n_sp = int(round(spike_frac * ntok))
    for b in range(batch):
        kk = torch.randn((hkv, ntok, d), generator=g, device=device) * sig_k
        if n_sp:
            pos = torch.randperm(ntok, generator=g, device=device)[:n_sp]
            kk[:, pos] *= spike_scale
        k[b] = kk.to(torch.bfloat16)
        v[b] = (torch.randn((hkv, ntok, d), generator=g, device=device) * sig_v).to(torch.bfloat16)
    return k, v


def decode_queries(batch: int, hq: int, d: int, seed: int) -> np.ndarray:
    """Decode-step queries, bf16 bits [batch, hq, d] ~ N(0,1)."""
    g = gen(seed + 777)
    return f32_to_bf16_bits(g.standard_normal((batch, hq, d), dtype=np.float32))


def search_set(n: int, d_in: int, seed: int, power: float = 0.3) -> np.ndarray:
    """n vectors x ~ N(0, diag(sigma^2)), sigma_i = i^-power (i = 1..d_in), scaled to unit
    length; returned as fp32 [n, d_in]."""
    g = gen(seed)
    sig = np.arange(1, d_in + 1, dtype=np.float64) ** (-power)
    out = np.empty((n, d_in), dtype=np.float32)
    step = 1 << 16
    for s in range(0, n, step):
        e = min(n, s + step)
        x = g.standard_normal((e - s, d_in)) * sig
        x /= np.linalg.norm(x, axis=1, keepdims=True)
        out[s:e] = x.astype(np.float32)
    return out
