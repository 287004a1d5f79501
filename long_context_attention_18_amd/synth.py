"""Seeded synthetic inputs shared by the GPU path's tests/benchmark and the oracle.

This module draws random numbers and converts them to the storage types the
library consumes (BF16 bits, fp32). It holds none of the method's arithmetic:
no pooling, RoPE, quantisation, scoring, selection or attention.

Streams are indexed by position so that any sub-range can be regenerated on
its own: every tensor is drawn in chunks of ``CHUNK`` positions from
``np.random.default_rng(SeedSequence([2026, workload, layer, tensor, seq, chunk]))``.

Distributions (the workload descriptions: hidden states N(0,1), projection
weights N(0, 0.02^2), BF16 storage):
  * per-token projected inputs kv, gate (128 wide) and, for CSA, ik, ig (64
    wide) are drawn directly as N(0, sigma^2) with sigma = 0.02*sqrt(hidden),
    the marginal law of h.W; this stands in for the 10^13 host MACs that a
    1M-token cache fill through real projections would cost. A workload that
    states its inputs as N(0,1) uses sigma = 1.
  * queries go through a real projection: h ~ N(0,1) [hidden], q = h.Wq,
    qI = h.WqI (rounded to BF16), w = h.Ww (fp32), W* ~ N(0, 0.02^2).
  * learned positional biases ~ N(0, 0.02^2), fp32.
"""
from __future__ import annotations

import numpy as np

CHUNK = 4096

# tensor ids inside the seed sequence
T_KV, T_GATE, T_IK, T_IG, T_HID, T_WQ, T_WQI, T_WW, T_BIAS, T_IBIAS = range(10)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bfloat16 bit patterns, round to nearest even (storage conversion)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    r = (u >> 16) & 1          # new array; u (a view of x) is not modified
    r += 0x7FFF
    r += u                     # no uint32 overflow for finite inputs
    r >>= 16
    out = r.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _rng(*key) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([2026, *[int(k) for k in key]]))


class TokenStream:
    """Per-token projected inputs of one layer and one sequence, by position."""

    def __init__(self, workload: int, layer: int, seq: int, csa: bool, sigma: float):
        self.workload, self.layer, self.seq, self.csa, self.sigma = workload, layer, seq, csa, float(sigma)

    def _chunk(self, tensor: int, ci: int, width: int) -> np.ndarray:
        g = _rng(self.workload, self.layer, tensor, self.seq, ci)
        x = g.standard_normal((CHUNK, width), dtype=np.float32)
        x *= np.float32(self.sigma)
        return bf16_bits(x)

    def _range(self, tensor: int, pos0: int, n: int, width: int) -> np.ndarray:
        out = np.empty((n, width), np.uint16)
        p = pos0
        while p < pos0 + n:
            ci = p // CHUNK
            lo = p - ci * CHUNK
            hi = min(CHUNK, pos0 + n - ci * CHUNK)
            out[p - pos0: p - pos0 + (hi - lo)] = self._chunk(tensor, ci, width)[lo:hi]
            p += hi - lo
        return out

    def tokens(self, pos0: int, n: int) -> dict:
        d = {"kv": self._range(T_KV, pos0, n, 128), "gate": self._range(T_GATE, pos0, n, 128)}
        if self.csa:
            d["ik"] = self._range(T_IK, pos0, n, 64)
            d["ig"] = self._range(T_IG, pos0, n, 64)
        return d


def token_batch(streams, pos0: int, n: int) -> dict:
    """Stack TokenStream.tokens over sequences -> arrays [B][n][width]."""
    parts = [s.tokens(pos0, n) for s in streams]
    return {k: np.stack([p[k] for p in parts]) for k in parts[0]}


class QueryProjector:
    """Query-side inputs through a real projection of seeded hidden states."""

    def __init__(self, workload: int, layer: int, hidden: int, n_heads: int, idx_heads: int, head_dim: int = 128,
                 idx_dim: int = 64):
        self.workload, self.layer, self.hidden = workload, layer, hidden
        self.H, self.HI, self.d, self.dI = n_heads, idx_heads, head_dim, idx_dim
        self.Wq = (_rng(workload, layer, T_WQ).standard_normal((hidden, n_heads * head_dim), dtype=np.float32)
                   * np.float32(0.02))
        self.WqI = None
        self.Ww = None
        if idx_heads:
            self.WqI = (_rng(workload, layer, T_WQI).standard_normal((hidden, idx_heads * idx_dim), dtype=np.float32)
                        * np.float32(0.02))
            self.Ww = (_rng(workload, layer, T_WW).standard_normal((hidden, idx_heads), dtype=np.float32)
                       * np.float32(0.02))

    def hidden_states(self, seq: int, positions) -> np.ndarray:
        rows = []
        for p in positions:
            rows.append(_rng(self.workload, self.layer, T_HID, seq, int(p)).standard_normal(self.hidden,
                                                                                           dtype=np.float32))
        return np.stack(rows)

    def queries(self, seq: int, positions) -> dict:
        """q [n][H][128] BF16 bits; qI [n][H_I][64] BF16 bits; w [n][H_I] f32."""
        h = self.hidden_states(seq, positions)
        n = h.shape[0]
        out = {"q": bf16_bits(h @ self.Wq).reshape(n, self.H, self.d)}
        if self.HI:
            out["qI"] = bf16_bits(h @ self.WqI).reshape(n, self.HI, self.dI)
            out["w"] = np.ascontiguousarray((h @ self.Ww).astype(np.float32)).reshape(n, self.HI)
        return out


def direct_queries(workload: int, layer: int, seq: int, pos0: int, n: int, n_heads: int, idx_heads: int,
                   sigma: float) -> dict:
    """Query-side inputs drawn directly (for workloads stated as N(0,1) inputs)."""
    g = _rng(workload, layer, T_HID, seq, pos0, n)
    q = g.standard_normal((n, n_heads, 128), dtype=np.float32) * np.float32(sigma)
    out = {"q": bf16_bits(q)}
    if idx_heads:
        qI = g.standard_normal((n, idx_heads, 64), dtype=np.float32) * np.float32(sigma)
        w = g.standard_normal((n, idx_heads), dtype=np.float32) * np.float32(sigma)
        out["qI"] = bf16_bits(qI)
        out["w"] = w.astype(np.float32)
    return out


def biases(workload: int, layer: int, m: int, csa: bool) -> dict:
    out = {"bias": (_rng(workload, layer, T_BIAS).standard_normal((m, 128), dtype=np.float32)
                    * np.float32(0.02)).astype(np.float32)}
    if csa:
        out["idx_bias"] = (_rng(workload, layer, T_IBIAS).standard_normal((m, 64), dtype=np.float32)
                           * np.float32(0.02)).astype(np.float32)
    return out
