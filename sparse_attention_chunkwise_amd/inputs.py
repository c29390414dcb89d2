"""Seeded synthetic inputs for the LoLA layer workloads.

This module only draws random numbers and rounds them to the storage dtype.
It holds none of the layer's arithmetic, so both the HIP path and the CPU
oracle take their inputs from here without sharing any method code.

Workloads (all synthetic; the pages measure accuracy on RULER / commonsense
suites that need trained weights, and these shapes only imitate their
structure):

  1  tiny fp32:           B1, Hq=Hkv=1, D64, feature half 32, w16, C16, L16, T512
  2  collision stress:    B1, Hq=Hkv=4, D64, half 32, w32, C32, L32, T2048, fp32,
                          clustered keys + 16 planted near-orthogonal needles
  3  4K bf16 prefill:     B1, Hq32/Hkv8, D128, half 64, w64, C256, L64, T4096
  4  bf16 decode:         64 sequences of cfg3 shape, 4096-token prefill, then
                          256 single-token steps with fresh q/k/v
  5  64K bf16 prefill:    B4, Hq32/Hkv8, D128, half 64, w64, C512, L128, T65536,
                          clustered keys with 5% planted needles

Random stream: numpy Generator(PCG64(1000*cfg + b)) for sequence b.  The
generator of sequence 0 first draws the feature-map weights W (feat_half x D,
entries N(0, 1/D)), then every sequence draws Q [T,Hq,D], K [T,Hkv,D],
V [T,Hkv,D] in that order.  Decode steps (cfg 4) use a second stream
PCG64(1000*cfg + 500 + b) per sequence, drawing q/k/v per step; the mixed
(continuous-batching) steps over the cfg 4 sequences use PCG64(1000*cfg + 700).
"N(0, x)" means variance x.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np


@dataclasses.dataclass(frozen=True)
class LayerConfig:
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    feat_half: int
    window: int
    cache_cap: int
    chunk: int
    io_dtype: str  # "f32" or "bf16"
    softmax_scale: float = 0.0  # 0 -> 1/sqrt(head_dim)
    policy: int = 0  # scoring / cache policy: 0 SRE, 1 stale SRE (min-heap), 2 FIFO, 3 attention weight, 4 softmax error
    decode_mode: int = 0  # 0 decode steps rescore the cache, 1 they update stored scores (same result)

    @property
    def feat_dim(self) -> int:
        return 2 * self.feat_half

    @property
    def scale(self) -> float:
        return self.softmax_scale if self.softmax_scale > 0 else 1.0 / math.sqrt(self.head_dim)

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads


@dataclasses.dataclass(frozen=True)
class Workload:
    cfg_id: int
    name: str
    layer: LayerConfig
    batch: int
    seq_len: int
    keys: str  # "gauss" or "clustered"
    n_needles: int = 0
    decode_steps: int = 0


WORKLOADS = {
    1: Workload(1, "tiny-fp32-d64-w16-c16-l16-t512",
                LayerConfig(1, 1, 64, 32, 16, 16, 16, "f32"), 1, 512, "gauss"),
    2: Workload(2, "collision-fp32-h4-d64-w32-c32-l32-t2048",
                LayerConfig(4, 4, 64, 32, 32, 32, 32, "f32"), 1, 2048, "clustered", n_needles=16),
    3: Workload(3, "prefill-bf16-h32kv8-d128-w64-c256-l64-t4096-b1",
                LayerConfig(32, 8, 128, 64, 64, 256, 64, "bf16"), 1, 4096, "gauss"),
    4: Workload(4, "decode-bf16-h32kv8-d128-w64-c256-b64-ctx4096-steps256",
                LayerConfig(32, 8, 128, 64, 64, 256, 64, "bf16"), 64, 4096, "gauss",
                decode_steps=256),
    5: Workload(5, "prefill-bf16-h32kv8-d128-w64-c512-l128-t65536-b4",
                LayerConfig(32, 8, 128, 64, 64, 512, 128, "bf16"), 4, 65536, "clustered",
                n_needles=round(0.05 * 65536)),
}


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32).astype(np.uint64)
    rounded = (bits + 0x7FFF + ((bits >> 16) & 1)) >> 16 << 16
    out = (rounded & 0xFFFFFFFF).astype(np.uint32).view(np.float32)
    nan = np.isnan(x)
    if nan.any():
        out = out.copy()
        out[nan] = np.nan
    return out


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Upper 16 bits of float32 values that are already exact bfloat16 numbers."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


def to_storage(x: np.ndarray, io_dtype: str) -> np.ndarray:
    return round_to_bf16(x) if io_dtype == "bf16" else np.ascontiguousarray(x, dtype=np.float32)


def draw_feature_weights(rng: np.random.Generator, feat_half: int, head_dim: int) -> np.ndarray:
    return (rng.standard_normal((feat_half, head_dim)) / math.sqrt(head_dim)).astype(np.float32)


def _clustered_keys(rng: np.random.Generator, T: int, D: int, n_needles: int, window: int):
    """Keys drawn around 8 centres, plus needles orthogonal to the centres' span."""
    centres = rng.standard_normal((8, D))
    z = rng.integers(0, 8, size=T)
    keys = centres[z] + math.sqrt(0.1) * rng.standard_normal((T, D))
    hi = max(T - window, 1)
    n = min(n_needles, hi)
    pos = np.sort(rng.choice(hi, size=n, replace=False))
    g = rng.standard_normal((n, D))
    q, _ = np.linalg.qr(centres.T)  # D x 8 orthonormal basis of the centres' span
    g = g - (g @ q) @ q.T
    g *= math.sqrt(D) / np.linalg.norm(g, axis=1, keepdims=True)
    keys[pos] = g
    return keys, pos


def make_sequence(wl: Workload, b: int, seq_len: int | None = None):
    """Draw (W or None, Q, K, V, needle positions) for sequence b, all float32 in storage precision.

    W is returned only for b == 0 (it is the first draw of that stream).
    seq_len shortens the draw (the first seq_len tokens of a shorter stream,
    not a prefix of the full one) for quick cases.
    """
    L = wl.layer
    T = wl.seq_len if seq_len is None else seq_len
    rng = np.random.Generator(np.random.PCG64(1000 * wl.cfg_id + b))
    W = draw_feature_weights(rng, L.feat_half, L.head_dim) if b == 0 else None
    Q = rng.standard_normal((T, L.n_q_heads, L.head_dim), dtype=np.float32)
    needles = []
    if wl.keys == "gauss":
        K = rng.standard_normal((T, L.n_kv_heads, L.head_dim), dtype=np.float32)
    else:
        K = np.empty((T, L.n_kv_heads, L.head_dim), dtype=np.float32)
        for g in range(L.n_kv_heads):
            kg, pos = _clustered_keys(rng, T, L.head_dim, wl.n_needles, L.window)
            K[:, g, :] = kg
            needles.append(pos)
    V = rng.standard_normal((T, L.n_kv_heads, L.head_dim), dtype=np.float32)
    io = L.io_dtype
    return (None if W is None else W), to_storage(Q, io), to_storage(K, io), to_storage(V, io), needles


def make_batch(wl: Workload, seq_len: int | None = None, batch: int | None = None):
    """Return W [Hkv,feat_half,D] (one W broadcast to every KV head) and Q [B,T,Hq,D], K, V [B,T,Hkv,D]."""
    B = wl.batch if batch is None else batch
    Ws, Qs, Ks, Vs = None, [], [], []
    for b in range(B):
        W, Q, K, V, _ = make_sequence(wl, b, seq_len)
        if b == 0:
            Ws = W
        Qs.append(Q)
        Ks.append(K)
        Vs.append(V)
    L = wl.layer
    Wfull = np.ascontiguousarray(np.broadcast_to(Ws, (L.n_kv_heads,) + Ws.shape), dtype=np.float32)
    return Wfull, np.stack(Qs), np.stack(Ks), np.stack(Vs)


def make_decode_steps(wl: Workload, steps: int, batch: int | None = None):
    """Fresh N(0,1) q [S,B,Hq,D], k, v [S,B,Hkv,D] for single-token decode steps."""
    L = wl.layer
    B = wl.batch if batch is None else batch
    q = np.empty((steps, B, L.n_q_heads, L.head_dim), np.float32)
    k = np.empty((steps, B, L.n_kv_heads, L.head_dim), np.float32)
    v = np.empty_like(k)
    for b in range(B):
        rng = np.random.Generator(np.random.PCG64(1000 * wl.cfg_id + 500 + b))
        for s in range(steps):
            q[s, b] = rng.standard_normal((L.n_q_heads, L.head_dim), dtype=np.float32)
            k[s, b] = rng.standard_normal((L.n_kv_heads, L.head_dim), dtype=np.float32)
            v[s, b] = rng.standard_normal((L.n_kv_heads, L.head_dim), dtype=np.float32)
    io = L.io_dtype
    return to_storage(q, io), to_storage(k, io), to_storage(v, io)


def make_mixed_steps(wl: Workload, steps: int, chunk_tokens: int, n_prefill: int):
    """Mixed (continuous-batching) steps over the decode workload's sequences: in step s,
    sequences (s * n_prefill + j) mod B for j < n_prefill advance by a chunk of
    `chunk_tokens` tokens, every other sequence by one token.  Returns int32 counts [S,B]
    and N(0,1) q [S,B,chunk,Hq,D], k, v [S,B,chunk,Hkv,D], zero past each count."""
    L = wl.layer
    B = wl.batch
    counts = np.ones((steps, B), np.int32)
    q = np.zeros((steps, B, chunk_tokens, L.n_q_heads, L.head_dim), np.float32)
    k = np.zeros((steps, B, chunk_tokens, L.n_kv_heads, L.head_dim), np.float32)
    v = np.zeros_like(k)
    rng = np.random.Generator(np.random.PCG64(1000 * wl.cfg_id + 700))
    for s in range(steps):
        for j in range(n_prefill):
            counts[s, (s * n_prefill + j) % B] = chunk_tokens
        for b in range(B):
            n = int(counts[s, b])
            q[s, b, :n] = rng.standard_normal((n, L.n_q_heads, L.head_dim), dtype=np.float32)
            k[s, b, :n] = rng.standard_normal((n, L.n_kv_heads, L.head_dim), dtype=np.float32)
            v[s, b, :n] = rng.standard_normal((n, L.n_kv_heads, L.head_dim), dtype=np.float32)
    io = L.io_dtype
    return counts, to_storage(q, io), to_storage(k, io), to_storage(v, io)


def random_case(seed: int, layer: LayerConfig, batch: int, T: int):
    """Plain N(0,1) inputs for an arbitrary layer shape (edge-case tests)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    W = draw_feature_weights(rng, layer.feat_half, layer.head_dim)
    Wfull = np.ascontiguousarray(np.broadcast_to(W, (layer.n_kv_heads,) + W.shape), dtype=np.float32)
    Q = rng.standard_normal((batch, T, layer.n_q_heads, layer.head_dim), dtype=np.float32)
    K = rng.standard_normal((batch, T, layer.n_kv_heads, layer.head_dim), dtype=np.float32)
    V = rng.standard_normal((batch, T, layer.n_kv_heads, layer.head_dim), dtype=np.float32)
    io = layer.io_dtype
    return Wfull, to_storage(Q, io), to_storage(K, io), to_storage(V, io)
