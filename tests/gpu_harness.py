"""Parity harness: the HIP library (through its C ABI) against the fp64 oracle.

Selection rule (per sequence, KV head and interval): with the oracle's own
scores sorted e(1) >= e(2) >= ..., margin mu = (e(C) - e(C+1)) / e(C).  Where
mu > 1e-5 the GPU's kept set must equal the oracle's.  Where mu <= 1e-5 both
sets are correct if the GPU set has C candidates whose smallest score is at
least the largest left-out score minus 1e-5 * e(C); the oracle then adopts
the GPU set (teacher forcing) and both continue from the same memories.

Tolerances: outputs, max over rows of ||o_gpu - o_ref|| / ||o_ref||; H and s,
per chain ||.||_F relative: 1e-4 for fp32 io, 2e-2 for bf16 io.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
from sparse_attention_chunkwise_amd import lola

MARGIN = 1e-5


def tol_for(layer) -> float:
    return 1e-4 if layer.io_dtype == "f32" else 2e-2


def dev(x: np.ndarray, layer) -> torch.Tensor:
    """Device tensor in the io dtype from float32 values exact in that dtype."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to("cuda")
    return t.to(torch.bfloat16) if layer.io_dtype == "bf16" else t


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def row_rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    num = np.linalg.norm(got - ref, axis=-1)
    den = np.linalg.norm(ref, axis=-1)
    return float((num / np.maximum(den, 1e-300)).max()) if num.size else 0.0


def fro_rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / den) if den > 0 else float(np.linalg.norm(got))


def check_selection(log, b, g, ci, gpu_set, C):
    """Apply the margin rule to one interval.  Returns (ok, forced_needed, text)."""
    nU = int(log["n_cand"][b, g, ci])
    pos = [int(p) for p in log["cand_pos"][b, g, ci, :nU]]
    sre = dict(zip(pos, log["cand_sre"][b, g, ci, :nU].tolist()))
    own = set(int(p) for p in log["own_kept"][b, g, ci] if p >= 0) if C > 0 else set()
    gpu = set(gpu_set)
    if gpu == own:
        return True, False, ""
    if nU <= C:
        return False, False, f"all {nU} candidates fit but the gpu kept {len(gpu)} of them differently"
    if not gpu.issubset(sre) or len(gpu) != min(C, nU):
        return False, False, f"gpu set not a selection of the candidates: {sorted(gpu - set(sre))[:5]}"
    es = sorted(sre.values(), reverse=True)
    eC, eC1 = es[C - 1], es[C]
    mu = 0.0 if eC == 0 else (eC - eC1) / eC
    kept_min = min(sre[p] for p in gpu)
    out_max = max(sre[p] for p in set(sre) - gpu)
    if mu <= MARGIN and kept_min >= out_max - MARGIN * eC:
        return True, True, f"near tie mu={mu:.3g} adopted"
    return False, False, f"selection differs with margin mu={mu:.3g} (kept min {kept_min}, left-out max {out_max})"


class Stepper:
    """A GPU state and an oracle advanced together, one interval per call."""

    def __init__(self, layer, B: int, W: np.ndarray):
        self.layer = layer
        self.B = B
        self.W = W
        self.state = lola.init_state(layer, B, torch.from_numpy(W).to("cuda"))
        self.orc = oracle.Oracle(layer, B, W)
        self.forced_count = 0

    def gpu_cache_sets(self):
        rc = lola.read_cache(self.layer, self.state, self.B, want_kv=False, want_state=False)
        cnt = rc["count"].cpu().numpy()
        pos = rc["pos"].cpu().numpy()
        return [[[int(p) for p in pos[b, g, : cnt[b, g]]] for g in range(self.layer.n_kv_heads)]
                for b in range(self.B)]

    def step(self, q, k, v, decode: bool = False, row_mask=None, chain_mask=None):
        """Run one interval (n <= chunk tokens, or one decode token) on both sides.

        q [B,n,Hq,D], k, v [B,n,Hkv,D] float32 arrays exact in the io dtype.
        Returns (gpu_out, ref_out) as float64 arrays [B,n,Hq,D]; asserts the
        selection rule on every chain.
        """
        L = self.layer
        n = k.shape[1]
        assert n <= L.chunk or (decode and n == 1)
        if decode:
            out = lola.decode(L, self.state, dev(q[:, 0], L), dev(k[:, 0], L), dev(v[:, 0], L))
            gout = host(out)[:, None]
        else:
            out = lola.prefill(L, self.state, dev(q, L), dev(k, L), dev(v, L))
            gout = host(out)
        self.last_out = out  # device tensor of this step's outputs
        sets = self.gpu_cache_sets()
        C = L.cache_cap
        forced = np.full((self.B, L.n_kv_heads, 1, max(C, 1)), -1, np.int64)
        for b in range(self.B):
            for g in range(L.n_kv_heads):
                s = sets[b][g]
                forced[b, g, 0, : len(s)] = s
        ref, log = self.orc.run(q, k, v, log=True, forced=forced if C > 0 else None,
                                row_mask=row_mask, chain_mask=chain_mask)
        for b in range(self.B):
            for g in range(L.n_kv_heads):
                if chain_mask is not None and not chain_mask[b, g]:
                    continue
                ok, fc, txt = check_selection(log, b, g, 0, sets[b][g], C)
                assert ok, f"chain ({b},{g}) at t0={self.orc.tokens_seen(b) - n}: {txt}"
                self.forced_count += int(fc)
        return gout, ref

    def healthy(self) -> bool:
        """The state header is intact and no scan gave up waiting (synchronises)."""
        return lola.check_state(self.layer, self.state, self.B) == 0

    def compare_state(self, chain_mask=None):
        """H, s relative errors (max over chains) and exact cache key/value equality."""
        L = self.layer
        rc = lola.read_cache(L, self.state, self.B)
        H, s = host(rc["H"]), host(rc["s"])
        K, V, cnt = host(rc["k"]), host(rc["v"]), rc["count"].cpu().numpy()
        eh = es = 0.0
        for b in range(self.B):
            for g in range(L.n_kv_heads):
                if chain_mask is not None and not chain_mask[b, g]:
                    continue
                ch = self.orc.chain(b, g)
                eh = max(eh, fro_rel_err(H[b, g], ch["H"]))
                es = max(es, fro_rel_err(s[b, g], ch["s"]))
                c = int(cnt[b, g])
                assert c == ch["cache_n"]
                np.testing.assert_array_equal(K[b, g, :c], ch["cache_k"])
                np.testing.assert_array_equal(V[b, g, :c], ch["cache_v"])
        return eh, es


def min_margin(log, C):
    """Smallest selection margin over every full interval of a log (inf if none)."""
    best = np.inf
    nc = log["n_cand"]
    for idx in np.ndindex(nc.shape):
        nU = int(nc[idx])
        if nU <= C or C == 0:
            continue
        es = np.sort(log["cand_sre"][idx][:nU])[::-1]
        eC, eC1 = es[C - 1], es[C]
        mu = 0.0 if eC == 0 else (eC - eC1) / eC
        best = min(best, mu)
    return best
