"""ctypes front end of the fp64 CPU oracle (lola_oracle.c).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's CPU
baseline leg use it; the product path never imports it.  It shares no code
with the HIP library.

Parity status of each oracle function (what pins it, see tests/):
  lo_phi  -- closed forms (halves sum to 1, W = 0 gives uniform 2/F, softmax
             shift invariance) and a NumPy restatement.
  lo_sre  -- closed forms (zero for a state holding only that pair, mean-value
             state, scale invariance, empty state).
  lo_run  -- (policies other than the SRE: closed forms for the FIFO cache,
             the attention-weight scorer with one query head and the
             approximation-error scorer with a constant feature map, and an
             independent NumPy replay of every policy)
             reductions to causal softmax attention (w >= T) and to causal
             linear attention (w = 0, C = 0), chunk-size independence at
             C = 0, per-key-weight brute force, from-scratch recomputation of
             every interval's scores and ranking, conservation laws, a hand
             worked trajectory under tests/golden/, split-call and
             decode-step equivalences.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "lola_oracle.c")
LIB = os.path.join(_HERE, "liblola_oracle.so")

_lib = None


def build(src: str = SRC, out: str = LIB) -> str:
    """Compile the oracle with gcc (plain -O2, no fast-math)."""
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-shared", "-fPIC", "-o", out, src, "-lm", "-lpthread"]
    subprocess.run(cmd, check=True)
    return out


class _Cfg(ctypes.Structure):
    _fields_ = [("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("feat_half", ctypes.c_int32),
                ("window", ctypes.c_int32), ("cache_cap", ctypes.c_int32),
                ("chunk", ctypes.c_int32), ("policy", ctypes.c_int32), ("scale", ctypes.c_double)]


class _Log(ctypes.Structure):
    _fields_ = [("max_intervals", ctypes.c_int32), ("max_cand", ctypes.c_int32),
                ("n_cand", ctypes.c_void_p), ("cand_pos", ctypes.c_void_p),
                ("cand_sre", ctypes.c_void_p), ("own_kept", ctypes.c_void_p)]


def load(path: str = LIB):
    """Load the oracle library (compiling it first if it is not built)."""
    global _lib
    if _lib is not None and path == LIB:
        return _lib
    if not os.path.exists(path) or (path == LIB and os.path.getmtime(path) < os.path.getmtime(SRC)):
        build(SRC, path)
    lib = ctypes.CDLL(path)
    vp, i32, dbl = ctypes.c_void_p, ctypes.c_int, ctypes.c_double
    lib.lo_phi.argtypes = [vp, i32, i32, vp, vp]
    lib.lo_phi.restype = None
    lib.lo_sre.argtypes = [i32, i32, vp, vp, vp, vp]
    lib.lo_sre.restype = dbl
    lib.lo_create.argtypes = [ctypes.POINTER(_Cfg), i32, vp]
    lib.lo_create.restype = vp
    lib.lo_clone.argtypes = [vp]
    lib.lo_clone.restype = vp
    lib.lo_destroy.argtypes = [vp]
    lib.lo_destroy.restype = None
    lib.lo_tokens_seen.argtypes = [vp, i32]
    lib.lo_tokens_seen.restype = ctypes.c_int64
    lib.lo_get_chain.argtypes = [vp, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.lo_get_chain.restype = None
    lib.lo_run.argtypes = [vp, i32, vp, vp, vp, vp, vp, ctypes.POINTER(_Log), vp, vp, i32]
    lib.lo_run.restype = i32
    if path == LIB:
        _lib = lib
    return lib


def _f64(x):
    return np.ascontiguousarray(x, dtype=np.float64)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def phi(W, x, lib=None):
    """phi(x) = [softmax(W x); softmax(-W x)] for one vector x (W is feat_half x D)."""
    lib = lib or load()
    W, x = _f64(W), _f64(x)
    out = np.empty(2 * W.shape[0], np.float64)
    lib.lo_phi(_ptr(W), W.shape[0], W.shape[1], _ptr(x), _ptr(out))
    return out


def sre(H, s, phik, v, lib=None):
    """Self-recall error of the pair (k, v) against the state (H, s); phik = phi(k)."""
    lib = lib or load()
    H, s, phik, v = _f64(H), _f64(s), _f64(phik), _f64(v)
    return lib.lo_sre(H.shape[0], H.shape[1], _ptr(H), _ptr(s), _ptr(phik), _ptr(v))


class Oracle:
    """A batch of LoLA layer states advanced token interval by token interval in fp64."""

    def __init__(self, layer, batch: int, W, lib=None, _handle=None):
        self.lib = lib or load()
        self.layer = layer
        self.B = batch
        L = layer
        self._cfg = _Cfg(L.n_q_heads, L.n_kv_heads, L.head_dim, L.feat_half, L.window,
                         L.cache_cap, L.chunk, int(L.policy), float(L.softmax_scale))
        if _handle is None:
            W = _f64(W)
            assert W.shape == (L.n_kv_heads, L.feat_half, L.head_dim), W.shape
            self._W = W
            self._h = self.lib.lo_create(ctypes.byref(self._cfg), batch, _ptr(W))
            if not self._h:
                raise ValueError("oracle rejected the configuration")
        else:
            self._W = W
            self._h = _handle

    def __del__(self):
        h = getattr(self, "_h", None)
        if h:
            self.lib.lo_destroy(h)
            self._h = None

    def clone(self) -> "Oracle":
        return Oracle(self.layer, self.B, self._W, self.lib, _handle=self.lib.lo_clone(self._h))

    def tokens_seen(self, b: int = 0) -> int:
        return int(self.lib.lo_tokens_seen(self._h, b))

    def run(self, q, k, v, want_out: bool = True, forced=None, log: bool = False,
            chain_mask=None, row_mask=None, nthreads: int | None = None):
        """Advance every sequence by n = k.shape[1] tokens.

        q [B,n,Hq,D], k, v [B,n,Hkv,D].  Returns (out or None, log dict or None).
        forced: int64 [B,Hkv,NI,C] kept positions per interval (-1 padded).
        """
        L = self.layer
        k, v = _f64(k), _f64(v)
        B, n = k.shape[0], k.shape[1]
        assert B == self.B and k.shape[2:] == (L.n_kv_heads, L.head_dim)
        q = _f64(q) if q is not None else None
        out = np.zeros((B, n, L.n_q_heads, L.head_dim), np.float64) if want_out else None
        NI = (n + L.chunk - 1) // L.chunk
        maxU = L.cache_cap + L.chunk
        lg = None
        logd = None
        if log:
            logd = {
                "n_cand": np.zeros((B, L.n_kv_heads, NI), np.int32),
                "cand_pos": np.full((B, L.n_kv_heads, NI, maxU), -1, np.int64),
                "cand_sre": np.zeros((B, L.n_kv_heads, NI, maxU), np.float64),
                "own_kept": np.full((B, L.n_kv_heads, NI, max(L.cache_cap, 1)), -1, np.int64),
            }
            lg = _Log(NI, maxU, _ptr(logd["n_cand"]).value, _ptr(logd["cand_pos"]).value,
                      _ptr(logd["cand_sre"]).value,
                      _ptr(logd["own_kept"]).value if L.cache_cap > 0 else None)
        if forced is not None:
            forced = np.ascontiguousarray(forced, dtype=np.int64)
            assert forced.shape == (B, L.n_kv_heads, NI, L.cache_cap), forced.shape
        cm = None if chain_mask is None else np.ascontiguousarray(chain_mask, dtype=np.uint8)
        rm = None if row_mask is None else np.ascontiguousarray(row_mask, dtype=np.uint8)
        nt = nthreads or min(os.cpu_count() or 1, B * L.n_kv_heads, 16)
        rc = self.lib.lo_run(self._h, n, _ptr(q), _ptr(k), _ptr(v),
                             _ptr(out), _ptr(forced), ctypes.byref(lg) if lg is not None else None,
                             _ptr(cm), _ptr(rm), nt)
        if rc == -2:
            raise ValueError("forced selection is not a valid choice for this interval")
        if rc != 0:
            raise RuntimeError(f"oracle lo_run failed: {rc}")
        return out, logd

    def chain(self, b: int, g: int) -> dict:
        L = self.layer
        F, D, C, w = L.feat_dim, L.head_dim, L.cache_cap, L.window
        H = np.zeros((F, D))
        s = np.zeros(F)
        cn = ctypes.c_int32(0)
        cpos = np.full(max(C, 1), -1, np.int64)
        ck = np.zeros((max(C, 1), D))
        cv = np.zeros((max(C, 1), D))
        wn = ctypes.c_int32(0)
        wpos = np.full(max(w, 1), -1, np.int64)
        wk = np.zeros((max(w, 1), D))
        wv = np.zeros((max(w, 1), D))
        nf = ctypes.c_int64(0)
        self.lib.lo_get_chain(self._h, b, g, _ptr(H), _ptr(s), ctypes.byref(cn), _ptr(cpos), _ptr(ck),
                              _ptr(cv), ctypes.byref(wn), _ptr(wpos), _ptr(wk), _ptr(wv), ctypes.byref(nf))
        c, m = cn.value, wn.value
        return {"H": H, "s": s, "cache_n": c, "cache_pos": cpos[:c].copy(), "cache_k": ck[:c].copy(),
                "cache_v": cv[:c].copy(), "win_n": m, "win_pos": wpos[:m].copy(), "win_k": wk[:m].copy(),
                "win_v": wv[:m].copy(), "n_folded": int(nf.value)}
