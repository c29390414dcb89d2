"""Pins of the fp64 oracle: checks against what the definitions and the
mathematics fix, written independently of the oracle's C code.

Each check_* function takes the loaded oracle library (so the mutation test
can run the same checks against a copy with a planted mistake) and raises
AssertionError on a mismatch.

Sources for what is checked: the SRE equation of the "Self-Recall Error"
section and steps 1-4 of the "Inferentiestrategie" section of the LoLA
technical summary (gist.science), the three-memory split of the paper's
abstract, and the reductions the layer definition implies (window covering
the whole sequence -> causal softmax attention; no window and no cache ->
causal linear attention; no cache -> independent of the interval length).
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import scipy.special
import torch

import oracle
from sparse_attention_chunkwise_amd.inputs import LayerConfig, random_case

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# --------------------------------------------------------------------------
# independent NumPy restatements used by the checks
# --------------------------------------------------------------------------

def phi_rows(W, X):
    """Feature map of every row of X via scipy's softmax: [softmax(Wx); softmax(-Wx)]."""
    Z = np.asarray(X, np.float64) @ np.asarray(W, np.float64).T
    return np.concatenate([scipy.special.softmax(Z, axis=-1), scipy.special.softmax(-Z, axis=-1)], axis=-1)


def brute_outputs(layer, W, Q, K, V, cache_sets, t_start=0):
    """Per-key-weight form of the read.

    Every past key j <= t contributes exactly once with weight
      exp(tau q.k_j)     if j is in the last-w window of t or in the cache set
                         active for t's interval,
      phi(q).phi(k_j)    otherwise (folded or still pending: both linear),
    and o_t = sum_j kappa_j v_j / sum_j kappa_j.  cache_sets[b][g][c] is the
    cache content (positions) during interval c.
    """
    B, T = K.shape[0], K.shape[1]
    G = layer.group
    tau = layer.scale
    w, L = layer.window, layer.chunk
    out = np.zeros(Q.shape, np.float64)
    for b in range(B):
        for g in range(layer.n_kv_heads):
            phK = phi_rows(W[g], K[b, :, g])
            for t in range(T):
                c = t // L
                S = cache_sets[b][g][c]
                j = np.arange(t + 1)
                soft = (j >= t - w + 1) | np.isin(j, list(S))
                for h in range(g * G, (g + 1) * G):
                    q = Q[b, t, h].astype(np.float64)
                    logit = tau * (K[b, : t + 1, g].astype(np.float64) @ q)
                    kap_lin = phK[: t + 1] @ phi_rows(W[g], q[None])[0]
                    kap = np.where(soft, np.exp(logit), kap_lin)
                    out[b, t, h] = kap @ V[b, : t + 1, g].astype(np.float64) / kap.sum()
    return out


def replay_selection(layer, W, K, V, T, choose=None, Q=None):
    """Recompute every interval's candidates, scores and kept set from scratch.

    Candidates at interval [a, e): the cache plus positions max(0,a-w)..e-1-w.
    State: H = sum over folded pairs of phi(k) v^T, s = sum of phi(k),
    rebuilt from the folded set (not updated in place).  Scores: the
    Nadaraya-Watson form of the SRE, r = sum_f kappa_f v_f / sum_f kappa_f
    with kappa_f = phi(k).phi(k_f) (0 when nothing is folded).
    choose(b, g, c, U, scores, own) may replace the kept set `own` (the first
    min(C, |U|) by score descending, position ascending) by another list of
    positions; the rest of the candidates are folded.
    layer.policy other than 0 replaces the SRE as the score (Q gives the
    queries of the query-based scorers): 1 a cached pair keeps the score it
    had when it left the window, 2 the position, 3 the sum over the KV head's
    query heads of the softmax weight the interval's last query gives the
    candidate among all candidates, 4 the sum of |softmax weight - linear
    weight| with linear weight phi(q).phi(k) normalised over the candidates.
    Returns per chain a list of dicts (cand positions, scores, own and kept
    sets) and, per chain, the folded positions in fold order.
    """
    w, C, L = layer.window, layer.cache_cap, layer.chunk
    B = K.shape[0]
    res = []
    for b in range(B):
        per_b = []
        for g in range(layer.n_kv_heads):
            phK = phi_rows(W[g], K[b, :, g])
            Vg = V[b, :, g].astype(np.float64)
            folded, S, steps = [], [], []
            kept_score = {}
            for a in range(0, T, L):
                e = min(a + L, T)
                E = list(range(max(0, a - w), e - w))
                U = list(S) + E
                if folded:
                    kap = phK[U] @ phK[folded].T  # |U| x |folded|
                    r = kap @ Vg[folded] / kap.sum(axis=1, keepdims=True)
                else:
                    r = np.zeros((len(U), Vg.shape[1]))
                sc = ((r - Vg[U]) ** 2).sum(axis=1) if U else np.zeros(0)
                if layer.policy == 1:
                    sc = np.array([kept_score[u] if u in kept_score else x for u, x in zip(U, sc)])
                elif layer.policy == 2:
                    sc = np.array(U, np.float64)
                elif layer.policy in (3, 4) and U:
                    G = layer.group
                    sc = np.zeros(len(U))
                    for h in range(g * G, (g + 1) * G):
                        q = Q[b, e - 1, h].astype(np.float64)
                        p = scipy.special.softmax(layer.scale * (K[b, U, g].astype(np.float64) @ q))
                        if layer.policy == 3:
                            sc += p
                        else:
                            lin = phK[U] @ phi_rows(W[g], q[None])[0]
                            sc += np.abs(p - lin / lin.sum())
                order = sorted(range(len(U)), key=lambda i: (-sc[i], U[i]))
                own = [U[i] for i in order[: min(C, len(U))]]
                keep = own if choose is None else list(choose(b, g, len(steps), U, sc, own))
                gone = [u for u in U if u not in set(keep)]
                kept_score = {u: x for u, x in zip(U, sc) if u in set(keep)}
                steps.append({"U": U, "sre": sc, "keep": set(keep), "own": set(own), "order": order,
                              "folded": list(folded)})
                folded.extend(gone)
                S = keep
            steps_final = {"folded": folded}
            per_b.append(steps + [steps_final])
        res.append(per_b)
    return res


def cache_sets_from_log(log, B, Hkv):
    """Cache content during each interval, from the oracle's own kept sets."""
    sets = []
    for b in range(B):
        per_b = []
        for g in range(Hkv):
            seq = [set()]
            for c in range(log["own_kept"].shape[2]):
                seq.append(set(int(p) for p in log["own_kept"][b, g, c] if p >= 0))
            per_b.append(seq)
        sets.append(per_b)
    return sets


def _case(layer, T, B=1, seed=11):
    W, Q, K, V = random_case(seed, layer, B, T)
    return W, Q.astype(np.float64), K.astype(np.float64), V.astype(np.float64)


# --------------------------------------------------------------------------
# feature map and SRE closed forms
# --------------------------------------------------------------------------

def check_phi(lib):
    rng = np.random.default_rng(1)
    for Fh, D in [(1, 3), (4, 8), (32, 64), (64, 128)]:
        W = rng.standard_normal((Fh, D)) / math.sqrt(D)
        for _ in range(3):
            x = rng.standard_normal(D) * 3
            p = oracle.phi(W, x, lib)
            assert p.shape == (2 * Fh,)
            assert np.all(p > 0)
            assert abs(p[:Fh].sum() - 1) < 1e-14 and abs(p[Fh:].sum() - 1) < 1e-14
            np.testing.assert_allclose(p[:Fh], scipy.special.softmax(W @ x), rtol=1e-13, atol=1e-300)
            np.testing.assert_allclose(p[Fh:], scipy.special.softmax(-(W @ x)), rtol=1e-13, atol=1e-300)
        p0 = oracle.phi(np.zeros((Fh, D)), rng.standard_normal(D), lib)
        np.testing.assert_allclose(p0, np.full(2 * Fh, 1.0 / Fh), rtol=0, atol=1e-15)


def check_sre_closed_forms(lib):
    rng = np.random.default_rng(2)
    for Fh, D in [(2, 3), (32, 64), (64, 128)]:
        F = 2 * Fh
        W = rng.standard_normal((Fh, D)) / math.sqrt(D)
        k = rng.standard_normal(D)
        v = rng.standard_normal(D)
        pk = oracle.phi(W, k, lib)
        # a state that holds only this pair recalls it exactly
        e0 = oracle.sre(np.outer(pk, v), pk, pk, v, lib)
        assert e0 <= 1e-24 * max(1.0, v @ v), e0
        # every folded value equal: the prediction is that value
        vbar = rng.standard_normal(D)
        s = rng.random(F) + 0.1
        e1 = oracle.sre(np.outer(s, vbar), s, pk, v, lib)
        assert abs(e1 - ((vbar - v) ** 2).sum()) <= 1e-12 * (vbar - v) @ (vbar - v)
        # empty state predicts zero
        e2 = oracle.sre(np.zeros((F, D)), np.zeros(F), pk, v, lib)
        assert abs(e2 - v @ v) <= 1e-13 * (v @ v)
        # a state built from folded pairs: the prediction is the kernel-weighted
        # mean of their values (Nadaraya-Watson form), and scaling H, s together
        # changes nothing
        ks = rng.standard_normal((7, D))
        vs = rng.standard_normal((7, D))
        P = phi_rows(W, ks)
        H = P.T @ vs
        sv = P.sum(0)
        kap = P @ pk
        r = kap @ vs / kap.sum()
        e3 = oracle.sre(H, sv, pk, v, lib)
        assert abs(e3 - ((r - v) ** 2).sum()) <= 1e-11 * ((r - v) ** 2).sum()
        e4 = oracle.sre(3.5 * H, 3.5 * sv, pk, v, lib)
        assert abs(e4 - e3) <= 1e-12 * e3


# --------------------------------------------------------------------------
# reductions of the whole layer
# --------------------------------------------------------------------------

def check_full_window_is_causal_softmax(lib):
    """Window covering the whole sequence (any cache, any interval): exact causal softmax."""
    for (Hq, Hkv, C, L) in [(2, 1, 0, 5), (4, 2, 3, 4), (1, 1, 8, 1)]:
        layer = LayerConfig(Hq, Hkv, 16, 4, 64, C, L, "f32")
        T = 40
        W, Q, K, V = _case(layer, T, B=2, seed=3)
        o, _ = oracle.Oracle(layer, 2, W, lib).run(Q, K, V)
        G = Hq // Hkv
        q = torch.from_numpy(Q).permute(0, 2, 1, 3)
        k = torch.from_numpy(K).permute(0, 2, 1, 3).repeat_interleave(G, dim=1)
        v = torch.from_numpy(V).permute(0, 2, 1, 3).repeat_interleave(G, dim=1)
        ref = torch.nn.functional.scaled_dot_product_attention(
            q, k, v, is_causal=True, scale=layer.scale).permute(0, 2, 1, 3).numpy()
        np.testing.assert_allclose(o, ref, rtol=1e-11, atol=1e-12)


def check_no_window_no_cache_is_linear_attention(lib):
    """w = 0, C = 0: causal linear attention with the feature map, any interval length."""
    for L in (1, 3, 8):
        layer = LayerConfig(2, 1, 16, 4, 0, 0, L, "f32")
        T = 30
        W, Q, K, V = _case(layer, T, seed=4)
        o, _ = oracle.Oracle(layer, 1, W, lib).run(Q, K, V)
        pk = phi_rows(W[0], K[0, :, 0])
        Sk = np.cumsum(pk[:, :, None] * V[0, :, 0][:, None, :], axis=0)  # T x F x D
        sk = np.cumsum(pk, axis=0)
        for h in range(2):
            pq = phi_rows(W[0], Q[0, :, h])
            ref = np.einsum("tf,tfd->td", pq, Sk) / np.einsum("tf,tf->t", pq, sk)[:, None]
            np.testing.assert_allclose(o[0, :, h], ref, rtol=1e-11, atol=1e-13)


def check_no_cache_independent_of_interval(lib):
    """C = 0: outputs and final state do not depend on the interval length."""
    T = 37
    ref = None
    for L in (1, 4, 9, 37):
        layer = LayerConfig(2, 2, 8, 3, 5, 0, L, "f32")
        W, Q, K, V = _case(layer, T, seed=5)
        orc = oracle.Oracle(layer, 1, W, lib)
        o, _ = orc.run(Q, K, V)
        ch = orc.chain(0, 1)
        if ref is None:
            ref = (o, ch)
        else:
            np.testing.assert_allclose(o, ref[0], rtol=1e-11, atol=1e-13)
            np.testing.assert_allclose(ch["H"], ref[1]["H"], rtol=1e-11, atol=1e-13)
            np.testing.assert_allclose(ch["s"], ref[1]["s"], rtol=1e-11, atol=1e-13)


def check_per_key_weights(lib, layer=None, T=None, B=1, seed=6):
    """Every output equals the per-key-weight brute force under the oracle's own selections."""
    cases = [(layer, T)] if layer is not None else [
        (LayerConfig(1, 1, 16, 4, 3, 2, 4, "f32"), 29),
        (LayerConfig(4, 2, 8, 2, 0, 3, 2, "f32"), 23),
        (LayerConfig(2, 1, 8, 4, 6, 4, 9, "f32"), 31),
        (LayerConfig(2, 2, 16, 8, 2, 5, 1, "f32"), 20),
    ]
    for lay, TT in cases:
        W, Q, K, V = _case(lay, TT, B=B, seed=seed)
        o, log = oracle.Oracle(lay, B, W, lib).run(Q, K, V, log=True)
        sets = cache_sets_from_log(log, B, lay.n_kv_heads)
        ref = brute_outputs(lay, W, Q, K, V, sets)
        np.testing.assert_allclose(o, ref, rtol=1e-10, atol=1e-12)


def check_selection_replay(lib, layer=None, T=None, B=1, seed=7, keys=None):
    """Candidates, scores and kept sets equal a from-scratch recomputation."""
    cases = [(layer, T)] if layer is not None else [
        (LayerConfig(1, 1, 16, 4, 3, 2, 4, "f32"), 41),
        (LayerConfig(2, 2, 8, 2, 0, 3, 2, "f32"), 23),
        (LayerConfig(2, 1, 8, 4, 6, 4, 9, "f32"), 47),
        (LayerConfig(1, 1, 12, 3, 1, 1, 1, "f32"), 15),
    ]
    for lay, TT in cases:
        if keys is None:
            W, Q, K, V = _case(lay, TT, B=B, seed=seed)
        else:
            W, Q, K, V = keys
        _, log = oracle.Oracle(lay, B, W, lib).run(Q, K, V, want_out=False, log=True)
        rep = replay_selection(lay, W, K, V, TT)
        for b in range(B):
            for g in range(lay.n_kv_heads):
                for c, st in enumerate(rep[b][g][:-1]):
                    nU = int(log["n_cand"][b, g, c])
                    pos = [int(p) for p in log["cand_pos"][b, g, c, :nU]]
                    assert sorted(pos) == sorted(st["U"]), (b, g, c, pos, st["U"])
                    got = dict(zip(pos, log["cand_sre"][b, g, c, :nU]))
                    for u, e in zip(st["U"], st["sre"]):
                        assert abs(got[u] - e) <= 1e-9 * max(1.0, abs(e)), (u, got[u], e)
                    kept = set(int(p) for p in log["own_kept"][b, g, c] if p >= 0) if lay.cache_cap else set()
                    assert kept == st["keep"], (b, g, c, kept, st["keep"])


def check_forced_selection(lib):
    """Teacher forcing: the oracle adopts a kept set given from outside.

    Several chains (2 sequences x 2 KV heads, which share candidate positions)
    run many intervals in one call; in a third of the intervals, with an offset
    that differs per chain, the kept set is a seeded random valid choice instead
    of the top C.  The candidates and scores the oracle logs, the outputs, and
    the final H, s must equal an independent replay that makes the same choices
    (outputs through the per-key-weight brute force with those cache sets), and
    the oracle must still log its own top-C choice.  Invalid forced sets (a
    position that is not a candidate, a repeated position, too few positions)
    are rejected."""
    layer = LayerConfig(2, 2, 8, 3, 3, 3, 4, "f32")
    B, T, C, Hkv = 2, 37, layer.cache_cap, layer.n_kv_heads
    NI = (T + layer.chunk - 1) // layer.chunk
    W, Q, K, V = _case(layer, T, B=B, seed=13)
    rng = np.random.default_rng(14)
    differs = []

    def choose(b, g, c, U, sc, own):
        if len(U) > C and (c + b + 2 * g) % 3 == 0:
            pick = sorted(int(x) for x in rng.choice(U, size=C, replace=False))
            differs.append(set(pick) != set(own))
            return pick
        return own

    rep = replay_selection(layer, W, K, V, T, choose=choose)
    assert sum(differs) >= 4, "the forcing changed too few intervals to test anything"
    forced = np.full((B, Hkv, NI, C), -1, np.int64)
    sets = []
    for b in range(B):
        per_b = []
        for g in range(Hkv):
            seq = [set()]
            for c in range(NI):
                kp = sorted(rep[b][g][c]["keep"])
                forced[b, g, c, :len(kp)] = kp
                seq.append(set(kp))
            per_b.append(seq)
        sets.append(per_b)
    # forced sets of different chains and intervals differ: a wrong offset cannot pass
    assert any(set(forced[0, 0, c]) != set(forced[0, 1, c]) for c in range(NI))
    assert any(set(forced[0, 0, c]) != set(forced[1, 0, c]) for c in range(NI))
    orc = oracle.Oracle(layer, B, W, lib)
    o, log = orc.run(Q, K, V, forced=forced, log=True)
    for b in range(B):
        for g in range(Hkv):
            for c in range(NI):
                st = rep[b][g][c]
                nU = int(log["n_cand"][b, g, c])
                pos = [int(p) for p in log["cand_pos"][b, g, c, :nU]]
                assert sorted(pos) == sorted(st["U"]), (b, g, c)
                got = dict(zip(pos, log["cand_sre"][b, g, c, :nU]))
                for u, e in zip(st["U"], st["sre"]):
                    assert abs(got[u] - e) <= 1e-9 * max(1.0, abs(e)), (b, g, c, u)
                own = set(int(p) for p in log["own_kept"][b, g, c] if p >= 0)
                assert own == st["own"], (b, g, c)
            ch = orc.chain(b, g)
            folded = rep[b][g][-1]["folded"]
            pk = phi_rows(W[g], K[b, folded, g])
            np.testing.assert_allclose(ch["H"], pk.T @ V[b, folded, g], rtol=1e-11, atol=1e-12)
            np.testing.assert_allclose(ch["s"], pk.sum(0), rtol=1e-11, atol=1e-12)
            assert sorted(ch["cache_pos"].tolist()) == sorted(rep[b][g][NI - 1]["keep"])
    ref = brute_outputs(layer, W, Q, K, V, sets)
    np.testing.assert_allclose(o, ref, rtol=1e-10, atol=1e-12)
    # invalid forced sets
    _, lg0 = oracle.Oracle(layer, B, W, lib).run(None, K[:, :12], V[:, :12], want_out=False, log=True)
    c_full = next(c for c in range(3) if int(lg0["n_cand"][0, 0, c]) > C)
    base = np.full((B, Hkv, 3, C), -1, np.int64)
    for b in range(B):
        for g in range(Hkv):
            for c in range(3):
                kp = [int(p) for p in lg0["own_kept"][b, g, c] if p >= 0]
                base[b, g, c, :len(kp)] = kp
    oracle.Oracle(layer, B, W, lib).run(None, K[:, :12], V[:, :12], want_out=False, forced=base)
    for bad in ("not_a_candidate", "repeated", "too_few"):
        f = base.copy()
        if bad == "not_a_candidate":
            f[1, 1, c_full, 0] = T + 5
        elif bad == "repeated":
            f[1, 1, c_full, 1] = f[1, 1, c_full, 0]
        else:
            f[1, 1, c_full, C - 1] = -1
        try:
            oracle.Oracle(layer, B, W, lib).run(None, K[:, :12], V[:, :12], want_out=False, forced=f)
        except ValueError:
            continue
        raise AssertionError(f"forced set with a {bad} entry accepted")


POLICY_LAYERS = [
    # (layer without the policy, T): several query heads per KV head, L = 1, L > w
    (LayerConfig(4, 2, 8, 3, 3, 3, 4, "f32"), 37),
    (LayerConfig(2, 1, 8, 4, 2, 2, 1, "f32"), 21),
    (LayerConfig(3, 1, 16, 4, 2, 4, 6, "f32"), 44),
]


def _with_policy(layer, policy):
    return LayerConfig(layer.n_q_heads, layer.n_kv_heads, layer.head_dim, layer.feat_half, layer.window,
                       layer.cache_cap, layer.chunk, layer.io_dtype, layer.softmax_scale, policy)


def check_policy_replay(lib):
    """Every scoring / cache policy: candidates, logged scores and kept sets equal an
    independent NumPy replay of the policy, and the outputs equal the per-key-weight
    brute force under the oracle's own cache sets."""
    for policy in (1, 2, 3, 4):
        for base, T in POLICY_LAYERS:
            lay = _with_policy(base, policy)
            B = 2
            W, Q, K, V = _case(lay, T, B=B, seed=20 + policy)
            o, log = oracle.Oracle(lay, B, W, lib).run(Q, K, V, log=True)
            rep = replay_selection(lay, W, K, V, T, Q=Q)
            for b in range(B):
                for g in range(lay.n_kv_heads):
                    for c, st in enumerate(rep[b][g][:-1]):
                        nU = int(log["n_cand"][b, g, c])
                        pos = [int(p) for p in log["cand_pos"][b, g, c, :nU]]
                        assert sorted(pos) == sorted(st["U"]), (policy, b, g, c)
                        got = dict(zip(pos, log["cand_sre"][b, g, c, :nU]))
                        for u, x in zip(st["U"], st["sre"]):
                            assert abs(got[u] - x) <= 1e-9 * max(1.0, abs(x)), (policy, b, g, c, u, got[u], x)
                        kept = set(int(p) for p in log["own_kept"][b, g, c] if p >= 0)
                        assert kept == st["keep"], (policy, b, g, c, kept, st["keep"])
            ref = brute_outputs(lay, W, Q, K, V, cache_sets_from_log(log, B, lay.n_kv_heads))
            np.testing.assert_allclose(o, ref, rtol=1e-10, atol=1e-12)


def check_fifo_closed_form(lib):
    """FIFO: after the interval [a, e) the cache holds exactly the C most recent
    positions that have left the window, [max(0, e-w-C), e-w), and the state holds
    every older pair."""
    lay = _with_policy(LayerConfig(2, 2, 8, 3, 3, 4, 5, "f32"), 2)
    T = 41
    W, Q, K, V = _case(lay, T, seed=31)
    orc = oracle.Oracle(lay, 1, W, lib)
    for a in range(0, T, lay.chunk):
        e = min(a + lay.chunk, T)
        orc.run(Q[:, a:e], K[:, a:e], V[:, a:e])
        hi = e - lay.window
        want = list(range(max(0, hi - lay.cache_cap), max(0, hi)))
        for g in range(2):
            ch = orc.chain(0, g)
            assert ch["cache_pos"].tolist() == want, (a, g, ch["cache_pos"].tolist(), want)
            old = list(range(0, max(0, hi - lay.cache_cap)))
            pk = phi_rows(W[g], K[0, old, g]) if old else np.zeros((0, 6))
            np.testing.assert_allclose(ch["H"], pk.T @ V[0, old, g] if old else 0 * ch["H"], atol=1e-12)


def check_attn_one_head_is_top_dot(lib):
    """Attention-weight scorer with one query head per KV head: softmax is monotone, so
    the kept set is the C candidates with the largest q.k for the interval's last query
    (older position first on a tie)."""
    lay = _with_policy(LayerConfig(2, 2, 8, 3, 3, 3, 4, "f32"), 3)
    T = 33
    W, Q, K, V = _case(lay, T, seed=32)
    _, log = oracle.Oracle(lay, 1, W, lib).run(Q, K, V, log=True)
    for g in range(2):
        for c in range(log["n_cand"].shape[2]):
            nU = int(log["n_cand"][0, g, c])
            if nU <= lay.cache_cap:
                continue
            pos = [int(p) for p in log["cand_pos"][0, g, c, :nU]]
            e = min((c + 1) * lay.chunk, T)
            dots = K[0, pos, g] @ Q[0, e - 1, g]
            order = sorted(range(nU), key=lambda i: (-dots[i], pos[i]))
            want = set(pos[i] for i in order[: lay.cache_cap])
            kept = set(int(p) for p in log["own_kept"][0, g, c] if p >= 0)
            assert kept == want, (g, c)


def check_kerr_constant_features(lib):
    """Softmax-approximation-error scorer with W = 0: every feature vector is the same,
    so the linear weight of each candidate is 1/|U| and the score is
    sum_h |softmax weight - 1/|U||."""
    lay = _with_policy(LayerConfig(4, 2, 8, 3, 3, 3, 4, "f32"), 4)
    T = 30
    _, Q, K, V = _case(lay, T, seed=33)
    W = np.zeros((2, 3, 8))
    _, log = oracle.Oracle(lay, 1, W, lib).run(Q, K, V, log=True)
    G = lay.group
    for g in range(2):
        for c in range(log["n_cand"].shape[2]):
            nU = int(log["n_cand"][0, g, c])
            if nU == 0:
                continue
            pos = [int(p) for p in log["cand_pos"][0, g, c, :nU]]
            e = min((c + 1) * lay.chunk, T)
            want = np.zeros(nU)
            for h in range(g * G, (g + 1) * G):
                p = scipy.special.softmax(lay.scale * (K[0, pos, g] @ Q[0, e - 1, h]))
                want += np.abs(p - 1.0 / nU)
            np.testing.assert_allclose(log["cand_sre"][0, g, c, :nU], want, rtol=1e-12, atol=1e-15)


def check_stale_scores_never_change(lib):
    """Stale-score min-heap: the score logged for a cached pair in every later interval
    is the SRE it had in the interval in which it left the window."""
    lay = _with_policy(LayerConfig(2, 1, 8, 3, 2, 3, 3, "f32"), 1)
    T = 45
    W, Q, K, V = _case(lay, T, seed=34)
    _, log = oracle.Oracle(lay, 1, W, lib).run(Q, K, V, log=True)
    first = {}
    for c in range(log["n_cand"].shape[2]):
        nU = int(log["n_cand"][0, 0, c])
        for p, x in zip(log["cand_pos"][0, 0, c, :nU], log["cand_sre"][0, 0, c, :nU]):
            p = int(p)
            if p in first:
                assert x == first[p], (c, p)
            else:
                first[p] = x
    assert len(first) > lay.cache_cap + 5


def check_conservation(lib):
    """1^T s = 2 * folded count, column sums of H = 2 * sum of folded values,
    and window + cache + folded counts add up to the tokens seen."""
    layer = LayerConfig(2, 2, 8, 3, 4, 3, 5, "f32")
    T = 53
    W, Q, K, V = _case(layer, T, seed=8)
    orc = oracle.Oracle(layer, 1, W, lib)
    orc.run(Q, K, V, want_out=False)
    for g in range(2):
        ch = orc.chain(0, g)
        assert ch["win_n"] + ch["cache_n"] + ch["n_folded"] == T
        assert list(ch["win_pos"]) == list(range(T - layer.window, T))
        held = set(ch["win_pos"].tolist()) | set(ch["cache_pos"].tolist())
        folded = [j for j in range(T) if j not in held]
        assert len(folded) == ch["n_folded"]
        assert abs(ch["s"].sum() - 2 * len(folded)) < 1e-11
        np.testing.assert_allclose(ch["H"].sum(0), 2 * V[0, folded, g].sum(0), rtol=1e-11, atol=1e-11)
        np.testing.assert_array_equal(ch["cache_k"], K[0, ch["cache_pos"], g])
        np.testing.assert_array_equal(ch["cache_v"], V[0, ch["cache_pos"], g])


def check_kept_outrank_folded(lib):
    """In every interval the kept scores are at least every folded score."""
    layer = LayerConfig(2, 1, 16, 4, 3, 4, 6, "f32")
    T = 60
    W, Q, K, V = _case(layer, T, seed=9)
    _, log = oracle.Oracle(layer, 1, W, lib).run(Q, K, V, want_out=False, log=True)
    for c in range(log["n_cand"].shape[2]):
        nU = int(log["n_cand"][0, 0, c])
        pos = log["cand_pos"][0, 0, c, :nU]
        e = log["cand_sre"][0, 0, c, :nU]
        kept = set(int(p) for p in log["own_kept"][0, 0, c] if p >= 0)
        assert len(kept) == min(layer.cache_cap, nU)
        ke = [x for p, x in zip(pos, e) if int(p) in kept]
        fe = [x for p, x in zip(pos, e) if int(p) not in kept]
        if ke and fe:
            assert min(ke) >= max(fe)


def check_tie_order(lib):
    """Exact ties (every value equal, one-entry feature halves so phi is constant):
    the kept set is the oldest candidates (reading: the older pair wins a tie)."""
    layer = LayerConfig(1, 1, 2, 1, 1, 2, 3, "f32")
    T = 14
    rng = np.random.default_rng(12)
    W = rng.standard_normal((1, 1, 2))
    K = rng.standard_normal((1, T, 1, 2))
    V = np.ones((1, T, 1, 2))
    _, log = oracle.Oracle(layer, 1, W, lib).run(None, K, V, want_out=False, log=True)
    for c in range(log["n_cand"].shape[2]):
        nU = int(log["n_cand"][0, 0, c])
        pos = sorted(int(p) for p in log["cand_pos"][0, 0, c, :nU])
        kept = sorted(int(p) for p in log["own_kept"][0, 0, c] if p >= 0)
        assert kept == pos[: layer.cache_cap], (c, pos, kept)


def check_split_and_step_equivalence(lib):
    """Two calls (first a whole number of intervals) equal one call; T one-token
    calls equal one call with one-token intervals; a clone continues identically."""
    layer = LayerConfig(2, 1, 8, 3, 3, 2, 4, "f32")
    T, n1 = 30, 12
    W, Q, K, V = _case(layer, T, seed=10)
    one = oracle.Oracle(layer, 1, W, lib)
    o_ref, _ = one.run(Q, K, V)
    two = oracle.Oracle(layer, 1, W, lib)
    o1, _ = two.run(Q[:, :n1], K[:, :n1], V[:, :n1])
    cl = two.clone()
    o2, _ = two.run(Q[:, n1:], K[:, n1:], V[:, n1:])
    o3, _ = cl.run(Q[:, n1:], K[:, n1:], V[:, n1:])
    np.testing.assert_array_equal(np.concatenate([o1, o2], axis=1), o_ref)
    np.testing.assert_array_equal(o3, o2)
    np.testing.assert_array_equal(two.chain(0, 0)["H"], one.chain(0, 0)["H"])

    lay1 = LayerConfig(2, 1, 8, 3, 3, 2, 1, "f32")
    ref1, _ = oracle.Oracle(lay1, 1, W, lib).run(Q, K, V)
    dec = oracle.Oracle(layer, 1, W, lib)  # interval length 4, fed one token per call
    outs = [dec.run(Q[:, t:t + 1], K[:, t:t + 1], V[:, t:t + 1])[0] for t in range(T)]
    np.testing.assert_array_equal(np.concatenate(outs, axis=1), ref1)


def check_golden_hand_trajectory(lib):
    """Hand-worked 4-token trajectory (tests/golden/hand_trajectory.json)."""
    with open(os.path.join(GOLDEN, "hand_trajectory.json")) as f:
        gold = json.load(f)
    for case in gold["cases"]:
        lay = LayerConfig(1, 1, 2, 1, 1, 1, 1, "f32", softmax_scale=1.0)
        W = np.array(gold["W"], np.float64).reshape(1, 1, 2)
        Q = np.array(case["q"], np.float64).reshape(1, 4, 1, 2)
        K = np.array(case["k"], np.float64).reshape(1, 4, 1, 2)
        V = np.array(gold["v"], np.float64).reshape(1, 4, 1, 2)
        orc = oracle.Oracle(lay, 1, W, lib)
        outs, sres, kept = [], [], []
        for t in range(4):
            o, log = orc.run(Q[:, t:t + 1], K[:, t:t + 1], V[:, t:t + 1], log=True)
            outs.append(o[0, 0, 0])
            nU = int(log["n_cand"][0, 0, 0])
            sres.append(sorted(zip(log["cand_pos"][0, 0, 0, :nU].tolist(), log["cand_sre"][0, 0, 0, :nU].tolist())))
            kept.append([int(p) for p in log["own_kept"][0, 0, 0] if p >= 0])
        exp_out = [[eval_frac(x) for x in row] for row in case["out"]]
        np.testing.assert_allclose(np.array(outs), np.array(exp_out), rtol=1e-13, atol=1e-14)
        for got, want in zip(sres, gold["sre"]):
            assert [p for p, _ in got] == [p for p, _ in want]
            np.testing.assert_allclose([e for _, e in got], [e for _, e in want], rtol=1e-13)
        assert kept == gold["kept"]
        ch = orc.chain(0, 0)
        np.testing.assert_allclose(ch["H"], np.array(gold["H_final"], np.float64), atol=1e-13)
        np.testing.assert_allclose(ch["s"], np.array(gold["s_final"], np.float64), atol=1e-13)
        assert ch["cache_pos"].tolist() == gold["cache_final"]
        assert ch["win_pos"].tolist() == gold["window_final"]


def eval_frac(x):
    if isinstance(x, str):
        n, d = x.split("/")
        return float(n) / float(d)
    return float(x)


ALL_CHECKS = [
    check_phi,
    check_sre_closed_forms,
    check_full_window_is_causal_softmax,
    check_no_window_no_cache_is_linear_attention,
    check_no_cache_independent_of_interval,
    check_per_key_weights,
    check_selection_replay,
    check_forced_selection,
    check_policy_replay,
    check_fifo_closed_form,
    check_attn_one_head_is_top_dot,
    check_kerr_constant_features,
    check_stale_scores_never_change,
    check_conservation,
    check_kept_outrank_folded,
    check_tie_order,
    check_split_and_step_equivalence,
    check_golden_hand_trajectory,
]
