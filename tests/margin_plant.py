"""Plant selection margins just above the exact-selection threshold.

The parity rule demands the GPU's kept set equal the oracle's wherever the
margin mu = (e(C) - e(C+1)) / e(C) of an interval exceeds 1e-5.  Random inputs
rarely put an interval near that edge, so this module edits inputs until chosen
intervals have mu in a given band (default [2e-5, 1e-4]), using the oracle only.

How: the state at the start of interval c does not depend on the value of a key
that first becomes a candidate in interval c.  So for one such leaving key p
the oracle's scores of every other candidate are fixed, and the key's own
score e_p = || r_p - v_p ||^2, with r_p = H^T phi(k_p) / (s . phi(k_p)) from the
oracle's interval-start state, is set through v_p alone: v_p is placed so that
p sits next to the score now ranked C-th among the others (just above or just
below it), then moved one storage-dtype ulp at a time until the margin falls
in the band.
The final margins are re-read from an oracle run over the edited inputs.
"""
from __future__ import annotations

import numpy as np

import oracle


def _round(x, io):
    x = np.asarray(x, np.float32)
    if io != "bf16":
        return x.astype(np.float64)
    u = x.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def _ulp(x, io):
    """Spacing of the storage dtype at each entry of x."""
    x = np.abs(np.asarray(x, np.float64)) + 1e-30
    bits = 7 if io == "bf16" else 23
    return 2.0 ** (np.floor(np.log2(x)) - bits)


def _margin(e_sorted, C):
    eC, eC1 = e_sorted[C - 1], e_sorted[C]
    return 0.0 if eC == 0 else (eC - eC1) / eC


def plant(layer, W, K, V, B, interval, band=(2e-5, 1e-4), target=5e-5, seed=0, decode=False, calls=None):
    """Edit V (a copy is returned) so that interval `interval` of every chain has its
    selection margin in `band`.  Prefill: intervals of layer.chunk tokens from position
    0, one call.  decode=True: the one-token interval at position `interval` (a decode
    step), after calls of the given sizes (default: one call of `interval` tokens).
    Returns (V_new, margins[b][g])."""
    rng = np.random.default_rng(seed)
    L = layer
    C, w, D = L.cache_cap, L.window, L.head_dim
    V = np.array(V, np.float32, copy=True)
    if decode:
        a, e = interval, interval + 1
    else:
        a, e = interval * L.chunk, min((interval + 1) * L.chunk, K.shape[1])
    calls = list(calls) if calls is not None else ([a] if a > 0 else [])
    assert sum(calls) == a

    def advance(o, VV):
        t = 0
        for n in calls:
            o.run(None, K[:, t:t + n], VV[:, t:t + n], want_out=False)
            t += n

    orc = oracle.Oracle(L, B, W)
    advance(orc, V)
    chains = [[orc.chain(b, g) for g in range(L.n_kv_heads)] for b in range(B)]
    probe = orc.clone()
    _, log = probe.run(None, K[:, a:e], V[:, a:e], want_out=False, log=True)
    margins = [[None] * L.n_kv_heads for _ in range(B)]
    for b in range(B):
        for g in range(L.n_kv_heads):
            nU = int(log["n_cand"][b, g, 0])
            pos = [int(x) for x in log["cand_pos"][b, g, 0, :nU]]
            sre = log["cand_sre"][b, g, 0, :nU]
            leaving = [p for p in pos if p >= a - w]
            assert nU > C and leaving, f"interval {interval} of chain ({b},{g}) does not select"
            # p goes just above the score ranked C-th among the others (then that one
            # ranks C+1-th) or just below it (then p ranks C+1-th): whichever has room
            for p in rng.permutation(leaving):
                p = int(p)
                others = np.sort(np.array([s for q, s in zip(pos, sre) if q != p]))[::-1]
                oC = others[C - 1]
                up = others[C - 2] if C >= 2 else np.inf
                down = others[C] if C < len(others) else 0.0
                if oC * (1.0 + 3 * target) < up:
                    goal, lim = oC * (1.0 + target), (oC, up)
                    break
                if oC * (1.0 - 3 * target) > down:
                    goal, lim = oC * (1.0 - target), (down, oC)
                    break
            else:
                raise AssertionError(f"chain ({b},{g}): no room next to the C-th score")
            ch = chains[b][g]
            ph = oracle.phi(W[g], K[b, p, g])
            den = ph @ ch["s"]
            r = ph @ ch["H"] / den if den > 0 else np.zeros(D)
            u = rng.standard_normal(D)
            u /= np.linalg.norm(u)
            v = _round(r + np.sqrt(goal) * u, L.io_dtype)

            def err(vv):
                return float(((r - vv) ** 2).sum())

            def mu_of(vv):
                ep = err(vv)
                allv = np.sort(np.append(others, ep))[::-1]
                return _margin(allv, C), ep

            mu, ep = mu_of(v)
            for _ in range(4000):
                if band[0] <= mu <= band[1] and lim[0] < ep < lim[1]:
                    break
                # one ulp on the component that moves e_p closest to the goal
                step = _ulp(v, L.io_dtype)
                best = None
                for sgn in (1.0, -1.0):
                    cand = v + sgn * step
                    de = (r - cand) ** 2 - (r - v) ** 2
                    j = int(np.argmin(np.abs(ep + de - goal)))
                    if best is None or abs(ep + de[j] - goal) < best[0]:
                        best = (abs(ep + de[j] - goal), j, cand[j])
                nv = v.copy()
                nv[best[1]] = _round(best[2], L.io_dtype)
                if np.array_equal(nv, v):
                    break
                v = nv
                mu, ep = mu_of(v)
            assert band[0] <= mu <= band[1], f"chain ({b},{g}): could not plant a margin (got {mu:.3g})"
            V[b, p, g] = v.astype(np.float32)
            margins[b][g] = mu
    # re-read from the oracle on the edited inputs
    orc2 = oracle.Oracle(L, B, W)
    advance(orc2, V)
    _, log2 = orc2.run(None, K[:, a:e], V[:, a:e], want_out=False, log=True)
    for b in range(B):
        for g in range(L.n_kv_heads):
            nU = int(log2["n_cand"][b, g, 0])
            es = np.sort(log2["cand_sre"][b, g, 0, :nU])[::-1]
            mu = _margin(es, C)
            assert band[0] <= mu <= band[1], f"chain ({b},{g}): oracle margin {mu:.3g} outside {band}"
            margins[b][g] = mu
    return V, margins
