"""Incremental decode scores (decode_mode = LOLA_DECODE_INCREMENTAL, include/lola.h):
the state keeps n = H^T phi(k) and d = s . phi(k) per cached pair and each decode
step updates them with the one folded pair instead of rescoring the cache.  The
result is the method's (needs an MI355X):

  * stepped against the oracle: kept sets under the selection rule, outputs and
    H, s within the bf16 tolerance, across prefill calls that mark the stored
    scores stale in between decode steps;
  * against the rescoring step on the same history: the same cache positions at
    every step and, since the victims agree, bit-identical outputs, H and s (only
    the scores of the cached pairs are computed differently);
  * on a planted near-margin eviction (margins in [2e-5, 1e-4]).
"""
import numpy as np
import pytest
import torch

from sparse_attention_chunkwise_amd import inputs as I
from sparse_attention_chunkwise_amd import lola
from tests.gpu_harness import Stepper, dev, host, min_margin, row_rel_err, tol_for

pytestmark = pytest.mark.gpu


def _inc(layer, mode=1):
    return I.LayerConfig(layer.n_q_heads, layer.n_kv_heads, layer.head_dim, layer.feat_half, layer.window,
                         layer.cache_cap, layer.chunk, layer.io_dtype, layer.softmax_scale, layer.policy, mode)


LAYERS = [
    ("gqa", I.LayerConfig(16, 2, 128, 64, 16, 32, 16, "bf16"), 2, 100, 40),
    ("d64_f128", I.LayerConfig(4, 2, 64, 64, 6, 9, 8, "bf16"), 2, 50, 40),
    ("no_window", I.LayerConfig(4, 1, 128, 64, 0, 12, 8, "bf16"), 2, 40, 30),
    ("cold_start", I.LayerConfig(4, 1, 64, 32, 8, 6, 8, "bf16"), 3, 0, 40),
]


@pytest.mark.parametrize("name,layer,B,T,steps", LAYERS, ids=[x[0] for x in LAYERS])
def test_incremental_decode_against_oracle(name, layer, B, T, steps):
    layer = _inc(layer)
    W, Q, K, V = I.random_case(1300 + len(name), layer, B, T + steps + 12)
    st = Stepper(layer, B, W)
    tol = tol_for(layer)
    for a in range(0, T, layer.chunk):
        e = min(a + layer.chunk, T)
        g, r = st.step(Q[:, a:e], K[:, a:e], V[:, a:e])
        assert row_rel_err(g, r) <= tol
    t = T
    for s in range(steps):
        if s == steps // 2:  # a prefill call in between: the stored scores become stale
            for a in range(t, t + 12, layer.chunk):
                e = min(a + layer.chunk, t + 12)
                g, r = st.step(Q[:, a:e], K[:, a:e], V[:, a:e])
                assert row_rel_err(g, r) <= tol
            t += 12
        g, r = st.step(Q[:, t:t + 1], K[:, t:t + 1], V[:, t:t + 1], decode=True)
        err = row_rel_err(g, r)
        assert err <= tol, f"{name} step {t}: {err:.3g}"
        t += 1
    eh, es = st.compare_state()
    assert eh <= tol and es <= tol
    assert st.healthy()


CMP = [
    ("gqa", I.LayerConfig(16, 2, 128, 64, 16, 32, 16, "bf16"), 2, 100, 60),
    ("decode_workload_shapes", I.WORKLOADS[4].layer, 4, 320, 64),
]


@pytest.mark.parametrize("name,layer,B,T,steps", CMP, ids=[x[0] for x in CMP])
def test_incremental_equals_rescoring(name, layer, B, T, steps):
    W, Q, K, V = I.random_case(1400 + len(name), layer, B, T + steps)
    Wd = torch.from_numpy(W).to("cuda")
    res = {}
    for mode in (0, 1):
        lay = _inc(layer, mode)
        state = lola.init_state(lay, B, Wd)
        lola.prefill(lay, state, dev(Q[:, :T], lay), dev(K[:, :T], lay), dev(V[:, :T], lay))
        outs, sets = [], []
        for t in range(T, T + steps):
            outs.append(lola.decode(lay, state, dev(Q[:, t], lay), dev(K[:, t], lay), dev(V[:, t], lay)))
            sets.append(lola.read_cache(lay, state, B, want_kv=False, want_state=False)["pos"].cpu())
        assert lola.check_state(lay, state, B) == 0
        res[mode] = (outs, sets, lola.read_cache(lay, state, B))
    for s in range(steps):
        assert torch.equal(res[0][1][s], res[1][1][s]), f"{name} step {s}: kept positions differ"
        assert torch.equal(res[0][0][s], res[1][0][s]), f"{name} step {s}: outputs differ"
    for key in ("count", "pos", "k", "v", "H", "s", "tokens_seen"):
        assert torch.equal(res[0][2][key], res[1][2][key]), key


def test_incremental_planted_near_margin():
    """Evictions whose margin is planted in [2e-5, 1e-4]: the stored-score path must
    still evict the oracle's choice."""
    from tests.margin_plant import plant
    layer = _inc(I.LayerConfig(16, 2, 128, 64, 16, 32, 16, "bf16"))
    B, T = 2, 100
    W, Q, K, V = I.random_case(1500, layer, B, T + 8)
    V, _ = plant(layer, W, K, V, B, T + 2, seed=1, decode=True, calls=[T, 1, 1])
    V, _ = plant(layer, W, K, V, B, T + 5, seed=2, decode=True, calls=[T, 1, 1, 1, 1, 1])
    st = Stepper(layer, B, W)
    tol = tol_for(layer)
    out = lola.prefill(layer, st.state, dev(Q[:, :T], layer), dev(K[:, :T], layer), dev(V[:, :T], layer))
    ref, log = st.orc.run(Q[:, :T], K[:, :T], V[:, :T], log=True)
    assert min_margin(log, layer.cache_cap) > 1e-5
    assert row_rel_err(host(out), ref) <= tol
    for t in range(T, T + 8):
        g, r = st.step(Q[:, t:t + 1], K[:, t:t + 1], V[:, t:t + 1], decode=True)
        assert row_rel_err(g, r) <= tol, f"step {t}"
        assert st.forced_count == 0, f"step {t}: a near tie was adopted"
