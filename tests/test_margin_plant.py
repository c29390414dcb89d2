"""The margin planter (tests/margin_plant.py) against the oracle alone: planted
intervals have their selection margin inside the band, every other interval is
unchanged in its candidates, and a plant at one interval leaves earlier ones alone."""
import numpy as np
import pytest

import oracle
from sparse_attention_chunkwise_amd import inputs as I
from tests.margin_plant import plant


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_planted_margins_in_band(io):
    layer = I.LayerConfig(4, 2, 64, 32, 8, 12, 16, io)
    B, T = 2, 160
    W, Q, K, V = I.random_case(61, layer, B, T)
    V2, mus = plant(layer, W, K, V, B, interval=5, seed=3)
    V3, mus2 = plant(layer, W, K, V2, B, interval=8, seed=4)
    for row in mus + mus2:
        for mu in row:
            assert 2e-5 <= mu <= 1e-4
    # only values of keys that leave the window in the planted intervals changed
    changed = np.argwhere(np.any(V3 != V, axis=-1))
    lo5, hi5 = 5 * 16 - 8, 6 * 16 - 8
    lo8, hi8 = 8 * 16 - 8, 9 * 16 - 8
    for b, t, g in changed:
        assert lo5 <= t < hi5 or lo8 <= t < hi8, (b, t, g)
    # both planted margins survive in one run over the final inputs
    _, log = oracle.Oracle(layer, B, W).run(None, K, V3, want_out=False, log=True)
    for c in (5, 8):
        for b in range(B):
            for g in range(layer.n_kv_heads):
                nU = int(log["n_cand"][b, g, c])
                es = np.sort(log["cand_sre"][b, g, c, :nU])[::-1]
                C = layer.cache_cap
                mu = (es[C - 1] - es[C]) / es[C - 1]
                assert 2e-5 <= mu <= 1e-4, (c, b, g, mu)


def test_planted_decode_margin():
    layer = I.LayerConfig(4, 1, 64, 32, 6, 10, 8, "bf16")
    B, T = 2, 60
    W, Q, K, V = I.random_case(62, layer, B, T + 1)
    V2, mus = plant(layer, W, K, V, B, interval=T - 4, seed=5, decode=True)
    V3, mus2 = plant(layer, W, K, V2, B, interval=T - 1, seed=6, decode=True, calls=[T - 4, 1, 1, 1])
    for row in mus + mus2:
        for mu in row:
            assert 2e-5 <= mu <= 1e-4
