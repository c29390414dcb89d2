"""Scoring and cache-policy variants (lola_policy in include/lola.h) on the GPU
against the oracle's readings of them (needs an MI355X): stale-score min-heap,
FIFO, attention-weight magnitude, softmax approximation error.

Each runs interval by interval with the selection rule of the SRE policy (kept
sets equal the oracle's wherever the margin of its scores exceeds 1e-5, else
any set within that margin is adopted), outputs and H, s within the io dtype's
tolerance; one call over the whole sequence equals the stepped run bit for bit;
lola_decode_step rejects these policies (lola_prefill_chunk with one token runs
them)."""
import numpy as np
import pytest
import torch

from sparse_attention_chunkwise_amd import inputs as I
from sparse_attention_chunkwise_amd import lola
from tests.gpu_harness import Stepper, dev, row_rel_err, tol_for

pytestmark = pytest.mark.gpu

POLICIES = {1: "stale", 2: "fifo", 3: "attn", 4: "softmax_err"}


def _layer(base, policy):
    return I.LayerConfig(base.n_q_heads, base.n_kv_heads, base.head_dim, base.feat_half, base.window,
                         base.cache_cap, base.chunk, base.io_dtype, base.softmax_scale, policy)


BASES = [
    ("f32", I.LayerConfig(4, 2, 64, 32, 8, 12, 16, "f32"), 2, 150),
    ("bf16", I.LayerConfig(8, 2, 128, 64, 16, 24, 32, "bf16"), 2, 230),
    ("bf16_interval_1", I.LayerConfig(4, 1, 64, 32, 4, 6, 1, "bf16"), 1, 40),
]
CASES = [(f"{POLICIES[p]}-{n}", _layer(base, p), B, T) for p in POLICIES for (n, base, B, T) in BASES]


@pytest.mark.parametrize("name,layer,B,T", CASES, ids=[c[0] for c in CASES])
def test_policy_stepped(name, layer, B, T):
    W, Q, K, V = I.random_case(600 + len(name), layer, B, T)
    st = Stepper(layer, B, W)
    tol = tol_for(layer)
    for ci, a in enumerate(range(0, T, layer.chunk)):
        e = min(a + layer.chunk, T)
        g, r = st.step(Q[:, a:e], K[:, a:e], V[:, a:e])
        err = row_rel_err(g, r)
        assert err <= tol, f"{name} interval {ci}: output rel err {err:.3g}"
        if ci % 4 == 3 or e == T:
            eh, es = st.compare_state()
            assert eh <= tol and es <= tol, f"{name} interval {ci}: H {eh:.3g} s {es:.3g}"
    assert st.healthy()
    print(f"{name}: near ties adopted {st.forced_count}", flush=True)


@pytest.mark.parametrize("name,layer,B,T", CASES, ids=[c[0] for c in CASES])
def test_policy_one_call_equals_stepped(name, layer, B, T):
    W, Q, K, V = I.random_case(650 + len(name), layer, B, T)
    Wd = torch.from_numpy(W).to("cuda")
    s1, s2 = lola.init_state(layer, B, Wd), lola.init_state(layer, B, Wd)
    o1 = lola.prefill(layer, s1, dev(Q, layer), dev(K, layer), dev(V, layer))
    outs = []
    for a in range(0, T, layer.chunk):
        e = min(a + layer.chunk, T)
        outs.append(lola.prefill(layer, s2, dev(Q[:, a:e], layer), dev(K[:, a:e], layer), dev(V[:, a:e], layer)))
    assert torch.equal(o1, torch.cat(outs, dim=1))
    assert torch.equal(s1, s2)


def test_policy_4k_shapes_attention_weight():
    """The attention-weight scorer at the 4K workload's shapes (32/8 heads, D 128,
    C 256, L 64) over 1024 tokens, interval by interval."""
    layer = _layer(I.WORKLOADS[3].layer, 3)
    W, Q, K, V = I.make_batch(I.WORKLOADS[3], seq_len=1024)
    st = Stepper(layer, 1, W)
    tol = tol_for(layer)
    for a in range(0, 1024, layer.chunk):
        g, r = st.step(Q[:, a:a + layer.chunk], K[:, a:a + layer.chunk], V[:, a:a + layer.chunk])
        assert row_rel_err(g, r) <= tol
    eh, es = st.compare_state()
    assert eh <= tol and es <= tol


@pytest.mark.parametrize("policy", sorted(POLICIES))
def test_decode_step_rejects_policy(policy):
    layer = _layer(BASES[1][1], policy)
    W, Q, K, V = I.random_case(7, layer, 1, 40)
    state = lola.init_state(layer, 1, torch.from_numpy(W).to("cuda"))
    lola.prefill(layer, state, dev(Q, layer), dev(K, layer), dev(V, layer))
    before = state.clone()
    with pytest.raises(lola.LolaError) as ei:
        lola.decode(layer, state, dev(Q[:, -1], layer), dev(K[:, -1], layer), dev(V[:, -1], layer))
    assert ei.value.status == -2
    torch.cuda.synchronize()
    assert torch.equal(state, before)
