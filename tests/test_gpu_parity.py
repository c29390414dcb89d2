"""HIP path against the fp64 oracle, through the C ABI (needs an MI355X)."""
import numpy as np
import pytest
import torch

import oracle
from sparse_attention_chunkwise_amd import inputs as I
from sparse_attention_chunkwise_amd import lola
from tests.gpu_harness import Stepper, dev, fro_rel_err, host, min_margin, row_rel_err, tol_for

pytestmark = pytest.mark.gpu


def _stepped(layer, B, W, Q, K, V, state_every=8, label=""):
    """Whole sequence one interval per call; returns the stepper."""
    st = Stepper(layer, B, W)
    T = K.shape[1]
    tol = tol_for(layer)
    worst = 0.0
    for ci, a in enumerate(range(0, T, layer.chunk)):
        e = min(a + layer.chunk, T)
        g, r = st.step(Q[:, a:e], K[:, a:e], V[:, a:e])
        err = row_rel_err(g, r)
        worst = max(worst, err)
        assert err <= tol, f"{label} interval {ci}: output rel err {err:.3g} > {tol}"
        if state_every and (ci % state_every == state_every - 1 or e == T):
            eh, es = st.compare_state()
            assert eh <= tol and es <= tol, f"{label} interval {ci}: H {eh:.3g} s {es:.3g}"
    assert st.healthy(), f"{label}: state marked faulted"
    print(f"{label}: worst output rel err {worst:.3g}, near ties adopted {st.forced_count}", flush=True)
    return st


def _full(layer, B, W, Q, K, V, calls=None):
    """GPU run as one call (or the given split); returns (out, read_cache dict, state)."""
    state = lola.init_state(layer, B, torch.from_numpy(W).to("cuda"))
    T = K.shape[1]
    calls = calls or [T]
    outs, a = [], 0
    for n in calls:
        outs.append(lola.prefill(layer, state, dev(Q[:, a:a + n], layer), dev(K[:, a:a + n], layer),
                                 dev(V[:, a:a + n], layer)))
        a += n
    out = torch.cat(outs, dim=1)
    assert lola.check_state(layer, state, B) == 0, "state marked faulted"
    return out, lola.read_cache(layer, state, B), state


@pytest.mark.parametrize("cfg", [1, 2])
def test_small_configs_stepped(cfg):
    wl = I.WORKLOADS[cfg]
    W, Q, K, V = I.make_batch(wl)
    _stepped(wl.layer, wl.batch, W, Q, K, V, label=f"cfg{cfg}")


@pytest.mark.parametrize("cfg", [1, 2])
def test_small_configs_one_call(cfg):
    """One call over the whole sequence against the oracle's own trajectory
    (these workloads have no sub-margin tie, so no forcing is needed)."""
    wl = I.WORKLOADS[cfg]
    L = wl.layer
    W, Q, K, V = I.make_batch(wl)
    ref, log = oracle.Oracle(L, wl.batch, W).run(Q, K, V, log=True)
    assert min_margin(log, L.cache_cap) > 1e-5
    out, rc, _ = _full(L, wl.batch, W, Q, K, V)
    tol = tol_for(L)
    assert row_rel_err(host(out), ref) <= tol
    orc = oracle.Oracle(L, wl.batch, W)
    orc.run(Q, K, V, want_out=False)
    for g in range(L.n_kv_heads):
        ch = orc.chain(0, g)
        c = int(rc["count"][0, g])
        assert rc["pos"][0, g, :c].cpu().tolist() == ch["cache_pos"].tolist()
        assert fro_rel_err(host(rc["H"])[0, g], ch["H"]) <= tol
        assert fro_rel_err(host(rc["s"])[0, g], ch["s"]) <= tol


@pytest.mark.parametrize("cfg", [1, 2, 3])
def test_one_call_equals_stepped_bitwise(cfg):
    """A call over many intervals equals the same intervals one call each, bit for bit."""
    wl = I.WORKLOADS[cfg]
    L = wl.layer
    T = 1024 if cfg == 3 else wl.seq_len
    W, Q, K, V = I.make_batch(wl, seq_len=T)
    o1, r1, _ = _full(L, wl.batch, W, Q, K, V)
    o2, r2, _ = _full(L, wl.batch, W, Q, K, V, calls=[L.chunk] * (T // L.chunk))
    assert torch.equal(o1, o2)
    for key in ("count", "pos", "H", "s", "k", "v", "tokens_seen"):
        assert torch.equal(r1[key], r2[key]), key


def test_cfg3_prefill_stepped():
    """4K bf16 GQA prefill, interval by interval with the margin rule."""
    wl = I.WORKLOADS[3]
    W, Q, K, V = I.make_batch(wl)
    _stepped(wl.layer, wl.batch, W, Q, K, V, state_every=16, label="cfg3")


EDGE = [
    # (name, layer, B, T)
    ("no_cache", I.LayerConfig(4, 2, 64, 32, 8, 0, 8, "f32"), 2, 75),
    ("no_window", I.LayerConfig(2, 2, 64, 32, 0, 6, 8, "f32"), 1, 61),
    ("no_window_no_cache", I.LayerConfig(2, 1, 64, 32, 0, 0, 5, "f32"), 1, 40),
    ("interval_1", I.LayerConfig(2, 1, 64, 32, 4, 5, 1, "f32"), 1, 37),
    ("window_beyond_seq", I.LayerConfig(4, 4, 64, 32, 100, 8, 16, "f32"), 1, 70),
    ("cache_beyond_seq", I.LayerConfig(2, 1, 64, 32, 4, 128, 8, "f32"), 1, 90),
    ("interval_longer_than_window", I.LayerConfig(4, 1, 128, 64, 5, 7, 24, "f32"), 2, 101),
    ("d64_f128", I.LayerConfig(2, 1, 64, 64, 6, 9, 10, "f32"), 1, 55),
    ("d128_f64", I.LayerConfig(2, 2, 128, 32, 6, 9, 10, "f32"), 1, 55),
    ("group16", I.LayerConfig(16, 1, 64, 32, 7, 9, 11, "f32"), 1, 50),
    ("bf16_ragged", I.LayerConfig(8, 2, 128, 64, 16, 24, 32, "bf16"), 2, 203),
    ("bf16_d64", I.LayerConfig(4, 4, 64, 32, 8, 12, 16, "bf16"), 1, 130),
    ("max_interval", I.LayerConfig(2, 1, 64, 32, 16, 40, 256, "f32"), 1, 600),
    ("max_cache", I.LayerConfig(2, 1, 64, 32, 8, 1024, 128, "bf16"), 1, 1500),
    # bf16 io runs the scan with each chain spread over head_dim/16 workgroups
    ("bf16_no_window", I.LayerConfig(2, 2, 64, 32, 0, 6, 8, "bf16"), 1, 61),
    ("bf16_no_cache", I.LayerConfig(2, 1, 64, 32, 4, 0, 8, "bf16"), 1, 40),
    ("bf16_interval_1", I.LayerConfig(2, 1, 64, 32, 4, 5, 1, "bf16"), 1, 37),
    ("bf16_cache_beyond_seq", I.LayerConfig(2, 1, 64, 32, 4, 128, 8, "bf16"), 1, 90),
    ("bf16_interval_longer_than_window", I.LayerConfig(4, 1, 128, 64, 5, 7, 24, "bf16"), 2, 101),
    ("bf16_d128_f64", I.LayerConfig(2, 2, 128, 32, 6, 9, 10, "bf16"), 1, 55),
    ("bf16_d64_f128", I.LayerConfig(2, 1, 64, 64, 6, 9, 10, "bf16"), 1, 55),
    ("bf16_twelve_chains", I.LayerConfig(4, 4, 64, 32, 8, 12, 16, "bf16"), 3, 90),
    ("bf16_max_interval", I.LayerConfig(2, 1, 64, 32, 16, 40, 256, "bf16"), 1, 600),
    ("bf16_max_window", I.LayerConfig(2, 1, 64, 32, 8192, 16, 64, "bf16"), 1, 8300),
    ("bf16_group16", I.LayerConfig(16, 1, 64, 32, 7, 9, 11, "bf16"), 1, 50),
    # logits with a spread of tens (scale 2 instead of 1/sqrt(128)): the output pass's
    # softmax reference must move across key blocks, in the window-span blocks and in
    # the cache blocks (64-key blocks: one straddling span and cache, one full cache
    # block, one partial)
    ("bf16_sharp_softmax", I.LayerConfig(8, 2, 128, 64, 16, 96, 32, "bf16", softmax_scale=2.0), 1, 300),
]


@pytest.mark.parametrize("name,layer,B,T", EDGE, ids=[e[0] for e in EDGE])
def test_edge_stepped(name, layer, B, T):
    W, Q, K, V = I.random_case(100 + len(name), layer, B, T)
    _stepped(layer, B, W, Q, K, V, state_every=4, label=name)


ONE_BLOCK = [e for e in EDGE if e[0] in ("bf16_ragged", "bf16_d64", "bf16_max_interval", "bf16_no_cache",
                                          "bf16_sharp_softmax")]


@pytest.mark.parametrize("name,layer,B,T", ONE_BLOCK, ids=[e[0] for e in ONE_BLOCK])
def test_edge_stepped_one_block_scan(name, layer, B, T, monkeypatch):
    """bf16 io with the scan forced to one workgroup per chain (the path large batches take)."""
    monkeypatch.setenv("LOLA_SCAN_SPLIT", "0")
    W, Q, K, V = I.random_case(100 + len(name), layer, B, T)
    _stepped(layer, B, W, Q, K, V, state_every=4, label=name + "/one-block")


# draws whose first seed holds a sub-margin tie in some interval (the comparison
# below would be skipped): another seed of the same shapes
SPLIT_SEED = {"max_cache": 1200 + len("max_cache"), "bf16_twelve_chains": 1200 + len("bf16_twelve_chains")}


@pytest.mark.parametrize("name,layer,B,T", EDGE, ids=[e[0] for e in EDGE])
def test_edge_split_calls(name, layer, B, T):
    """Calls of uneven sizes (each starts its own interval grid) against the oracle."""
    W, Q, K, V = I.random_case(SPLIT_SEED.get(name, 200 + len(name)), layer, B, T)
    cuts = [max(1, T // 3), max(1, T // 5), 1]
    calls = cuts + [T - sum(cuts)]
    orc = oracle.Oracle(layer, B, W)
    refs, logs, a = [], [], 0
    for n in calls:
        r, lg = orc.run(Q[:, a:a + n], K[:, a:a + n], V[:, a:a + n], log=True)
        refs.append(r)
        logs.append(lg)
        a += n
    if min(min_margin(lg, layer.cache_cap) for lg in logs) <= 1e-5:
        pytest.skip("sub-margin tie in this draw; covered by the stepped test")
    out, rc, _ = _full(layer, B, W, Q, K, V, calls=calls)
    tol = tol_for(layer)
    assert row_rel_err(host(out), np.concatenate(refs, axis=1)) <= tol
    for b in range(B):
        for g in range(layer.n_kv_heads):
            ch = orc.chain(b, g)
            c = int(rc["count"][b, g])
            assert rc["pos"][b, g, :c].cpu().tolist() == ch["cache_pos"].tolist()
            assert fro_rel_err(host(rc["H"])[b, g], ch["H"]) <= tol
    assert rc["tokens_seen"].cpu().tolist() == [T] * B


DECODE_EDGE = [
    ("decode_basic", I.LayerConfig(4, 2, 64, 32, 6, 5, 8, "f32"), 2, 40, 30),
    ("decode_no_window", I.LayerConfig(2, 1, 64, 32, 0, 4, 8, "f32"), 1, 20, 20),
    ("decode_no_cache", I.LayerConfig(2, 2, 128, 64, 5, 0, 4, "f32"), 1, 20, 20),
    ("decode_cold_start", I.LayerConfig(4, 1, 64, 32, 8, 6, 8, "bf16"), 3, 0, 40),
    ("decode_bf16_group16", I.LayerConfig(16, 1, 128, 64, 8, 12, 16, "bf16"), 2, 60, 20),
    ("decode_bf16_gqa", I.LayerConfig(16, 2, 128, 64, 16, 32, 16, "bf16"), 2, 100, 24),
]


@pytest.mark.parametrize("name,layer,B,T,steps", DECODE_EDGE, ids=[e[0] for e in DECODE_EDGE])
def test_decode_steps(name, layer, B, T, steps):
    W, Q, K, V = I.random_case(300 + len(name), layer, B, T + steps)
    st = Stepper(layer, B, W)
    tol = tol_for(layer)
    for a in range(0, T, layer.chunk):
        e = min(a + layer.chunk, T)
        g, r = st.step(Q[:, a:e], K[:, a:e], V[:, a:e])
        assert row_rel_err(g, r) <= tol
    for t in range(T, T + steps):
        g, r = st.step(Q[:, t:t + 1], K[:, t:t + 1], V[:, t:t + 1], decode=True)
        err = row_rel_err(g, r)
        assert err <= tol, f"{name} step {t}: {err:.3g}"
    eh, es = st.compare_state()
    assert eh <= tol and es <= tol


def test_decode_after_one_block_scan(monkeypatch):
    """Decode steps on a state prefilled by the one-workgroup bf16 scan: its state-out
    must also leave the cached keys' feature rows that a decode step scores with."""
    name, layer, B, T, steps = DECODE_EDGE[-1]
    W, Q, K, V = I.random_case(500 + len(name), layer, B, T + steps)
    st = Stepper(layer, B, W)
    tol = tol_for(layer)
    monkeypatch.setenv("LOLA_SCAN_SPLIT", "0")
    for a in range(0, T, layer.chunk):
        e = min(a + layer.chunk, T)
        g, r = st.step(Q[:, a:e], K[:, a:e], V[:, a:e])
        assert row_rel_err(g, r) <= tol
    monkeypatch.delenv("LOLA_SCAN_SPLIT")
    for t in range(T, T + steps):
        g, r = st.step(Q[:, t:t + 1], K[:, t:t + 1], V[:, t:t + 1], decode=True)
        err = row_rel_err(g, r)
        assert err <= tol, f"{name} one-block prefill, decode step {t}: {err:.3g}"
    eh, es = st.compare_state()
    assert eh <= tol and es <= tol


def test_decode_equals_one_token_prefill():
    """lola_decode_step and lola_prefill_chunk(n=1) agree on outputs and state."""
    layer = I.LayerConfig(8, 2, 128, 64, 16, 24, 32, "bf16")
    B, T = 2, 150
    W, Q, K, V = I.random_case(77, layer, B, T + 20)
    sa = lola.init_state(layer, B, torch.from_numpy(W).to("cuda"))
    sb = lola.init_state(layer, B, torch.from_numpy(W).to("cuda"))
    for s in (sa, sb):
        lola.prefill(layer, s, dev(Q[:, :T], layer), dev(K[:, :T], layer), dev(V[:, :T], layer))
    for t in range(T, T + 20):
        oa = lola.decode(layer, sa, dev(Q[:, t], layer), dev(K[:, t], layer), dev(V[:, t], layer))
        ob = lola.prefill(layer, sb, dev(Q[:, t:t + 1], layer), dev(K[:, t:t + 1], layer), dev(V[:, t:t + 1], layer))
        assert row_rel_err(host(oa), host(ob)[:, 0]) <= 2e-2
    ra, rb = lola.read_cache(layer, sa, B), lola.read_cache(layer, sb, B)
    assert torch.equal(ra["pos"], rb["pos"]) and torch.equal(ra["k"], rb["k"])
    assert fro_rel_err(host(ra["H"]), host(rb["H"])) <= 1e-5


def test_cfg4_decode_shapes():
    """The decode workload's trajectory: 4 of its 64 sequences, the 4096-token prefill
    interval by interval (state only on the oracle side), then all 256 decode steps the
    benchmark times, each step's outputs, kept sets (selection rule) and, every 32
    steps, H and s against the oracle."""
    wl = I.WORKLOADS[4]
    L = wl.layer
    B, steps = 4, 256
    W, Q, K, V = I.make_batch(wl, batch=B)
    qd, kd, vd = I.make_decode_steps(wl, steps, batch=B)
    st = Stepper(L, B, W)
    tol = tol_for(L)
    for a in range(0, wl.seq_len, L.chunk):
        st.step(Q[:, a:a + L.chunk], K[:, a:a + L.chunk], V[:, a:a + L.chunk],
                row_mask=np.zeros(L.chunk, np.uint8))
    print(f"cfg4: prefill done, {st.forced_count} near ties adopted", flush=True)
    worst = 0.0
    for s in range(steps):
        g, r = st.step(qd[s][:, None], kd[s][:, None], vd[s][:, None], decode=True)
        err = row_rel_err(g, r)
        worst = max(worst, err)
        assert err <= tol, f"decode step {s}: output rel err {err:.3g}"
        if s % 32 == 31:
            eh, es = st.compare_state()
            assert eh <= tol and es <= tol, f"decode step {s}: H {eh:.3g} s {es:.3g}"
    assert st.healthy()
    print(f"cfg4: {steps} decode steps, worst rel err {worst:.3g}, forced {st.forced_count}", flush=True)


def test_state_errors():
    layer = I.LayerConfig(2, 1, 64, 32, 4, 4, 4, "f32")
    W = np.zeros((1, 32, 64), np.float32)
    st = lola.init_state(layer, 2, torch.from_numpy(W).to("cuda"))
    assert lola.check_state(layer, st, 2) == 0
    assert lola.check_state(layer, st, 3) == -3
    other = I.LayerConfig(2, 1, 64, 32, 5, 4, 4, "f32")
    assert lola.check_state(other, st, 2) == -3
    junk = torch.zeros_like(st)
    assert lola.check_state(layer, junk, 2) == -3
    q = torch.zeros((2, 8, 2, 64), device="cuda")
    k = torch.zeros((2, 8, 1, 64), device="cuda")
    small = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(lola.LolaError) as ei:
        lola.prefill(layer, st, q, k, k, workspace=small)
    assert ei.value.status == -4


def test_determinism():
    """Two runs on fresh states give identical bits (no races in LDS or slot updates)."""
    wl = I.WORKLOADS[3]
    W, Q, K, V = I.make_batch(wl, seq_len=1024)
    o1, r1, _ = _full(wl.layer, 1, W, Q, K, V)
    o2, r2, _ = _full(wl.layer, 1, W, Q, K, V)
    assert torch.equal(o1, o2) and torch.equal(r1["H"], r2["H"]) and torch.equal(r1["pos"], r2["pos"])


def test_cfg5_long_context_sampled():
    """64K-token bf16 prefill (4 sequences, cache 512, interval 128, clustered keys
    with 5% needles) at full size.  The whole sequence in one call (as the bench
    runs a prefill) equals the same intervals one call each, bit for bit.  The
    stepped run's kept sets of every interval of all 32 chains are then given to
    the oracle in one state-and-sampled-rows run (teacher forcing): every set must
    satisfy the selection rule against the oracle's own scores, 4 sampled token
    rows of every interval must match in every head, and the final H, s and cache
    of every chain must match."""
    from tests.gpu_harness import check_selection
    wl = I.WORKLOADS[5]
    L = wl.layer
    B, T, C = wl.batch, wl.seq_len, wl.layer.cache_cap
    NI = T // L.chunk
    W, Q, K, V = I.make_batch(wl)
    Wd = torch.from_numpy(W).to("cuda")
    # one call over the whole sequence
    s_one = lola.init_state(L, B, Wd)
    out_one = lola.prefill(L, s_one, dev(Q, L), dev(K, L), dev(V, L))
    assert lola.check_state(L, s_one, B) == 0
    # interval by interval, recording each interval's kept sets and the sampled rows
    rng = np.random.Generator(np.random.PCG64(5005))
    rows = np.zeros(T, np.uint8)
    forced = np.full((B, L.n_kv_heads, NI, C), -1, np.int64)
    state = lola.init_state(L, B, Wd)
    for ci in range(NI):
        a, e = ci * L.chunk, (ci + 1) * L.chunk
        rows[a + rng.choice(e - a, size=4, replace=False)] = 1
        o = lola.prefill(L, state, dev(Q[:, a:e], L), dev(K[:, a:e], L), dev(V[:, a:e], L))
        assert torch.equal(out_one[:, a:e], o), f"interval {ci}: one call differs from stepped"
        rc = lola.read_cache(L, state, B, want_kv=False, want_state=False)
        cnt, pos = rc["count"].cpu().numpy(), rc["pos"].cpu().numpy()
        for b in range(B):
            for g in range(L.n_kv_heads):
                forced[b, g, ci, :cnt[b, g]] = pos[b, g, :cnt[b, g]]
        if ci % 64 == 63:
            print(f"cfg5: GPU interval {ci}", flush=True)
    assert lola.check_state(L, state, B) == 0
    r1, r2 = lola.read_cache(L, s_one, B), lola.read_cache(L, state, B)
    for key in ("count", "pos", "k", "v", "H", "s", "tokens_seen"):
        assert torch.equal(r1[key], r2[key]), key
    # the oracle over all 32 chains in one call, adopting the GPU's sets
    orc = oracle.Oracle(L, B, W)
    ref, log = orc.run(Q, K, V, forced=forced, log=True, row_mask=rows)
    print("cfg5: oracle done", flush=True)
    adopted = 0
    for b in range(B):
        for g in range(L.n_kv_heads):
            for ci in range(NI):
                gset = [int(p) for p in forced[b, g, ci] if p >= 0]
                ok, fc, txt = check_selection(log, b, g, ci, gset, C)
                assert ok, f"chain ({b},{g}) interval {ci}: {txt}"
                adopted += int(fc)
    sel = np.flatnonzero(rows)
    g_out = host(out_one[:, sel])
    err = row_rel_err(g_out, ref[:, sel])
    tol = tol_for(L)
    assert err <= tol, f"sampled rows: output rel err {err:.3g}"
    H, S = host(r1["H"]), host(r1["s"])
    Kc, Vc, cnt = host(r1["k"]), host(r1["v"]), r1["count"].cpu().numpy()
    eh = es = 0.0
    for b in range(B):
        for g in range(L.n_kv_heads):
            ch = orc.chain(b, g)
            eh = max(eh, fro_rel_err(H[b, g], ch["H"]))
            es = max(es, fro_rel_err(S[b, g], ch["s"]))
            c = int(cnt[b, g])
            assert c == ch["cache_n"]
            assert r1["pos"][b, g, :c].cpu().tolist() == ch["cache_pos"].tolist()
            np.testing.assert_array_equal(Kc[b, g, :c], ch["cache_k"])
            np.testing.assert_array_equal(Vc[b, g, :c], ch["cache_v"])
    assert eh <= tol and es <= tol, (eh, es)
    print(f"cfg5: all 32 chains, sampled output rel err {err:.3g}, H {eh:.3g}, s {es:.3g}, "
          f"near ties adopted {adopted}", flush=True)


NEAR_MARGIN = [
    # (name, layer, B, T, planted intervals, one-workgroup scan)
    ("bf16_split", I.LayerConfig(8, 4, 128, 64, 16, 32, 32, "bf16"), 2, 320, (4, 7), False),
    ("bf16_one_block", I.LayerConfig(8, 4, 128, 64, 16, 32, 32, "bf16"), 2, 320, (4, 7), True),
    ("bf16_4k_shapes", I.WORKLOADS[3].layer, 1, 1024, (6, 11), False),
    ("f32", I.LayerConfig(4, 2, 64, 32, 8, 12, 16, "f32"), 2, 192, (5, 9), False),
]


@pytest.mark.parametrize("name,layer,B,T,planted,one_block", NEAR_MARGIN, ids=[x[0] for x in NEAR_MARGIN])
def test_planted_near_margin(name, layer, B, T, planted, one_block, monkeypatch):
    """Intervals whose selection margin is planted in [2e-5, 1e-4] on every chain (just
    above the 1e-5 edge of the exact-selection rule, where the 16-bit operand splits of
    the SRE contraction are tightest): the GPU's kept sets must equal the oracle's."""
    from tests.margin_plant import plant
    if one_block:
        monkeypatch.setenv("LOLA_SCAN_SPLIT", "0")
    W, Q, K, V = I.random_case(700 + len(name), layer, B, T)
    for i, c in enumerate(planted):
        V, mus = plant(layer, W, K, V, B, c, seed=i)
        print(f"{name}: interval {c} margins {min(min(r) for r in mus):.3g}..{max(max(r) for r in mus):.3g}",
              flush=True)
    st = Stepper(layer, B, W)
    tol = tol_for(layer)
    for ci, a in enumerate(range(0, T, layer.chunk)):
        e = min(a + layer.chunk, T)
        g, r = st.step(Q[:, a:e], K[:, a:e], V[:, a:e])
        assert row_rel_err(g, r) <= tol, f"interval {ci}"
        if ci <= max(planted):
            assert st.forced_count == 0, f"interval {ci}: a near tie was adopted before a planted interval"
    eh, es = st.compare_state()
    assert eh <= tol and es <= tol


DECODE_MARGIN = [
    ("bf16", I.LayerConfig(16, 2, 128, 64, 16, 32, 16, "bf16"), 2, 100),
    ("f32", I.LayerConfig(4, 2, 64, 32, 6, 5, 8, "f32"), 2, 40),
]


@pytest.mark.parametrize("name,layer,B,T", DECODE_MARGIN, ids=[x[0] for x in DECODE_MARGIN])
def test_planted_near_margin_decode(name, layer, B, T):
    """Decode steps whose eviction margin is planted in [2e-5, 1e-4] on every chain."""
    from tests.margin_plant import plant
    W, Q, K, V = I.random_case(800 + len(name), layer, B, T + 6)
    V, _ = plant(layer, W, K, V, B, T, seed=1, decode=True)
    V, _ = plant(layer, W, K, V, B, T + 3, seed=2, decode=True, calls=[T, 1, 1, 1])
    st = Stepper(layer, B, W)
    tol = tol_for(layer)
    # the prefix as one call, as the planter assumed; it holds no sub-margin tie, so the
    # oracle follows its own choices and the two sides must hold the same cache after it
    out = lola.prefill(layer, st.state, dev(Q[:, :T], layer), dev(K[:, :T], layer), dev(V[:, :T], layer))
    ref, log = st.orc.run(Q[:, :T], K[:, :T], V[:, :T], log=True)
    assert min_margin(log, layer.cache_cap) > 1e-5
    assert row_rel_err(host(out), ref) <= tol
    sets = st.gpu_cache_sets()
    for b in range(B):
        for g in range(layer.n_kv_heads):
            assert sets[b][g] == st.orc.chain(b, g)["cache_pos"].tolist()
    for t in range(T, T + 6):
        g, r = st.step(Q[:, t:t + 1], K[:, t:t + 1], V[:, t:t + 1], decode=True)
        assert row_rel_err(g, r) <= tol, f"step {t}"
        assert st.forced_count == 0, f"step {t}: a near tie was adopted"
    eh, es = st.compare_state()
    assert eh <= tol and es <= tol


RAGGED = [
    ("bf16_split", I.LayerConfig(8, 2, 128, 64, 16, 24, 32, "bf16"), True),
    ("bf16_one_block", I.LayerConfig(8, 2, 128, 64, 16, 24, 32, "bf16"), False),
    ("f32", I.LayerConfig(4, 2, 64, 32, 16, 16, 16, "f32"), True),
]


@pytest.mark.parametrize("name,layer,split", RAGGED, ids=[r[0] for r in RAGGED])
def test_ragged_mixed_batch(name, layer, split, monkeypatch):
    """lola_prefill_ragged: in one call each sequence advances by its own count (a
    prefill chunk, one token, none).  Bitwise equal to lola_prefill_chunk on each
    sequence alone; within tolerance of the oracle (selection rule per interval);
    rows past a sequence's count are not written; 0 tokens leaves a sequence as is."""
    from tests.gpu_harness import check_selection
    if not split:
        monkeypatch.setenv("LOLA_SCAN_SPLIT", "0")
    L, B, C = layer.chunk, 3, layer.cache_cap
    rounds = [[L, 1, 0], [7, L, 1], [0, 5, L], [L, L, L], [1, 0, L - 3], [3 * L + 5, 2 * L, 0]]
    total = [sum(r[b] for r in rounds) for b in range(B)]
    W, Q, K, V = I.random_case(900 + len(name), layer, B, max(total))
    Wd = torch.from_numpy(W).to("cuda")
    rag = lola.init_state(layer, B, Wd)
    singles = [lola.init_state(layer, 1, Wd) for _ in range(B)]
    orcs = [oracle.Oracle(layer, 1, W) for _ in range(B)]
    tol = tol_for(layer)
    at = [0] * B
    for ri, counts in enumerate(rounds):
        m = max(counts)
        seg = [(Q[b, at[b]:at[b] + counts[b]], K[b, at[b]:at[b] + counts[b]], V[b, at[b]:at[b] + counts[b]])
               for b in range(B)]

        def padded(i):
            X = (Q, K, V)[i]
            P = np.zeros((B, m) + X.shape[2:], np.float32)
            for b in range(B):
                P[b, :counts[b]] = seg[b][i]
            return dev(P, layer)

        print(f"{name} round {ri}: counts {counts}", flush=True)
        n_dev = torch.tensor(counts, dtype=torch.int32, device="cuda")
        out = dev(np.full((B, m, layer.n_q_heads, layer.head_dim), 7.0, np.float32), layer)
        lola.prefill_ragged(layer, rag, n_dev, padded(0), padded(1), padded(2), out=out)
        rc = lola.read_cache(layer, rag, B, want_kv=False, want_state=False)
        for b in range(B):
            n = counts[b]
            assert bool(torch.all(out[b, n:] == 7.0)), f"round {ri}: rows past {n} of sequence {b} written"
            if n == 0:
                continue
            o1 = lola.prefill(layer, singles[b], dev(seg[b][0][None], layer), dev(seg[b][1][None], layer),
                              dev(seg[b][2][None], layer))
            assert torch.equal(out[b, :n], o1[0]), f"round {ri}: sequence {b} differs from its own call"
            if m > L:
                continue  # several intervals in one call: no per-interval cache sets to check against
            forced = np.full((1, layer.n_kv_heads, 1, max(C, 1)), -1, np.int64)
            sets = []
            for g in range(layer.n_kv_heads):
                s = [int(p) for p in rc["pos"][b, g, : int(rc["count"][b, g])].cpu().numpy()] if C > 0 else []
                forced[0, g, 0, : len(s)] = s
                sets.append(s)
            ref, log = orcs[b].run(seg[b][0][None], seg[b][1][None], seg[b][2][None], log=True,
                                   forced=forced if C > 0 else None)
            for g in range(layer.n_kv_heads):
                ok, _, txt = check_selection(log, 0, g, 0, sets[g], C)
                assert ok, f"round {ri} chain ({b},{g}): {txt}"
            err = row_rel_err(host(out[b:b + 1, :n]), ref)
            assert err <= tol, f"round {ri} sequence {b}: output rel err {err:.3g}"
        at = [at[b] + counts[b] for b in range(B)]
    assert lola.check_state(layer, rag, B) == 0
    ra = lola.read_cache(layer, rag, B)
    assert ra["tokens_seen"].cpu().tolist() == total
    for b in range(B):
        rb = lola.read_cache(layer, singles[b], 1)
        for key in ("count", "pos", "k", "v", "H", "s", "tokens_seen"):
            assert torch.equal(ra[key][b:b + 1], rb[key]), f"sequence {b}: {key} differs from its own calls"


def test_ragged_mixed_batch_decode_shapes(monkeypatch):
    """The mixed-batch launch that bench.py times: the decode workload's layer over 64
    sequences (512 chains, past what the split scan holds at once, so the one-workgroup
    scan runs), each prefilled with 320 tokens (window and cache full), then one
    lola_prefill_ragged call in which sequences 8..15 take 64 tokens and the rest one.
    Sampled sequences equal their own calls bitwise (the one-sequence states are forced
    onto the same one-workgroup scan: the split scan folds with other rounding); two
    follow the oracle."""
    monkeypatch.setenv("LOLA_SCAN_SPLIT", "0")
    wl = I.WORKLOADS[4]
    layer, B, T0, m = wl.layer, wl.batch, 320, 64
    W, Q, K, V = I.random_case(4242, layer, B, T0 + m)
    Wd = torch.from_numpy(W).to("cuda")
    rag = lola.init_state(layer, B, Wd)
    lola.prefill(layer, rag, dev(Q[:, :T0], layer), dev(K[:, :T0], layer), dev(V[:, :T0], layer))
    counts = np.ones(B, np.int32)
    counts[8:16] = m
    pad = lambda X: dev(np.where((np.arange(m)[None, :] < counts[:, None])[..., None, None], X[:, T0:T0 + m], 0.0), layer)
    out = dev(np.full((B, m, layer.n_q_heads, layer.head_dim), 7.0, np.float32), layer)
    lola.prefill_ragged(layer, rag, torch.from_numpy(counts).to("cuda"), pad(Q), pad(K), pad(V), out=out)
    assert lola.check_state(layer, rag, B) == 0
    ra = lola.read_cache(layer, rag, B)
    C, tol = layer.cache_cap, tol_for(layer)
    for b in (0, 9, 63):
        n = int(counts[b])
        print(f"mixed batch: sequence {b}, {n} tokens", flush=True)
        assert bool(torch.all(out[b, n:] == 7.0))
        one = lola.init_state(layer, 1, Wd)
        lola.prefill(layer, one, dev(Q[b:b + 1, :T0], layer), dev(K[b:b + 1, :T0], layer), dev(V[b:b + 1, :T0], layer))
        o1 = lola.prefill(layer, one, dev(Q[b:b + 1, T0:T0 + n], layer), dev(K[b:b + 1, T0:T0 + n], layer),
                          dev(V[b:b + 1, T0:T0 + n], layer))
        assert torch.equal(out[b, :n], o1[0]), f"sequence {b} differs from its own calls"
        rb = lola.read_cache(layer, one, 1)
        for key in ("count", "pos", "k", "v", "H", "s", "tokens_seen"):
            assert torch.equal(ra[key][b:b + 1], rb[key]), f"sequence {b}: {key}"
        if b == 63:
            continue
        # the oracle over the same history: the 320-token prefill as five intervals with the
        # GPU's cache sets adopted under the margin rule, then this call's interval
        st = Stepper(layer, 1, W)
        for a in range(0, T0, layer.chunk):
            st.step(Q[b:b + 1, a:a + layer.chunk], K[b:b + 1, a:a + layer.chunk], V[b:b + 1, a:a + layer.chunk])
        g_out, r_out = st.step(Q[b:b + 1, T0:T0 + n], K[b:b + 1, T0:T0 + n], V[b:b + 1, T0:T0 + n])
        assert torch.equal(st.last_out[0], out[b, :n]), f"sequence {b}: stepped GPU run differs"
        err = row_rel_err(g_out, r_out)
        assert err <= tol, f"sequence {b}: output rel err {err:.3g}"
        eh, es = st.compare_state()
        assert eh <= tol and es <= tol


def test_decode_full_batch_launch(monkeypatch):
    """The decode launch that bench.py times: 64 sequences of the decode layer (512
    workgroups, two rounds of 256 CUs), window and cache full (320-token prefill), then
    four decode steps.  Sampled sequences equal a one-sequence run of the same history
    bitwise (both prefilled by the one-workgroup scan, which 512 chains need), and that
    run follows the oracle step by step."""
    monkeypatch.setenv("LOLA_SCAN_SPLIT", "0")
    wl = I.WORKLOADS[4]
    layer, B, T0, steps = wl.layer, wl.batch, 320, 4
    W, Q, K, V = I.random_case(5151, layer, B, T0 + steps)
    Wd = torch.from_numpy(W).to("cuda")
    full = lola.init_state(layer, B, Wd)
    lola.prefill(layer, full, dev(Q[:, :T0], layer), dev(K[:, :T0], layer), dev(V[:, :T0], layer))
    outs = [lola.decode(layer, full, dev(Q[:, t], layer), dev(K[:, t], layer), dev(V[:, t], layer))
            for t in range(T0, T0 + steps)]
    assert lola.check_state(layer, full, B) == 0
    tol = tol_for(layer)
    for b in (5, 62):
        print(f"decode full batch: sequence {b}", flush=True)
        st = Stepper(layer, 1, W)
        for a in range(0, T0, layer.chunk):
            st.step(Q[b:b + 1, a:a + layer.chunk], K[b:b + 1, a:a + layer.chunk], V[b:b + 1, a:a + layer.chunk])
        for i, t in enumerate(range(T0, T0 + steps)):
            g, r = st.step(Q[b:b + 1, t:t + 1], K[b:b + 1, t:t + 1], V[b:b + 1, t:t + 1], decode=True)
            assert torch.equal(st.last_out[0], outs[i][b]), f"sequence {b} step {t}: differs from its own run"
            err = row_rel_err(g, r)
            assert err <= tol, f"sequence {b} step {t}: output rel err {err:.3g}"
        eh, es = st.compare_state()
        assert eh <= tol and es <= tol
