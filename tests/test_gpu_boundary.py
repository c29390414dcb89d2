"""The C ABI's state contract on the GPU: header tests inside the kernels, and
saving / restoring a state between calls (needs an MI355X).

A state initialised for another configuration or batch, or one an earlier call
marked faulted, must be left exactly as it is by every call that advances a
state: no state byte, output row or workspace byte written, and
lola_check_state reports it.  A state copied out between calls and copied back
into another buffer continues exactly as the uninterrupted one.
"""
import numpy as np
import pytest
import torch

from sparse_attention_chunkwise_amd import inputs as I
from sparse_attention_chunkwise_amd import lola
from tests.gpu_harness import dev

pytestmark = pytest.mark.gpu

BAD_STATE = -3
FAULT_OFFSET = 20  # int32 fault word of the 32-byte state header

LAYERS = [
    # (name, call config, the other config the buffer is initialised for)
    ("bf16_split", I.LayerConfig(8, 2, 128, 64, 16, 24, 32, "bf16"), I.LayerConfig(8, 2, 128, 64, 8, 24, 32, "bf16")),
    ("f32", I.LayerConfig(4, 2, 64, 32, 8, 12, 16, "f32"), I.LayerConfig(4, 2, 64, 32, 8, 12, 8, "f32")),
]


def _filled(shape, dtype, value):
    return torch.full(shape, value, dtype=dtype, device="cuda")


def _assert_call_wrote_nothing(layer, state, before, B, T, seed, what):
    """prefill, ragged prefill, decode and read-out on `state`: nothing written anywhere."""
    W, Q, K, V = I.random_case(seed, layer, B, T + 1)
    dt = lola.torch_dtype(layer)
    out = _filled((B, T, layer.n_q_heads, layer.head_dim), dt, 7.0)
    ws = torch.full((lola.workspace_bytes(layer, B, T),), 0x5A, dtype=torch.uint8, device="cuda")
    ws_before = ws.clone()
    lola.prefill(layer, state, dev(Q[:, :T], layer), dev(K[:, :T], layer), dev(V[:, :T], layer), out=out,
                 workspace=ws)
    counts = torch.full((B,), T, dtype=torch.int32, device="cuda")
    lola.prefill_ragged(layer, state, counts, dev(Q[:, :T], layer), dev(K[:, :T], layer), dev(V[:, :T], layer),
                        out=out, workspace=ws)
    dout = _filled((B, layer.n_q_heads, layer.head_dim), dt, 7.0)
    lola.decode(layer, state, dev(Q[:, T], layer), dev(K[:, T], layer), dev(V[:, T], layer), out=dout)
    torch.cuda.synchronize()
    assert torch.equal(state, before), f"{what}: state bytes changed"
    assert bool(torch.all(out == 7.0)), f"{what}: prefill output written"
    assert bool(torch.all(dout == 7.0)), f"{what}: decode output written"
    assert torch.equal(ws, ws_before), f"{what}: workspace written"
    assert lola.check_state(layer, state, B) == BAD_STATE


@pytest.mark.parametrize("name,layer,other", LAYERS, ids=[x[0] for x in LAYERS])
def test_state_of_other_config_left_untouched(name, layer, other):
    """A buffer sized for the call's config but initialised for another one (a smaller
    window, or another batch): every call leaves it and its outputs untouched."""
    B, T = 2, 40
    W, _, _, _ = I.random_case(1, layer, B, 1)
    Wd = torch.from_numpy(W).to("cuda")
    for init_layer, init_B in ((other, B), (layer, 1)):
        nbytes = lola.state_bytes(layer, B)
        assert lola.state_bytes(init_layer, init_B) <= nbytes
        state = torch.full((nbytes,), 0xA5, dtype=torch.uint8, device="cuda")
        lola.init_state(init_layer, init_B, Wd, state=state)
        torch.cuda.synchronize()
        assert lola.check_state(init_layer, state, init_B) == 0
        before = state.clone()
        _assert_call_wrote_nothing(layer, state, before, B, T, 17, f"{name} init for {init_layer}, batch {init_B}")
        # the read-out leaves its outputs unwritten as well
        rc = lola.read_cache(layer, state, B)
        torch.cuda.synchronize()
        assert bool(torch.all(rc["count"] == 0)) and bool(torch.all(rc["pos"] == -1))
        assert bool(torch.all(rc["H"] == 0)) and bool(torch.all(rc["tokens_seen"] == 0))
        # and the state is still the other config's, intact
        assert lola.check_state(init_layer, state, init_B) == 0


@pytest.mark.parametrize("name,layer,other", LAYERS, ids=[x[0] for x in LAYERS])
def test_faulted_state_left_untouched(name, layer, other):
    """A state whose fault word is set (as a split scan that gave up waiting leaves it;
    here set from the host) is not advanced any further, but can still be read out."""
    B, T = 2, 70
    W, Q, K, V = I.random_case(23, layer, B, T)
    state = lola.init_state(layer, B, torch.from_numpy(W).to("cuda"))
    lola.prefill(layer, state, dev(Q, layer), dev(K, layer), dev(V, layer))
    torch.cuda.synchronize()
    good = lola.read_cache(layer, state, B)
    state[FAULT_OFFSET:FAULT_OFFSET + 4] = torch.tensor([1, 0, 0, 0], dtype=torch.uint8, device="cuda")
    before = state.clone()
    _assert_call_wrote_nothing(layer, state, before, B, 33, 29, f"{name} faulted")
    rc = lola.read_cache(layer, state, B)
    for key in ("count", "pos", "H", "s", "k", "v", "tokens_seen"):
        assert torch.equal(rc[key], good[key]), key


SAVE_RESTORE = [
    ("4k_split_scan", I.WORKLOADS[3].layer, 1, 1024, 512),
    ("ragged_cut", I.LayerConfig(8, 2, 128, 64, 16, 24, 32, "bf16"), 2, 300, 160),
    ("f32", I.LayerConfig(4, 2, 64, 32, 8, 12, 16, "f32"), 2, 200, 96),
]


@pytest.mark.parametrize("name,layer,B,T,cut", SAVE_RESTORE, ids=[x[0] for x in SAVE_RESTORE])
def test_save_restore_continues_bitwise(name, layer, B, T, cut):
    """Copy the state bytes to host memory after `cut` tokens, overwrite the device buffer,
    copy them back into a fresh buffer and continue: outputs and every memory equal the
    uninterrupted run bit for bit (the cut is a whole number of intervals, so both runs
    use the same interval grid), and so do eight decode steps after it."""
    W, Q, K, V = I.random_case(41, layer, B, T + 8)
    Wd = torch.from_numpy(W).to("cuda")
    assert cut % layer.chunk == 0

    def rows(a, b):  # densely packed device copies of token rows [a, b)
        return dev(Q[:, a:b], layer), dev(K[:, a:b], layer), dev(V[:, a:b], layer)

    def tok(t):
        return dev(Q[:, t], layer), dev(K[:, t], layer), dev(V[:, t], layer)

    ref_state = lola.init_state(layer, B, Wd)
    ref_out = lola.prefill(layer, ref_state, *rows(0, T))
    ref_dec = [lola.decode(layer, ref_state, *tok(t)) for t in range(T, T + 8)]

    s1 = lola.init_state(layer, B, Wd)
    o1 = lola.prefill(layer, s1, *rows(0, cut))
    saved = s1.cpu()
    s1.fill_(0x3C)  # the old buffer is reused for something else
    s2 = torch.empty_like(s1)
    s2.copy_(saved.to("cuda"))
    assert lola.check_state(layer, s2, B) == 0
    o2 = lola.prefill(layer, s2, *rows(cut, T))
    dec = [lola.decode(layer, s2, *tok(t)) for t in range(T, T + 8)]
    assert lola.check_state(layer, s2, B) == 0
    assert torch.equal(torch.cat([o1, o2], dim=1), ref_out)
    for a, b in zip(dec, ref_dec):
        assert torch.equal(a, b)
    ra, rb = lola.read_cache(layer, s2, B), lola.read_cache(layer, ref_state, B)
    for key in ("count", "pos", "k", "v", "H", "s", "tokens_seen"):
        assert torch.equal(ra[key], rb[key]), key
    if not torch.equal(s2, ref_state):
        diff = torch.nonzero(s2 != ref_state).flatten().cpu().numpy()
        raise AssertionError(f"state bytes differ from the uninterrupted run at {len(diff)} bytes: "
                             + ", ".join(describe_offset(layer, B, int(o)) for o in diff[:6]))


def _align(x, a=256):
    return (x + a - 1) // a * a


def describe_offset(layer, B, off):
    """Field of the state layout (as include/lola.h describes it) holding byte `off`."""
    D, F, Fh, w, C, Hkv = layer.head_dim, 2 * layer.feat_half, layer.feat_half, layer.window, layer.cache_cap, \
        layer.n_kv_heads
    es = 2 if layer.io_dtype == "bf16" else 4
    o = 256
    Woff = o
    o = _align(o + 4 * Hkv * Fh * D)
    Wboff = o
    o = _align(o + 2 * 3 * Hkv * Fh * D)
    chains = o
    fields = [("tok+count", 256), ("H", 4 * F * D), ("s", 4 * F), ("cache_pos", 4 * max(C, 1)),
              ("ring_k", es * w * D), ("ring_v", es * w * D), ("cache_k", es * C * D), ("cache_v", es * C * D),
              ("cache_phi", 2 * 2 * F * C if es == 2 else 0)]
    if off < Woff:
        return f"header+{off}"
    if off < chains:
        return f"W@{off}"
    cb = sum(_align(n) for _, n in fields)
    ci, r = divmod(off - chains, cb)
    for name, n in fields:
        if r < _align(n):
            return f"chain {ci} {name}+{r}"
        r -= _align(n)
    return f"chain {ci} ?"
