"""C ABI checks that need no GPU: the library loads, exports every symbol the
header declares, sizes its buffers and rejects bad arguments before any launch."""
import ctypes
import os
import re

import pytest

from sparse_attention_chunkwise_amd import inputs as I
from sparse_attention_chunkwise_amd import lola

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_symbols():
    with open(os.path.join(ROOT, "include", "lola.h")) as f:
        src = f.read()
    return sorted(set(re.findall(r"\b(lola_[a-z_]+)\s*\(", src)))


def test_exports_every_declared_symbol():
    lib = lola.lib()
    names = declared_symbols()
    assert set(names) == set(lola.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_sizes():
    for cfg, wl in I.WORKLOADS.items():
        sb = lola.state_bytes(wl.layer, wl.batch)
        wb = lola.workspace_bytes(wl.layer, wl.batch, wl.seq_len)
        assert sb > 0 and wb > 0 and sb % 256 == 0
        L = wl.layer
        per_chain = (4 * 2 * L.feat_half * L.head_dim + (2 if L.io_dtype == "bf16" else 4)
                     * 2 * (L.window + L.cache_cap) * L.head_dim)
        assert sb >= wl.batch * L.n_kv_heads * per_chain
    # workspace grows with the call length
    L = I.WORKLOADS[3].layer
    assert lola.workspace_bytes(L, 1, 8192) > lola.workspace_bytes(L, 1, 4096)


@pytest.mark.parametrize("bad,status", [
    (dict(head_dim=96), -2), (dict(feat_half=48), -2), (dict(n_q_heads=3), -1),
    (dict(n_q_heads=64, n_kv_heads=2), -2), (dict(chunk=0), -1), (dict(chunk=512), -2),
    (dict(window=-1), -1), (dict(cache_cap=2048), -2), (dict(window=9000), -2),
])
def test_config_rejected(bad, status):
    base = dict(n_q_heads=4, n_kv_heads=2, head_dim=64, feat_half=32, window=8, cache_cap=8, chunk=8,
                io_dtype="f32")
    base.update(bad)
    layer = I.LayerConfig(**base)
    assert lola.state_bytes(layer, 1) == 0
    lib = lola.lib()
    cfg = lola.config(layer)
    fake = ctypes.c_void_p(4096)
    rc = lib.lola_prefill_chunk(ctypes.byref(cfg), fake, 1, 8, fake, fake, fake, fake, fake, 1 << 30, None)
    assert rc == status


def test_bad_arguments_rejected_before_launch():
    layer = I.WORKLOADS[1].layer
    lib = lola.lib()
    cfg = lola.config(layer)
    p = ctypes.c_void_p(4096)
    mis = ctypes.c_void_p(4100)
    ws = lola.workspace_bytes(layer, 1, 16)
    assert lib.lola_prefill_chunk(None, p, 1, 16, p, p, p, p, p, ws, None) == -1
    assert lib.lola_prefill_chunk(ctypes.byref(cfg), p, 0, 16, p, p, p, p, p, ws, None) == -1
    assert lib.lola_prefill_chunk(ctypes.byref(cfg), p, 1, 0, p, p, p, p, p, ws, None) == -1
    assert lib.lola_prefill_chunk(ctypes.byref(cfg), None, 1, 16, p, p, p, p, p, ws, None) == -1
    assert lib.lola_prefill_chunk(ctypes.byref(cfg), p, 1, 16, mis, p, p, p, p, ws, None) == -1
    assert lib.lola_prefill_chunk(ctypes.byref(cfg), p, 1, 16, p, p, p, p, p, ws - 1, None) == -4
    cnt, cmis = ctypes.c_void_p(8192), ctypes.c_void_p(8194)
    assert lib.lola_prefill_ragged(ctypes.byref(cfg), p, 1, 16, None, p, p, p, p, p, ws, None) == -1
    assert lib.lola_prefill_ragged(ctypes.byref(cfg), p, 1, 16, cmis, p, p, p, p, p, ws, None) == -1
    assert lib.lola_prefill_ragged(ctypes.byref(cfg), p, 1, 0, cnt, p, p, p, p, p, ws, None) == -1
    assert lib.lola_prefill_ragged(ctypes.byref(cfg), p, 1, 16, cnt, mis, p, p, p, p, ws, None) == -1
    assert lib.lola_prefill_ragged(ctypes.byref(cfg), p, 1, 16, cnt, p, p, p, p, p, ws - 1, None) == -4
    assert lib.lola_decode_step(ctypes.byref(cfg), p, 1, None, p, p, p, None) == -1
    assert lib.lola_decode_step(ctypes.byref(cfg), p, -3, p, p, p, p, None) == -1
    assert lib.lola_init_state(ctypes.byref(cfg), 1, None, p, None) == -1
    assert lib.lola_read_cache(ctypes.byref(cfg), None, 1, None, None, None, None, None, None, None, None) == -1
    assert lib.lola_check_state(ctypes.byref(cfg), None, 1, None) == -1


def test_status_strings():
    for s in (0, -1, -2, -3, -4, -5, 7):
        assert isinstance(lola.status_string(s), str) and lola.status_string(s)


def test_policy_checks():
    """Policies outside the enum are rejected; lola_decode_step takes only the SRE policy."""
    lib = lola.lib()
    fake = ctypes.c_void_p(4096)
    bad = I.LayerConfig(4, 2, 64, 32, 8, 8, 8, "f32", policy=7)
    assert lola.state_bytes(bad, 1) == 0
    for p in (1, 2, 3, 4):
        layer = I.LayerConfig(4, 2, 64, 32, 8, 8, 8, "f32", policy=p)
        assert lola.state_bytes(layer, 1) > 0
        rc = lib.lola_decode_step(ctypes.byref(lola.config(layer)), fake, 1, fake, fake, fake, fake, None)
        assert rc == -2
