"""lola_prefill_chunk_noalloc (the entry point that allocates nothing: its workspace is
the library's static per-GPU device array) against lola_prefill_chunk with a caller
workspace, through the C ABI (needs an MI355X).  Two calls in a row, the second with
a smaller input, must give identical outputs and state bytes; a call whose workspace
would not fit the array is rejected before anything is enqueued."""
import numpy as np
import pytest
import torch

from sparse_attention_chunkwise_amd import inputs as I
from sparse_attention_chunkwise_amd import lola
from tests.gpu_harness import dev

pytestmark = pytest.mark.gpu

CASES = [
    # (name, layer, B, first call, second call)
    ("bf16_4k_split_scan", I.WORKLOADS[3].layer, 1, 4096, 1000),
    ("bf16_one_block_scan", I.LayerConfig(8, 2, 128, 64, 16, 24, 32, "bf16"), 40, 300, 77),
    ("f32", I.LayerConfig(4, 2, 64, 32, 8, 12, 16, "f32"), 3, 400, 123),
]


@pytest.mark.parametrize("name,layer,B,n1,n2", CASES, ids=[c[0] for c in CASES])
def test_noalloc_equals_workspace_call(name, layer, B, n1, n2):
    assert lola.workspace_bytes(layer, B, n1) <= lola.NOALLOC_SCRATCH_BYTES
    W, Q, K, V = I.random_case(321 + len(name), layer, B, n1 + n2)
    Wd = torch.from_numpy(W).to("cuda")
    sa = lola.init_state(layer, B, Wd)   # static scratch
    sb = lola.init_state(layer, B, Wd)   # caller workspace
    for a, e in ((0, n1), (n1, n1 + n2)):
        print(f"{name}: tokens [{a}, {e})", flush=True)
        q, k, v = dev(Q[:, a:e], layer), dev(K[:, a:e], layer), dev(V[:, a:e], layer)
        oa = lola.prefill_noalloc(layer, sa, q, k, v)
        ob = lola.prefill(layer, sb, q, k, v)
        torch.cuda.synchronize()
        assert torch.equal(oa, ob), f"{name} [{a}, {e}): outputs differ"
        assert torch.equal(sa, sb), f"{name} [{a}, {e}): state bytes differ"
    assert lola.check_state(layer, sa, B) == 0


def test_noalloc_rejects_calls_beyond_its_scratch():
    layer = I.WORKLOADS[3].layer
    n = 16384
    assert lola.workspace_bytes(layer, 1, n) > lola.NOALLOC_SCRATCH_BYTES
    W, Q, K, V = I.random_case(5, layer, 1, 8)
    state = lola.init_state(layer, 1, torch.from_numpy(W).to("cuda"))
    before = state.clone()
    q = torch.zeros((1, n, layer.n_q_heads, layer.head_dim), dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros((1, n, layer.n_kv_heads, layer.head_dim), dtype=torch.bfloat16, device="cuda")
    out = torch.full_like(q, 7.0)
    with pytest.raises(lola.LolaError) as ei:
        lola.prefill_noalloc(layer, state, q, kv, kv, out=out)
    assert ei.value.status == -4
    torch.cuda.synchronize()
    assert torch.equal(state, before) and bool(torch.all(out == 7.0))
