"""LOLA_TRACE=1 (a roctx range around every kernel launch) must not change any result:
the same small prefill and decode steps run in two child processes, one with the
variable set, and their outputs and final state bytes must be equal (needs an MI355X).
Without a profiler attached the roctx calls record nothing.

The children use the one-workgroup scan (LOLA_SCAN_SPLIT=0): the split scan's
cooperative launch failed (LOLA_ERR_HIP) in a child while this test process, which had
run split scans in earlier tests, was alive on the same GPU."""
import hashlib
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import hashlib, sys
sys.path.insert(0, {root!r})
import torch
from sparse_attention_chunkwise_amd import inputs as I
from sparse_attention_chunkwise_amd import lola
from tests.gpu_harness import dev
h = hashlib.sha256()
for layer in (I.LayerConfig(8, 2, 128, 64, 16, 24, 32, "bf16"), I.LayerConfig(4, 2, 64, 32, 8, 12, 16, "f32")):
    B, T = 2, 100
    W, Q, K, V = I.random_case(11, layer, B, T + 3)
    state = lola.init_state(layer, B, torch.from_numpy(W).to("cuda"))
    out = lola.prefill(layer, state, dev(Q[:, :T], layer), dev(K[:, :T], layer), dev(V[:, :T], layer))
    h.update(out.view(torch.uint8).cpu().numpy().tobytes())
    for t in range(T, T + 3):
        o = lola.decode(layer, state, dev(Q[:, t], layer), dev(K[:, t], layer), dev(V[:, t], layer))
        h.update(o.view(torch.uint8).cpu().numpy().tobytes())
    torch.cuda.synchronize()
    assert lola.check_state(layer, state, B) == 0
    h.update(state.cpu().numpy().tobytes())
print("digest", h.hexdigest(), flush=True)
"""


def _digest(trace: bool) -> str:
    env = dict(os.environ)
    env.pop("LOLA_TRACE", None)
    env["LOLA_SCAN_SPLIT"] = "0"
    if trace:
        env["LOLA_TRACE"] = "1"
    res = subprocess.run([sys.executable, "-c", CHILD.format(root=ROOT)], env=env, capture_output=True, text=True,
                         timeout=240)
    assert res.returncode == 0, res.stdout + res.stderr
    lines = [ln for ln in res.stdout.splitlines() if ln.startswith("digest ")]
    assert lines, res.stdout + res.stderr
    return lines[-1].split()[1]


def test_trace_ranges_change_nothing():
    assert _digest(trace=True) == _digest(trace=False)
