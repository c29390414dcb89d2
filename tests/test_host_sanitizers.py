"""The host side of liblola (argument checks, sizes, layouts; everything that runs
before a launch) built with AddressSanitizer and UndefinedBehaviorSanitizer on the
host pass only (-Xarch_host: the GPU code is built as usual), running the C-ABI
checks that need no GPU in a child process."""
import glob
import os
import subprocess
import sys

import pytest

from sparse_attention_chunkwise_amd import build as hipbuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import sys
sys.path.insert(0, {root!r})
from sparse_attention_chunkwise_amd import lola
lola.LIB_PATH = {so!r}
from tests import test_abi as T
T.test_exports_every_declared_symbol()
T.test_sizes()
for bad, st in [(dict(head_dim=96), -2), (dict(feat_half=48), -2), (dict(n_q_heads=3), -1),
                (dict(n_q_heads=64, n_kv_heads=2), -2), (dict(chunk=0), -1), (dict(chunk=512), -2),
                (dict(window=-1), -1), (dict(cache_cap=2048), -2), (dict(window=9000), -2)]:
    T.test_config_rejected(bad, st)
T.test_policy_checks()
print("host checks ok", flush=True)
"""


def test_host_checks_under_asan_and_ubsan(tmp_path):
    rt = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not rt:
        pytest.skip("the ROCm clang AddressSanitizer runtime is not installed")
    so = str(tmp_path / "liblola_host_san.so")
    csrc = os.path.join(ROOT, "sparse_attention_chunkwise_amd", "csrc")
    cmd = [hipbuild.hipcc(), "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-shared", "-fPIC",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(ROOT, "include"), "-I", csrc, "-o", so, os.path.join(csrc, "lola_api.hip")]
    subprocess.run(cmd, check=True, capture_output=True)
    env = dict(os.environ, LD_PRELOAD=rt[-1], ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    res = subprocess.run([sys.executable, "-c", CHILD.format(root=ROOT, so=so)], env=env, capture_output=True,
                         text=True, timeout=600)
    assert res.returncode == 0, res.stdout[-2000:] + res.stderr[-4000:]
    assert "ERROR: AddressSanitizer" not in res.stderr and "runtime error" not in res.stderr, res.stderr[-4000:]
    assert "host checks ok" in res.stdout
