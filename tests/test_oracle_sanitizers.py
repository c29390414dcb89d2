"""The oracle built with AddressSanitizer and UndefinedBehaviorSanitizer (gcc, CPU
only) runs a set of its pins in a child process: no out-of-bounds access, use after
free or undefined behaviour in the C code that every parity claim rests on."""
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import sys
sys.path.insert(0, {root!r})
import oracle
from tests import oracle_pins as P
lib = oracle.load({so!r})
for check in (P.check_sre_closed_forms, P.check_per_key_weights, P.check_selection_replay,
              P.check_forced_selection, P.check_policy_replay, P.check_split_and_step_equivalence,
              P.check_golden_hand_trajectory):
    check(lib)
    print("ok", check.__name__, flush=True)
"""


def test_oracle_under_asan_and_ubsan(tmp_path):
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(asan) or not os.path.exists(asan):
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    so = str(tmp_path / "liblola_oracle_san.so")
    subprocess.run(["gcc", "-O1", "-g", "-std=c11", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                    "-fno-omit-frame-pointer", "-shared", "-fPIC", "-o", so, oracle.SRC, "-lm", "-lpthread"],
                   check=True)
    env = dict(os.environ, LD_PRELOAD=asan, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    res = subprocess.run([sys.executable, "-c", CHILD.format(root=ROOT, so=so)], env=env, capture_output=True,
                         text=True, timeout=600)
    assert res.returncode == 0, res.stdout[-2000:] + res.stderr[-4000:]
    assert "ERROR: AddressSanitizer" not in res.stderr and "runtime error" not in res.stderr, res.stderr[-4000:]
    assert res.stdout.count("ok ") == 7
