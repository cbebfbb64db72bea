"""The step's host-side logic (validation, attention work lists, plan step
model) built from the library's host-only sources with AddressSanitizer and
UndefinedBehaviorSanitizer, and run over randomised valid and corrupted
batches (tests/host_fuzz.cpp).  CPU only: the device trusts these work lists'
indices, so every one of them is checked here."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "intra_operation_overlap_amd", "csrc")
OUT = os.path.join(HERE, "_build")


@pytest.fixture(scope="module")
def fuzzer():
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    os.makedirs(OUT, exist_ok=True)
    exe = os.path.join(OUT, "host_fuzz")
    sources = [os.path.join(HERE, "host_fuzz.cpp"), os.path.join(CSRC, "validate.cpp"),
               os.path.join(CSRC, "plan_model.cpp")]
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", *sources, "-o", exe]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert r.returncode == 0, r.stdout
    return exe


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_host_logic_under_sanitizers(fuzzer, seed):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([fuzzer, "4000", str(seed)], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True,
                       env=env, timeout=300)
    assert r.returncode == 0, r.stdout[-4000:]
    assert r.stdout.startswith("ok:"), r.stdout[-2000:]
    # the generator must reach both outcomes in quantity
    words = r.stdout.split()
    rejected, checked = int(words[3]), int(words[7])
    assert rejected > 400 and checked > 400, r.stdout
