"""The host side of the C ABI under AddressSanitizer and UndefinedBehaviorSanitizer.

Builds every library source with the sanitizers on the host code only (the
gfx950 device code is built as usual) and links tests/host_check/abi_fuzz.cpp
against it: a seeded walk over decode, explicit, per-head, quantiser and
projection requests around the documented limits that exercises the argument
validation and the workspace planning without making a GPU call.  CPU only.
"""
import concurrent.futures as cf
import os
import subprocess

import pytest

from rank_latent_attention_amd import build as B

HERE = os.path.dirname(os.path.abspath(__file__))
OUT = os.path.join(B.BUILD, "sanitize")
# each -fsanitize= applies to the host compilation only
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer", "-g"]


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")


@pytest.fixture(scope="module")
def fuzz_binary():
    try:
        hipcc = B.hipcc()
    except RuntimeError as e:
        pytest.skip(str(e))
    os.makedirs(OUT, exist_ok=True)
    srcs = [os.path.join(B.CSRC, s) for s in B.SOURCES] + [os.path.join(HERE, "host_check", "abi_fuzz.cpp")]

    def comp(src):
        obj = os.path.join(OUT, os.path.splitext(os.path.basename(src))[0] + ".o")
        lang = ["-x", "hip"] if src.endswith(".cpp") else []
        _run([hipcc, *B.CFLAGS, *SAN, *lang, "-c", src, "-o", obj])
        return obj

    with cf.ThreadPoolExecutor(max_workers=min(len(srcs), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(comp, srcs))
    exe = os.path.join(OUT, "abi_fuzz")
    _run([hipcc, f"--offload-arch={B.ARCH}", *SAN, *objs, "-o", exe])
    return exe


def test_abi_validation_and_planning_under_sanitizers(fuzz_binary):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    res = subprocess.run([fuzz_binary], capture_output=True, text=True, env=env, timeout=600)
    out = res.stdout + res.stderr
    print(out[-4000:])
    assert "ERROR: AddressSanitizer" not in out
    assert "runtime error:" not in out
    assert res.returncode == 0, out[-4000:]
    assert "0 failures" in res.stdout
