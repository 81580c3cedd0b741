"""Host code of libnanokv under AddressSanitizer and UndefinedBehaviorSanitizer.

Every source of the library is compiled again with the sanitizers on its
host code only (device code is unchanged), linked with the fuzz driver
tests/sanitize/abi_fuzz.cpp, and run: seeded random calls of every entry
point through argument validation, route building, workspace layout and
dispatch (up to the first kernel launch, which fails without a GPU), the
rollout policies and the storage account.  Any sanitizer report or failed
invariant fails the test.  Runs only where no GPU is visible: the driver
passes fake device pointers.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
from compressed_history_attention_amd import build  # noqa: E402

OUT = os.path.join(ROOT, "_build", "sanitize")
# sanitizers on the host side of every compile and of the link
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def _gpu_visible() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:  # noqa: BLE001
        return False


def _compile(src: str) -> str:
    obj = os.path.join(OUT, os.path.basename(src) + ".o")
    flags = [f for f in build.COMMON if f != "-O3"] + ["-O1", "-g"]
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [build.HIPCC, *flags, *SAN, *lang, "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed for {src}:\n{res.stderr[-4000:]}")
    return obj


@pytest.mark.skipif(_gpu_visible(), reason="the fuzz passes fake device pointers: host only")
def test_abi_fuzz_under_asan_ubsan():
    os.makedirs(OUT, exist_ok=True)
    srcs = build.sources() + [os.path.join(ROOT, "tests", "sanitize", "abi_fuzz.cpp")]
    with ThreadPoolExecutor(max_workers=8) as ex:
        objs = list(ex.map(_compile, srcs))
    exe = os.path.join(OUT, "abi_fuzz")
    cmd = [build.HIPCC, f"--offload-arch={build.ARCH}", *SAN, "-o", exe, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-4000:]
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    print(run.stdout[-2000:], run.stderr[-4000:])
    if run.returncode == 77:
        pytest.skip("a GPU is visible to the driver")
    assert run.returncode == 0, run.stderr[-4000:]
    assert "ERROR: AddressSanitizer" not in run.stderr
    assert "runtime error" not in run.stderr
    assert "abi_fuzz: 0 failed checks" in run.stdout
