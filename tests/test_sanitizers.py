"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

* The oracle's C (oracle/nf4_oracle.c) is built with gcc -fsanitize=address,undefined together
  with tests/sanitize/oracle_driver.c, which calls every oracle function on ragged sizes.
* The HIP library is built with the sanitizers on its host code only (-Xarch_host; the gfx950
  device code is unchanged) and linked with tests/sanitize/abi_driver.cpp, which runs the C ABI's
  host paths: the codebook builders, the workspace plans over the routing boundaries and every
  argument check (all of which return before any HIP call, so no GPU is needed).
Any sanitizer report fails the run (-fno-sanitize-recover=all).
"""
import concurrent.futures as cf
import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    _run(["gcc", "-std=c99", "-O1", "-g", "-ffp-contract=off", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=all", os.path.join(ROOT, "oracle", "nf4_oracle.c"),
          os.path.join(HERE, "oracle_driver.c"), "-o", exe, "-lm"])
    r = _run([exe])
    assert r.stdout.strip().endswith("ok")


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not found")
def test_abi_host_paths_under_asan_ubsan(tmp_path):
    flags = ["-std=c++17", "-O1", "-g", "-fPIC", "--offload-arch=gfx950", "-I", os.path.join(ROOT, "include"),
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wno-unused-command-line-argument",
             "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=all"]
    csrc = os.path.join(ROOT, "bit_nf4_quantized_codebook_amd", "csrc")
    srcs = sorted(glob.glob(os.path.join(csrc, "*.hip")) + glob.glob(os.path.join(csrc, "*.cpp")))
    srcs.append(os.path.join(HERE, "abi_driver.cpp"))

    def comp(src):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        _run([HIPCC] + flags + ["-x", "hip", "-c", src, "-o", obj])
        return obj

    with cf.ThreadPoolExecutor(max_workers=8) as ex:
        objs = list(ex.map(comp, srcs))
    exe = str(tmp_path / "abi_driver")
    _run([HIPCC, "--offload-arch=gfx950", "-Xarch_host", "-fsanitize=address", "-Xarch_host",
          "-fsanitize=undefined"] + objs + ["-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0")
    r = _run([exe], env=env)
    assert r.stdout.strip().endswith("ok")
