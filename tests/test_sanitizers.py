"""Host AddressSanitizer and UndefinedBehaviorSanitizer runs (CPU only).

* The oracle (oracle/losa_oracle.c) built with both sanitizers and driven
  through every entry point on small ragged inputs, every reading flag, an
  empty prefix and a partial page (tests/sanitize/oracle_driver.c).
* liblosa.so's host code -- argument checks, shape arithmetic, workspace
  carving, status strings, the allocation-free entry point's rejection -- built
  with both sanitizers on its host side only (the device code is unchanged), and
  driven by tests/sanitize/api_driver.c through calls that return before any
  launch, so no GPU is needed.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SAN = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def _run(cmd, env=None, cwd=None):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, env=env,
                       cwd=cwd)
    return r.returncode, r.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_san")
    rc, out = _run(["gcc", "-std=c99", "-O1", "-g", "-fno-omit-frame-pointer", "-ffp-contract=off",
                    *SAN, os.path.join(ROOT, "oracle", "losa_oracle.c"),
                    os.path.join(HERE, "sanitize", "oracle_driver.c"), "-lm", "-o", exe])
    assert rc == 0, out
    rc, out = _run([exe], env=ENV)
    assert rc == 0 and "oracle sanitizer run: ok" in out, out


def test_library_host_code_under_sanitizers(tmp_path):
    from sparse_attention_block_amd import build as B
    host_san = [x for f in SAN for x in ("-Xarch_host", f)]
    objs = []
    for src in B.SOURCES:
        o = str(tmp_path / (src + ".o"))
        rc, out = _run([B.HIPCC, *B.FLAGS, *host_san, "-g", "-c", os.path.join(B.CSRC, src), "-o", o])
        assert rc == 0, out
        objs.append(o)
    drv = str(tmp_path / "api_driver.o")
    rc, out = _run(["gcc", "-std=c99", "-O1", "-g", "-I", B.INCLUDE, "-c",
                    os.path.join(HERE, "sanitize", "api_driver.c"), "-o", drv])
    assert rc == 0, out
    exe = str(tmp_path / "api_san")
    rc, out = _run([B.HIPCC, f"--offload-arch={B.ARCH}", *host_san, *objs, drv, "-o", exe])
    assert rc == 0, out
    rc, out = _run([exe], env=ENV)
    assert rc == 0 and "api sanitizer run: 0 failed checks" in out, out
