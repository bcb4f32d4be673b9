"""The C oracle under the address and undefined-behaviour sanitizers (host
only).  oracle/sanitize_driver.c runs every entry point of oracle/pkv_oracle.c
once on the tiny paged case of the iThome article's section "手動畫一次 block
table", with every buffer at exactly its documented size, an empty sequence and
NaN in every unused cache slot; a read or write out of bounds, a leak or
undefined behaviour fails the run.  The driver also requires the paged and
the dense decode to agree bit for bit."""
import os
import shutil
import subprocess

import pytest

ORACLE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_sanitizers(tmp_path):
    exe = tmp_path / "sanitize_driver"
    cmd = ["gcc", "-O1", "-g", "-std=c11", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-Wall",
           "-Wno-unknown-pragmas", "-Wno-unused-parameter", "-o", str(exe),
           os.path.join(ORACLE, "pkv_oracle.c"), os.path.join(ORACLE, "sanitize_driver.c"), "-lm"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    res = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    out = res.stdout + res.stderr
    assert "Sanitizer" not in out and "runtime error" not in out, out
    assert res.returncode == 0, out
    assert "status 0" in res.stdout, out
