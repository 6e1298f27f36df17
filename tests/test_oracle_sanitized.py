"""The CPU oracle built with AddressSanitizer and UndefinedBehaviorSanitizer
(gcc, host only) and driven over exactly-sized buffers (no GPU)."""
import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def test_oracle_under_sanitizers(tmp_path):
    exe = tmp_path / "oracle_asan"
    cmd = ["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-ffp-contract=off",
           "-I", os.path.join(ROOT, "oracle"), os.path.join(ROOT, "oracle", "a2av_ref.c"),
           os.path.join(HERE, "oracle_asan_driver.c"), "-o", str(exe), "-lm"]
    try:
        subprocess.run(cmd, check=True, capture_output=True, text=True)
    except subprocess.CalledProcessError as e:
        if "asan" in (e.stderr or "").lower() and "cannot find" in (e.stderr or "").lower():
            pytest.skip("sanitizer runtime not installed")
        raise
    # the sanitizer runtime is linked statically into nothing else, so it need
    # not be first in the library list of the process
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0")
    p = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    assert p.returncode == 0, p.stderr[-3000:]
    assert "oracle sanitized: ok" in p.stdout
