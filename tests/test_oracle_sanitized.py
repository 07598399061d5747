"""The CPU oracle under AddressSanitizer and UndefinedBehaviorSanitizer: its C
source and a driver (tests/oracle_sanitize_driver.c) are built with gcc and
both sanitizers, then every entry point runs on exactly sized heap buffers
(small shapes, live counts below, at and past the row count, all element
types) and the codecs over every 16-bit pattern.  Host code only."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def _sanitizers_available(tmp_path):
    probe = tmp_path / "probe.c"
    probe.write_text("int main(void) { return 0; }\n")
    r = subprocess.run(["gcc", "-fsanitize=address,undefined", str(probe), "-o", str(tmp_path / "probe")],
                       capture_output=True, text=True)
    return r.returncode == 0


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no C compiler")
def test_oracle_under_asan_and_ubsan(tmp_path):
    if not _sanitizers_available(tmp_path):
        pytest.skip("gcc has no sanitizer runtime here")
    exe = tmp_path / "oracle_sanitized"
    cmd = ["gcc", "-std=gnu11", "-g", "-O1", "-ffp-contract=off", "-fno-fast-math",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
           os.path.join(ROOT, "oracle", "ga_oracle.c"), os.path.join(HERE, "oracle_sanitize_driver.c"),
           "-o", str(exe), "-lm"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    res = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=env)
    assert res.returncode == 0 and res.stdout.strip().endswith("ok"), res.stdout[-3000:] + res.stderr[-3000:]
