"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer.

- The CPU oracle: its C source and a driver (tests/oracle_sanitize_driver.c)
  built with gcc and both sanitizers; every entry point runs on exactly sized
  heap buffers (small shapes, live counts below, at and past the row count,
  all element types) and the codecs over every 16-bit pattern.
- The C-ABI's host code: csrc/api.hip (argument checks, planners, dispatch)
  built with the sanitizers on its host side only, linked into the C99 client
  of tests/c_abi_client.c, whose calls reach it before libga.so's own copy;
  the kernels' launchers come from libga.so.  Nothing is launched."""
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


ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


@pytest.mark.skipif(not os.path.exists(os.path.join(ROCM, "bin", "hipcc")), reason="no hipcc")
def test_abi_host_code_under_asan_and_ubsan(tmp_path):
    import gated_activation_amd as ga
    lib_dir = os.path.dirname(ga.library_path)
    clang = os.path.join(ROCM, "llvm", "bin", "clang")
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all"]
    api_o, client_o, exe = tmp_path / "api.o", tmp_path / "client.o", tmp_path / "client_sanitized"
    host_san = []
    for f in san:
        host_san += ["-Xarch_host", f]
    subprocess.run([os.path.join(ROCM, "bin", "hipcc"), "--offload-arch=gfx950", "-O1", "-g", "-std=c++17",
                    "-fPIC", "-I", os.path.join(ROOT, "include")] + host_san +
                   ["-c", os.path.join(ROOT, "gated_activation_amd", "csrc", "api.hip"), "-o", str(api_o)],
                   check=True, capture_output=True, text=True)
    subprocess.run([clang, "-std=c99", "-g", "-O1"] + san + ["-I", os.path.join(ROOT, "include"), "-c",
                    os.path.join(HERE, "c_abi_client.c"), "-o", str(client_o)],
                   check=True, capture_output=True, text=True)
    subprocess.run([clang + "++"] + san[:1] + [str(client_o), str(api_o), "-o", str(exe), "-L", lib_dir, "-lga",
                    "-L", os.path.join(ROCM, "lib"), "-lamdhip64", f"-Wl,-rpath,{lib_dir}",
                    f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}"],
                   check=True, capture_output=True, text=True)
    # the client's ga_* calls reach the instrumented copy
    syms = subprocess.run(["nm", str(exe)], capture_output=True, text=True, check=True).stdout
    assert " T ga_gelu_and_mul_sparse\n" in syms and " T ga_plan_gelu_and_mul_sparse\n" in syms
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    res = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=env)
    assert res.returncode == 0 and res.stdout.strip().endswith("ok"), res.stdout[-3000:] + res.stderr[-3000:]
