"""__graft_entry__.build() on a tree where nothing is built yet.

The packages load their built libraries when imported, so build() must not
import them before compiling.  This copies the sources (no built libraries)
into a temporary directory, runs build() there with hipcc cross-compiling
for gfx950 (no GPU needed) and checks that every library is produced and the
package imports.  About a minute and a half of compiling.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")


def _copy_sources(dst):
    """The tracked files of a fresh clone (git ls-files), else the sources by
    extension."""
    tops = ("gated_activation_amd", "oracle", "synth", "include")
    r = subprocess.run(["git", "ls-files", *tops], cwd=ROOT, capture_output=True, text=True)
    if r.returncode == 0 and r.stdout.strip():
        for rel in r.stdout.split():
            os.makedirs(os.path.join(dst, os.path.dirname(rel)), exist_ok=True)
            shutil.copy2(os.path.join(ROOT, rel), os.path.join(dst, rel))
        shutil.copy2(os.path.join(ROOT, "__graft_entry__.py"), dst)
        return
    keep = (".py", ".hip", ".h", ".inc", ".c", ".cpp")
    for top in tops:
        for dirpath, dirnames, filenames in os.walk(os.path.join(ROOT, top)):
            dirnames[:] = [d for d in dirnames if d != "__pycache__"]
            rel = os.path.relpath(dirpath, ROOT)
            os.makedirs(os.path.join(dst, rel), exist_ok=True)
            for f in filenames:
                if f.endswith(keep):
                    shutil.copy2(os.path.join(dirpath, f), os.path.join(dst, rel, f))
    shutil.copy2(os.path.join(ROOT, "__graft_entry__.py"), dst)


@pytest.mark.skipif(not os.path.exists(HIPCC) or shutil.which("gcc") is None, reason="needs hipcc and gcc")
def test_build_from_a_tree_with_nothing_built(tmp_path):
    _copy_sources(str(tmp_path))
    built = [os.path.join("gated_activation_amd", "libga.so"), os.path.join("oracle", "libga_oracle.so"),
             os.path.join("synth", "libsynth_core.so")]
    for b in built:
        assert not os.path.exists(tmp_path / b)
    env = dict(os.environ, PYTHONPATH=str(tmp_path))
    r = subprocess.run([sys.executable, "-c", "import __graft_entry__ as g; g.build(); "
                        "import gated_activation_amd as ga; print(ga.library_path)"],
                       cwd=str(tmp_path), env=env, capture_output=True, text=True, timeout=900)
    assert r.returncode == 0, r.stderr[-2000:]
    for b in built:
        assert os.path.exists(tmp_path / b), b
    assert str(tmp_path) in r.stdout
