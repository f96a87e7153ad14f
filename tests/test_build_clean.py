"""A clean copy of the source tree (what git tracks, plus files not yet committed that
.gitignore does not list; no built library) builds itself with ``__graft_entry__.build()``
and the built library loads.  CPU only: compiles for gfx950 with hipcc, launches nothing."""
import os
import shutil
import subprocess
import sys

import pytest

from tests.conftest import ROOT


def kvq_abi():
    """KVQ_ABI_VERSION as the header defines it."""
    import re
    return int(re.search(r"#define KVQ_ABI_VERSION (\d+)", open(os.path.join(ROOT, "include", "kvq.h")).read()).group(1))


def _source_files():
    if shutil.which("git") is None or not os.path.isdir(os.path.join(ROOT, ".git")):
        pytest.skip("needs the git checkout to list the source files")
    out = subprocess.run(["git", "ls-files", "-co", "--exclude-standard"], cwd=ROOT, check=True,
                         stdout=subprocess.PIPE, text=True).stdout.split("\n")
    return [f for f in out if f and os.path.isfile(os.path.join(ROOT, f))]


def test_clean_tree_builds_and_loads(tmp_path):
    if shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"):
        pytest.skip("hipcc not available")
    files = _source_files()
    assert not any(f.endswith(".so") for f in files), "a built library is part of the source tree"
    for f in files:
        dst = tmp_path / f
        dst.parent.mkdir(parents=True, exist_ok=True)
        shutil.copy2(os.path.join(ROOT, f), dst)
    assert not (tmp_path / "rotate_then_bit_amd" / "libkvq.so").exists()
    code = ("import __graft_entry__ as g; g.build(); import rotate_then_bit_amd as k; "
            "import os; assert os.path.dirname(k.library_path()) == os.path.join(os.getcwd(), 'rotate_then_bit_amd'); "
            "print('abi', k.abi_version())")
    env = dict(os.environ, PYTHONDONTWRITEBYTECODE="1")
    p = subprocess.run([sys.executable, "-c", code], cwd=str(tmp_path), env=env, stdout=subprocess.PIPE,
                       stderr=subprocess.STDOUT, text=True, timeout=900)
    assert p.returncode == 0, p.stdout[-4000:]
    assert f"abi {kvq_abi()}" in p.stdout
    assert (tmp_path / "rotate_then_bit_amd" / "libkvq.so").exists()
