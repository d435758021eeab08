"""A fresh checkout builds: ``__graft_entry__.build()`` and the documented
``python -m paged_attention_decode_photon_amd.build`` must work on a tree
that holds only the tracked sources (no built library)."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _tracked_files():
    try:
        out = subprocess.run(["git", "ls-files", "-z"], cwd=ROOT, capture_output=True, check=True)
    except (OSError, subprocess.CalledProcessError):
        return None
    return [f for f in out.stdout.decode().split("\0") if f]


def test_build_from_a_clean_checkout(tmp_path):
    if shutil.which("/opt/rocm/bin/hipcc") is None and not os.environ.get("HIPCC"):
        pytest.skip("hipcc is not installed")
    files = _tracked_files()
    if files is None:
        pytest.skip("not a git checkout")
    tree = tmp_path / "tree"
    for rel in files:
        src = os.path.join(ROOT, rel)
        if not os.path.isfile(src):  # deleted in the working tree
            continue
        dst = tree / rel
        dst.parent.mkdir(parents=True, exist_ok=True)
        shutil.copy2(src, dst)
    lib = tree / "paged_attention_decode_photon_amd" / "libphoton_decode.so"
    assert not lib.exists()
    env = dict(os.environ, PYTHONDONTWRITEBYTECODE="1")
    env.pop("PYTHONPATH", None)
    r = subprocess.run([sys.executable, "-c", "import __graft_entry__ as g; g.build()"],
                       cwd=tree, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-4000:]
    assert lib.exists()
    # the documented module command, on the same tree
    r = subprocess.run([sys.executable, "-m", "paged_attention_decode_photon_amd.build"],
                       cwd=tree, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-4000:]
    r = subprocess.run([sys.executable, "-c",
                        "import paged_attention_decode_photon_amd as pa; "
                        "print(pa.lib.photon_abi_version())"],
                       cwd=tree, env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-4000:]
    assert int(r.stdout.split()[-1]) > 0
