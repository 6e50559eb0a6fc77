"""Host logic of the launch code, built with hipcc as host-only C++ and run on
the CPU (no GPU, no HIP runtime call)."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def _hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    pytest.skip("hipcc not found")


def test_xcd_remap_covers_every_tile(tmp_path):
    """The grouped GEMMs remap block ids so that runs of tiles stay on one XCD;
    with the launch grid rounded up to a multiple of 8 every tile of any
    device-side count up to the grid is computed exactly once, and so it is
    when the last tiles of each XCD's share go through the work queues, in any
    order the blocks run (a fast XCD then takes tiles of the others')."""
    exe = str(tmp_path / "xcd_cover")
    subprocess.check_call([_hipcc(), "-O1", "-std=c++17", "-D__HIP_PLATFORM_AMD__",
                           f"-I{os.path.join(ROOT, 'include')}", os.path.join(HERE, "host", "xcd_cover.cpp"),
                           "-o", exe])
    r = subprocess.run([exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "reaches tile 41: 0" in r.stdout
    assert "a fast XCD took up to" in r.stdout
