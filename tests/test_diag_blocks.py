"""Host check of the engine's diagonal-tile rule (CPU).

On a diagonal tile of the symmetric products each wave leaves out the 32x32
blocks wholly below the diagonal (the stored result is the upper triangle
and its mirror). The rule is plain constexpr code in csrc/muon_device.hpp
(Keep, diag_form), shared with the engine; tests/native/diag_blocks.cpp
enumerates every wave of every engine layout and checks that each block on
or above the diagonal is computed by its wave with its fragments read, and
that the blocks left out are exactly the strictly lower ones (28 of 64 on a
256-tile, 6 of 16 on a 128-tile), the fractions the planner's executed-flop
count uses. The GPU tests compare the results of all layouts bit for bit.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_diagonal_tile_blocks(tmp_path):
    exe = tmp_path / "diag_blocks"
    cmd = ["g++", "-std=c++17", "-O1", "-Wall", "-Werror", f"-I{ROOT}/muon_newton_schulz_update_amd/csrc",
           f"{ROOT}/tests/native/diag_blocks.cpp", "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert run.returncode == 0, run.stdout
    lines = run.stdout.splitlines()
    assert len(lines) == 3 and all(l.endswith(" 0 errors") for l in lines), run.stdout
    assert "tile 256: 28 of 64" in lines[0] and "tile 128: 6 of 16" in lines[2], run.stdout
