"""The attention launch's workgroup-shape choice (waves per workgroup), built
with g++ from the same header the library uses, on a 256-CU part.  The GPU
parity tests rely on these shapes to run every kernel instance."""
import os
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "context_ring_ulysses_amd", "csrc")

# (splits, B, H, Sq) -> waves expected on 256 CUs
CASES = [
    # GPU parity test shapes (Sq = 300): one per workgroup shape
    ((1, 1, 128, 300), 8),
    ((1, 1, 150, 300), 4),
    ((1, 1, 8, 300), 2),
    # FLUX-1024 full forward: 432 tiles of 256 rows
    ((1, 1, 24, 4608), 8),
    # Ulysses share at degree 2: 12 heads at full length
    ((1, 1, 12, 4608), 8),
    # ring share at degree 8: one chunk per launch, then all 8 chunks fused
    ((1, 1, 24, 576), 2),
    ((8, 1, 24, 576), 4),
    # tiny inputs
    ((1, 1, 1, 1), 2),
]


def run_cases(cases):
    lines = "\n".join(f"  printf(\"%d\\n\", cru::attn_pick_waves({s * b * h}L, {sq}L, 256));"
                      for (s, b, h, sq), _ in cases)
    prog = "#include <cstdio>\n#include \"attn_shape.h\"\nint main() {\n" + lines + "\n  return 0;\n}\n"
    with tempfile.TemporaryDirectory() as tmp:
        src, exe = os.path.join(tmp, "s.cpp"), os.path.join(tmp, "s")
        open(src, "w").write(prog)
        r = subprocess.run(["g++", "-O1", "-std=c++17", "-I", CSRC, src, "-o", exe],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr
        out = subprocess.run([exe], capture_output=True, text=True, check=True).stdout.split()
    return [int(x) for x in out]


def test_workgroup_shapes():
    got = run_cases(CASES)
    for ((shape, want), w) in zip(CASES, got):
        assert w == want, f"splits,B,H,Sq={shape}: {w} waves, expected {want}"


@pytest.mark.parametrize("n_cu", [256])
def test_empty_launch_is_harmless(n_cu):
    # zero rows or zero heads: any shape, nothing is launched
    got = run_cases([((1, 1, 0, 300), 8), ((1, 1, 4, 0), 8)])
    assert all(w in (2, 4, 8) for w in got)
