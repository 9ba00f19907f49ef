"""Arithmetic identities the HIP kernels rely on, checked exhaustively on the
host (no GPU): the fused multiply-add division by 6 of the E4M3 block-scale
step (device_common.h `div6`) against the correctly rounded quotient, over
every finite non-negative fp32 input."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))


def test_div6_matches_correct_rounding(tmp_path):
    exe = str(tmp_path / "div6")
    subprocess.run(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-o", exe,
                    os.path.join(HERE, "exhaustive_div6.c"), "-lm", "-lpthread"], check=True)
    r = subprocess.run([exe, str(min(8, os.cpu_count() or 1))], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0 and r.stdout.startswith("OK"), r.stdout + r.stderr
