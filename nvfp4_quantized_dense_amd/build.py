"""Build libnvfp4_mi355x.so, the gfx950 HIP library, in-tree with hipcc.

Every translation unit compiles for gfx950 only, without fast-math (the
quantizer's divisions must be correctly rounded) and with packed-fp32
instructions disabled."""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libnvfp4_mi355x.so")
SOURCES = ["api.cpp", "quantize.hip", "repack.hip", "stream.hip", "stream_nt1.hip", "mid.hip", "gemv.hip", "fp4gemv.hip",
           "decode.hip", "decode16.hip", "tiled.hip", "tiled2.hip", "tiled16.hip", "silu_quant.hip", "prescale.hip"]
# LLVM instruction-scheduling strategy per translation unit, where another
# than the default measured faster on MI355X: the W4A16 tiled kernel with
# max-ilp (forward at 256 / 4096 tokens, hidden 5120: 208 -> 198 us, 1948 ->
# 1895 us), the one-token-group weight-streaming kernels with iterative-ilp
# (W4A16 forward at 16 tokens 60.5 -> 55.4 us; W4A4 at 4 / 16 tokens 37.8 /
# 42.9 -> 37.3 / 42.3 us). The same strategies made other kernels slower
# (max-ilp: the W4A4 tiled kernel 3.2 -> 5.5 ms; iterative-ilp: the 4-group
# streaming kernel at 64 tokens 77.5 -> 84.2 us), so they stay per file.
SCHED = {"tiled16.hip": "max-ilp", "stream_nt1.hip": "iterative-ilp"}
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMMON = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950", "-Wall",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", os.path.join(os.path.dirname(HERE), "include")]


def _compile(src: str, verbose: bool) -> str:
    out = os.path.join(OBJ, src + ".o")
    sched = ["-mllvm", "-amdgpu-sched-strategy=" + SCHED[src]] if src in SCHED else []
    cmd = [HIPCC] + COMMON + sched + ["-c", os.path.join(CSRC, src), "-o", out]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "not a recognized feature for this target" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{msg}")
    if msg.strip() and verbose:
        print(msg)
    return out


def build(verbose: bool = False, jobs: int = 0) -> str:
    os.makedirs(OBJ, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 1)
    with ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
