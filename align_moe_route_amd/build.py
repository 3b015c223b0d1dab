"""Build libmoe_route_sort.so for gfx950 with hipcc (in-tree, no JIT cache)."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRCS = [os.path.join(HERE, "csrc", f) for f in ("moe_route_sort.hip", "moe_gemm1.hip", "moe_gate.hip")]
OUT = os.path.join(HERE, "libmoe_route_sort.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-ffp-contract=off",          # every rounding step is the one the source spells out
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",  # no packed FP32 ops
    "-Wall",
]


GEN_SRC = os.path.join(HERE, "csrc", "gen_sig_table.cpp")
GEN_EXE = os.path.join(HERE, "csrc", "gen_sig_table")
TABLE_INC = os.path.join(HERE, "csrc", "sig_table.inc")


def _run(cmd, what):
    res = subprocess.run(cmd, capture_output=True, text=True)
    msg = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                    if "packed-fp32-ops" not in l and l.strip())
    if res.returncode != 0:
        raise RuntimeError(f"{what} failed ({res.returncode}):\n{msg}")
    return msg


def build_table(verbose: bool = False) -> str:
    """Generate sig_table.inc: the host program evaluates the library's own
    correctly rounded sigmoid on every BF16 pattern the table covers."""
    cmd = [HIPCC, "-x", "hip", "--offload-arch=gfx950", "-O2", "-std=c++17", "-ffp-contract=off",
           "-I", os.path.join(HERE, "csrc"), GEN_SRC, "-o", GEN_EXE]
    if verbose:
        print(" ".join(cmd), flush=True)
    _run(cmd, "compiling the table generator")
    _run([GEN_EXE, TABLE_INC + ".tmp"], "generating the sigmoid table")
    os.replace(TABLE_INC + ".tmp", TABLE_INC)
    os.remove(GEN_EXE)
    return TABLE_INC


def build(verbose: bool = False) -> str:
    build_table(verbose)
    cmd = [HIPCC, *FLAGS, "-I", os.path.join(ROOT, "include"), "-I", os.path.join(HERE, "csrc"), *SRCS,
           "-o", OUT + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    msg = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                    if "packed-fp32-ops" not in l and l.strip())
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{msg}")
    if verbose and msg:
        print(msg, flush=True)
    os.replace(OUT + ".tmp", OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose=True))
    sys.exit(0)
