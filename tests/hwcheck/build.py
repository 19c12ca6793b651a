"""Build the test-only sweep library (tests/hwcheck/libps_hwcheck.so) for
gfx950 with hipcc, with the library's own compiler flags."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

from drift_aware_kv_amd import build as libbuild  # noqa: E402

SRC = os.path.join(HERE, "ps_hwcheck.hip")
LIB = os.path.join(HERE, "libps_hwcheck.so")


def build(verbose: bool = False) -> str:
    cmd = [libbuild._hipcc(), *libbuild.FLAGS, "-shared", SRC, "-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {SRC}:\n{r.stdout}{r.stderr}")
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
