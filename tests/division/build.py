"""Build the GPU check of the kernels' reciprocal (tests/division/rcp_check) with hipcc."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
BIN = os.path.join(HERE, "rcp_check")


def build(verbose: bool = False) -> str:
    cmd = [os.environ.get("HIPCC", "/opt/rocm/bin/hipcc"), "--offload-arch=gfx950", "-O3", "-std=c++17",
           "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", os.path.join(HERE, "rcp_check.hip"), "-o", BIN + ".tmp"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"building the reciprocal check failed:\n{r.stdout}\n{r.stderr}")
    os.replace(BIN + ".tmp", BIN)
    if verbose:
        print("built", BIN)
    return BIN


if __name__ == "__main__":
    build(verbose=True)
