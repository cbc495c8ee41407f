"""Build the C++ client of the C ABI (tests/abi_c/ptq_path) against the in-tree libptq.so with hipcc."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
LIBDIR = os.path.join(ROOT, "post_int8_quantization_amd")
BIN = os.path.join(HERE, "ptq_path")


def build(verbose: bool = False) -> str:
    cmd = [os.environ.get("HIPCC", "/opt/rocm/bin/hipcc"), "-O2", "-std=c++17", "-I", os.path.join(ROOT, "include"),
           os.path.join(HERE, "ptq_path.cpp"), "-L", LIBDIR, "-lptq", "-Wl,-rpath,$ORIGIN/../../post_int8_quantization_amd", "-o", BIN + ".tmp"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"building the C client failed:\n{r.stdout}\n{r.stderr}")
    os.replace(BIN + ".tmp", BIN)
    if verbose:
        print("built", BIN)
    return BIN


if __name__ == "__main__":
    build(verbose=True)
