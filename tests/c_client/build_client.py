"""Build the plain-C client of the MX library (tests/c_client/c_client.c)
with gcc against include/mx.h, the built libmx.so and the HIP runtime.
Test infrastructure: run by the package build step and, if the binary is
missing, by the test that uses it."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "c_client.c")
EXE = os.path.join(HERE, "c_client")
LIBDIR = os.path.join(ROOT, "microscaling_fp4_block_mx_amd")


def build(verbose: bool = False) -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    if not os.path.exists(os.path.join(LIBDIR, "libmx.so")):
        raise RuntimeError("libmx.so is missing: build the package first")
    cmd = ["gcc", "-std=c99", "-O1", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(rocm, "include"),
           SRC, "-o", EXE + ".tmp",
           "-L", LIBDIR, "-l:libmx.so", "-L", os.path.join(rocm, "lib"), "-lamdhip64", "-lm",
           # the library is found next to the repository copy it was built in
           "-Wl,-rpath,$ORIGIN/../../microscaling_fp4_block_mx_amd",
           "-Wl,-rpath," + os.path.join(rocm, "lib")]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("gcc failed building the C client")
    os.replace(EXE + ".tmp", EXE)
    return EXE


if __name__ == "__main__":
    print(build(verbose=True))
