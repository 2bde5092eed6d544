"""Compile tests/c_abi/flce_c_check.c with the host C compiler against the HIP
runtime and the in-tree libflce.so (no hipcc, no torch): the C consumer the
GPU test runs.  Called by __graft_entry__.build() after the library is built."""
import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
BIN = os.path.join(HERE, "flce_c_check")


def build() -> str:
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        raise RuntimeError("no host C compiler for the C ABI check")
    pkg = os.path.join(ROOT, "linear_cross_entropy_bwd_amd")
    cmd = [cc, "-std=c11", "-O1", "-Wall", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"),
           os.path.join(HERE, "flce_c_check.c"), "-o", BIN,
           "-L", pkg, "-lflce", f"-Wl,-rpath,{pkg}",
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64", f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"C ABI check failed to build: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return BIN


if __name__ == "__main__":
    print(build())
