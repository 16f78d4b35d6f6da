"""Compile tests/c_abi/consumer.c with the system C compiler against
include/sgemm_f32.h and libsgemm_f32.so (a check that the boundary is plain C)."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
PKG = os.path.join(ROOT, "dense_fp32_matrix_f32_amd")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build(out: str = os.path.join(HERE, "consumer")) -> str:
    """Build the consumer next to its source (or at `out`, which must sit two
    directories below the repository root for the library to be found)."""
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"),
           os.path.join(HERE, "consumer.c"), "-o", out,
           "-L", PKG, "-lsgemm_f32", "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           # the library is found relative to the program, wherever the tree is
           "-Wl,-rpath,$ORIGIN/../../dense_fp32_matrix_f32_amd",
           f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    return out


if __name__ == "__main__":
    print(build())
