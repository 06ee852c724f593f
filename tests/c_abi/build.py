"""Build step for the plain-C check of the library (abi_from_c.c): gcc against
include/ssd.h, libssd.so and the HIP runtime, with the C oracle compiled in for the
comparison.  Run by the top-level build entry point after the library is built."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
EXE = os.path.join(HERE, "abi_from_c")


def build() -> str:
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-Wall", "-D__HIP_PLATFORM_AMD__",
           f"-I{ROCM}/include", f"-I{os.path.join(ROOT, 'include')}",
           os.path.join(HERE, "abi_from_c.c"), os.path.join(ROOT, "oracle", "ssd_oracle.c"),
           f"-L{os.path.join(ROOT, 'ssd_chunked_scan_03_amd')}", "-lssd", f"-L{ROCM}/lib", "-lamdhip64", "-lm",
           "-Wl,-rpath,$ORIGIN/../../ssd_chunked_scan_03_amd", f"-Wl,-rpath,{ROCM}/lib", "-o", EXE]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("gcc failed for the C check:\n" + r.stderr[-4000:])
    return EXE


if __name__ == "__main__":
    print(build())
