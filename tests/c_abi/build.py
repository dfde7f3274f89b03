"""Build the C program that uses libdit.so through include/dit.h alone
(tests/c_abi/abi_check.c), with gcc, next to its source."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "abi_check.c")
EXE = os.path.join(HERE, "abi_check")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build_abi_check() -> str:
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"), SRC,
           "-L", os.path.join(ROOT, "diffusion_transformer_video_amd"), "-ldit",
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-lm",
           "-Wl,-rpath,$ORIGIN/../../diffusion_transformer_video_amd", "-Wl,-rpath," + os.path.join(ROCM, "lib"),
           "-o", EXE]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"building {SRC} failed:\n{r.stdout}{r.stderr}")
    return EXE


if __name__ == "__main__":
    print(build_abi_check())
