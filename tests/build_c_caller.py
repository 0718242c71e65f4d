"""Builds tests/bin/c_gpu_prefill from tests/c_gpu_prefill.c: a plain C99
program that drives the HIP library through its C ABI with the HIP runtime
API, checked against the C oracle.  Called by __graft_entry__.build() after
the library and the oracle are built (the GPU test runs the binary; nothing
is compiled inside a test)."""
import os
import shutil
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "c_gpu_prefill.c")
BIN = os.path.join(ROOT, "tests", "bin", "c_gpu_prefill")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build():
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        raise RuntimeError("no C compiler found for tests/c_gpu_prefill.c")
    os.makedirs(os.path.dirname(BIN), exist_ok=True)
    pkg = os.path.join(ROOT, "linear_attention_lightning_amd")
    orc = os.path.join(ROOT, "oracle")
    cmd = [cc, "-std=c99", "-O1", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"),
           "-o", BIN + ".tmp", SRC,
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           "-L", pkg, "-l:liblightning_attn.so", "-L", orc, "-l:liboracle.so", "-lm",
           # found next to the binary wherever the tree is copied
           "-Wl,-rpath,$ORIGIN/../../linear_attention_lightning_amd",
           "-Wl,-rpath,$ORIGIN/../../oracle", "-Wl,-rpath," + os.path.join(ROCM, "lib")]
    subprocess.run(cmd, check=True)
    os.replace(BIN + ".tmp", BIN)
    return BIN


if __name__ == "__main__":
    print(build())
