"""CPU sanitizer runs (no GPU needed).

The oracle (oracle.c) is built with AddressSanitizer and
UndefinedBehaviorSanitizer and its pins (test_oracle.py, test_chunk_model.py)
run against that build; the HIP library is built with the sanitizers on its
host code only (argument validation, planning, the C ABI; the device code is
built as usual) and the C-ABI checks (test_abi.py) run against it.  Each
runs in a child process with the sanitizer runtime preloaded, and any report
fails it (halt on the first error).
"""
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _gcc_runtime(name):
    p = subprocess.run(["gcc", "-print-file-name=" + name], capture_output=True, text=True)
    path = p.stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def _run_child(tests, env_extra, preload, log_dir):
    env = dict(os.environ)
    env.update(env_extra)
    env["LD_PRELOAD"] = preload
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:log_path=%s/asan" % log_dir
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1:log_path=%s/ubsan" % log_dir
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        "-m", "not gpu"] + tests, cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=900)
    reports = ""
    for f in sorted(glob.glob(os.path.join(log_dir, "*san*"))):
        with open(f) as fh:
            reports += fh.read()
    assert r.returncode == 0 and not reports, (r.stdout[-3000:], r.stderr[-3000:], reports[:3000])


def test_oracle_under_asan_ubsan(tmp_path):
    asan, ubsan = _gcc_runtime("libasan.so"), _gcc_runtime("libubsan.so")
    if not (asan and ubsan):
        pytest.skip("gcc sanitizer runtimes not available")
    lib = str(tmp_path / "liboracle_san.so")
    subprocess.run(["gcc", "-O1", "-g", "-fPIC", "-shared", "-pthread", "-ffp-contract=off",
                    "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", "-o", lib, os.path.join(ROOT, "oracle",
                                                                         "oracle.c"), "-lm"],
                   check=True)
    logs = tmp_path / "logs"
    logs.mkdir()
    _run_child(["tests/test_oracle.py", "tests/test_chunk_model.py"], {"ORACLE_LIB": lib},
               asan + ":" + ubsan, str(logs))


def test_host_abi_under_asan_ubsan(tmp_path):
    from linear_attention_lightning_amd import build as hip_build
    rts = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    try:
        hipcc = hip_build.hipcc()
    except RuntimeError:
        hipcc = None
    if not rts or hipcc is None or shutil.which("nm") is None:
        pytest.skip("hipcc or its sanitizer runtime not available")
    lib = str(tmp_path / "liblightning_attn_san.so")
    host_only = []
    for f in ("-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all",
              "-fno-omit-frame-pointer"):
        host_only += ["-Xarch_host", f]
    hip_build.build(out=lib, extra=["-O1", "-g"] + host_only)
    logs = tmp_path / "logs"
    logs.mkdir()
    _run_child(["tests/test_abi.py"], {"LIGHTNING_ATTN_LIB": lib}, rts[0], str(logs))
