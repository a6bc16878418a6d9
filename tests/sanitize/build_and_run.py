"""Build the host-check driver with AddressSanitizer and UndefinedBehavior-
Sanitizer on the host code that validates arguments (glance.cpp and the
driver; the kernel objects are the library's own, built without them) and
run it.  Usage: python -m tests.sanitize.build_and_run [out_dir]"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
PKG = os.path.join(ROOT, "tree_verified_block_amd")
HIP_OBJS = ["tree.hip.o", "gemm.hip.o", "attn.hip.o", "walk.hip.o", "layer.hip.o"]
# each sanitizer applies to the host pass only
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-fno-omit-frame-pointer", "-g", "-O1"]


def build(out_dir: str) -> str:
    from tree_verified_block_amd.build import BUILD, build as build_lib, hipcc
    if not all(os.path.exists(os.path.join(BUILD, o)) for o in HIP_OBJS):
        build_lib(verbose=False)
    os.makedirs(out_dir, exist_ok=True)
    inc = [f"-I{os.path.join(ROOT, 'include')}", f"-I{os.path.join(PKG, 'csrc')}"]
    objs = []
    for src in (os.path.join(PKG, "csrc", "glance.cpp"), os.path.join(HERE, "host_checks.cpp")):
        obj = os.path.join(out_dir, os.path.basename(src) + ".o")
        subprocess.run([hipcc(), "-std=c++17", *SAN, *inc, "-c", src, "-o", obj], check=True,
                       capture_output=True, text=True)
        objs.append(obj)
    exe = os.path.join(out_dir, "host_checks")
    subprocess.run([hipcc(), *SAN, "--offload-arch=gfx950", *objs,
                    *[os.path.join(BUILD, o) for o in HIP_OBJS], "-o", exe], check=True,
                   capture_output=True, text=True)
    return exe


def run(exe: str) -> subprocess.CompletedProcess:
    env = dict(os.environ)
    # the HIP runtime keeps allocations until exit; leaks are not what is checked
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    return subprocess.run([exe], env=env, capture_output=True, text=True, timeout=300)


if __name__ == "__main__":
    exe = build(sys.argv[1] if len(sys.argv) > 1 else os.path.join(ROOT, "_work", "sanitize"))
    r = run(exe)
    sys.stdout.write(r.stdout)
    sys.stderr.write(r.stderr)
    sys.exit(r.returncode)
