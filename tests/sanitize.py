"""Host-code sanitizer pass: AddressSanitizer and UndefinedBehaviorSanitizer over the CPU oracle (gcc) and over
the host side of libconvrot_amd (hipcc, sanitizers on the host compilation only; the gfx950 code is built as
usual).  It builds sanitized copies beside the normal libraries and runs the CPU tests that exercise them, each
in a child process with the matching sanitizer runtime preloaded:

  * the oracle's pins and the host tables against liboracle_san.so (gcc's libasan);
  * the C ABI's exports and host-side argument validation against libconvrot_amd_san.so (clang's runtime).

Any report aborts the child (-fno-sanitize-recover=all) and fails the pass.  Leak detection is off: the
Python interpreter keeps its allocations to the end.  Not collected by pytest (it rebuilds the libraries);
run it by hand:  python tests/sanitize.py
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

SAN = ["address", "undefined"]


def build_oracle() -> str:
    import oracle.binding as ob
    out = os.path.join(ROOT, "oracle", "liboracle_san.so")
    flags = [f for f in ob.CFLAGS if not f.startswith("-O")] + ["-O1", "-g", "-fno-omit-frame-pointer",
                                                                 "-fno-sanitize-recover=all"]
    flags += ["-fsanitize=" + s for s in SAN]
    subprocess.run(["gcc", *flags, ob._SRC, "-o", out, "-lm"], check=True)
    return out


def build_library() -> str:
    from w8a8_rotated_int8_amd import build as b
    os.makedirs(b.BUILD, exist_ok=True)
    b.silu_table("inc")
    host = ["-g", "-fno-omit-frame-pointer", "-fno-sanitize-recover=all"]
    for s in SAN:
        host += ["-fsanitize=" + s]
    xflags = []
    for f in host:
        xflags += ["-Xarch_host", f]
    objs = []
    for src in b.SOURCES:
        obj = os.path.join(b.BUILD, os.path.splitext(src)[0] + "_san.o")
        subprocess.run([b.HIPCC, *b.FLAGS, *xflags, "-x", "hip", "-c", os.path.join(b.CSRC, src), "-o", obj],
                       check=True)
        objs.append(obj)
    out = os.path.join(b.PKG, "libconvrot_amd_san.so")
    subprocess.run([b.HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-shared-libsan", *xflags, *objs, "-o",
                    out], check=True)
    return out


def run(tests, env_extra, preload) -> int:
    env = dict(os.environ)
    env.update(env_extra)
    env["LD_PRELOAD"] = preload
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    cmd = [sys.executable, "-m", "pytest", "-q", "-m", "not gpu", "-p", "no:cacheprovider", *tests]
    print("+", " ".join(cmd), flush=True)
    return subprocess.run(cmd, cwd=ROOT, env=env).returncode


def main() -> int:
    gcc_asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    gcc_ubsan = subprocess.run(["gcc", "-print-file-name=libubsan.so"], capture_output=True,
                               text=True).stdout.strip()
    clang_rt = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not clang_rt:
        print("clang's AddressSanitizer runtime was not found", file=sys.stderr)
        return 2
    rc = run(["tests/test_oracle_pins.py", "tests/test_host_tables.py"], {"CONVROT_ORACLE_LIB": build_oracle()},
             f"{gcc_asan}:{gcc_ubsan}")
    if rc == 0:
        rc = run(["tests/test_abi.py"], {"CONVROT_AMD_LIB": build_library()}, clang_rt[-1])
    print("sanitizer pass:", "clean" if rc == 0 else f"FAILED ({rc})", flush=True)
    return rc


if __name__ == "__main__":
    sys.exit(main())
