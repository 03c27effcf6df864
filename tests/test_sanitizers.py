"""CPU builds under AddressSanitizer and UndefinedBehaviorSanitizer.

The oracle (oracle/gdn_oracle.c) is built with gcc and both sanitizers and run
through every entry point on small inputs, valid and invalid
(tests/sanitize/oracle_driver.c); the C-ABI library's sources are built with
the sanitizers on their host side only (hipcc -Xarch_host; GPU code is not
instrumented and nothing here reaches a device) and every entry point is called
with arguments the host checks refuse (tests/sanitize/abi_driver.cpp).  Any
out-of-bounds access, use after free, leak, signed overflow or misaligned
access aborts the run.  A planted overflow checks that the sanitizer is live.
"""
import concurrent.futures as fut
import glob
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
GCC_SAN = ["-g", "-O1", "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
HIP_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")


def _run(exe):
    return subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=300)


@pytest.mark.parametrize("san,body,report", [
    ("address", "int* p = malloc(4 * sizeof *p); volatile int i = 4; p[i] = 1; int r = p[0]; free(p); return r;",
     "heap-buffer-overflow"),
    ("undefined", "volatile int x = 2147483647; return x + argc;", "signed integer overflow"),
], ids=["asan", "ubsan"])
def test_sanitizers_are_live(tmp_path, san, body, report):
    """A planted mistake in a throwaway program, each sanitizer on its own."""
    src = tmp_path / "planted.c"
    src.write_text("#include <stdlib.h>\nint main(int argc, char** argv) { (void)argv; " + body + " }\n")
    exe = tmp_path / "planted"
    subprocess.check_call(["gcc", "-g", "-O1", "-fsanitize=" + san, "-fno-sanitize-recover=all", "-o", str(exe),
                           str(src)])
    r = _run(str(exe))
    assert r.returncode != 0 and report in r.stderr, r.stderr[-2000:]


def test_oracle_under_asan_and_ubsan(tmp_path):
    exe = tmp_path / "oracle_asan"
    subprocess.check_call(["gcc", "-std=c99", "-ffp-contract=off", *GCC_SAN, "-o", str(exe),
                           os.path.join(ROOT, "oracle", "gdn_oracle.c"), os.path.join(HERE, "oracle_driver.c"),
                           "-lm"])
    r = _run(str(exe))
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert "every call as expected" in r.stdout


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
def test_abi_host_checks_under_asan_and_ubsan(tmp_path):
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-ffp-contract=off",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "gated_deltanet_decode_amd", "csrc")]
    srcs = sorted(glob.glob(os.path.join(ROOT, "gated_deltanet_decode_amd", "csrc", "*.hip")))
    srcs.append(os.path.join(HERE, "abi_driver.cpp"))

    def compile_one(src):
        obj = tmp_path / (os.path.basename(src) + ".o")
        subprocess.run([HIPCC, *flags, *HIP_SAN, "-c", src, "-o", str(obj)], check=True, capture_output=True)
        return str(obj)

    with fut.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as pool:
        objs = list(pool.map(compile_one, srcs))
    exe = tmp_path / "abi_asan"
    subprocess.run([HIPCC, "--offload-arch=gfx950", *HIP_SAN, "-o", str(exe), *objs], check=True,
                   capture_output=True)
    r = _run(str(exe))
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert "every call refused as expected" in r.stdout
