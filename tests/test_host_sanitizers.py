"""Host-side AddressSanitizer + UndefinedBehaviorSanitizer runs (CPU only).

The host library's C++ sources (CSR build and validation, the plan, the
fast divide, cascade detection / split / layouts) and the C oracle are
rebuilt with gcc/g++ ``-fsanitize=address,undefined -fno-sanitize-recover``
into a temporary directory; the device entry points are replaced by stubs
that refuse (``tests/sanitize/device_stubs.cpp``).  The CSR, plan,
cascade-host, fast-divide and oracle test suites then run again in a child
process against those builds (``PAGED_DECODE_LIB`` / ``ORACLE_LIB``), with the
ASan runtime preloaded.  Any heap overflow, use after free, signed overflow,
misaligned access or out-of-range shift aborts the child, which fails this
test.  Tests that need the GPU, torch, or a kernel's answer (MLA plans,
kernel-kind queries, the block-selection table) are left out of the child
run; the ordinary run covers them.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "paged_attention_decode_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
       "-g", "-O1"]


def _runtime(name):
    path = subprocess.run(["gcc", "-print-file-name=" + name], capture_output=True,
                          text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.fixture(scope="module")
def san_libs(tmp_path_factory):
    if not shutil.which("gcc") or not shutil.which("g++"):
        pytest.skip("gcc/g++ not available")
    asan = _runtime("libasan.so")
    if asan is None:
        pytest.skip("no ASan runtime")
    d = tmp_path_factory.mktemp("san")
    host = str(d / "libpaged_decode_san.so")
    subprocess.check_call(
        ["g++", "-std=c++17", "-shared", "-fPIC"] + SAN +
        ["-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
         os.path.join(CSRC, "pd_host.cpp"), os.path.join(CSRC, "pd_cascade_host.cpp"),
         os.path.join(ROOT, "tests", "sanitize", "device_stubs.cpp"), "-o", host])
    orc = str(d / "liboracle_san.so")
    subprocess.check_call(["gcc", "-std=c11", "-shared", "-fPIC"] + SAN +
                          [os.path.join(ROOT, "oracle", "oracle.c"), "-o", orc, "-lm",
                           "-lpthread"])
    return host, orc, asan


SUITES = [
    ("tests/test_host_library.py",
     "csr or plan or fastdiv or q_heads or version or exports",
     "mla or noalloc or refuse or default_target"),
    ("tests/test_cascade_host.py", None, "subgroup"),
    ("tests/test_oracle_csr_plan.py", None, None),
    ("tests/test_oracle_chunks.py", None, None),
    ("tests/test_oracle_attention.py", None, "sdpa"),
    ("tests/test_oracle_mla.py", None, "sdpa"),
    ("tests/test_oracle_sparse.py", None, "sdpa"),
]


@pytest.mark.parametrize("suite,keep,drop", SUITES, ids=[s[0].split("/")[-1] for s in SUITES])
def test_suite_clean_under_asan_ubsan(san_libs, suite, keep, drop):
    host, orc, asan = san_libs
    env = dict(os.environ)
    env.update(PAGED_DECODE_LIB=host, ORACLE_LIB=orc, LD_PRELOAD=asan,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:detect_odr_violation=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    expr = []
    if keep:
        expr.append("(%s)" % keep)
    if drop:
        expr.append("not (%s)" % drop)
    # --capture=sys: a sanitizer report goes to the child's real stderr
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "--capture=sys", "-p",
           "no:cacheprovider", "-m", "not gpu", suite]
    if expr:
        cmd += ["-k", " and ".join(expr)]
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in r.stdout, out[-2000:]
