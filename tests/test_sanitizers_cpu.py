"""CPU sanitizer builds: the oracle and the library's host code (tables,
workspace planners, argument validation) built with AddressSanitizer and
UndefinedBehaviorSanitizer and driven by the small C programs under
tests/sanitize/.  The device code of the library is compiled as usual; the
sanitizers are applied to the host side only.  No GPU is needed: the
drivers never reach a kernel launch."""
import concurrent.futures
import os
import shutil
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
SAN_FLAGS = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=undefined",
             "-fno-omit-frame-pointer", "-g"]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    return r.returncode, r.stdout + r.stderr


def test_oracle_under_sanitizers():
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    with tempfile.TemporaryDirectory() as tmp:
        exe = os.path.join(tmp, "oracle_check")
        rc, out = _run(["gcc", "-O1", "-std=c11", "-ffp-contract=off", *SAN_FLAGS,
                        os.path.join(SAN, "oracle_check.c"), os.path.join(ROOT, "oracle", "oracle.c"),
                        "-o", exe, "-lm", "-lpthread"])
        assert rc == 0, out
        rc, out = _run([exe], env=dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0"))
        assert rc == 0 and "oracle sanitizer check ok" in out, out
        assert "runtime error" not in out and "AddressSanitizer" not in out, out


def test_library_host_code_under_sanitizers():
    sys.path.insert(0, ROOT)
    from chunked_prefill_causal_rope_amd import build as B
    try:
        cc = B.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    host_san = []
    for f in SAN_FLAGS:
        host_san += ["-Xarch_host", f]
    with tempfile.TemporaryDirectory() as tmp:
        def compile_one(src):
            obj = os.path.join(tmp, os.path.basename(src) + ".o")
            cmd = [cc, *B.COMMON_FLAGS, *B.FILE_FLAGS.get(os.path.basename(src), []), *host_san, "-c", src,
                   "-o", obj]
            rc, out = _run(cmd)
            return obj, rc, out
        with concurrent.futures.ThreadPoolExecutor(max_workers=6) as ex:
            res = list(ex.map(compile_one, B.sources()))
        for obj, rc, out in res:
            assert rc == 0, out
        drv = os.path.join(tmp, "abi_check.o")
        rc, out = _run(["clang" if shutil.which("clang") else "gcc", "-O1", "-std=c11", *SAN_FLAGS, "-I",
                        os.path.join(ROOT, "include"), "-c", os.path.join(SAN, "abi_check.c"), "-o", drv])
        if rc != 0:
            rc, out = _run(["gcc", "-O1", "-std=c11", *SAN_FLAGS, "-I", os.path.join(ROOT, "include"), "-c",
                            os.path.join(SAN, "abi_check.c"), "-o", drv])
        assert rc == 0, out
        exe = os.path.join(tmp, "abi_check")
        rc, out = _run([cc, f"--offload-arch={B.ARCH}", *host_san, drv, *[o for o, _, _ in res], "-o", exe])
        assert rc == 0, out
        # the HIP runtime keeps its allocations until exit: leaks are not ours
        rc, out = _run([exe], env=dict(os.environ, ASAN_OPTIONS="detect_leaks=0"))
        assert rc == 0 and "library host sanitizer check ok" in out, out
        assert "runtime error" not in out and "ERROR: AddressSanitizer" not in out, out
