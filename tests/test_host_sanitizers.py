"""Host AddressSanitizer + UndefinedBehaviorSanitizer runs of the C ABI's
host layer (argument validation, error codes, workspace sizing, split
planning), on the CPU: the library is rebuilt with -fsanitize on its host
compilation only (grouped_query_kv_amd.build.build_sanitized), then
  * the C99 program of test_c_header.py, built with the same sanitizers, runs
    against it, and
  * tests/test_abi.py runs in a Python process that loads it (the ASan
    runtime preloaded, since the interpreter is not instrumented).
Any sanitizer report fails the run.  Skipped where a preload is already in
place (the sanitizer runtime must come first) or no host clang exists."""
import os
import shutil
import subprocess
import sys
from pathlib import Path

import pytest

from grouped_query_kv_amd import build as bld

ROOT = Path(__file__).resolve().parent.parent
CLANG = str(Path(bld.HOST_CXX).with_name("clang"))
SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]

pytestmark = pytest.mark.skipif(
    bool(os.environ.get("LD_PRELOAD")) or not Path(bld.HOST_CXX).exists() or shutil.which(bld.HIPCC) is None
    and not Path(bld.HIPCC).exists(),
    reason="needs the host clang and hipcc, and no other preloaded library")


def _san_env():
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    return env


@pytest.fixture(scope="module")
def san_lib():
    stamp = bld.SAN_DIR / "build_id"
    if not (bld.SAN_LIB.exists() and stamp.exists() and stamp.read_text() == bld.build_id()):
        bld.build_sanitized(verbose=False)
        stamp.write_text(bld.build_id())
    return bld.SAN_LIB


def _clean(out: str) -> bool:
    return "AddressSanitizer" not in out and "runtime error:" not in out and "LeakSanitizer" not in out


def test_sanitizer_setup_catches_a_planted_overflow(tmp_path):
    """The toolchain and options used below do report a heap overflow (a
    throwaway host program, not library code)."""
    src = tmp_path / "bad.c"
    src.write_text("#include <stdlib.h>\nint main(void){ char* p = malloc(8); p[8] = 1; free(p); return 0; }\n")
    exe = tmp_path / "bad"
    subprocess.run([CLANG, *SAN_FLAGS, str(src), "-o", str(exe)], check=True, capture_output=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=_san_env(), timeout=60)
    assert r.returncode != 0 and "heap-buffer-overflow" in r.stderr


def test_c99_program_under_asan_ubsan(san_lib, tmp_path):
    from test_c_header import C_SRC
    src = tmp_path / "abi.c"
    src.write_text(C_SRC)
    exe = tmp_path / "abi"
    cmd = [CLANG, "-std=c99", *SAN_FLAGS, "-shared-libsan", f"-I{ROOT / 'include'}", str(src), f"-L{san_lib.parent}", "-lgqa",
           f"-Wl,-rpath,{san_lib.parent}", f"-Wl,-rpath,{Path(bld.asan_runtime()).parent}", "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=_san_env(), timeout=120)
    out = r.stdout + r.stderr
    assert r.returncode == 0 and r.stdout.strip().endswith("OK") and _clean(out), out[-3000:]


def test_abi_suite_under_asan_ubsan(san_lib):
    runner = (
        "import sys\n"
        f"sys.path[:0] = [{str(ROOT)!r}, {str(ROOT / 'tests')!r}]\n"
        "from grouped_query_kv_amd import _binding as B\n"
        f"lib = B.load_library({str(san_lib)!r})\n"
        f"assert lib._name == {str(san_lib)!r}\n"
        "import pytest\n"
        f"sys.exit(pytest.main(['-q', '-p', 'no:cacheprovider', {str(ROOT / 'tests' / 'test_abi.py')!r}]))\n")
    env = _san_env()
    env["LD_PRELOAD"] = bld.asan_runtime()
    r = subprocess.run([sys.executable, "-c", runner], capture_output=True, text=True, env=env, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0 and " passed" in r.stdout and _clean(out), out[-3000:]
