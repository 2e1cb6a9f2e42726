"""Build libgqa.so (the HIP kernels + C ABI) in-tree for gfx950.

    python -m grouped_query_kv_amd.build

Every .hip file under csrc/ is compiled with hipcc for gfx950 and the objects
are linked into grouped_query_kv_amd/libgqa.so.  Packed fp32 instructions are
disabled for all device code.

The library carries the SHA-256 of the code it was built from (every source
under csrc/ and include/gqa.h, comments and whitespace removed), returned by
gqa_build_id(); the binding refuses to load a library whose code hash
differs from that of the sources next to it.
"""
from __future__ import annotations

import hashlib
import os
import re
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
BUILD = PKG / "_build"
LIB = PKG / "libgqa.so"

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{ROOT / 'include'}", f"-I{CSRC}",
]


def sources() -> list[Path]:
    return sorted(CSRC.glob("*.hip"))


def code_sha256(paths) -> str:
    """SHA-256 of the code in the given files (absolute, or relative to the
    repository root), C/C++ comments removed and whitespace runs collapsed,
    so that an edit of comments alone leaves it unchanged."""
    h = hashlib.sha256()
    for src in paths:
        text = (ROOT / src).read_text(encoding="utf-8")
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(re.sub(r"\s+", " ", text).strip().encode())
        h.update(b"\0")
    return h.hexdigest()


def hashed_sources() -> list[str]:
    """The files whose code defines the library (repository-relative)."""
    files = sorted(CSRC.glob("*.hip")) + sorted(CSRC.glob("*.h")) + [ROOT / "include" / "gqa.h"]
    return [str(f.relative_to(ROOT)) for f in files]


def build_id() -> str:
    """Code hash of the sources in this tree (what gqa_build_id() must return)."""
    return code_sha256(hashed_sources())


def _compile(src: Path, bid: str) -> Path:
    obj = BUILD / (src.stem + ".o")
    cmd = [HIPCC, *CFLAGS, f'-DGQA_BUILD_ID="{bid}"', "-c", str(src), "-o", str(obj)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src.name}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def _check_launch_stubs(lib: Path) -> None:
    """Fail when a kernel's host launch stub is referenced but not defined.

    hipcc's host pass can drop a kernel's stub without a diagnostic (seen with
    a __bf16 source pointer passed to the global-to-LDS load builtin); the
    library then links but cannot be loaded."""
    nm = shutil.which("nm")
    if nm is None:
        return
    r = subprocess.run([nm, "-u", str(lib)], capture_output=True, text=True)
    missing = [ln.split()[-1] for ln in r.stdout.splitlines() if "__device_stub__" in ln]
    if missing:
        raise RuntimeError(f"{len(missing)} kernel launch stubs are undefined in {lib.name}, e.g. {missing[0]}")


def build(verbose: bool = True) -> Path:
    """Compile every source and link libgqa.so (always rebuilds)."""
    if not shutil.which(HIPCC) and not Path(HIPCC).exists():
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    BUILD.mkdir(exist_ok=True)
    srcs = sources()
    bid = build_id()
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda src: _compile(src, bid), srcs))
    tmp = LIB.with_suffix(".so.tmp")
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", str(tmp), *map(str, objs)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    _check_launch_stubs(tmp)
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} from {len(srcs)} sources", file=sys.stderr)
    return LIB


# Host-side AddressSanitizer + UndefinedBehaviorSanitizer build of the whole
# library, for the CPU tests of the C ABI's validation layer: every
# -fsanitize flag applies to the host compilation only (device code is
# built as usual), and the objects are linked by the host compiler.
SAN_DIR = BUILD / "san"
SAN_LIB = SAN_DIR / "libgqa.so"
SAN_HOST_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
HOST_CXX = os.environ.get("HOST_CXX", "/opt/rocm/llvm/bin/clang++")


def asan_runtime() -> str:
    """Path of the host compiler's shared AddressSanitizer runtime."""
    r = subprocess.run([HOST_CXX, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    return r.stdout.strip()


def build_sanitized(verbose: bool = True) -> Path:
    """Compile every source with host ASan/UBSan and link _build/san/libgqa.so."""
    SAN_DIR.mkdir(parents=True, exist_ok=True)
    bid = build_id()

    def comp(src: Path) -> Path:
        obj = SAN_DIR / (src.stem + ".o")
        cmd = [HIPCC, *CFLAGS, *SAN_HOST_FLAGS, f'-DGQA_BUILD_ID="{bid}"', "-c", str(src), "-o", str(obj)]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"sanitized compile failed for {src.name}:\n{r.stderr}")
        return obj

    srcs = sources()
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(comp, srcs))
    rt_dir = str(Path(asan_runtime()).parent)
    link = [HOST_CXX, "-shared", "-fPIC", "-fsanitize=address,undefined", "-shared-libsan", "-o", str(SAN_LIB),
            *map(str, objs), "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", f"-Wl,-rpath,{rt_dir}"]
    r = subprocess.run(link, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"sanitized link failed:\n{r.stderr}")
    if verbose:
        print(f"built {SAN_LIB} (host ASan/UBSan)", file=sys.stderr)
    return SAN_LIB


if __name__ == "__main__":
    if len(sys.argv) > 1 and sys.argv[1] == "sanitized":
        build_sanitized()
    else:
        build()
