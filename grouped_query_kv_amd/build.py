"""Build libgqa.so (the HIP kernels + C ABI) in-tree for gfx950.

    python -m grouped_query_kv_amd.build

Every .hip file under csrc/ is compiled with hipcc for gfx950 and the objects
are linked into grouped_query_kv_amd/libgqa.so.  Packed fp32 instructions are
disabled for all device code.
"""
from __future__ import annotations

import os
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


def _compile(src: Path) -> Path:
    obj = BUILD / (src.stem + ".o")
    cmd = [HIPCC, *CFLAGS, "-c", str(src), "-o", str(obj)]
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
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
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


if __name__ == "__main__":
    build()
