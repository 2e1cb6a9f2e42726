"""ctypes binding of libgqa (include/gqa.h), one Python function per entry point.

Argument marshalling only: the functions take torch tensors that live on the
GPU, check dtype/shape/contiguity/device, derive the integer sizes the C ABI
wants from the shapes, and pass raw device pointers plus the current HIP
stream.  Every step of the computation runs in the HIP kernels of libgqa.so;
if the library is missing the functions raise instead of computing anything
another way.
"""
from __future__ import annotations

import ctypes
import re
from pathlib import Path

import torch

PKG = Path(__file__).resolve().parent
LIB_PATH = PKG / "libgqa.so"
HEADER = PKG.parent / "include" / "gqa.h"

GQA_F32, GQA_BF16 = 0, 1
GQA_OK, GQA_ERR_INVALID, GQA_ERR_UNSUPPORTED, GQA_ERR_WORKSPACE, GQA_ERR_HIP = 0, -1, -2, -3, -4

_DTYPE_CODE = {torch.float32: GQA_F32, torch.bfloat16: GQA_BF16}

_c_void_p, _c_int, _c_int64, _c_size_t, _c_float = (
    ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float)

_SIGNATURES = {
    "gqa_abi_version": (_c_int, []),
    "gqa_build_id": (ctypes.c_char_p, []),
    "gqa_last_error": (ctypes.c_char_p, []),
    "gqa_set_timing_events": (_c_int, [_c_void_p, _c_void_p]),
    "gqa_kv_cache_bytes": (ctypes.c_uint64, [_c_int, _c_int, _c_int, _c_int, ctypes.c_uint64]),
    "gqa_kv_append": (_c_int, [_c_void_p] * 5 + [_c_int] * 5 + [_c_void_p]),
    "gqa_decode_workspace_bytes": (_c_size_t, [_c_int] * 5),
    "gqa_decode": (_c_int, [_c_void_p] * 6 + [_c_size_t] + [_c_int] * 6 + [_c_float, _c_int, _c_int, _c_void_p]),
    "gqa_decode_append": (_c_int, [_c_void_p] * 8 + [_c_size_t] + [_c_int] * 6 + [_c_float, _c_int, _c_int, _c_void_p]),
    "gqa_decode_append_noalloc": (_c_int, [_c_void_p] * 7 + [_c_int] * 6 + [_c_float, _c_int, _c_int, _c_void_p]),
    "gqa_kv_append_paged": (_c_int, [_c_void_p] * 6 + [_c_int] * 7 + [_c_void_p]),
    "gqa_decode_paged_workspace_bytes": (_c_size_t, [_c_int] * 6),
    "gqa_decode_paged": (_c_int, [_c_void_p] * 7 + [_c_size_t] + [_c_int] * 8 + [_c_float, _c_int, _c_int, _c_void_p]),
    "gqa_decode_append_paged": (_c_int, [_c_void_p] * 9 + [_c_size_t] + [_c_int] * 8 + [_c_float, _c_int, _c_int, _c_void_p]),
    "gqa_kv_quantize_int8": (_c_int, [_c_void_p] * 3 + [_c_int64, _c_int, _c_int, _c_void_p]),
    "gqa_kv_append_int8": (_c_int, [_c_void_p] * 7 + [_c_int] * 5 + [_c_void_p]),
    "gqa_decode_int8": (_c_int, [_c_void_p] * 8 + [_c_size_t] + [_c_int] * 6 + [_c_float, _c_int, _c_int, _c_void_p]),
    "gqa_decode_append_int8": (_c_int, [_c_void_p] * 10 + [_c_size_t] + [_c_int] * 6 + [_c_float, _c_int, _c_int, _c_void_p]),
    "gqa_prefill_chunk": (_c_int, [_c_void_p] * 5 + [_c_int] * 6 + [_c_float, _c_int, _c_int, _c_void_p]),
    "gqa_cross_attention": (_c_int, [_c_void_p] * 5 + [_c_int] * 6 + [_c_float, _c_int, _c_int, _c_void_p]),
    "gqa_kv_append_rows": (_c_int, [_c_void_p] * 5 + [_c_int] * 6 + [_c_void_p]),
    "gqa_kv_project": (_c_int, [_c_void_p] * 4 + [_c_int] * 6 + [_c_void_p]),
    "gqa_kv_project_workspace_bytes": (_c_size_t, [_c_int] * 5),
    "gqa_kv_project_append": (_c_int, [_c_void_p] * 6 + [_c_size_t] + [_c_int] * 7 + [_c_void_p]),
    "gqa_prefill_causal": (_c_int, [_c_void_p] * 4 + [_c_int] * 6 + [_c_float, _c_int, _c_int, _c_void_p]),
    "gqa_meanpool_convert": (_c_int, [_c_void_p, _c_void_p, _c_int64, _c_int, _c_int, _c_int64, _c_int, _c_void_p]),
}

_lib = None


class GQAError(RuntimeError):
    def __init__(self, fn: str, code: int, msg: str):
        super().__init__(f"{fn} returned {code}: {msg}")
        self.code = code


def header_symbols() -> list[str]:
    """Entry points declared in include/gqa.h."""
    text = HEADER.read_text()
    return sorted(set(re.findall(r"^\s*(?:[\w\*\s]+?)\b(gqa_\w+)\s*\(", text, flags=re.M)))


def load_library(path: Path | str = LIB_PATH) -> ctypes.CDLL:
    """Load libgqa.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    path = Path(path)
    if not path.exists():
        raise RuntimeError(
            f"{path} is missing: build it first (python -m grouped_query_kv_amd.build); "
            "there is no other implementation to fall back on")
    lib = ctypes.CDLL(str(path))
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    from .build import build_id

    built, here = lib.gqa_build_id().decode(), build_id()
    if built != here:
        raise RuntimeError(
            f"{path} was built from other sources (code hash {built[:16]}..., the sources here "
            f"hash to {here[:16]}...): rebuild it (python -m grouped_query_kv_amd.build)")
    _lib = lib
    return lib


def _check(fn: str, code: int) -> None:
    if code != GQA_OK:
        raise GQAError(fn, code, load_library().gqa_last_error().decode())


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


def _need(t: torch.Tensor, name: str, ndim: int, dtypes=(torch.float32, torch.bfloat16)):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")
    if t.dtype not in dtypes:
        raise ValueError(f"{name}: dtype {t.dtype} not supported")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


# ---------------------------------------------------------------------------
# entry points (same names as the C ABI)
# ---------------------------------------------------------------------------
def gqa_abi_version() -> int:
    return load_library().gqa_abi_version()


def gqa_build_id() -> str:
    return load_library().gqa_build_id().decode()


def gqa_last_error() -> str:
    return load_library().gqa_last_error().decode()


def gqa_kv_cache_bytes(layers: int, K: int, d: int, elem_bytes: int, tokens: int) -> int:
    return int(load_library().gqa_kv_cache_bytes(layers, K, d, elem_bytes, tokens))


_hip = None


def _hip_runtime() -> ctypes.CDLL:
    """The HIP runtime already loaded in this process (the one torch and
    libgqa share), for raw event handles."""
    global _hip
    if _hip is None:
        load_library()
        h = ctypes.CDLL("libamdhip64.so.7")
        h.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), _c_void_p, _c_void_p]
        h.hipEventSynchronize.argtypes = [_c_void_p]
        h.hipEventDestroy.argtypes = [_c_void_p]
        _hip = h
    return _hip


class HipEvent:
    """A raw timing hipEvent_t, recorded by the library's timing hook.  It is
    created without the system-scope fence on record (a timing-only event),
    so recording it does not write back and invalidate the caches between
    the kernels it brackets."""

    DISABLE_SYSTEM_FENCE = 0x20000000  # hipEventDisableSystemFence

    def __init__(self):
        self.handle = ctypes.c_void_p()
        if _hip_runtime().hipEventCreateWithFlags(ctypes.byref(self.handle), self.DISABLE_SYSTEM_FENCE) != 0:
            raise RuntimeError("hipEventCreateWithFlags failed")

    def elapsed_ms(self, end: "HipEvent") -> float:
        """Milliseconds between this event and `end` (waits for `end`)."""
        h = _hip_runtime()
        if h.hipEventSynchronize(end.handle) != 0:
            raise RuntimeError("hipEventSynchronize failed")
        ms = ctypes.c_float()
        if h.hipEventElapsedTime(ctypes.byref(ms), self.handle, end.handle) != 0:
            raise RuntimeError("hipEventElapsedTime failed (event not recorded?)")
        return float(ms.value)

    def __del__(self):
        if _hip is not None and self.handle:
            _hip.hipEventDestroy(self.handle)
            self.handle = ctypes.c_void_p()


def gqa_set_timing_events(begin: HipEvent | None = None, end: HipEvent | None = None) -> None:
    """Arm (or clear, with None) the begin/end events recorded around the
    main kernel of gqa_decode / gqa_prefill_causal on this thread."""
    b = None if begin is None else begin.handle
    e = None if end is None else end.handle
    _check("gqa_set_timing_events", load_library().gqa_set_timing_events(b, e))


def gqa_kv_append(k_new, v_new, k_cache, v_cache, seq_lens, stream=None) -> None:
    """Write k_new/v_new [B,K,d] at row seq_lens[b] of the caches [B,K,S_max,d]
    and increment seq_lens (int32 [B]), all on the GPU."""
    _need(k_cache, "k_cache", 4)
    B, K, S_max, d = k_cache.shape
    for t, nm in ((v_cache, "v_cache"),):
        _need(t, nm, 4)
        if t.shape != k_cache.shape or t.dtype != k_cache.dtype:
            raise ValueError("v_cache must match k_cache")
    for t, nm in ((k_new, "k_new"), (v_new, "v_new")):
        _need(t, nm, 3)
        if tuple(t.shape) != (B, K, d) or t.dtype != k_cache.dtype:
            raise ValueError(f"{nm} must be [B,K,d] of the cache dtype")
    _need(seq_lens, "seq_lens", 1, (torch.int32,))
    if seq_lens.numel() != B:
        raise ValueError("seq_lens must have B entries")
    lib = load_library()
    _check("gqa_kv_append", lib.gqa_kv_append(
        k_new.data_ptr(), v_new.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
        seq_lens.data_ptr(), B, K, S_max, d, _DTYPE_CODE[k_cache.dtype], _stream(stream)))


def gqa_decode_workspace_bytes(B: int, H: int, K: int, max_seq_len: int, d: int) -> int:
    return int(load_library().gqa_decode_workspace_bytes(B, H, K, max_seq_len, d))


def gqa_decode(q, k_cache, v_cache, seq_lens, out, workspace, max_seq_len: int,
               scale: float, stream=None) -> None:
    """One decode step: out [B,H,d] = GQA of q [B,H,d] over rows [0, seq_lens[b])
    of the caches [B,K,S_max,d].  workspace: uint8 GPU tensor of at least
    gqa_decode_workspace_bytes(...) bytes."""
    _need(q, "q", 3)
    _need(k_cache, "k_cache", 4)
    _need(v_cache, "v_cache", 4)
    _need(out, "out", 3)
    _need(seq_lens, "seq_lens", 1, (torch.int32,))
    _need(workspace, "workspace", 1, (torch.uint8,))
    B, H, d = q.shape
    Bk, K, S_max, dk = k_cache.shape
    if Bk != B or dk != d or v_cache.shape != k_cache.shape or tuple(out.shape) != (B, H, d):
        raise ValueError("shape mismatch between q, caches and out")
    if k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise ValueError("q and caches must share a dtype")
    if seq_lens.numel() != B:
        raise ValueError("seq_lens must have B entries")
    lib = load_library()
    _check("gqa_decode", lib.gqa_decode(
        q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), seq_lens.data_ptr(), out.data_ptr(),
        workspace.data_ptr(), workspace.numel(), B, H, K, S_max, int(max_seq_len), d, float(scale),
        _DTYPE_CODE[q.dtype], _DTYPE_CODE[out.dtype], _stream(stream)))


def gqa_decode_append(q, k_new, v_new, k_cache, v_cache, seq_lens, out, workspace,
                      max_seq_len: int, scale: float, stream=None) -> None:
    """gqa_kv_append followed by gqa_decode, fused into two kernel launches.
    max_seq_len bounds the lengths after the append."""
    _need(q, "q", 3)
    _need(k_cache, "k_cache", 4)
    _need(v_cache, "v_cache", 4)
    _need(out, "out", 3)
    _need(seq_lens, "seq_lens", 1, (torch.int32,))
    _need(workspace, "workspace", 1, (torch.uint8,))
    B, H, d = q.shape
    Bk, K, S_max, dk = k_cache.shape
    if Bk != B or dk != d or v_cache.shape != k_cache.shape or tuple(out.shape) != (B, H, d):
        raise ValueError("shape mismatch between q, caches and out")
    for t, nm in ((k_new, "k_new"), (v_new, "v_new")):
        _need(t, nm, 3)
        if tuple(t.shape) != (B, K, d) or t.dtype != k_cache.dtype:
            raise ValueError(f"{nm} must be [B,K,d] of the cache dtype")
    if k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise ValueError("q and caches must share a dtype")
    if seq_lens.numel() != B:
        raise ValueError("seq_lens must have B entries")
    lib = load_library()
    _check("gqa_decode_append", lib.gqa_decode_append(
        q.data_ptr(), k_new.data_ptr(), v_new.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
        seq_lens.data_ptr(), out.data_ptr(), workspace.data_ptr(), workspace.numel(), B, H, K,
        S_max, int(max_seq_len), d, float(scale), _DTYPE_CODE[q.dtype], _DTYPE_CODE[out.dtype],
        _stream(stream)))


def gqa_decode_append_noalloc(q, k_new, v_new, k_cache, v_cache, seq_lens, out, max_seq_len: int,
                              scale: float, stream=None) -> None:
    """gqa_decode_append without a workspace: the library's static device
    scratch holds the partials (for callers that cannot allocate; calls that
    overlap on one GPU race)."""
    _need(q, "q", 3)
    _need(k_cache, "k_cache", 4)
    _need(v_cache, "v_cache", 4)
    _need(out, "out", 3)
    _need(seq_lens, "seq_lens", 1, (torch.int32,))
    B, H, d = q.shape
    Bk, K, S_max, dk = k_cache.shape
    if Bk != B or dk != d or v_cache.shape != k_cache.shape or tuple(out.shape) != (B, H, d):
        raise ValueError("shape mismatch between q, caches and out")
    for t, nm in ((k_new, "k_new"), (v_new, "v_new")):
        _need(t, nm, 3)
        if tuple(t.shape) != (B, K, d) or t.dtype != k_cache.dtype:
            raise ValueError(f"{nm} must be [B,K,d] of the cache dtype")
    if k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise ValueError("q and caches must share a dtype")
    if seq_lens.numel() != B:
        raise ValueError("seq_lens must have B entries")
    _check("gqa_decode_append_noalloc", load_library().gqa_decode_append_noalloc(
        q.data_ptr(), k_new.data_ptr(), v_new.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
        seq_lens.data_ptr(), out.data_ptr(), B, H, K, S_max, int(max_seq_len), d, float(scale),
        _DTYPE_CODE[q.dtype], _DTYPE_CODE[out.dtype], _stream(stream)))


def _need_paged(k_pool, v_pool, block_table, seq_lens):
    _need(k_pool, "k_pool", 4)
    _need(v_pool, "v_pool", 4)
    if v_pool.shape != k_pool.shape or v_pool.dtype != k_pool.dtype:
        raise ValueError("v_pool must match k_pool")
    _need(block_table, "block_table", 2, (torch.int32,))
    _need(seq_lens, "seq_lens", 1, (torch.int32,))
    if seq_lens.numel() != block_table.shape[0]:
        raise ValueError("seq_lens must have one entry per block_table row")


def gqa_kv_append_paged(k_new, v_new, k_pool, v_pool, block_table, seq_lens, stream=None) -> None:
    """Write k_new/v_new [B,K,d] at logical row seq_lens[b] of the paged pools
    [num_blocks,K,block_size,d] through block_table [B,max_blocks] and
    increment seq_lens, all on the GPU."""
    _need_paged(k_pool, v_pool, block_table, seq_lens)
    num_blocks, K, block_size, d = k_pool.shape
    B, max_blocks = block_table.shape
    for t, nm in ((k_new, "k_new"), (v_new, "v_new")):
        _need(t, nm, 3)
        if tuple(t.shape) != (B, K, d) or t.dtype != k_pool.dtype:
            raise ValueError(f"{nm} must be [B,K,d] of the pool dtype")
    lib = load_library()
    _check("gqa_kv_append_paged", lib.gqa_kv_append_paged(
        k_new.data_ptr(), v_new.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(),
        block_table.data_ptr(), seq_lens.data_ptr(), B, K, num_blocks, block_size, max_blocks, d,
        _DTYPE_CODE[k_pool.dtype], _stream(stream)))


def gqa_decode_paged_workspace_bytes(B: int, H: int, K: int, max_seq_len: int, d: int,
                                     block_size: int) -> int:
    return int(load_library().gqa_decode_paged_workspace_bytes(B, H, K, max_seq_len, d, block_size))


def gqa_decode_paged(q, k_pool, v_pool, block_table, seq_lens, out, workspace, max_seq_len: int,
                     scale: float, stream=None) -> None:
    """One decode step over a paged cache: out [B,H,d] = GQA of q [B,H,d]
    over logical rows [0, seq_lens[b]) gathered through block_table."""
    _need(q, "q", 3, (torch.bfloat16,))
    _need_paged(k_pool, v_pool, block_table, seq_lens)
    _need(out, "out", 3)
    _need(workspace, "workspace", 1, (torch.uint8,))
    B, H, d = q.shape
    num_blocks, K, block_size, dk = k_pool.shape
    if dk != d or block_table.shape[0] != B or tuple(out.shape) != (B, H, d):
        raise ValueError("shape mismatch between q, pools, block_table and out")
    if k_pool.dtype != q.dtype:
        raise ValueError("q and pools must share a dtype")
    lib = load_library()
    _check("gqa_decode_paged", lib.gqa_decode_paged(
        q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(), block_table.data_ptr(),
        seq_lens.data_ptr(), out.data_ptr(), workspace.data_ptr(), workspace.numel(), B, H, K,
        num_blocks, block_size, block_table.shape[1], int(max_seq_len), d, float(scale),
        _DTYPE_CODE[q.dtype], _DTYPE_CODE[out.dtype], _stream(stream)))


def gqa_decode_append_paged(q, k_new, v_new, k_pool, v_pool, block_table, seq_lens, out, workspace,
                            max_seq_len: int, scale: float, stream=None) -> None:
    """gqa_kv_append_paged followed by gqa_decode_paged, fused into two kernel
    launches.  max_seq_len bounds the lengths after the append."""
    _need(q, "q", 3, (torch.bfloat16,))
    _need_paged(k_pool, v_pool, block_table, seq_lens)
    _need(out, "out", 3)
    _need(workspace, "workspace", 1, (torch.uint8,))
    B, H, d = q.shape
    num_blocks, K, block_size, dk = k_pool.shape
    if dk != d or block_table.shape[0] != B or tuple(out.shape) != (B, H, d):
        raise ValueError("shape mismatch between q, pools, block_table and out")
    if k_pool.dtype != q.dtype:
        raise ValueError("q and pools must share a dtype")
    for t, nm in ((k_new, "k_new"), (v_new, "v_new")):
        _need(t, nm, 3, (torch.bfloat16,))
        if tuple(t.shape) != (B, K, d):
            raise ValueError(f"{nm} must be [B,K,d]")
    _check("gqa_decode_append_paged", load_library().gqa_decode_append_paged(
        q.data_ptr(), k_new.data_ptr(), v_new.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(),
        block_table.data_ptr(), seq_lens.data_ptr(), out.data_ptr(), workspace.data_ptr(),
        workspace.numel(), B, H, K, num_blocks, block_size, block_table.shape[1], int(max_seq_len), d,
        float(scale), _DTYPE_CODE[q.dtype], _DTYPE_CODE[out.dtype], _stream(stream)))


def gqa_kv_quantize_int8(src, codes, scales, stream=None) -> None:
    """Quantise the rows of src [..., d] (fp32 or bf16) into int8 codes of
    the same shape and fp32 scales [...] (one per row)."""
    if not isinstance(src, torch.Tensor) or not src.is_cuda or not src.is_contiguous():
        raise ValueError("src must be a contiguous GPU tensor")
    if src.dtype not in _DTYPE_CODE:
        raise ValueError(f"src: dtype {src.dtype} not supported")
    d = src.shape[-1]
    rows = src.numel() // d
    _need(codes, "codes", src.dim(), (torch.int8,))
    _need(scales, "scales", src.dim() - 1, (torch.float32,))
    if codes.shape != src.shape or tuple(scales.shape) != tuple(src.shape[:-1]):
        raise ValueError("codes must match src, scales must be src.shape[:-1]")
    _check("gqa_kv_quantize_int8", load_library().gqa_kv_quantize_int8(
        src.data_ptr(), codes.data_ptr(), scales.data_ptr(), rows, d, _DTYPE_CODE[src.dtype],
        _stream(stream)))


def _need_int8_cache(k_codes, v_codes, k_scales, v_scales):
    _need(k_codes, "k_codes", 4, (torch.int8,))
    _need(v_codes, "v_codes", 4, (torch.int8,))
    _need(k_scales, "k_scales", 3, (torch.float32,))
    _need(v_scales, "v_scales", 3, (torch.float32,))
    if v_codes.shape != k_codes.shape or k_scales.shape != k_codes.shape[:3] or \
            v_scales.shape != k_codes.shape[:3]:
        raise ValueError("int8 cache: codes [B,K,S_max,d] and scales [B,K,S_max] must agree")


def gqa_kv_append_int8(k_new, v_new, k_codes, v_codes, k_scales, v_scales, seq_lens, stream=None) -> None:
    """Quantise k_new/v_new [B,K,d] and append them at row seq_lens[b] of an
    int8 cache; increment seq_lens."""
    _need_int8_cache(k_codes, v_codes, k_scales, v_scales)
    B, K, S_max, d = k_codes.shape
    for t, nm in ((k_new, "k_new"), (v_new, "v_new")):
        _need(t, nm, 3)
        if tuple(t.shape) != (B, K, d) or t.dtype != k_new.dtype:
            raise ValueError(f"{nm} must be [B,K,d]")
    _need(seq_lens, "seq_lens", 1, (torch.int32,))
    if seq_lens.numel() != B:
        raise ValueError("seq_lens must have B entries")
    _check("gqa_kv_append_int8", load_library().gqa_kv_append_int8(
        k_new.data_ptr(), v_new.data_ptr(), k_codes.data_ptr(), v_codes.data_ptr(),
        k_scales.data_ptr(), v_scales.data_ptr(), seq_lens.data_ptr(), B, K, S_max, d,
        _DTYPE_CODE[k_new.dtype], _stream(stream)))


def gqa_decode_int8(q, k_codes, v_codes, k_scales, v_scales, seq_lens, out, workspace,
                    max_seq_len: int, scale: float, stream=None) -> None:
    """One decode step over an int8 cache: out [B,H,d] = GQA of the bf16 q
    [B,H,d] over the dequantised rows [0, seq_lens[b])."""
    _need(q, "q", 3, (torch.bfloat16,))
    _need_int8_cache(k_codes, v_codes, k_scales, v_scales)
    _need(out, "out", 3)
    _need(seq_lens, "seq_lens", 1, (torch.int32,))
    _need(workspace, "workspace", 1, (torch.uint8,))
    B, H, d = q.shape
    Bk, K, S_max, dk = k_codes.shape
    if Bk != B or dk != d or tuple(out.shape) != (B, H, d) or seq_lens.numel() != B:
        raise ValueError("shape mismatch between q, cache, seq_lens and out")
    _check("gqa_decode_int8", load_library().gqa_decode_int8(
        q.data_ptr(), k_codes.data_ptr(), v_codes.data_ptr(), k_scales.data_ptr(), v_scales.data_ptr(),
        seq_lens.data_ptr(), out.data_ptr(), workspace.data_ptr(), workspace.numel(), B, H, K, S_max,
        int(max_seq_len), d, float(scale), GQA_BF16, _DTYPE_CODE[out.dtype], _stream(stream)))


def gqa_decode_append_int8(q, k_new, v_new, k_codes, v_codes, k_scales, v_scales, seq_lens, out,
                           workspace, max_seq_len: int, scale: float, stream=None) -> None:
    """gqa_kv_append_int8 followed by gqa_decode_int8, fused into two kernel
    launches (bf16 q, k_new, v_new).  max_seq_len bounds the lengths after
    the append."""
    _need(q, "q", 3, (torch.bfloat16,))
    _need_int8_cache(k_codes, v_codes, k_scales, v_scales)
    _need(out, "out", 3)
    _need(seq_lens, "seq_lens", 1, (torch.int32,))
    _need(workspace, "workspace", 1, (torch.uint8,))
    B, H, d = q.shape
    Bk, K, S_max, dk = k_codes.shape
    if Bk != B or dk != d or tuple(out.shape) != (B, H, d) or seq_lens.numel() != B:
        raise ValueError("shape mismatch between q, cache, seq_lens and out")
    for t, nm in ((k_new, "k_new"), (v_new, "v_new")):
        _need(t, nm, 3, (torch.bfloat16,))
        if tuple(t.shape) != (B, K, d):
            raise ValueError(f"{nm} must be [B,K,d]")
    _check("gqa_decode_append_int8", load_library().gqa_decode_append_int8(
        q.data_ptr(), k_new.data_ptr(), v_new.data_ptr(), k_codes.data_ptr(), v_codes.data_ptr(),
        k_scales.data_ptr(), v_scales.data_ptr(), seq_lens.data_ptr(), out.data_ptr(),
        workspace.data_ptr(), workspace.numel(), B, H, K, S_max, int(max_seq_len), d, float(scale),
        GQA_BF16, _DTYPE_CODE[out.dtype], _stream(stream)))


def _prefill_shapes(q, k, v, out):
    """Shapes of a prefill-family call: bf16 inputs (bf16 or fp32 output) or
    fp32 inputs and output; q/out [B,H,S,d], k/v [B,K,S_max,d]."""
    _need(q, "q", 4)
    _need(k, "k", 4)
    _need(v, "v", 4)
    _need(out, "out", 4)
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k and v must share a dtype")
    if q.dtype == torch.float32 and out.dtype != torch.float32:
        raise ValueError("fp32 inputs need an fp32 output")
    B, H, S, d = q.shape
    Bk, K, S_max, dk = k.shape
    if Bk != B or dk != d or v.shape != k.shape or tuple(out.shape) != (B, H, S, d):
        raise ValueError("shape mismatch between q, k, v and out")
    return B, H, S, d, K, S_max


def gqa_prefill_causal(q, k, v, out, scale: float, stream=None) -> None:
    """Causal GQA over a prefix: q/out [B,H,S,d], k/v [B,K,S_max,d] (rows < S used)."""
    B, H, S, d, K, S_max = _prefill_shapes(q, k, v, out)
    lib = load_library()
    _check("gqa_prefill_causal", lib.gqa_prefill_causal(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), B, H, K, S, S_max, d,
        float(scale), _DTYPE_CODE[q.dtype], _DTYPE_CODE[out.dtype], _stream(stream)))


def gqa_prefill_chunk(q, k_cache, v_cache, seq_lens, out, scale: float, stream=None) -> None:
    """Causal attention of the last S positions (q/out [B,H,S,d]) over caches
    [B,K,S_max,d] holding seq_lens[b] rows, the chunk included."""
    B, H, S, d, K, S_max = _prefill_shapes(q, k_cache, v_cache, out)
    _need(seq_lens, "seq_lens", 1, (torch.int32,))
    if seq_lens.numel() != B:
        raise ValueError("seq_lens must have B entries")
    _check("gqa_prefill_chunk", load_library().gqa_prefill_chunk(
        q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), seq_lens.data_ptr(), out.data_ptr(),
        B, H, K, S, S_max, d, float(scale), _DTYPE_CODE[q.dtype], _DTYPE_CODE[out.dtype], _stream(stream)))


def gqa_cross_attention(q, k, v, kv_lens, out, scale: float, stream=None) -> None:
    """Non-causal attention of q/out [B,H,S_q,d] over rows [0, kv_lens[b]) of
    k, v [B,K,S_max,d]."""
    B, H, S, d, K, S_max = _prefill_shapes(q, k, v, out)
    _need(kv_lens, "kv_lens", 1, (torch.int32,))
    if kv_lens.numel() != B:
        raise ValueError("kv_lens must have B entries")
    _check("gqa_cross_attention", load_library().gqa_cross_attention(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), kv_lens.data_ptr(), out.data_ptr(),
        B, H, K, S, S_max, d, float(scale), _DTYPE_CODE[q.dtype], _DTYPE_CODE[out.dtype], _stream(stream)))


def gqa_kv_append_rows(k_new, v_new, k_cache, v_cache, seq_lens, stream=None) -> None:
    """Append k_new/v_new [B,K,T,d] at rows [seq_lens[b], seq_lens[b] + T) of
    the caches [B,K,S_max,d] and add T to seq_lens."""
    _need(k_cache, "k_cache", 4)
    B, K, S_max, d = k_cache.shape
    _need(v_cache, "v_cache", 4)
    if v_cache.shape != k_cache.shape or v_cache.dtype != k_cache.dtype:
        raise ValueError("v_cache must match k_cache")
    _need(k_new, "k_new", 4)
    _need(v_new, "v_new", 4)
    T = k_new.shape[2]
    for t, nm in ((k_new, "k_new"), (v_new, "v_new")):
        if tuple(t.shape) != (B, K, T, d) or t.dtype != k_cache.dtype:
            raise ValueError(f"{nm} must be [B,K,T,d] of the cache dtype")
    _need(seq_lens, "seq_lens", 1, (torch.int32,))
    if seq_lens.numel() != B:
        raise ValueError("seq_lens must have B entries")
    _check("gqa_kv_append_rows", load_library().gqa_kv_append_rows(
        k_new.data_ptr(), v_new.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), seq_lens.data_ptr(),
        B, K, T, S_max, d, _DTYPE_CODE[k_cache.dtype], _stream(stream)))


def gqa_kv_project(x, w_kv, k_out, v_out, stream=None) -> None:
    """Project x [B,T,d_model] by W_KV [K,2d,d_model] into K and V rows
    k_out, v_out [B,K,T,d] (bf16)."""
    _need(x, "x", 3, (torch.bfloat16,))
    _need(w_kv, "w_kv", 3, (torch.bfloat16,))
    _need(k_out, "k_out", 4, (torch.bfloat16,))
    _need(v_out, "v_out", 4, (torch.bfloat16,))
    B, T, dm = x.shape
    K, d2, dmw = w_kv.shape
    d = d2 // 2
    if dmw != dm or tuple(k_out.shape) != (B, K, T, d) or v_out.shape != k_out.shape:
        raise ValueError("shape mismatch between x, w_kv and the outputs")
    _check("gqa_kv_project", load_library().gqa_kv_project(
        x.data_ptr(), w_kv.data_ptr(), k_out.data_ptr(), v_out.data_ptr(), B, T, dm, K, d, GQA_BF16,
        _stream(stream)))


def gqa_kv_project_workspace_bytes(B: int, T: int, d_model: int, K: int, d: int) -> int:
    return int(load_library().gqa_kv_project_workspace_bytes(B, T, d_model, K, d))


def gqa_kv_project_append(x, w_kv, k_cache, v_cache, seq_lens, workspace, stream=None) -> None:
    """Project x [B,T,d_model] by W_KV [K,2d,d_model] and append the K/V rows
    at seq_lens[b] of the caches [B,K,S_max,d]; add T to seq_lens.
    workspace: uint8 GPU tensor of gqa_kv_project_workspace_bytes(...) bytes."""
    _need(x, "x", 3, (torch.bfloat16,))
    _need(w_kv, "w_kv", 3, (torch.bfloat16,))
    _need(k_cache, "k_cache", 4, (torch.bfloat16,))
    _need(v_cache, "v_cache", 4, (torch.bfloat16,))
    _need(seq_lens, "seq_lens", 1, (torch.int32,))
    B, T, dm = x.shape
    Bk, K, S_max, d = k_cache.shape
    if v_cache.shape != k_cache.shape or Bk != B or tuple(w_kv.shape) != (K, 2 * d, dm) or seq_lens.numel() != B:
        raise ValueError("shape mismatch between x, w_kv, caches and seq_lens")
    _need(workspace, "workspace", 1, (torch.uint8,))
    _check("gqa_kv_project_append", load_library().gqa_kv_project_append(
        x.data_ptr(), w_kv.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), seq_lens.data_ptr(),
        workspace.data_ptr(), workspace.numel(), B, T, dm, K, S_max, d, GQA_BF16, _stream(stream)))


def gqa_meanpool_convert(src, dst, stream=None) -> None:
    """dst [outer,K,inner] = mean over each group of G consecutive heads of src [outer,H,inner]."""
    _need(src, "src", 3)
    _need(dst, "dst", 3)
    outer, H, inner = src.shape
    K = dst.shape[1]
    if dst.shape[0] != outer or dst.shape[2] != inner or dst.dtype != src.dtype:
        raise ValueError("dst must be [outer,K,inner] of the src dtype")
    lib = load_library()
    _check("gqa_meanpool_convert", lib.gqa_meanpool_convert(
        src.data_ptr(), dst.data_ptr(), outer, H, K, inner, _DTYPE_CODE[src.dtype], _stream(stream)))
