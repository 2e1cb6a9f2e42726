"""The C-ABI library: it loads, exports what include/gqa.h declares, and its
host-side logic (sizes, validation, error codes) behaves -- all without a GPU.

Every call here fails validation (or is host-only), so nothing is enqueued.
"""
import ctypes
import json
from pathlib import Path

import pytest

import grouped_query_kv_amd as gqa
from grouped_query_kv_amd import _binding as B
from grouped_query_kv_amd import _binding as B_

GOLDEN = Path(__file__).resolve().parent / "golden" / "kv_cache_bytes.json"
FAKE = 0x10000  # 16-byte aligned, never dereferenced (validation fails first)


@pytest.fixture(scope="module")
def lib():
    return gqa.load_library()


def test_exports_every_declared_symbol(lib):
    declared = gqa.header_symbols()
    assert {"gqa_kv_append", "gqa_decode", "gqa_decode_append", "gqa_prefill_causal",
            "gqa_meanpool_convert"} <= set(declared)
    for name in declared:
        assert hasattr(lib, name), f"libgqa.so does not export {name}"


def test_binding_signatures_match_header():
    """Every declaration in include/gqa.h has a binding signature with the
    same number of parameters and pointer/integer/float kinds."""
    import re
    text = B.HEADER.read_text()
    decls = re.findall(r"^(?:int|size_t|uint64_t|const char\s*\*)\s*(gqa_\w+)\s*\(([^;()]*)\)\s*;", text,
                       flags=re.M)
    assert len(decls) == len(B._SIGNATURES), sorted(set(B._SIGNATURES) ^ {n for n, _ in decls})
    for name, params in decls:
        ps = [x.strip() for x in params.replace("\n", " ").split(",")]
        ps = [] if ps == ["void"] else ps
        argtypes = B._SIGNATURES[name][1]
        assert len(ps) == len(argtypes), f"{name}: header {len(ps)} params, binding {len(argtypes)}"
        for decl, at in zip(ps, argtypes):
            if "*" in decl:
                kind = ctypes.c_void_p
            elif decl.startswith("float"):
                kind = ctypes.c_float
            elif decl.startswith(("int64_t", "uint64_t", "size_t")):
                kind = (ctypes.c_int64, ctypes.c_uint64, ctypes.c_size_t)
            else:
                kind = ctypes.c_int
            ok = at in kind if isinstance(kind, tuple) else at == kind
            assert ok, f"{name}: parameter '{decl}' bound as {at}"


def test_abi_version(lib):
    assert lib.gqa_abi_version() == 1


def test_kv_cache_bytes_matches_pages(lib):
    for e in json.loads(GOLDEN.read_text())["entries"]:
        got = gqa.gqa_kv_cache_bytes(e["layers"], e["kv_heads"], e["head_dim"], e["elem_bytes"], e["tokens"])
        if "exact_bytes" in e:
            assert got == e["exact_bytes"], e["what"]
        else:
            assert round(got / e["unit_bytes"], e["round_to"]) == e["approx"], e["what"]
    assert gqa.gqa_kv_cache_bytes(-1, 8, 128, 2, 1) == 0


def test_workspace_bytes(lib):
    assert gqa.gqa_decode_workspace_bytes(16, 32, 8, 8193, 128) > 0
    # invalid shapes -> 0
    assert gqa.gqa_decode_workspace_bytes(16, 30, 8, 8193, 128) == 0
    assert gqa.gqa_decode_workspace_bytes(16, 32, 8, 8193, 96) == 0
    assert gqa.gqa_decode_workspace_bytes(0, 32, 8, 8193, 128) == 0
    # grows with the context
    assert gqa.gqa_decode_workspace_bytes(4, 32, 8, 131072, 128) >= gqa.gqa_decode_workspace_bytes(4, 32, 8, 1024, 128)


def _decode(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, sl=FAKE, out=FAKE, ws=FAKE, wsb=1 << 30, B=2, H=8, K=2,
             S_max=64, max_seq_len=64, d=128, scale=0.088, dtype=B.GQA_BF16, out_dtype=B.GQA_BF16)
    a.update(kw)
    return lib.gqa_decode(a["q"], a["k"], a["v"], a["sl"], a["out"], a["ws"], a["wsb"], a["B"], a["H"],
                          a["K"], a["S_max"], a["max_seq_len"], a["d"], a["scale"], a["dtype"],
                          a["out_dtype"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), B.GQA_ERR_INVALID),
    (dict(out=None), B.GQA_ERR_INVALID),
    (dict(H=9, K=2), B.GQA_ERR_INVALID),
    (dict(H=2, K=4), B.GQA_ERR_INVALID),
    (dict(B=0), B.GQA_ERR_INVALID),
    (dict(d=96), B.GQA_ERR_UNSUPPORTED),
    (dict(dtype=7), B.GQA_ERR_UNSUPPORTED),
    (dict(dtype=B.GQA_F32, out_dtype=B.GQA_BF16), B.GQA_ERR_UNSUPPORTED),
    (dict(max_seq_len=65), B.GQA_ERR_INVALID),
    (dict(scale=float("nan")), B.GQA_ERR_INVALID),
    (dict(scale=-0.5), B.GQA_ERR_INVALID),
    (dict(scale=0.0), B.GQA_ERR_INVALID),
    (dict(q=FAKE + 2), B.GQA_ERR_INVALID),
    (dict(wsb=16), B.GQA_ERR_WORKSPACE),
    (dict(ws=None), B.GQA_ERR_WORKSPACE),
])
def test_decode_rejects(lib, kw, code):
    assert _decode(lib, **kw) == code
    assert lib.gqa_last_error().decode().startswith("gqa_decode")


@pytest.mark.parametrize("kn,vn,code", [(None, FAKE, B.GQA_ERR_INVALID), (FAKE, None, B.GQA_ERR_INVALID),
                                         (FAKE + 4, FAKE, B.GQA_ERR_INVALID)])
def test_decode_append_rejects(lib, kn, vn, code):
    rc = lib.gqa_decode_append(FAKE, kn, vn, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, 2, 8, 2, 64, 64, 128,
                               0.088, B.GQA_BF16, B.GQA_BF16, None)
    assert rc == code and lib.gqa_last_error().decode().startswith("gqa_decode_append")


@pytest.mark.parametrize("args,code", [
    ((None, FAKE, FAKE, FAKE, FAKE, 2, 8, 16, 128, B.GQA_BF16), B.GQA_ERR_INVALID),
    ((FAKE, FAKE, FAKE, FAKE, FAKE, 0, 8, 16, 128, B.GQA_BF16), B.GQA_ERR_INVALID),
    ((FAKE, FAKE, FAKE, FAKE, FAKE, 2, 8, 16, 80, B.GQA_BF16), B.GQA_ERR_UNSUPPORTED),
    ((FAKE, FAKE, FAKE, FAKE, FAKE, 2, 8, 16, 128, 5), B.GQA_ERR_UNSUPPORTED),
    ((FAKE, FAKE, FAKE + 8, FAKE, FAKE, 2, 8, 16, 128, B.GQA_BF16), B.GQA_ERR_INVALID),
    ((FAKE, FAKE, FAKE, FAKE, FAKE + 2, 2, 8, 16, 128, B.GQA_BF16), B.GQA_ERR_INVALID),
])
def test_append_rejects(lib, args, code):
    assert lib.gqa_kv_append(*args, None) == code


@pytest.mark.parametrize("args,code", [
    ((FAKE, FAKE, FAKE, FAKE, 1, 8, 2, 8, 16, 128, 0.1, B.GQA_F32, B.GQA_BF16), B.GQA_ERR_UNSUPPORTED),
    ((FAKE, FAKE, FAKE, FAKE, 1, 8, 2, 8, 16, 128, 0.1, 7, B.GQA_F32), B.GQA_ERR_UNSUPPORTED),
    ((FAKE, FAKE, FAKE, FAKE, 1, 8, 2, 8, 16, 128, float("nan"), B.GQA_F32, B.GQA_F32), B.GQA_ERR_INVALID),
    ((FAKE, FAKE, FAKE, FAKE, 1, 8, 3, 16, 16, 128, 0.1, B.GQA_F32, B.GQA_F32), B.GQA_ERR_INVALID),
    ((FAKE, FAKE, FAKE, FAKE, 1, 8, 2, 16, 8, 128, 0.1, B.GQA_BF16, B.GQA_BF16), B.GQA_ERR_INVALID),
    ((FAKE, FAKE, FAKE, FAKE, 1, 8, 3, 16, 16, 128, 0.1, B.GQA_BF16, B.GQA_BF16), B.GQA_ERR_INVALID),
    ((FAKE, FAKE, FAKE, None, 1, 8, 2, 16, 16, 128, 0.1, B.GQA_BF16, B.GQA_BF16), B.GQA_ERR_INVALID),
    ((FAKE, FAKE, FAKE, FAKE, 1, 8, 2, 16, 16, 32, 0.1, B.GQA_BF16, B.GQA_BF16), B.GQA_ERR_UNSUPPORTED),
    ((FAKE, FAKE, FAKE, FAKE, 1, 8, 2, 0, 16, 128, 0.1, B.GQA_BF16, B.GQA_BF16), B.GQA_ERR_INVALID),
])
def test_prefill_rejects(lib, args, code):
    assert lib.gqa_prefill_causal(*args, None) == code


@pytest.mark.parametrize("args,code", [
    ((None, FAKE, 4, 8, 2, 16, B.GQA_BF16), B.GQA_ERR_INVALID),
    ((FAKE, FAKE, 0, 8, 2, 16, B.GQA_BF16), B.GQA_ERR_INVALID),
    ((FAKE, FAKE, 4, 8, 3, 16, B.GQA_BF16), B.GQA_ERR_INVALID),
    ((FAKE, FAKE, 4, 8, 2, 16, 9), B.GQA_ERR_UNSUPPORTED),
    ((FAKE, FAKE + 4, 4, 8, 2, 16, B.GQA_F32), B.GQA_ERR_INVALID),
])
def test_meanpool_rejects(lib, args, code):
    assert lib.gqa_meanpool_convert(*args, None) == code


def _decode_paged(lib, **kw):
    a = dict(q=FAKE, kp=FAKE, vp=FAKE, bt=FAKE, sl=FAKE, out=FAKE, ws=FAKE, wsb=1 << 30, B=2, H=32, K=8,
             num_blocks=64, block_size=16, max_blocks=8, max_seq_len=128, d=128, scale=0.088,
             dtype=B.GQA_BF16, out_dtype=B.GQA_BF16)
    a.update(kw)
    return lib.gqa_decode_paged(a["q"], a["kp"], a["vp"], a["bt"], a["sl"], a["out"], a["ws"], a["wsb"],
                                a["B"], a["H"], a["K"], a["num_blocks"], a["block_size"], a["max_blocks"],
                                a["max_seq_len"], a["d"], a["scale"], a["dtype"], a["out_dtype"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(bt=None), B.GQA_ERR_INVALID),
    (dict(block_size=8), B.GQA_ERR_UNSUPPORTED),
    (dict(block_size=24), B.GQA_ERR_UNSUPPORTED),
    (dict(num_blocks=0), B.GQA_ERR_INVALID),
    (dict(max_blocks=0), B.GQA_ERR_INVALID),
    (dict(max_seq_len=129), B.GQA_ERR_INVALID),
    (dict(dtype=B.GQA_F32, out_dtype=B.GQA_F32), B.GQA_ERR_UNSUPPORTED),
    (dict(H=30), B.GQA_ERR_INVALID),
    (dict(scale=float("inf")), B.GQA_ERR_INVALID),
    (dict(bt=FAKE + 2), B.GQA_ERR_INVALID),
    (dict(wsb=64), B.GQA_ERR_WORKSPACE),
])
def test_decode_paged_rejects(lib, kw, code):
    assert _decode_paged(lib, **kw) == code
    assert lib.gqa_last_error().decode().startswith("gqa_decode_paged")


def _decode_append_paged(lib, **kw):
    a = dict(q=FAKE, kn=FAKE, vn=FAKE, kp=FAKE, vp=FAKE, bt=FAKE, sl=FAKE, out=FAKE, ws=FAKE, wsb=1 << 30, B=2,
             H=32, K=8, num_blocks=64, block_size=16, max_blocks=8, max_seq_len=128, d=128, scale=0.088,
             dtype=B.GQA_BF16, out_dtype=B.GQA_BF16)
    a.update(kw)
    return lib.gqa_decode_append_paged(a["q"], a["kn"], a["vn"], a["kp"], a["vp"], a["bt"], a["sl"], a["out"],
                                       a["ws"], a["wsb"], a["B"], a["H"], a["K"], a["num_blocks"],
                                       a["block_size"], a["max_blocks"], a["max_seq_len"], a["d"], a["scale"],
                                       a["dtype"], a["out_dtype"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(kn=None), B.GQA_ERR_INVALID),
    (dict(vn=None), B.GQA_ERR_INVALID),
    (dict(kn=FAKE + 8), B.GQA_ERR_INVALID),
    (dict(bt=None), B.GQA_ERR_INVALID),
    (dict(block_size=24), B.GQA_ERR_UNSUPPORTED),
    (dict(max_seq_len=129), B.GQA_ERR_INVALID),
    (dict(dtype=B.GQA_F32, out_dtype=B.GQA_F32), B.GQA_ERR_UNSUPPORTED),
    (dict(wsb=64), B.GQA_ERR_WORKSPACE),
])
def test_decode_append_paged_rejects(lib, kw, code):
    assert _decode_append_paged(lib, **kw) == code
    assert lib.gqa_last_error().decode().startswith("gqa_decode_append_paged")


def test_paged_workspace_bytes(lib):
    # partitions are capped at 63 blocks, so a long context with few heads
    # needs more partial rows than the contiguous plan
    assert lib.gqa_decode_paged_workspace_bytes(1, 8, 8, 1 << 20, 128, 16) > 0
    assert lib.gqa_decode_paged_workspace_bytes(64, 8, 8, 1 << 17, 128, 16) > \
        lib.gqa_decode_workspace_bytes(64, 8, 8, 1 << 17, 128)
    assert lib.gqa_decode_paged_workspace_bytes(1, 8, 8, 100, 128, 8) == 0
    assert lib.gqa_decode_paged_workspace_bytes(1, 8, 3, 100, 128, 16) == 0


@pytest.mark.parametrize("args,code", [
    ((None, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 8, 64, 16, 8, 128, B.GQA_BF16), B.GQA_ERR_INVALID),
    ((FAKE, FAKE, FAKE, FAKE, None, FAKE, 2, 8, 64, 16, 8, 128, B.GQA_BF16), B.GQA_ERR_INVALID),
    ((FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 8, 64, 12, 8, 128, B.GQA_BF16), B.GQA_ERR_UNSUPPORTED),
    ((FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 8, 0, 16, 8, 128, B.GQA_BF16), B.GQA_ERR_INVALID),
    ((FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 8, 64, 16, 8, 96, B.GQA_BF16), B.GQA_ERR_UNSUPPORTED),
    ((FAKE, FAKE, FAKE, FAKE, FAKE, FAKE + 2, 2, 8, 64, 16, 8, 128, B.GQA_BF16), B.GQA_ERR_INVALID),
])
def test_append_paged_rejects(lib, args, code):
    assert lib.gqa_kv_append_paged(*args, None) == code
    assert lib.gqa_last_error().decode().startswith("gqa_kv_append_paged")


def _decode_int8(lib, **kw):
    a = dict(q=FAKE, kc=FAKE, vc=FAKE, ks=FAKE, vs=FAKE, sl=FAKE, out=FAKE, ws=FAKE, wsb=1 << 30, B=2, H=32,
             K=8, S_max=128, max_seq_len=100, d=128, scale=0.088, q_dtype=B.GQA_BF16, out_dtype=B.GQA_BF16)
    a.update(kw)
    return lib.gqa_decode_int8(a["q"], a["kc"], a["vc"], a["ks"], a["vs"], a["sl"], a["out"], a["ws"], a["wsb"],
                               a["B"], a["H"], a["K"], a["S_max"], a["max_seq_len"], a["d"], a["scale"],
                               a["q_dtype"], a["out_dtype"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(ks=None), B.GQA_ERR_INVALID),
    (dict(S_max=130, max_seq_len=100), B.GQA_ERR_INVALID),   # scale rows need S_max % 4 == 0
    (dict(max_seq_len=129), B.GQA_ERR_INVALID),
    (dict(q_dtype=B.GQA_F32), B.GQA_ERR_UNSUPPORTED),
    (dict(out_dtype=5), B.GQA_ERR_UNSUPPORTED),
    (dict(d=96), B.GQA_ERR_UNSUPPORTED),
    (dict(vs=FAKE + 4), B.GQA_ERR_INVALID),
    (dict(scale=-1.0), B.GQA_ERR_INVALID),
    (dict(wsb=32), B.GQA_ERR_WORKSPACE),
])
def test_decode_int8_rejects(lib, kw, code):
    assert _decode_int8(lib, **kw) == code
    assert lib.gqa_last_error().decode().startswith("gqa_decode_int8")


def _decode_append_int8(lib, **kw):
    a = dict(q=FAKE, kn=FAKE, vn=FAKE, kc=FAKE, vc=FAKE, ks=FAKE, vs=FAKE, sl=FAKE, out=FAKE, ws=FAKE,
             wsb=1 << 30, B=2, H=32, K=8, S_max=128, max_seq_len=100, d=128, scale=0.088,
             dtype=B.GQA_BF16, out_dtype=B.GQA_BF16)
    a.update(kw)
    return lib.gqa_decode_append_int8(a["q"], a["kn"], a["vn"], a["kc"], a["vc"], a["ks"], a["vs"], a["sl"],
                                      a["out"], a["ws"], a["wsb"], a["B"], a["H"], a["K"], a["S_max"],
                                      a["max_seq_len"], a["d"], a["scale"], a["dtype"], a["out_dtype"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(kn=None), B.GQA_ERR_INVALID),
    (dict(vn=None), B.GQA_ERR_INVALID),
    (dict(vn=FAKE + 8), B.GQA_ERR_INVALID),
    (dict(dtype=B.GQA_F32), B.GQA_ERR_UNSUPPORTED),
    (dict(S_max=130, max_seq_len=100), B.GQA_ERR_INVALID),
    (dict(d=96), B.GQA_ERR_UNSUPPORTED),
    (dict(wsb=32), B.GQA_ERR_WORKSPACE),
])
def test_decode_append_int8_rejects(lib, kw, code):
    assert _decode_append_int8(lib, **kw) == code
    assert lib.gqa_last_error().decode().startswith("gqa_decode_append_int8")


@pytest.mark.parametrize("args,code", [
    ((None, FAKE, FAKE, 10, 128, B.GQA_BF16), B.GQA_ERR_INVALID),
    ((FAKE, FAKE, FAKE, 0, 128, B.GQA_BF16), B.GQA_ERR_INVALID),
    ((FAKE, FAKE, FAKE, 10, 32, B.GQA_BF16), B.GQA_ERR_UNSUPPORTED),
    ((FAKE, FAKE, FAKE, 10, 128, 3), B.GQA_ERR_UNSUPPORTED),
    ((FAKE + 8, FAKE, FAKE, 10, 128, B.GQA_BF16), B.GQA_ERR_INVALID),
    ((FAKE, FAKE + 4, FAKE, 10, 128, B.GQA_BF16), B.GQA_ERR_INVALID),
])
def test_quantize_int8_rejects(lib, args, code):
    assert lib.gqa_kv_quantize_int8(*args, None) == code


@pytest.mark.parametrize("args,code", [
    ((FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, 2, 8, 16, 128, B.GQA_BF16), B.GQA_ERR_INVALID),
    ((FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 8, 0, 128, B.GQA_BF16), B.GQA_ERR_INVALID),
    ((FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 8, 16, 128, 7), B.GQA_ERR_UNSUPPORTED),
    ((FAKE, FAKE, FAKE + 2, FAKE, FAKE, FAKE, FAKE, 2, 8, 16, 128, B.GQA_BF16), B.GQA_ERR_INVALID),
])
def test_append_int8_rejects(lib, args, code):
    assert lib.gqa_kv_append_int8(*args, None) == code


@pytest.mark.parametrize("args,code", [
    ((None, FAKE, FAKE, FAKE, 16, 1, 4096, 8, 128, B.GQA_BF16), B.GQA_ERR_INVALID),
    ((FAKE, FAKE, FAKE, FAKE, 16, 1, 100, 8, 128, B.GQA_BF16), B.GQA_ERR_UNSUPPORTED),
    ((FAKE, FAKE, FAKE, FAKE, 16, 0, 4096, 8, 128, B.GQA_BF16), B.GQA_ERR_INVALID),
    ((FAKE, FAKE + 8, FAKE, FAKE, 16, 1, 4096, 8, 128, B.GQA_BF16), B.GQA_ERR_INVALID),
    ((FAKE, FAKE, FAKE + 1, FAKE, 16, 1, 4096, 8, 128, B.GQA_BF16), B.GQA_ERR_INVALID),
])
def test_project_only_rejects(lib, args, code):
    assert lib.gqa_kv_project(*args, None) == code



@pytest.mark.parametrize("args,code", [
    ((None, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, 2, 1, 4096, 8, 64, 128, B.GQA_BF16), B.GQA_ERR_INVALID),
    ((FAKE, FAKE, FAKE, FAKE, None, FAKE, 1 << 30, 2, 1, 4096, 8, 64, 128, B.GQA_BF16), B.GQA_ERR_INVALID),
    ((FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, 2, 0, 4096, 8, 64, 128, B.GQA_BF16), B.GQA_ERR_INVALID),
    ((FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, 2, 1, 4004, 8, 64, 128, B.GQA_BF16), B.GQA_ERR_UNSUPPORTED),
    ((FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, 2, 1, 4096, 8, 64, 96, B.GQA_BF16), B.GQA_ERR_UNSUPPORTED),
    ((FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, 2, 1, 4096, 8, 64, 128, B.GQA_F32), B.GQA_ERR_UNSUPPORTED),
    ((FAKE + 2, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, 2, 1, 4096, 8, 64, 128, B.GQA_BF16), B.GQA_ERR_INVALID),
    ((FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1024, 2, 1, 4096, 8, 64, 128, B.GQA_BF16), B.GQA_ERR_WORKSPACE),
    ((FAKE, FAKE, FAKE, FAKE, FAKE, None, 1 << 30, 2, 1, 4096, 8, 64, 128, B.GQA_BF16), B.GQA_ERR_WORKSPACE),
])
def test_project_rejects(lib, args, code):
    assert lib.gqa_kv_project_append(*args, None) == code
    assert lib.gqa_last_error().decode().startswith("gqa_kv_project_append")


def test_project_workspace_bytes(lib):
    # the projected K and V rows, bf16
    assert lib.gqa_kv_project_workspace_bytes(16, 1, 4096, 8, 128) == 2 * 16 * 8 * 128 * 2
    assert lib.gqa_kv_project_workspace_bytes(2, 2048, 4096, 8, 128) == 2 * 2 * 2048 * 8 * 128 * 2
    assert lib.gqa_kv_project_workspace_bytes(16, 1, 4004, 8, 128) == 0
    assert lib.gqa_kv_project_workspace_bytes(16, 1, 4096, 8, 96) == 0


@pytest.mark.parametrize("fn", ["gqa_prefill_chunk", "gqa_cross_attention"])
@pytest.mark.parametrize("kw,code", [
    (dict(lens=None), B.GQA_ERR_INVALID),
    (dict(S=0), B.GQA_ERR_INVALID),
    (dict(H=12, K=8), B.GQA_ERR_INVALID),
    (dict(d=80), B.GQA_ERR_UNSUPPORTED),
    (dict(dtype=B.GQA_F32), B.GQA_ERR_UNSUPPORTED),
    (dict(scale=0.0), B.GQA_ERR_INVALID),
    (dict(lens=FAKE + 2), B.GQA_ERR_INVALID),
])
def test_chunk_cross_reject(lib, fn, kw, code):
    a = dict(lens=FAKE, S=64, H=32, K=8, d=128, dtype=B.GQA_BF16, scale=0.088)
    a.update(kw)
    f = getattr(lib, fn)
    if fn == "gqa_prefill_chunk":
        rc = f(FAKE, FAKE, FAKE, a["lens"], FAKE, 2, a["H"], a["K"], a["S"], 128, a["d"], a["scale"],
               a["dtype"], B.GQA_BF16, None)
    else:
        rc = f(FAKE, FAKE, FAKE, a["lens"], FAKE, 2, a["H"], a["K"], a["S"], 128, a["d"], a["scale"],
               a["dtype"], B.GQA_BF16, None)
    assert rc == code and lib.gqa_last_error().decode().startswith(fn)


@pytest.mark.parametrize("args,code", [
    ((None, FAKE, FAKE, FAKE, FAKE, 2, 8, 4, 64, 128, B.GQA_BF16), B.GQA_ERR_INVALID),
    ((FAKE, FAKE, FAKE, FAKE, FAKE, 2, 8, 0, 64, 128, B.GQA_BF16), B.GQA_ERR_INVALID),
    ((FAKE, FAKE, FAKE, FAKE, FAKE, 2, 8, 4, 64, 32, B.GQA_BF16), B.GQA_ERR_UNSUPPORTED),
    ((FAKE, FAKE, FAKE, FAKE, FAKE + 1, 2, 8, 4, 64, 128, B.GQA_BF16), B.GQA_ERR_INVALID),
])
def test_append_rows_rejects(lib, args, code):
    assert lib.gqa_kv_append_rows(*args, None) == code


def test_timing_events_need_both(lib):
    assert lib.gqa_set_timing_events(FAKE, None) == B.GQA_ERR_INVALID
    assert lib.gqa_set_timing_events(None, None) == B.GQA_OK


def test_binding_refuses_cpu_tensors():
    import torch
    x = torch.zeros(2, 8, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        gqa.gqa_meanpool_convert(torch.zeros(2, 8, 4), torch.zeros(2, 2, 4))
    with pytest.raises(ValueError):
        gqa.gqa_decode(x, x[:, None], x[:, None], torch.zeros(2, dtype=torch.int32), x,
                       torch.zeros(16, dtype=torch.uint8), 8, scale=0.1)


def test_binding_needs_an_explicit_scale():
    """The binding passes the caller's scale through; it never derives one."""
    import inspect
    for fn in (gqa.gqa_decode, gqa.gqa_decode_append, gqa.gqa_decode_paged, gqa.gqa_decode_append_paged,
               gqa.gqa_decode_int8, gqa.gqa_decode_append_int8, gqa.gqa_prefill_causal,
               gqa.gqa_prefill_chunk, gqa.gqa_cross_attention):
        p = inspect.signature(fn).parameters["scale"]
        assert p.default is inspect.Parameter.empty, fn.__name__


def test_build_id_matches_the_sources(lib):
    """The loaded library was built from the sources in this tree."""
    from grouped_query_kv_amd.build import build_id
    assert lib.gqa_build_id().decode() == build_id()
    assert len(build_id()) == 64


def test_stale_library_is_refused(monkeypatch):
    """A library whose code hash differs from the tree's sources is not used."""
    import grouped_query_kv_amd.build as bld
    monkeypatch.setattr(B, "_lib", None)
    monkeypatch.setattr(bld, "build_id", lambda: "0" * 64)
    with pytest.raises(RuntimeError, match="built from other sources"):
        B.load_library()
    monkeypatch.undo()
    B._lib = None
    B.load_library()


def test_build_id_ignores_comments_only(tmp_path):
    from grouped_query_kv_amd.build import code_sha256
    a = tmp_path / "a.hip"
    a.write_text("int f() { return 1; }  // one\n")
    h0 = code_sha256([a])
    a.write_text("/* note */ int f() {\n  return 1;\n}\n")
    assert code_sha256([a]) == h0
    a.write_text("int f() { return 2; }\n")
    assert code_sha256([a]) != h0


def test_missing_library_fails_loudly(tmp_path, monkeypatch):
    monkeypatch.setattr(B, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        B.load_library(tmp_path / "nope.so")


def test_library_has_every_kernel_launch_stub(lib):
    """No kernel's host launch stub is left undefined in the built library."""
    import subprocess
    from grouped_query_kv_amd.build import LIB
    r = subprocess.run(["nm", "-u", str(LIB)], capture_output=True, text=True, check=True)
    assert "__device_stub__" not in r.stdout


def test_build_rejects_undefined_launch_stub(tmp_path):
    """The build's link check fails on a library that references a launch
    stub it does not define (what a silently dropped host stub looks like)."""
    import shutil
    import subprocess
    from grouped_query_kv_amd.build import _check_launch_stubs
    if shutil.which("gcc") is None or shutil.which("nm") is None:
        pytest.skip("gcc / nm not available")
    src = tmp_path / "stub.c"
    src.write_text("extern void _ZN3gqa20__device_stub__probeEv(void);\n"
                   "void call_it(void) { _ZN3gqa20__device_stub__probeEv(); }\n")
    so = tmp_path / "libstub.so"
    subprocess.run(["gcc", "-shared", "-fPIC", "-o", str(so), str(src)], check=True)
    with pytest.raises(RuntimeError, match="launch stubs are undefined"):
        _check_launch_stubs(so)


def test_noalloc_rejects_sizes_beyond_the_static_scratch(lib):
    """gqa_decode_append_noalloc refuses sizes whose partials exceed its
    64 MiB static scratch, on the host, before any HIP call."""
    B, H, K, d = 4096, 128, 8, 128
    assert lib.gqa_decode_workspace_bytes(B, H, K, 4096, d) > 64 << 20
    code = lib.gqa_decode_append_noalloc(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, B, H, K, 4096, 4096, d,
                                         0.1, B_.GQA_BF16, B_.GQA_BF16, None)
    assert code == B_.GQA_ERR_WORKSPACE
    assert "static scratch holds" in lib.gqa_last_error().decode()
    # invalid arguments are still reported as such (validation comes first)
    assert lib.gqa_decode_append_noalloc(FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 8, 2, 64, 64, 128,
                                         0.1, B_.GQA_BF16, B_.GQA_BF16, None) == B_.GQA_ERR_INVALID
    assert lib.gqa_decode_append_noalloc(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 8, 3, 64, 64, 128,
                                         0.1, B_.GQA_BF16, B_.GQA_BF16, None) == B_.GQA_ERR_INVALID
