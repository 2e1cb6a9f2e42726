"""include/gqa.h is a plain C header: a C99 program that includes it compiles
with warnings as errors, links against libgqa.so and gets the documented
error codes back from host-side validation (no GPU needed)."""
import shutil
import subprocess

import pytest

from grouped_query_kv_amd import _binding as B

C_SRC = r"""
#include <stdio.h>
#include <string.h>
#include "gqa.h"

int main(void) {
  int fails = 0;
  if (gqa_abi_version() != 1) { puts("abi version"); fails++; }
  /* null pointers are rejected before anything is enqueued */
  if (gqa_decode(NULL, NULL, NULL, NULL, NULL, NULL, 0, 2, 32, 8, 64, 64, 128, 0.088f,
                 GQA_BF16, GQA_BF16, NULL) != GQA_ERR_INVALID) { puts("decode null"); fails++; }
  if (strncmp(gqa_last_error(), "gqa_decode", 10) != 0) { puts("last error"); fails++; }
  /* unsupported head dimension */
  if (gqa_prefill_causal((void*)0x10000, (void*)0x10000, (void*)0x10000, (void*)0x10000, 1, 8, 2, 16,
                         16, 96, 0.1f, GQA_BF16, GQA_BF16, NULL) != GQA_ERR_UNSUPPORTED) { puts("prefill d"); fails++; }
  /* the pages' KV-cache closed form: 32 layers, 32 KV heads, d = 128, bf16 */
  if (gqa_kv_cache_bytes(32, 32, 128, 2, 1) != 524288u) { puts("kv bytes"); fails++; }
  if (gqa_decode_workspace_bytes(16, 32, 8, 8193, 128) == 0) { puts("workspace"); fails++; }
  if (gqa_decode_workspace_bytes(16, 30, 8, 8193, 128) != 0) { puts("workspace H%K"); fails++; }
  printf("%s\n", fails ? "FAIL" : "OK");
  return fails;
}
"""


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no C compiler")
def test_header_is_c99_and_links(tmp_path):
    if not B.LIB_PATH.exists():
        pytest.skip("libgqa.so not built")
    src = tmp_path / "abi.c"
    src.write_text(C_SRC)
    exe = tmp_path / "abi"
    lib_dir = B.LIB_PATH.parent
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", f"-I{B.HEADER.parent}", str(src),
           f"-L{lib_dir}", "-lgqa", f"-Wl,-rpath,{lib_dir}", "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0 and r.stdout.strip().endswith("OK"), r.stdout + r.stderr
