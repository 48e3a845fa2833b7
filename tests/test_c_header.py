"""The C ABI from C: include/pfa_attn.h compiles as strict C99 (no HIP or C++
headers needed) and a C program linked against the library gets the
documented status codes from argument checks that fail before any launch
(runs without a GPU)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INCLUDE = os.path.join(ROOT, "include")
LIBDIR = os.path.join(ROOT, "precision_flash_attention_attn_amd", "_lib")

PROGRAM = r"""
#include <stdio.h>
#include <string.h>
#include "pfa_attn.h"

#define CHECK(cond) do { if (!(cond)) { printf("FAIL line %d: %s\n", __LINE__, #cond); return 1; } } while (0)

int main(void) {
  void* fake = (void*)0x10000;  /* 16-byte aligned, never dereferenced: the checks fail first */
  size_t need;
  pfa_tie_opts opts;
  CHECK(strncmp(attn_version(), "pfa_attn", 8) == 0);
  CHECK(strcmp(attn_strerror(PFA_OK), "ok") == 0);
  CHECK(attn_bwd_workspace_bytes(1, 16, 8192, 128, PFA_BF16_OUT) == (size_t)16 * 8192 * 4);
  CHECK(attn_bwd_workspace_bytes(1, 1, 1, 96, PFA_BF16_OUT) == 0);
  CHECK(attn_bwd_noalloc_max_bytes() == ((size_t)72 << 20));
  /* forward: NULL q, unsupported head size, bad tie options */
  CHECK(attn_fwd(NULL, fake, fake, fake, fake, NULL, 1, 1, 128, 64, 1, 0.125f, PFA_BF16_OUT, NULL, NULL)
        == PFA_ERR_INVALID);
  CHECK(attn_fwd(fake, fake, fake, fake, fake, NULL, 1, 1, 128, 80, 1, 0.125f, PFA_BF16_OUT, NULL, NULL)
        == PFA_ERR_UNSUPPORTED);
  opts.beta = 0.5f;
  opts.eps = 1e-3f;
  CHECK(attn_fwd(fake, fake, fake, fake, fake, NULL, 1, 1, 128, 64, 1, 0.125f, PFA_TIE_AWARE_SOFTMAX, &opts,
                 NULL) == PFA_ERR_INVALID);
  /* backward: too small a workspace, unknown mode */
  need = attn_bwd_workspace_bytes(1, 1, 128, 64, PFA_BF16_OUT);
  CHECK(attn_bwd(fake, fake, fake, fake, fake, (const float*)fake, fake, fake, fake, NULL, fake, need - 1,
                 1, 1, 128, 64, 1, 0.125f, PFA_BF16_OUT, NULL) == PFA_ERR_INVALID);
  CHECK(attn_bwd(fake, fake, fake, fake, fake, (const float*)fake, fake, fake, fake, NULL, fake, need,
                 1, 1, 128, 64, 1, 0.125f, 7, NULL) == PFA_ERR_INVALID);
  CHECK(attn_bwd_dq_delta(fake, fake, fake, NULL, fake, (const float*)fake, fake, NULL, fake, need,
                          1, 1, 128, 64, 1, 0.125f, PFA_BF16_OUT, NULL) == PFA_ERR_INVALID);
  /* the allocation-free backward refuses problems beyond its static scratch */
  CHECK(attn_bwd_noalloc(fake, fake, fake, fake, fake, (const float*)fake, fake, fake, fake, NULL,
                         64, 64, 8192, 128, 1, 0.088f, PFA_FP32_OUT, NULL) == PFA_ERR_SCRATCH);
  printf("ok\n");
  return 0;
}
"""


@pytest.fixture(scope="module")
def lib_built():
    so = os.path.join(LIBDIR, "libpfa_attn.so")
    if not os.path.exists(so):
        from precision_flash_attention_attn_amd.build import build_library
        build_library()
    return so


def test_header_is_plain_c99(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no C compiler")
    src = tmp_path / "h.c"
    src.write_text('#include "pfa_attn.h"\nint main(void) { return PFA_OK; }\n')
    r = subprocess.run([gcc, "-std=c99", "-pedantic", "-Wall", "-Wextra", "-Werror", f"-I{INCLUDE}", "-c",
                        str(src), "-o", str(tmp_path / "h.o")], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_c_program_gets_the_documented_status_codes(tmp_path, lib_built):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no C compiler")
    src = tmp_path / "prog.c"
    src.write_text(PROGRAM)
    exe = tmp_path / "prog"
    r = subprocess.run([gcc, "-std=c99", "-Wall", "-Werror", f"-I{INCLUDE}", str(src), "-o", str(exe),
                        f"-L{LIBDIR}", "-lpfa_attn", f"-Wl,-rpath,{LIBDIR}"], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0 and run.stdout.strip().endswith("ok"), run.stdout + run.stderr
