"""The boundary from C: include/kda.h compiles as C99 with warnings as errors, a C
program links against libkda.so and calls the host-only entry points (workspace
sizes, the scan plan, the status strings) and the argument checks of the launching
ones, which reject bad arguments on the host before touching the GPU.  Runs on the CPU."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIBDIR = os.path.join(ROOT, "gated_delta_rule_chunked_amd")

C_SRC = r"""
#include <stdio.h>
#include <string.h>
#include "kda.h"

static int fail(const char* what) { fprintf(stderr, "FAIL %s\n", what); return 1; }

int main(void) {
  kda_fwd_args a;
  size_t bytes = 0;
  int32_t plan = -1;
  memset(&a, 0, sizeof a);
  a.B = 1; a.T = 8192; a.HQK = 32; a.HV = 32; a.K = 128; a.V = 128; a.N = 1;
  a.scale = 0.08838834764831845f;
  if (kda_fwd_workspace_bytes(&a, &bytes) != KDA_OK || bytes == 0) return fail("workspace size");
  if (kda_fwd_scan_plan(&a, &plan) != KDA_OK || plan != 32) return fail("scan plan");
  a.K = 96;
  if (kda_fwd_workspace_bytes(&a, &bytes) != KDA_ERR_UNSUPPORTED) return fail("K = 96 rejected");
  a.K = 128;
  /* no tensors: the launching entry points refuse on the host */
  if (kda_fwd(&a) != KDA_ERR_INVALID_ARG) return fail("kda_fwd without tensors");
  if (kda_fwd_no_alloc(&a) != KDA_ERR_TOO_LARGE) return fail("kda_fwd_no_alloc beyond its scratch");
  a.T = 256; a.HQK = 2; a.HV = 2;
  if (kda_fwd_no_alloc(&a) != KDA_ERR_INVALID_ARG) return fail("kda_fwd_no_alloc without tensors");
  a.T = 8192; a.HQK = 32; a.HV = 32;
  if (kda_fwd(NULL) != KDA_ERR_INVALID_ARG) return fail("kda_fwd(NULL)");
  {
    kda_bwd_dhu_args b;
    memset(&b, 0, sizeof b);
    b.B = 1; b.T = 8192; b.HV = 32; b.K = 128; b.V = 128; b.N = 1;
    if (kda_bwd_dhu_workspace_bytes(&b, &bytes) != KDA_OK) return fail("bwd workspace size");
    if (kda_bwd_dhu(&b) != KDA_ERR_INVALID_ARG) return fail("kda_bwd_dhu without tensors");
  }
  if (strlen(kda_strerror(KDA_ERR_TOO_LARGE)) == 0 || strlen(kda_strerror(KDA_OK)) == 0) return fail("strerror");
  printf("ok %zu %d\n", bytes, (int)plan);
  return 0;
}
"""


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_header_compiles_as_c99_and_links(tmp_path):
    lib = os.path.join(LIBDIR, "libkda.so")
    if not os.path.exists(lib):
        pytest.skip("libkda.so not built")
    src = tmp_path / "use_kda.c"
    src.write_text(C_SRC)
    exe = tmp_path / "use_kda"
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I", os.path.join(ROOT, "include"),
           str(src), "-L", LIBDIR, "-lkda", f"-Wl,-rpath,{LIBDIR}", "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.startswith("ok ")
