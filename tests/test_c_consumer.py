"""A plain C99 program built against include/ssm_scan.h and linked with libssmscan.so (no GPU
needed: it calls only the entry points that answer on the host, and the argument checks that
run before any launch)."""
import os
import shutil
import subprocess

import pytest

from selective_state_space_76_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

PROGRAM = r"""
#include <stdio.h>
#include <string.h>
#include "ssm_scan.h"

int main(void) {
  if (ssm_abi_version() != SSM_ABI_VERSION) return 1;
  if (strcmp(ssm_status_str(SSM_OK), "ok") != 0) return 2;
  ssm_shape s = {8, 1536, 16, 2048, SSM_BF16, 0};
  if (ssm_scan_workspace_size(&s) != 0) return 3;             /* enough channels: no split */
  if (ssm_scan_bwd_workspace_size(&s) <= ssm_scan_bwd_saved_workspace_size(&s)) return 4;
  ssm_shape longseq = {1, 1024, 16, 1 << 20, SSM_BF16, 0};
  if (ssm_scan_workspace_size(&longseq) == 0) return 5;      /* few channels, long sequence: split */
  if (ssm_scan_fwd(NULL, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0) != SSM_ERR_NULL) return 6;
  ssm_shape bad = {2, 64, 65, 128, SSM_BF16, 0};              /* dstate above 64 */
  char buf[64];
  void* p = (void*)(((unsigned long)buf + 15) & ~15ul);
  if (ssm_scan_fwd(&bad, p, p, p, p, p, 0, 0, 0, 0, p, 0, 0, 0, 0) != SSM_ERR_SHAPE) return 7;
  if (ssm_state_update(1, 1, 16, 7, 0, p, p, p, p, p, p, 0, 0, 0, p, 0) != SSM_ERR_DTYPE) return 8;
  if (ssm_conv1d_fwd(1, 4, 16, 5, SSM_BF16, p, p, 0, 0, p, 0, 0) != SSM_ERR_SHAPE) return 9;
  printf("c consumer ok\n");
  return 0;
}
"""


def test_c_program_against_header_and_library(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no gcc")
    L.load()  # raises when the library has not been built
    src = tmp_path / "consumer.c"
    src.write_text(PROGRAM)
    exe = tmp_path / "consumer"
    libdir = os.path.dirname(L.LIB_PATH)
    cmd = [gcc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-I", os.path.join(ROOT, "include"), str(src),
           "-o", str(exe), "-L", libdir, "-lssmscan", "-Wl,-rpath," + libdir]
    subprocess.run(cmd, check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, (r.returncode, r.stdout, r.stderr)
    assert "c consumer ok" in r.stdout
