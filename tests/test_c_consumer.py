"""The boundary from plain C (no GPU needed): include/fa.h compiles as C99, and a C program linked against
libfa.so takes the address of every declared entry point and gets validation errors back without a device."""
import os
import re
import shutil
import subprocess

import pytest

from tiled_online_softmax_amd import fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    text = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "fa.h")).read(), flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z0-9_]+)\s*\(", text)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_c_program_links_and_validates(tmp_path):
    names = _declared()
    src = tmp_path / "consumer.c"
    refs = ("  typedef void (*fn)(void);\n  fn volatile table[] = {" + ", ".join(f"(fn){n}" for n in names) + "};\n"
            f"  for (int i = 0; i < {len(names)}; ++i)\n    if (!table[i]) return 10;")
    src.write_text(f"""#include <stdio.h>
#include <string.h>
#include "fa.h"
int main(void) {{
{refs}
  /* a NULL pointer fails validation before any HIP call */
  int s = fa_fwd(NULL, NULL, NULL, NULL, NULL, 1, 1, 16, 64, 0, 0.125f, FA_BF16, NULL);
  if (s != FA_ERR_INVALID_ARG) return 1;
  if (strstr(fa_last_error(), "NULL") == NULL) return 2;
  if (strcmp(fa_status_string(FA_OK), "FA_OK") != 0) return 3;
  if (fa_bwd_workspace_size(1, 1, 16, 64, FA_F32, FA_BWD_DETERMINISTIC) != 0) return 4;  /* invalid: not bf16 */
  if (fa_bwd_workspace_size(1, 1, 16, 64, FA_BF16, FA_BWD_DETERMINISTIC) == 0) return 5;
  printf("ok %d\\n", (int)(sizeof(void*)));
  return 0;
}}
""")
    libdir = os.path.dirname(fa.LIB_PATH)
    exe = tmp_path / "consumer"
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-I", os.path.join(ROOT, "include"), str(src),
           fa.LIB_PATH, f"-Wl,-rpath,{libdir}", "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0 and r.stdout.startswith("ok"), (r.returncode, r.stdout, r.stderr)
