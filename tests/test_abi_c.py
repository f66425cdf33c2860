"""The C ABI from plain C: a C11 program includes include/sa.h (compiled by gcc
as C, not C++), links libsa.so and calls the admission and error paths, which
return before touching a GPU.  This checks that the header is valid C and that
every status comes back through the C calling convention."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIBDIR = os.path.join(ROOT, "causal_streaming_attention_amd")

C_SRC = r"""
#include <stdio.h>
#include <string.h>
#include "sa.h"

static int fails = 0;
#define EXPECT(cond) do { if (!(cond)) { printf("FAILED: %s (line %d)\n", #cond, __LINE__); ++fails; } } while (0)

int main(void) {
    sa_shape s;
    memset(&s, 0, sizeof s);
    s.batch = 1; s.T = 128; s.heads = 4; s.kv_heads = 2; s.causal = 1;
    EXPECT(sa_check_shape(&s) == SA_OK);
    EXPECT(sa_backward_workspace_bytes(&s) == (size_t)4 * 3 * 64 * 64 * 2);   /* 2 x 2 causal tiles: 3 */
    s.T = 100;
    EXPECT(sa_check_shape(&s) == SA_ERR_SHAPE);
    EXPECT(sa_backward_workspace_bytes(&s) == 0);
    s.T = 128; s.heads = 3;
    EXPECT(sa_check_shape(&s) == SA_ERR_SHAPE);
    s.heads = 4;
    EXPECT(sa_check_shape(NULL) == SA_ERR_NULL);
    /* pointer checks come before any launch */
    void* fake = (void*)0x10000;
    EXPECT(sa_forward_ex(&s, fake, fake, fake, NULL, (float*)fake, 0.18f, NULL) == SA_ERR_NULL);
    EXPECT(sa_forward_ex(&s, fake, fake, (char*)fake + 4, fake, (float*)fake, 0.18f, NULL) == SA_ERR_ALIGN);
    EXPECT(sa_forward_ex(&s, fake, fake, fake, fake, (float*)fake, -1.0f, NULL) == SA_ERR_ARGUMENT);
    EXPECT(sa_forward(fake, fake, fake, fake, (float*)fake, 0.18f, 100, 4, 2, NULL) == SA_ERR_SHAPE);
    EXPECT(sa_dq_pass_rotated(&s, fake, fake, 0, 0.125f, (const float*)fake, (const float*)fake, fake, 512, NULL)
           == SA_ERR_WORKSPACE);
    EXPECT(strcmp(sa_status_string(SA_OK), "ok") == 0);
    EXPECT(strcmp(sa_status_string(12345), "unknown status") == 0);
    printf("%s\n", fails ? "c-abi: failures" : "c-abi: ok");
    return fails != 0;
}
"""


def test_header_compiles_as_c_and_statuses_round_trip(tmp_path):
    lib = os.path.join(LIBDIR, "libsa.so")
    if not os.path.exists(lib):
        pytest.skip("libsa.so not built")
    src = tmp_path / "abi.c"
    src.write_text(C_SRC)
    exe = tmp_path / "abi"
    subprocess.run(["gcc", "-std=c11", "-Wall", "-Wextra", "-Werror", "-I", os.path.join(ROOT, "include"),
                    str(src), "-L", LIBDIR, "-lsa", f"-Wl,-rpath,{LIBDIR}", "-o", str(exe)], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    sys.stdout.write(r.stdout)
    assert r.returncode == 0 and "c-abi: ok" in r.stdout, r.stdout + r.stderr
