"""The C ABI from C: include/tide.h compiles as C11 (gcc -Wall -Werror -pedantic)
and a C program linked against libtide.so creates a plan, reads its geometry
and gets the documented error codes.  No GPU call is made (plan functions are
host only, and the failing calls are rejected before any HIP call)."""
import os
import shutil
import subprocess

import pytest

from parameter_layout_collectives_amd._lib import LIB_PATH

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

PROGRAM = r"""
#include <stdio.h>
#include "tide.h"

int main(void) {
    /* the tiny workload: [5,7], [16], [33,4] over 4 ranks */
    const int64_t dim0[3] = {5, 16, 33}, inner[3] = {7, 1, 4};
    tide_plan *plan = NULL;
    if (tide_plan_create(4, 3, dim0, inner, 1, &plan) != TIDE_OK) return 1;
    int64_t off, c, seg, src, L;
    if (tide_plan_param(plan, 2, &off, &c, &seg) != TIDE_OK) return 2;
    if (tide_plan_real(plan, 3, 2, &src, &L) != TIDE_OK) return 3;
    printf("%lld %d %d %lld %lld %lld %lld %lld\n", (long long)tide_plan_shard_numel(plan),
           tide_plan_world(plan), tide_plan_nparams(plan), (long long)off, (long long)c,
           (long long)seg, (long long)src, (long long)L);
    /* errors: a bad rank, unknown flag bits, a bad element size */
    const void *grads[12] = {0};
    float *out = (float *)0x1000;
    const int st_rank = (int)tide_rs(plan, 4, grads, out, 0, 0, NULL);
    const int st_flags = (int)tide_rs(plan, 0, grads, out, 0x40u, 0, NULL);
    const int st_elem =
        (int)tide_ag(plan, (const void *const *)grads, (void *const *)grads, 3, 0, 0, NULL);
    const char *msg = tide_last_error();
    printf("%d %d %d %s %s\n", st_rank, st_flags, st_elem, tide_status_string(TIDE_E_INVALID),
           msg);
    tide_plan_destroy(plan);
    return 0;
}
"""


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_c_program_against_the_header_and_library(tmp_path):
    src = tmp_path / "consumer.c"
    src.write_text(PROGRAM)
    exe = tmp_path / "consumer"
    libdir = os.path.dirname(LIB_PATH)
    cmd = ["gcc", "-std=c11", "-Wall", "-Wextra", "-Werror", "-pedantic",
           "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe),
           "-L", libdir, "-ltide", f"-Wl,-rpath,{libdir}"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stderr
    line1, line2 = r.stdout.strip().splitlines()
    # S = 54; param 2 ([33,4]): off 18, c 9, seg 36; rank 3 holds 6 rows from element 108
    assert line1.split() == ["54", "4", "3", "18", "9", "36", "108", "24"]
    st_rank, st_flags, st_elem, name, msg = line2.split(" ", 4)
    assert (st_rank, st_flags, st_elem, name) == ("1", "2", "1", "TIDE_E_INVALID")
    assert "elem_bytes" in msg
