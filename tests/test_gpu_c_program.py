"""A C program drives the library on the GPU with no Python or PyTorch in
between: HIP runtime allocations, tide_rs for every rank and tide_ag on the
null stream, each result compared bit for bit with the C oracle
(liboracle.so) in the same program.  The tiny workload's shapes, 4 ranks,
seeded bf16 patterns whose sums stay finite (so no NaN payload is compared)."""
import os
import shutil
import subprocess

import pytest
import torch

from parameter_layout_collectives_amd._lib import LIB_PATH
from gpu_helpers import note

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")

PROGRAM = r"""
#include <stdio.h>
#include <stdint.h>
#include <string.h>
#include <stdlib.h>
#include <hip/hip_runtime_api.h>
#include "tide.h"

int oracle_rs(int32_t N, int32_t P, const int64_t *d0, const int64_t *inner, int64_t align,
              int32_t R, const uint16_t *const *grads, float *out);
int oracle_ag(int32_t N, int32_t P, const int64_t *d0, const int64_t *inner, int64_t align,
              int32_t elem_bytes, const void *const *rank_src, void *const *params);

#define CHECK(x) do { if ((x) != hipSuccess) { printf("hip error line %d\n", __LINE__); return 2; } } while (0)

static uint32_t lcg = 12345u;
static uint16_t finite_bf16(void) {   /* random sign, exponent 100..154 (no sum overflows) */
    lcg = lcg * 1664525u + 1013904223u;
    uint32_t x = lcg >> 8;
    uint16_t e = (uint16_t)(100 + (x % 55u));
    return (uint16_t)(((x >> 8) & 1u) << 15 | e << 7 | ((x >> 9) & 0x7fu));
}

int main(void) {
    enum { N = 4, P = 3 };
    const int64_t d0[P] = {5, 16, 33}, inner[P] = {7, 1, 4};
    tide_plan *plan = NULL;
    if (tide_plan_create(N, P, d0, inner, 1, &plan) != TIDE_OK) return 3;
    const int64_t S = tide_plan_shard_numel(plan);
    uint16_t *host[N * P];
    void *dev[N * P];
    for (int r = 0; r < N; r++)
        for (int i = 0; i < P; i++) {
            const int64_t n = d0[i] * inner[i];
            host[r * P + i] = malloc((size_t)n * 2);
            for (int64_t k = 0; k < n; k++) host[r * P + i][k] = finite_bf16();
            CHECK(hipMalloc(&dev[r * P + i], (size_t)n * 2));
            CHECK(hipMemcpy(dev[r * P + i], host[r * P + i], (size_t)n * 2, hipMemcpyHostToDevice));
        }
    float *blocks;
    CHECK(hipMalloc((void **)&blocks, (size_t)(N * S) * 4));
    float *got = malloc((size_t)S * 4), *want = malloc((size_t)(N * S) * 4);
    for (int R = 0; R < N; R++) {
        if (tide_rs(plan, R, (const void *const *)dev, blocks + R * S, 0, 0, NULL) != TIDE_OK) {
            printf("tide_rs: %s\n", tide_last_error());
            return 4;
        }
        CHECK(hipDeviceSynchronize());
        CHECK(hipMemcpy(got, blocks + R * S, (size_t)S * 4, hipMemcpyDeviceToHost));
        if (oracle_rs(N, P, d0, inner, 1, R, (const uint16_t *const *)host, want + R * S)) return 5;
        if (memcmp(got, want + R * S, (size_t)S * 4)) { printf("rank %d differs\n", R); return 6; }
    }
    /* all-gather of the fp32 blocks into full fp32 tensors */
    const void *src[N];
    const void *hsrc[N];
    void *params[P], *hparams[P];
    for (int r = 0; r < N; r++) { src[r] = blocks + r * S; hsrc[r] = want + r * S; }
    for (int i = 0; i < P; i++) {
        CHECK(hipMalloc(&params[i], (size_t)(d0[i] * inner[i]) * 4));
        hparams[i] = calloc((size_t)(d0[i] * inner[i]), 4);
    }
    if (tide_ag(plan, src, params, 4, 0, 0, NULL) != TIDE_OK) {
        printf("tide_ag: %s\n", tide_last_error());
        return 7;
    }
    CHECK(hipDeviceSynchronize());
    if (oracle_ag(N, P, d0, inner, 1, 4, hsrc, hparams)) return 8;
    for (int i = 0; i < P; i++) {
        const size_t bytes = (size_t)(d0[i] * inner[i]) * 4;
        void *g = malloc(bytes);
        CHECK(hipMemcpy(g, params[i], bytes, hipMemcpyDeviceToHost));
        if (memcmp(g, hparams[i], bytes)) { printf("param %d differs\n", i); return 9; }
        free(g);
        CHECK(hipFree(params[i]));
    }
    tide_plan_destroy(plan);
    for (int k = 0; k < N * P; k++) CHECK(hipFree(dev[k]));
    CHECK(hipFree(blocks));
    printf("ok S=%lld\n", (long long)S);
    return 0;
}
"""


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_c_program_on_the_gpu(tmp_path, orc):
    src = tmp_path / "tide_c.c"
    src.write_text(PROGRAM)
    exe = tmp_path / "tide_c"
    libdir = os.path.dirname(LIB_PATH)
    orcdir = os.path.dirname(orc.path)
    cmd = ["gcc", "-std=c11", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"),
           str(src), "-o", str(exe),
           "-L", libdir, "-ltide", "-L", orcdir, "-loracle",
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           f"-Wl,-rpath,{libdir}:{orcdir}:{os.path.join(ROCM, 'lib')}"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    note("C program: tide_rs x4 + tide_ag on the null stream")
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.startswith("ok"), (r.returncode, r.stdout, r.stderr)
