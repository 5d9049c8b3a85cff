"""include/rlca.h is a C header: a C99 program that includes it compiles with
gcc (-std=c99 -Wall -Wextra -Werror; not -pedantic, which ROCm's own
hip_runtime_api.h does not pass), links against librlca.so and runs on the
host.  The program checks the rlca_call layout as the C compiler lays it out
against the ctypes binding's, the batch limit, and calls that return before
anything is enqueued (status strings, size queries, failed argument checks,
empty calls).  No GPU is used."""
import ctypes
import os
import shutil
import subprocess

import pytest

from linear_recurrence_scan_row_amd import rlca as binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "linear_recurrence_scan_row_amd")
ROCM_INCLUDE = "/opt/rocm/include"

PROGRAM = r"""
#include "rlca.h"
#include <stddef.h>
#include <stdio.h>
#include <string.h>

#define EXPECT(cond) do { if (!(cond)) { printf("failed: %%s\n", #cond); return 1; } } while (0)

int main(void) {
    /* layout of one batch record, as the ctypes binding declares it */
    EXPECT(sizeof(rlca_call) == %(size)d);
    EXPECT(offsetof(rlca_call, gamma) == %(gamma)d);
    EXPECT(offsetof(rlca_call, out0) == %(out0)d);
    EXPECT(offsetof(rlca_call, dtype) == %(dtype)d);
    EXPECT(RLCA_MAX_BATCH == %(max_batch)d);

    /* every status has its own message */
    for (int a = RLCA_OK; a <= RLCA_ERR_HIP; ++a) {
        EXPECT(rlca_status_string((rlca_status)a) != NULL);
        for (int b = RLCA_OK; b < a; ++b)
            EXPECT(strcmp(rlca_status_string((rlca_status)a), rlca_status_string((rlca_status)b)) != 0);
    }

    /* checks that fail before anything is enqueued (fake, never dereferenced addresses) */
    float *r = (float *)0x10000000, *v = (float *)0x20000000, *adv = (float *)0x40000000;
    const uint8_t *term = (const uint8_t *)0x30000000;
    EXPECT(rlca_gae(NULL, v, term, NULL, NULL, NULL, 0.99f, 0.95f, 4, 8, adv, NULL, NULL) == RLCA_ERR_NULL_POINTER);
    EXPECT(rlca_gae(r, v, term, NULL, NULL, NULL, 0.99f, 0.95f, -1, 8, adv, NULL, NULL) == RLCA_ERR_INVALID_SIZE);
    EXPECT(rlca_gae(r, v, term, NULL, NULL, NULL, 1.5f, 0.95f, 4, 8, adv, NULL, NULL) == RLCA_ERR_INVALID_VALUE);
    EXPECT(rlca_gae(r, v, term, NULL, NULL, NULL, 0.99f, 0.95f, 4, 8, (float *)r, NULL, NULL) == RLCA_ERR_ALIASING);
    EXPECT(rlca_gae((float *)((char *)r + 2), v, term, NULL, NULL, NULL, 0.99f, 0.95f, 4, 8, adv, NULL, NULL) == RLCA_ERR_MISALIGNED);
    EXPECT(rlca_gae(r, v, term, NULL, NULL, NULL, 0.99f, 0.95f, 0, 8, adv, NULL, NULL) == RLCA_OK);

    /* batches: empty, over the limit */
    rlca_call calls[RLCA_MAX_BATCH + 1];
    memset(calls, 0, sizeof calls);
    EXPECT(rlca_run_batch(calls, 0, NULL) == RLCA_OK);
    EXPECT(rlca_run_batch(calls, RLCA_MAX_BATCH, NULL) == RLCA_OK);      /* all empty */
    EXPECT(rlca_run_batch(calls, RLCA_MAX_BATCH + 1, NULL) == RLCA_ERR_INVALID_SIZE);

    /* workspace queries are host arithmetic */
    EXPECT(rlca_gae_stats_workspace_size(4096, 128) > 0);
    EXPECT(rlca_gae_stats_workspace_size(0, 128) == 0);
    EXPECT(rlca_ppo_clip_loss_workspace_size(4096, 128) > 0);
    printf("ok %%zu %%zu\n", rlca_gae_stats_workspace_size(4096, 128),
           rlca_ppo_clip_loss_workspace_size(4096, 128));
    return 0;
}
"""


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no gcc")
def test_header_compiles_as_c99_and_links(tmp_path):
    lib = os.path.join(PKG, "librlca.so")
    if not os.path.exists(lib):
        pytest.fail("librlca.so is not built")
    src = tmp_path / "uses_rlca.c"
    src.write_text(PROGRAM % {
        "size": ctypes.sizeof(binding.RlcaCall),
        "gamma": binding.RlcaCall.gamma.offset,
        "out0": binding.RlcaCall.out0.offset,
        "dtype": binding.RlcaCall.dtype.offset,
        "max_batch": binding.MAX_BATCH,
    })
    exe = tmp_path / "uses_rlca"
    build = subprocess.run(
        ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
         "-I", os.path.join(ROOT, "include"), "-I", ROCM_INCLUDE, str(src),
         "-L", PKG, "-lrlca", f"-Wl,-rpath,{PKG}", "-o", str(exe)],
        capture_output=True, text=True)
    assert build.returncode == 0, build.stderr[-3000:]
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0, run.stdout + run.stderr[-2000:]
    sizes = [int(x) for x in run.stdout.split()[1:3]]
    lib_py = binding.lib()
    assert sizes == [lib_py.rlca_gae_stats_workspace_size(4096, 128),
                     lib_py.rlca_ppo_clip_loss_workspace_size(4096, 128)]
