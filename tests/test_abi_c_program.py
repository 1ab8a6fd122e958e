"""The C ABI from a plain C program, with no Python or torch in the process: include/lcattn.h compiles as C99 with
warnings as errors, and a program linked against liblcattn.so gets the ABI version, the workspace sizes and the
documented status codes for invalid arguments. Every call is a size query or is rejected on the host before any
device work, so no GPU is needed."""
import os
import shutil
import subprocess

import pytest

import long_context_attention_causal_amd as lca

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

PROGRAM = r"""
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "lcattn.h"

static int fails = 0;
#define CHECK(cond)                                                          \
    do {                                                                     \
        if (!(cond)) {                                                       \
            printf("FAIL line %d: %s (%s)\n", __LINE__, #cond, attn_last_error()); \
            ++fails;                                                         \
        }                                                                    \
    } while (0)

int main(void) {
    /* aligned, non-null and never dereferenced: validation fails before any launch */
    void* fake = (void*)(uintptr_t)(1u << 20);
    void* misaligned = (void*)(uintptr_t)((1u << 20) + 4);

    CHECK(attn_abi_version() == LCATTN_ABI_VERSION);
    CHECK(strcmp(attn_status_string(ATTN_OK), attn_status_string(ATTN_ERR_SHAPE)) != 0);

    attn_shape_t s = {1, 4, 2, 128, 128, 0.1f, ATTN_BF16};
    CHECK(attn_prefill_dense(NULL, fake, fake, fake, fake, NULL, NULL) == ATTN_ERR_NULL);
    CHECK(attn_prefill_dense(&s, NULL, fake, fake, fake, NULL, NULL) == ATTN_ERR_NULL);
    CHECK(attn_prefill_dense(&s, misaligned, fake, fake, fake, NULL, NULL) == ATTN_ERR_ALIGN);
    attn_shape_t bad = s;
    bad.heads_q = 3;
    CHECK(attn_prefill_dense(&bad, fake, fake, fake, fake, NULL, NULL) == ATTN_ERR_SHAPE);
    bad = s;
    bad.head_dim = 96;
    CHECK(attn_prefill_dense(&bad, fake, fake, fake, fake, NULL, NULL) == ATTN_ERR_UNSUPPORTED);
    bad = s;
    bad.scale = INFINITY;
    CHECK(attn_prefill_dense(&bad, fake, fake, fake, fake, NULL, NULL) == ATTN_ERR_SHAPE);
    bad = s;
    bad.seq_len = 1 << 24; /* one head's K slab would reach 2^31 bytes */
    CHECK(attn_prefill_dense(&bad, fake, fake, fake, fake, NULL, NULL) == ATTN_ERR_UNSUPPORTED);

    /* the 32K block-64 mask problem: a positive workspace that grows with the block count */
    attn_shape_t m32 = {1, 32, 4, 32768, 128, 0.08838835f, ATTN_BF16};
    attn_mask_params_t mp = {64, 100, 1.0, 50, 90, 0};
    const size_t ws32 = attn_block_mask_workspace_bytes(&m32, &mp);
    attn_shape_t m64 = m32;
    m64.seq_len = 65536;
    const size_t ws64 = attn_block_mask_workspace_bytes(&m64, &mp);
    CHECK(ws32 > 0 && ws64 > ws32 && ws32 % 256 == 0);
    attn_mask_params_t badp = mp;
    badp.block_size = 48;
    CHECK(attn_block_mask_workspace_bytes(&m32, &badp) == 0);
    CHECK(attn_block_mask_build(&m32, &mp, fake, fake, fake, fake, fake, NULL, NULL, 0, NULL) == ATTN_ERR_WORKSPACE);

    /* decode: a positive workspace; a missing one is refused */
    attn_decode_shape_t d = {32, 64, 8, 64, 16, 2048, 65536, 512, 0.125f};
    CHECK(attn_decode_workspace_bytes(&d, 32768) > 0);
    CHECK(attn_decode_paged(&d, fake, fake, fake, fake, fake, 32768, fake, NULL, NULL, 0, NULL) == ATTN_ERR_WORKSPACE);

    printf("c-abi checks done, %d failed\n", fails);
    return fails != 0;
}
"""


@pytest.fixture(scope="module")
def lib_dir():
    if not os.path.exists(lca.LIB_PATH):
        from long_context_attention_causal_amd import build
        build.build(verbose=False)
    return os.path.dirname(lca.LIB_PATH)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no C compiler")
def test_c_program_uses_the_abi(tmp_path, lib_dir):
    src = tmp_path / "abi_check.c"
    exe = tmp_path / "abi_check"
    src.write_text(PROGRAM)
    # the library's own dependencies (the HIP runtime) resolve through its RUNPATH; the linker gets the same directory
    hip_lib = "/opt/rocm/lib"
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I", os.path.join(ROOT, "include"),
           str(src), "-o", str(exe), "-L", lib_dir, "-llcattn", f"-Wl,-rpath,{lib_dir}", f"-Wl,-rpath-link,{hip_lib}",
           "-lm"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "0 failed" in run.stdout
