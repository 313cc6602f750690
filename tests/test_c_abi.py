"""The boundary from C: include/wmk.h compiles as C99 (gcc, no C++), a C program links
against libwmk.so and calls it -- a size query, an error with its message, and a dry-run
append whose plan it reads back.  No GPU: these calls only check arguments and plan."""
import os
import shutil
import subprocess

import pytest

import kv_cache_attention_02_amd as wmk

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

PROGRAM = r"""
#include "wmk.h"
#include <stdio.h>
#include <string.h>

int main(void) {
    wmk_cache_desc d = {1, 12, 128, 1508, 6, 8, 4, WMK_BF16};
    size_t bytes = wmk_cache_bytes(&d);
    wmk_cache* c = NULL;
    wmk_status bad = wmk_cache_init(&d, NULL, NULL, bytes, &c);
    int has_msg = strlen(wmk_last_error()) > 0;
    /* fake 16-byte aligned device addresses: the dry run only checks and plans */
    wmk_status ok = wmk_cache_init(&d, (void*)0x10000000, (void*)0x20000000, bytes, &c);
    wmk_status app = wmk_cache_append_evict(c, 0, (const void*)0x30000000, (const void*)0x40000000, 4, NULL);
    int64_t slots[14];
    int64_t frames = -1;
    wmk_status sl = wmk_cache_slots(c, 0, slots, &frames);
    printf("%zu %d %d %d %d %d %lld %lld %lld\n", bytes, (int)bad, has_msg, (int)ok, (int)app, (int)sl,
           (long long)frames, (long long)slots[3], (long long)slots[4]);
    wmk_cache_destroy(c);
    return 0;
}
"""


def test_header_compiles_as_c_and_the_library_links(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc is not installed")
    if not os.path.exists(wmk.LIB_PATH):
        pytest.skip("libwmk.so is not built")
    src = tmp_path / "use.c"
    src.write_text(PROGRAM)
    exe = tmp_path / "use"
    libdir = os.path.dirname(wmk.LIB_PATH)
    cc = subprocess.run([gcc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
                         "-I", "/opt/rocm/include", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe),
                         "-L", libdir, "-lwmk", f"-Wl,-rpath,{libdir}"], capture_output=True, text=True)
    assert cc.returncode == 0, cc.stderr
    env = dict(os.environ, WMK_DRY_RUN=str(tmp_path / "launches.log"))
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=60)
    assert r.returncode == 0, r.stderr
    bytes_, bad, has_msg, ok, app, sl, frames, s3, s4 = (int(x) for x in r.stdout.split())
    assert bytes_ == 14 * 1508 * 12 * 128 * 2
    assert bad == wmk.WMK_ERR_NULL and has_msg == 1
    assert ok == app == sl == wmk.WMK_OK
    assert (frames, s3, s4) == (4, 3, -1)
    assert (tmp_path / "launches.log").read_text().startswith("append layer=0 F=0 n=4 ranges=1")
