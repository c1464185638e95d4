"""The C ABI's host code under the address and undefined-behaviour sanitizers
(CPU only, no GPU needed).

fam_api.cpp (argument validation, the budget plan, Soft-TopK, the ratio
floors, workspace sizes, the dispatch) is compiled with the host sanitizers
and linked with the library's kernel objects into tests/native/
abi_host_checks.cpp, which calls every host-only function on ordinary and
edge inputs and every device entry point with invalid arguments (their
validation fails before anything is launched, so no pointer is used). The
program must exit cleanly with no sanitizer report.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BUILD = os.path.join(ROOT, "_build")
OUT = os.path.join(BUILD, "sanitized")
CSRC = os.path.join(ROOT, "future_attention_scoring_amd", "csrc")
KERNEL_OBJECTS = ["fam_lse", "fam_mass", "kvpop_target", "kv_cache", "ranking", "topk_cutoff", "evict_select",
                  "evict_select_long", "kv_compact"]
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
FLAGS = ["-O1", "-g", "-std=c++17", "--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang",
         "-packed-fp32-ops", "-I" + os.path.join(ROOT, "include"), "-I" + CSRC]


def hipcc():
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    pytest.skip("hipcc not available")


def run(cmd, **kw):
    res = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert res.returncode == 0, f"{' '.join(cmd[:4])} ... failed:\n{res.stdout[-3000:]}\n{res.stderr[-3000:]}"
    return res


def test_abi_host_code_under_sanitizers():
    objs = [os.path.join(BUILD, n + ".o") for n in KERNEL_OBJECTS]
    if not all(os.path.exists(o) for o in objs):
        pytest.skip("library objects not built (run the package build first)")
    cc = hipcc()
    os.makedirs(OUT, exist_ok=True)
    api = os.path.join(OUT, "fam_api.o")
    run([cc, "-x", "hip", "-c", os.path.join(CSRC, "fam_api.cpp"), "-o", api, "-fPIC"] + FLAGS + SAN)
    main_o = os.path.join(OUT, "abi_host_checks.o")
    run([cc, "-c", os.path.join(ROOT, "tests", "native", "abi_host_checks.cpp"), "-o", main_o] + FLAGS + SAN)
    exe = os.path.join(OUT, "abi_host_checks")
    run([cc, "--hip-link", main_o, api] + objs + ["-o", exe, "--offload-arch=gfx950"] + SAN)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", HIP_VISIBLE_DEVICES="")
    res = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    out = res.stdout + res.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert res.returncode == 0, out[-4000:]
    assert "all host checks passed" in res.stdout
