"""The library's host code (geometry validation, token widths, workspace
sizing and layouts, every entry point's argument checks) under
AddressSanitizer and UndefinedBehaviorSanitizer: all sources compiled by
hipcc with the sanitizers on the host side only, driven through the C ABI
by tests/sanitize/lib_host_sanitized_main.c on paths that are decided on
the host (no GPU).  Any report fails the run."""
import concurrent.futures as cf
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "learned_sparse_attention_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SOURCES = ["qsa_api", "index_score", "index_score_prefill", "topk", "sparse_attn", "append"]
# sanitizers for the host pass only (each flag behind -Xarch_host)
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_library_host_code_under_asan_and_ubsan(tmp_path):
    common = ["-O1", "-g", "--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang",
              "-packed-fp32-ops", *SAN, "-I", os.path.join(ROOT, "include"), "-I", CSRC]

    def compile_one(src):
        obj = str(tmp_path / f"{src}.o")
        r = subprocess.run([HIPCC, "-std=c++17", *common, "-c", os.path.join(CSRC, src + ".hip"),
                            "-o", obj], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr
        return obj

    with cf.ThreadPoolExecutor(max_workers=6) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    main_obj = str(tmp_path / "main.o")
    r = subprocess.run([HIPCC, "-x", "c", "-std=c11", *common, "-c",
                        os.path.join(ROOT, "tests", "sanitize", "lib_host_sanitized_main.c"),
                        "-o", main_obj], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    exe = str(tmp_path / "lib_host_sanitized")
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", *SAN, "-o", exe, main_obj, *objs],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "library host code sanitized run: ok" in run.stdout
