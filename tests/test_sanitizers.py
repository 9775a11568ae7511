"""The host code of the library (graph builder, C ABI host paths) built with
AddressSanitizer and UndefinedBehaviorSanitizer and exercised host-only by
tests/native/host_only_driver.cpp: decoder graphs of every benchmark shape
and build option, random task/region programs through the rewrite pipeline,
and argument errors.  The graph sizes it reports must equal those of the
library as built for use."""
import os
import shutil
import subprocess

import pytest

import synth
import task_graph_runtime_amd as mpk

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
CSRC = os.path.join(ROOT, "task_graph_runtime_amd", "csrc")


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.exists(os.path.join(ROCM, "lib", "libamdhip64.so")):
        pytest.skip("g++ or the HIP runtime library is not available")
    exe = str(tmp_path_factory.mktemp("sanitize") / "host_only_driver")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-omit-frame-pointer",
           "-fno-sanitize-recover=all", "-D__HIP_PLATFORM_AMD__", "-I" + os.path.join(ROCM, "include"),
           "-I" + os.path.join(ROOT, "include"), "-I" + CSRC, os.path.join(ROOT, "tests", "native", "host_only_driver.cpp"),
           os.path.join(CSRC, "capi.cpp"), os.path.join(CSRC, "builder.cpp"), "-L" + os.path.join(ROCM, "lib"),
           "-lamdhip64", "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise AssertionError("sanitizer build failed:\n" + r.stderr[-4000:])
    return exe


def test_host_paths_clean_under_asan_ubsan(driver):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([driver], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-6000:]
    assert r.stdout.strip().endswith("ok")
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr
    sizes = {}
    for line in r.stdout.splitlines():
        if line.startswith("graph "):
            _, name, *v = line.split()
            sizes[name] = tuple(int(x) for x in v)
    # the same graphs built by the library as used
    for name, shape, B, params in [("tiny_b3", "tiny", 3, {}), ("qwen3_8b_b1", "qwen3_8b", 1, {}),
                                   ("qwen3_8b_b16_hybrid", "qwen3_8b_b16", 16, dict(attn_jit=1)),
                                   ("tiny_b3_no_fusion", "tiny", 3, dict(fusion_order=1, n_workers=8, s_attn=4)),
                                   ("qwen3_30b_a3b_b16", "qwen3_30b_a3b_b16", 16, {})]:
        s = synth.SHAPES[shape]
        g = mpk.TGraph(s.cfg(), B, s.page_size, params, host_only=True)
        h = g.header()
        g.close()
        assert sizes[name] == (h["n_tasks"], h["n_events"], h["n_empty"], h["n_aot"]), name
