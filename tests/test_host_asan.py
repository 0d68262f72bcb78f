"""The host library (argument checks, launch plan, workspace layout, the
shifted weight / bias base of a vocabulary-range launch, row chunking) built
with g++ under AddressSanitizer and UndefinedBehaviorSanitizer against a fake
HIP runtime whose stand-in kernels touch exactly the bytes the real kernels
would (tests/host_asan/).  CPU only.  Planted mistakes in a copy of the
host source must make the harness fail, so it is known to catch them; so must
a launch plan that disagrees with the launch."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HOST = os.path.join(ROOT, "invariant_linear_log_amd", "csrc", "bilogp_host.cpp")
HARNESS = os.path.join(ROOT, "tests", "host_asan", "harness.cpp")
FAKE = os.path.join(ROOT, "tests", "host_asan", "fake_hip")
FLAGS = ["-std=c++17", "-g", "-O1", "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]


def _gxx():
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    return gxx


def _sanitizers_available(tmp_path):
    """Whether g++ can build and run a trivial program with the sanitizers
    (a missing runtime skips the tests; a broken harness must fail them)."""
    src = tmp_path / "probe.cpp"
    src.write_text("int main() { return 0; }\n")
    exe = tmp_path / "probe"
    r = subprocess.run([_gxx(), *FLAGS, str(src), "-o", str(exe)], capture_output=True, text=True)
    if r.returncode != 0:
        return False, r.stderr[-300:]
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    return r.returncode == 0, r.stderr[-300:]


def _build(tmp_path, host_src, name):
    ok, why = _sanitizers_available(tmp_path)
    if not ok:
        pytest.skip("g++ sanitizer runtime not available: " + why)
    exe = tmp_path / name
    cmd = [_gxx(), *FLAGS, "-I", FAKE, "-I", os.path.join(ROOT, "include"), "-I",
           os.path.join(ROOT, "invariant_linear_log_amd", "csrc"), str(host_src), HARNESS,
           "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    return exe


def _run(exe):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    return subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)


def test_host_library_clean_under_asan_ubsan(tmp_path):
    r = _run(_build(tmp_path, HOST, "harness"))
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert "cases passed" in r.stdout


MUTATIONS = {
    # a vocabulary-range launch that forgets to shift the weight base by col0
    "weight_base_not_shifted": ("(uintptr_t)col0 * (uintptr_t)c.H * 2u);",
                                "(uintptr_t)0 * (uintptr_t)c.H * 2u);"),
    # row chunks whose partials start one row late
    "chunk_partials_one_row_late": ("q.part = p.part + r0 * p.S;",
                                    "q.part = p.part + (r0 + 1) * p.S;"),
    # a launch plan that counts the 128-token stages with two buffers instead of
    # the three the forward launches with
    "launch_plan_wrong_buffer_count": ("  plan_projection(p, cu_count, 3);",
                                       "  plan_projection(p, cu_count, 2);"),
    # a split schedule whose big launch also runs the splits of the second launch
    "main_launch_overlaps_tail": ("  q.split1 = p.splitT;\n", "  q.split1 = p.split1;\n"),
    # a second launch that starts one split late
    "tail_launch_skips_a_split": ("  q.split0 = p.splitT;\n", "  q.split0 = p.splitT + 1;\n"),
    # a second launch sized from 256-token row blocks (its last rows never run)
    "tail_launch_too_few_row_blocks": ("  q.R = (int32_t)((p.N + 127) / 128);",
                                       "  q.R = (int32_t)((p.N + 255) / 256);"),
    # a bf16 bias read directly where V cuts its last 16-byte chunk
    "direct_bf16_bias_chunk_cut": ("  if (bias_dtype == BILOGP_BIAS_BF16) return V % 8 == 0;",
                                   "  if (bias_dtype == BILOGP_BIAS_BF16) return V % 4 == 0;"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_harness_catches_planted_mistakes(tmp_path, name):
    find, repl = MUTATIONS[name]
    src = open(HOST).read()
    assert src.count(find) == 1, f"mutation anchor not found: {find!r}"
    mutant = tmp_path / "bilogp_host_mutant.cpp"
    # the mutant is compiled from another directory: point its relative
    # include of the public header back at the repository
    mutant.write_text(src.replace(find, repl).replace('#include "../../include/bilogp.h"',
                                                      '#include "bilogp.h"'))
    r = _run(_build(tmp_path, mutant, "mutant"))
    assert r.returncode != 0, f"the harness did not catch {name}"
