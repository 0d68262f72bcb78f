"""The C ABI from a C program: include/bilogp.h compiles as C99 (and as C++),
and a C program linked against the built libbilogp.so calls the host-only
entry points (versions, split policy, workspace size, status strings,
fail-closed argument checks) without a GPU."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INC = os.path.join(ROOT, "include")
LIBDIR = os.path.join(ROOT, "invariant_linear_log_amd")

PROGRAM = r"""
#include <stdio.h>
#include <string.h>
#include "bilogp.h"

int main(void) {
  /* V = 128256: 501 tiles of 256 columns, 2 per split, 251 splits */
  printf("abi %d contract %d\n", bilogp_abi_version(), bilogp_bit_contract_version());
  printf("splits %d vps %d\n", bilogp_num_vocab_splits(128256), bilogp_vtiles_per_split(128256));
  printf("ws %zu\n", bilogp_workspace_bytes(4096, 128256));
  printf("empty %zu bad %d\n", bilogp_workspace_bytes(0, 1000),
         bilogp_workspace_bytes(-1, 1000) == (size_t)-1);
  /* fail closed before any device work: a null hidden pointer */
  float out[2];
  long long t[1] = {0};
  bilogp_status st = bilogp_forward_ex(NULL, NULL, (const int64_t*)t, NULL, BILOGP_BIAS_NONE,
                                       out, out + 1, 1, 64, 1000, NULL, 0, NULL);
  printf("null %d %s | %s\n", (int)st, bilogp_status_string(st), bilogp_last_error());
  return 0;
}
"""


def _lib():
    path = os.path.join(LIBDIR, "libbilogp.so")
    if not os.path.exists(path):
        pytest.fail("libbilogp.so is not built (run __graft_entry__.build())")
    return path


@pytest.mark.parametrize("std,compiler", [("c99", "gcc"), ("c11", "gcc"), ("c++11", "g++")])
def test_header_compiles(tmp_path, std, compiler):
    if shutil.which(compiler) is None:
        pytest.fail(f"{compiler} not found")
    src = tmp_path / "h.c"
    src.write_text('#include "bilogp.h"\nint main(void) { return bilogp_abi_version() > 0 ? 0 : 1; }\n')
    lang = ["-x", "c++"] if compiler == "g++" else []
    r = subprocess.run([compiler, f"-std={std}", "-Wall", "-Wextra", "-pedantic", "-Werror",
                        "-fsyntax-only", *lang, "-I", INC, str(src)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_c_program_calls_the_library(tmp_path):
    lib = _lib()
    src = tmp_path / "consumer.c"
    exe = tmp_path / "consumer"
    src.write_text(PROGRAM)
    r = subprocess.run(["gcc", "-std=c99", "-Wall", "-I", INC, str(src), "-o", str(exe),
                        "-L", LIBDIR, "-lbilogp", f"-Wl,-rpath,{LIBDIR}"],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ)
    env.setdefault("HIP_VISIBLE_DEVICES", "")
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120, env=env)
    assert r.returncode == 0, r.stderr
    lines = r.stdout.splitlines()
    assert lines[0] == "abi 4 contract 4"
    assert lines[1] == "splits 251 vps 2"
    # [N, S] (max, sum) pairs + [N] target logits + the padded fp32 bias, 256-byte parts
    assert lines[2] == f"ws {4096 * 251 * 8 + 4096 * 4 + 128256 * 4}"
    assert lines[3] == "empty 0 bad 1"
    assert lines[4].startswith("null 1 invalid argument | ")
