"""CPU checks of bench.py's bookkeeping: the algorithmic byte count behind the
roofline's GB/s, the code digest that keys the measured traffic, and the
one-GPU contract of the command line."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_algorithmic_bytes_of_the_headline():
    # W and hidden once, the targets, the [N, S] partials written and read back,
    # the target logits written and read, and the two outputs (S = 251 at V = 128256)
    N, H, V, S = 4096, 4096, 128256, 251
    expected = (V * H * 2) + (N * H * 2) + N * 8 + 2 * (N * S * 8) + 2 * (N * 4) + 2 * (N * 4)
    assert bench.algorithmic_bytes(N, H, V, S, 0) == expected == 1_100_775_424
    # a bf16 bias adds its 2 V bytes
    assert bench.algorithmic_bytes(N, H, 151936, 198, 151936 * 2) - \
        bench.algorithmic_bytes(N, H, 151936, 198, 0) == 151936 * 2


def test_code_digest_ignores_comments_and_whitespace(tmp_path):
    a = tmp_path / "a.hip"
    b = tmp_path / "b.hip"
    c = tmp_path / "c.hip"
    a.write_text("int f(int x) {\n  return x + 1;  // one more\n}\n")
    b.write_text("/* header */ int f(int x)\n{ return x + 1; }\n")
    c.write_text("int f(int x) { return x + 2; }\n")
    assert bench.code_digest(str(a)) == bench.code_digest(str(b))
    assert bench.code_digest(str(a)) != bench.code_digest(str(c))


def test_traffic_records_are_keyed_by_workload_and_digest():
    for (workload, digest), rec in bench.MEASURED_TRAFFIC.items():
        assert workload == "headline" and len(digest) == 16
        assert rec["fetch_bytes"] > 0 and rec["write_bytes"] > 0
    # an unknown workload or code never reports traffic
    assert bench.measured_traffic("no-such-workload") is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)
