"""Host logic of bench.py (no GPU): the contract's refusal of several GPUs,
the committed traffic counts picked by workload and kernel build, and a
kernel hash that does not depend on where the repository sits."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

LONGSEQ = "hstu_attn_bf16_longseq_b16_sl0.85_h8_d128"
JAGGED = "hstu_attn_bf16_b64_l256-1024_h4_d128"


def test_traffic_is_picked_by_workload():
    a, b = bench.measured_traffic(LONGSEQ), bench.measured_traffic(JAGGED)
    assert isinstance(a, int) and isinstance(b, int) and a != b
    assert bench.measured_traffic("mfalcon_bf16_b8_n2048_bm512_h4_d128") is None


def test_traffic_is_dropped_when_the_kernel_build_changes(monkeypatch):
    from hstu_sequential_transducer_causal_amd import build
    monkeypatch.setitem(build.EXTRA_FLAGS, "attn_bf16.hip", ["-O1"])
    assert bench.measured_traffic(LONGSEQ) is None


def test_kernel_hash_independent_of_the_working_directory(tmp_path):
    here = bench.kernel_hash()
    code = f"import sys; sys.path.insert(0, {ROOT!r}); import bench; print(bench.kernel_hash())"
    out = subprocess.run([sys.executable, "-c", code], cwd=tmp_path, capture_output=True, text=True,
                         check=True).stdout.strip()
    assert out == here


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True)
    assert r.returncode == 2 and "one GPU only" in r.stderr


def test_kernel_hash_ignores_comments_but_not_code():
    src = "int f(int x) {  // the input\n    /* twice */ return 2 * x;\n}\n"
    same = "// a header\nint f(int x) {\n    return 2 * x;   /* doubled */\n}\n"
    other = "int f(int x) {\n    return 3 * x;\n}\n"
    assert bench._code_only(src) == bench._code_only(same)
    assert bench._code_only(src) != bench._code_only(other)
