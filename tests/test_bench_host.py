"""bench.py's host-side contract, on the CPU: one GPU only (a request for
more exits with a JSON error line and status 2), the traffic figure is read
from the committed counter summary only while it matches the attention
kernel source and workload, and the reported kernel is the template
instance the library launches for each workload."""
import json
import os
import subprocess
import sys

import pytest

import bench
from synth import BY_NAME

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    rec = json.loads(r.stdout.strip().splitlines()[-1])
    assert rec["n_gpus"] == 2 and "one GPU" in rec["error"]


def test_traffic_record_follows_the_kernel_source(monkeypatch):
    got = bench.read_traffic("llama8b_128k", True)
    assert isinstance(got, int) and got > 0
    assert bench.read_traffic("llama8b_128k", False) is None          # other plan options
    assert bench.read_traffic("llama8b_32k", True) is None            # other workload
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "0" * 16)
    assert bench.read_traffic("llama8b_128k", True) is None           # kernel changed since


def test_source_hash_ignores_comments(tmp_path, monkeypatch):
    src = tmp_path / "csrc"
    src.mkdir()
    (src / "attn_kernels.hip").write_text("int a; // one\n\n// two\nint b;\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "ATTN_SOURCES", ("attn_kernels.hip",))
    os.makedirs(tmp_path / "sparse_long_context_last_amd", exist_ok=True)
    os.replace(src, tmp_path / "sparse_long_context_last_amd" / "csrc")
    h1 = bench.kernel_source_hash()
    (tmp_path / "sparse_long_context_last_amd" / "csrc" / "attn_kernels.hip").write_text(
        "int a;   // edited comment\nint b;\n")
    assert bench.kernel_source_hash() == h1
    (tmp_path / "sparse_long_context_last_amd" / "csrc" / "attn_kernels.hip").write_text("int a;\nint c;\n")
    assert bench.kernel_source_hash() != h1


@pytest.mark.parametrize("name,token,want", [
    ("llama8b_128k", False, "fp::k_attn_bf16<128, true, false, false, 128>"),
    ("llama8b_128k", True, "fp::k_attn_bf16<128, true, true, false, 128>"),
    ("glm9b_64k_bs64", False, "fp::k_attn_bf16<64, true, false, true, 128>"),
    ("tiny_fp32_4k", False, "fp::k_attn_f32<128, true, false, 128>"),
])
def test_kernel_names(name, token, want):
    assert bench.attention_kernel_name(BY_NAME[name], token) == want
