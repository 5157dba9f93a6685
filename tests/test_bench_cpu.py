"""bench.py's measured-traffic field: taken from the committed rocprofv3
counter summary only while the attention kernel source is the one the
counters were collected on."""

import importlib.util
import os
import shutil

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_traffic_follows_source_hash(tmp_path):
    b = _bench()
    md = tmp_path / "counters.md"
    src = tmp_path / "k_attn.hip"
    shutil.copy(b.ATTN_SRC, src)
    import hashlib
    h = hashlib.sha256(src.read_bytes()).hexdigest()
    md.write_text("- traffic_bytes_per_launch (k_attn_mla): 123456\n"
                  f"- source_sha256 (ragged_verification_amd/csrc/k_attn.hip): {h}\n")
    b.COUNTERS_MD, b.ATTN_SRC = str(md), str(src)
    assert b.measured_traffic() == 123456
    src.write_bytes(src.read_bytes() + b"\n// changed\n")
    assert b.measured_traffic() is None
    b.COUNTERS_MD = str(tmp_path / "missing.md")
    assert b.measured_traffic() is None


def test_gqa_traffic_is_keyed_by_workload(tmp_path):
    b = _bench()
    md = tmp_path / "gqa.md"
    import hashlib
    h = hashlib.sha256(open(b.ATTN_SRC, "rb").read()).hexdigest()
    md.write_text("- traffic_bytes_per_launch (k_attn_gqa, gqa_bf16): 111\n"
                  "- traffic_bytes_per_launch (k_attn_gqa, rejection_bf16): 222\n"
                  f"- source_sha256 (ragged_verification_amd/csrc/k_attn.hip): {h}\n")
    assert b.measured_traffic(str(md), "k_attn_gqa, gqa_bf16") == 111
    assert b.measured_traffic(str(md), "k_attn_gqa, rejection_bf16") == 222
    assert b.measured_traffic(str(md), "k_attn_gqa, sweep_gqa") is None


def test_gpus_other_than_one_exit():
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2 and "one GPU" in r.stderr
