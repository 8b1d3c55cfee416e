"""Host-side behaviour of bench.py that needs no GPU: the one-GPU refusal and the
lookup of committed HBM-traffic figures by kernel source hash."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("n", [2, 8])
def test_more_than_one_gpu_is_refused(n):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", str(n)], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr and r.stdout == ""


def test_read_traffic_needs_a_matching_source_hash(tmp_path, monkeypatch):
    sys.path.insert(0, ROOT)
    import bench
    from exact_attention_48_amd import kernel_sources
    prof = tmp_path / "profiles"
    prof.mkdir()
    f = prof / "bwd_dkdv_kernel__w__hbm_traffic.txt"
    f.write_text("# header: ignored\nhbm_bytes_per_launch: 12345\nsource_hash: 0000000000000000\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.read_traffic("bwd_dkdv_kernel", "w") is None          # stale hash: no figure
    f.write_text(f"hbm_bytes_per_launch: 12345\nsource_hash: {kernel_sources.source_hash('bwd_dkdv_kernel')}\n")
    assert bench.read_traffic("bwd_dkdv_kernel", "w") == 12345.0
    assert bench.read_traffic("bwd_dq_kernel", "w") is None            # no file
