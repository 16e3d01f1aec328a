"""Host-side pieces of bench.py (no GPU): the kernel-source digest that gates
the committed traffic records, and the refusal of more than one GPU."""
import json
import os
import subprocess
import sys

import dense_gemm_run_amd as dg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_every_configuration_has_a_kernel_source_digest():
    names = [dg.gemm_config_info(i)["name"] for i in range(dg.gemm_config_count())]
    digests = {n: bench.kernel_source_digest(n) for n in names}
    assert all(len(d) == 16 for d in digests.values())
    # configurations of one kernel file differ by their table entries
    assert len(set(digests.values())) == len(names)
    # split forms add the reduction and the split count
    assert bench.kernel_source_digest("mfma16x16_64x128x32_adma_split8") != digests["mfma16x16_64x128x32_adma"]


def test_traffic_records_name_existing_summaries():
    for f in os.listdir(os.path.join(ROOT, "profiles")):
        if f.startswith("traffic_") and f.endswith(".json"):
            rec = json.load(open(os.path.join(ROOT, "profiles", f)))
            assert os.path.exists(os.path.join(ROOT, rec["summary"])), f
            assert rec["hbm_bytes_per_launch"] > 0


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)
