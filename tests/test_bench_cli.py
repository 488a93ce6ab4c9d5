"""Host-side checks of bench.py: its byte accounting against the closed-form
sizes of the MXFP8 layers, and the one-GPU contract of its command line."""
import os
import subprocess
import sys

import bench
from moe_decode_gate_amd import inputs as gen

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_expert_bytes_closed_form():
    # Qwen-3-style layer: 2 x 768 rows of 2048 codes + 64 E8M0 bytes each; 2048 rows of 768 + 24
    gu, dn = bench.expert_bytes(gen.CONFIGS["qwen3"]["spec"])
    assert gu == 2 * 768 * 2048 + 2 * 768 * 64 == 3_244_032
    assert dn == 2048 * 768 + 2048 * 24 == 1_622_016
    # the H 4096 / I 1536 layer: 19,464,192 bytes per expert in all
    gu, dn = bench.expert_bytes(gen.CONFIGS["large"]["spec"])
    assert gu + dn == 19_464_192
    # agrees with the generator's own accounting of one expert
    for name in ("tiny", "qwen3", "large"):
        spec = gen.CONFIGS[name]["spec"]
        assert sum(bench.expert_bytes(spec)) == gen.expert_bytes(spec)


def test_more_than_one_gpu_is_refused():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert p.returncode == 2
    assert "one GPU" in p.stderr or "single MI355X" in p.stderr
