"""bench.py's host side without a GPU: the refusal of more than one GPU, the algorithmic bytes against the
per-unit figures of the layer written out by hand, and the HBM traffic it takes from the committed counter
summaries only while their kernel source digest matches the sources."""

import os
import re
import subprocess
import sys

import bench
from moe_synth import CONFIGS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, "bench.py", "--gpus", "2"], cwd=ROOT, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_unit_bytes_of_the_full_size_layer():
    """One token of H = 5120, I = I_s = 2304, 384 experts, top-6, MXFP4 (half a byte per code, one E8M0 byte
    per 32 codes), bf16 shared expert and activations, fp32 router rows."""
    cfg = CONFIGS["decode_t1_h5120_e384"]
    h, i, e = 5120, 2304, 384
    gate_up = 2 * i * (h // 2) + 2 * i * (h // 32)  # 12,533,760
    down = h * (i // 2) + h * (i // 32)  # 6,266,880
    assert (gate_up, down) == (12_533_760, 6_266_880)
    b = bench.algorithmic_bytes(cfg, touched=6)
    assert b["routed_gate_up"] == 6 * gate_up + h * 2 + 6 * i * 2  # weights, x, six h rows
    assert b["routed_down"] == 6 * down + 6 * i * 2 + 6 * h * 2  # weights, six h rows, six output rows
    assert b["shared_gate_up"] == 2 * i * h * 2 + h * 2 + i * 2
    assert b["shared_down"] == h * i * 2 + i * 2 + h * 2
    assert b["router_logits"] == e * h * 4 + h * 2 + e * 4
    # the whole layer: six experts, the shared expert's three matrices, the router rows, x in and y out
    assert bench.layer_bytes(cfg, 6) == 6 * (gate_up + down) + 3 * i * h * 2 + e * h * 4 + 2 * h * 2
    # MXFP8 codes are one byte each
    b8 = bench.algorithmic_bytes(CONFIGS["decode_t1_h5120_e384_fp8"], touched=6)
    assert b8["routed_gate_up"] == 6 * (2 * i * h + 2 * i * (h // 32)) + h * 2 + 6 * i * 2


def test_traffic_only_on_matching_digest():
    digest = bench.kernel_source_digest()
    assert re.fullmatch(r"[0-9a-f]{16}", digest) and digest == bench.kernel_source_digest()
    path = os.path.join(ROOT, "profiles", "pmc_decode_t1_h5120_e384.md")
    text = open(path).read()
    m = re.search(r"^\|\s*route_gate_up_shared_down\s*\|[^|]*\|[^|]*\|\s*([0-9.eE+]+)\s*\|", text, flags=re.M)
    assert m, "the summary lists the dominant one-token launch"
    stored = re.search(r"kernel source digest:\s*([0-9a-f]+)", text).group(1)
    got = bench.traffic_from_profile("route_gate_up_shared_down", "decode_t1_h5120_e384", stored)
    assert got == float(m.group(1))
    assert bench.traffic_from_profile("route_gate_up_shared_down", "decode_t1_h5120_e384", "0" * 16) is None
    assert bench.traffic_from_profile("route_gate_up_shared_down", "no_such_workload", stored) is None
