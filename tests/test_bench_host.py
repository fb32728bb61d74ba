"""Host logic of bench.py (no GPU): the algorithmic byte counts behind the
HBM fraction, the comment-blind source hash that keys the traffic record, and
the lookup of that record."""

import json
import sys

import pytest

import workloads


@pytest.fixture(scope="module")
def bench():
    argv = sys.argv
    sys.argv = ["bench.py"]
    try:
        import bench as b
    finally:
        sys.argv = argv
    return b


def test_algorithmic_bytes_closed_forms(bench):
    # MLP hidden layer: X (256, 32, 1024) f32, W (1024, 1024) f32, b (1024,), int64 seeds, Y (256, 32, 1024)
    wl = workloads.make(2)
    x = 256 * 32 * 1024 * 4
    w = 1024 * 1024 * 4 + 1024 * 4
    y = 256 * 32 * 1024 * 4
    assert bench.algorithmic_bytes(wl, "forward0", [], 0) == x + w + 256 * 8 + y
    n = 1024 * 1024 + 1024
    assert bench.algorithmic_bytes(wl, "grad_flat", [], n) == 256 * 4 + 256 * 8 + n * 4
    # large batch: one X (4096, 4096) bf16 shared by all 16 individuals, no bias
    wl6 = workloads.make(6)
    assert bench.algorithmic_bytes(wl6, "forward0", [], 0) == \
        4096 * 4096 * 2 + 4096 * 4096 * 2 + 16 * 8 + 16 * 4096 * 4096 * 4
    # 3-layer MLP, second layer: its input is the first layer's fp32 output
    wl4 = workloads.make(4)
    assert bench.algorithmic_bytes(wl4, "forward1", [], 0) == \
        512 * 64 * 256 * 4 + (256 * 256 * 4 + 256 * 4) + 512 * 8 + 512 * 64 * 256 * 4


def test_source_hash_ignores_comments_only(bench):
    code = "int f(int a) {\n  return a + 1;  // one more\n}\n"
    assert bench.code_without_comments(code) == bench.code_without_comments(
        "/* header */\nint f(int a) {\n\n  return a + 1;\n}\n")
    assert bench.code_without_comments(code) != bench.code_without_comments(code.replace("+ 1", "+ 2"))


def test_recorded_traffic_follows_the_source_hash(bench, tmp_path, monkeypatch):
    rec = {"source_hash": bench.kernel_source_hash(),
           "entries": {"2:forward0": {"hbm_bytes_per_launch": 123}}}
    f = tmp_path / "traffic.json"
    f.write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.recorded_traffic(2, "forward0") == 123
    assert bench.recorded_traffic(2, "grad_flat") is None
    rec["source_hash"] = "0" * 16                 # kernels changed since the counters were taken
    f.write_text(json.dumps(rec))
    assert bench.recorded_traffic(2, "forward0") is None


def test_committed_traffic_record_matches_the_kernels(bench):
    """While the committed record describes the kernels as they are, it holds
    the bench's default workload; once the kernels change, bench.py reports
    no traffic until the counters are taken again."""
    with open(bench.TRAFFIC_FILE) as fh:
        rec = json.load(fh)
    if rec.get("source_hash") != bench.kernel_source_hash():
        assert bench.recorded_traffic(5, "forward0") is None
        pytest.skip("kernel sources changed since the traffic counters were taken: bench.py reports null")
    assert bench.recorded_traffic(5, "forward0") is not None


def test_build_scratch_check_reads_the_resource_remarks():
    """The build's scratch check picks out kernels with nonzero ScratchSize
    from the compiler's resource-usage remarks (format of hipcc's output)."""
    from virtual_noise_perturbed_amd import build as b
    remarks = "\n".join([
        "vn_kernels.hip:10:1: remark: Function Name: _ZN2vn1aEv [-Rpass-analysis=kernel-resource-usage]",
        "vn_kernels.hip:10:1: remark:     VGPRs: 128 [-Rpass-analysis=kernel-resource-usage]",
        "vn_kernels.hip:10:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]",
        "vn_kernels.hip:20:1: remark: Function Name: _ZN2vn1bEv [-Rpass-analysis=kernel-resource-usage]",
        "vn_kernels.hip:20:1: remark:     ScratchSize [bytes/lane]: 128 [-Rpass-analysis=kernel-resource-usage]",
    ])
    assert b.kernels_with_scratch(remarks) == {"_ZN2vn1bEv": 128}
