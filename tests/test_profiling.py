"""A measured HBM-traffic record reaches the bench line only for its own
kernel, its own workload and the kernel sources it was measured on."""
import json

from block_draft_decoding_amd import profiling as P


def _record(tmp_path, **over):
    rec = {"tag": "gemm_gate_up", "workload": "traj2d3d", "traffic_bytes": 123,
           "source_digest": P.source_digest(P.kernel_files("gemm_gate_up"))}
    rec.update(over)
    p = tmp_path / "traffic.md"
    p.write_text("# traffic\n\n```json\n" + json.dumps(rec) + "\n```\n")
    return str(p)


def test_record_applies_to_its_kernel_and_workload_only(tmp_path):
    p = _record(tmp_path)
    assert P.read_traffic("gemm_gate_up", "traj2d3d", p) == 123
    assert P.read_traffic("gemm_gate_up", "traj2d", p) is None
    assert P.read_traffic("attention", "traj2d3d", p) is None


def test_record_of_other_sources_or_without_workload_is_ignored(tmp_path):
    assert P.read_traffic("gemm_gate_up", "traj2d3d", _record(tmp_path, source_digest="0" * 16)) is None
    assert P.read_traffic("gemm_gate_up", "traj2d3d", _record(tmp_path, workload=None)) is None


def test_missing_file_gives_no_traffic(tmp_path):
    assert P.read_traffic("gemm_gate_up", "traj2d3d", str(tmp_path / "absent.md")) is None
