"""bench.py's host-side accounting, on the CPU: the algorithmic bytes follow
their definition (touched weights, activations, index tables), the stored
traffic summaries are only used while the kernels' sources still hash as
measured, and the copy calibration scales them."""
import json
import os

import pytest

import bench
from sparse_mixture_experts_amd import inputs


def test_prefill_accounting_matches_its_definition():
    spec = inputs.workload("q4-prefill-t2048")
    acc = bench.accounting(spec, 512)
    T, D, F, E, K = spec.T, spec.d_model, spec.d_ff, spec.n_experts, spec.top_k
    # 4-bit codes plus one bf16 scale and one bf16 bias per group of 64
    per_matrix = lambda n, k: n * k // 2 + 2 * 2 * n * (k // 64)  # noqa: E731
    expert = per_matrix(2 * F, D) + per_matrix(D, F)
    assert bench.expert_bytes(spec) == expert
    assert acc["kernels"]["gateup_mfma"]["bytes"] == 512 * per_matrix(2 * F, D) + T * D * 2
    assert acc["kernels"]["down_mfma"]["bytes"] == 512 * per_matrix(D, F)
    assert acc["kernels"]["combine"]["bytes"] == T * D * 2 + T * K * 8
    assert acc["layer_bytes"] == 512 * expert + D * E * 2 + 2 * T * D * 2
    assert acc["expert_flops"] == 2 * T * K * 3 * D * F
    assert abs(acc["sparse_dense_flop_ratio"] - K / E) < 1e-12


def test_traffic_needs_matching_sources(tmp_path, monkeypatch):
    root = tmp_path
    (root / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(root))
    # the digest reads the real sources
    monkeypatch.setattr(bench, "kernel_sources_digest", lambda k: "h-" + k)
    rec = {"copy_calibration": {"bytes": 1 << 30, "fetch_kib": (1 << 20) / 2, "write_kib": 1 << 20},
           "kernels": {"gateup_mfma": {"fetch_kib": 1000.0, "write_kib": 10.0, "sources_sha256": "h-gateup_mfma"},
                       "down_mfma": {"fetch_kib": 1000.0, "write_kib": 10.0, "sources_sha256": "stale"}}}
    (root / "profiles" / "traffic_w.json").write_text(json.dumps(rec))
    # FETCH_SIZE read half the copy's bytes: its KiB count twice, WRITE_SIZE once
    assert bench.measured_traffic("w", "gateup_mfma") == int(1000 * 1024 * 2 + 10 * 1024)
    assert bench.measured_traffic("w", "down_mfma") is None
    assert bench.measured_traffic("w", "combine") is None
    assert bench.measured_traffic("other", "gateup_mfma") is None


@pytest.mark.parametrize("name", list(inputs.CONFIGS))
def test_committed_traffic_summaries_are_complete(name):
    """Every workload has a stored FETCH/WRITE summary with the copy
    calibration and a source hash per stage."""
    path = os.path.join(bench.ROOT, "profiles", f"traffic_{name}.json")
    with open(path) as fh:
        rec = json.load(fh)
    cal = rec["copy_calibration"]
    assert cal["bytes"] > 0 and cal["fetch_kib"] > 0 and cal["write_kib"] > 0
    assert rec["kernels"]
    for st, k in rec["kernels"].items():
        assert st in bench.STAGE_SOURCES
        assert len(k["sources_sha256"]) == 64 and k["fetch_kib"] >= 0 and k["write_kib"] >= 0
