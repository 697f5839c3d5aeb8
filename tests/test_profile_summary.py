"""Host logic of the rocprofv3 summaries (no GPU): the MFMA-utilisation
figures are computed from synthetic counter rows whose answers are known."""
import csv
import os

import pytest

from gqa_attention_flashattention_amd import profile_summary as ps


def _write_counters(path, rows):
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, ["Dispatch_Id", "Kernel_Name", "Grid_Size", "Counter_Name",
                               "Counter_Value"])
        w.writeheader()
        for r in rows:
            w.writerow(r)


def test_mfma_table_normalisation(tmp_path):
    name = "void gqa::(anonymous namespace)::prefill_bf16_kernel<128, 1, false>(...)"
    cycles = 1000.0
    rows = []
    for disp in (1, 2, 3):
        def row(c, v):
            return {"Dispatch_Id": disp, "Kernel_Name": name, "Grid_Size": 4096,
                    "Counter_Name": c, "Counter_Value": v}
        # GRBM_GUI_ACTIVE comes as one value per XCD; the busy counter as
        # per-SE shares that the reader sums
        rows += [row("GRBM_GUI_ACTIVE", cycles) for _ in range(ps.XCDS)]
        rows += [row("SQ_VALU_MFMA_BUSY_CYCLES", 0.25 * ps.SIMDS * cycles) for _ in range(2)]
        rows.append(row("SQ_INSTS_MFMA", 100.0))
        rows.append(row("SQ_INSTS_VALU", 450.0))
        # half the peak rate: 0.5 * 1024 flops per SIMD cycle over every SIMD
        rows.append(row("SQ_INSTS_VALU_MFMA_MOPS_BF16",
                        0.5 * ps.BF16_FLOPS_PER_SIMD_CYCLE * ps.SIMDS * cycles / ps.FLOPS_PER_MOP))
    _write_counters(str(tmp_path / "a"), rows)
    t = ps.mfma_table([str(tmp_path / "a")])
    rec = t["prefill_bf16_kernel<128,1,false>@4096"]
    assert rec["dispatches"] == 3
    assert rec["cycles"] == pytest.approx(cycles)
    assert rec["mfma_busy"] == pytest.approx(0.5)
    assert rec["valu_insts_per_mfma"] == pytest.approx(4.5)
    assert rec["mfma_rate_frac"] == pytest.approx(0.5)
    assert rec["counted_mfma_flops"] == pytest.approx(0.5 * 1024 * ps.SIMDS * cycles)
    assert "mfma_valu_coexec" not in rec


def test_mfma_table_skips_kernels_without_mfma(tmp_path):
    rows = [{"Dispatch_Id": 1, "Kernel_Name": "__amd_rocclr_copyBuffer", "Grid_Size": 64,
             "Counter_Name": c, "Counter_Value": v}
            for c, v in (("GRBM_GUI_ACTIVE", 10.0), ("SQ_VALU_MFMA_BUSY_CYCLES", 0.0))]
    _write_counters(str(tmp_path / "b"), rows)
    assert ps.mfma_table([str(tmp_path / "b")]) == {}


def test_committed_mfma_record_is_well_formed():
    """profiles/mfma.json, where present, holds fractions in (0, 1] and the
    source hash bench.py compares before reporting a record."""
    import json
    if not os.path.exists(ps.MFMA_JSON):
        pytest.skip("no MFMA record committed")
    rec = json.load(open(ps.MFMA_JSON))
    for k, r in rec.items():
        assert len(r["source_sha256"]) == 64, k
        assert 0.0 < r["mfma_busy"] <= 1.0
        assert r["dispatches"] >= 1 and r["cycles"] > 0
