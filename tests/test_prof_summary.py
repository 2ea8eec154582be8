"""Host logic of the profile summariser (mamba_ssd_layer_amd.prof_summary) on
small synthetic rocprofv3 counter files: per-dispatch averages of counters
summed over their instances, the largest instance of GRBM_GUI_ACTIVE, and the
ratios the `busy` table prints."""
import csv
import os

from mamba_ssd_layer_amd import prof_summary as ps

FIELDS = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]


def _write(d, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for r in rows:
            w.writerow(dict(zip(FIELDS, r)))


def test_counter_per_dispatch_sums_instances_and_averages_dispatches(tmp_path):
    d = str(tmp_path / "c")
    k = "void ssd::foo_kernel<256>(ssd::P)"
    _write(d, [(1, k, "SQ_INSTS_LDS", 10), (1, k, "SQ_INSTS_LDS", 30),  # two instances: 40
               (2, k, "SQ_INSTS_LDS", 60),                               # dispatch 2: 60
               (3, "other_kernel", "SQ_INSTS_LDS", 1000)])
    assert ps._counter_per_dispatch(d, "foo_kernel", "SQ_INSTS_LDS") == 50.0
    assert ps._counter_per_dispatch(d, "foo_kernel", "SQ_INSTS_LDS", "max") == 45.0  # (30 + 60) / 2


def test_busy_table_ratios(tmp_path):
    d = str(tmp_path / "sq")
    k = "void ssd::bar_kernel<128>(ssd::P)"
    active = 8 * 1000.0  # GRBM_GUI_ACTIVE summed over the 8 dies: 1000 clocks per die
    busy = 0.25 * 1000.0 * ps.SIMDS  # a quarter of every SIMD's clocks
    _write(d, [(7, k, "SQ_VALU_MFMA_BUSY_CYCLES", busy), (7, k, "SQ_INSTS_VALU_MFMA_MOPS_BF16", 2e6),
               (7, k, "GRBM_GUI_ACTIVE", active), (7, k, "GRBM_GUI_ACTIVE", 100.0),  # largest taken
               (7, k, "SQ_WAIT_INST_ANY", 30.0),
               (7, k, "SQ_WAVE_CYCLES", 120.0), (7, k, "SQ_INSTS_LDS", 3.5e6)])
    row = ps.busy_table(d, ["bar_kernel"]).splitlines()[2]
    cells = [c.strip() for c in row.strip("|").split("|")]
    assert cells[1] == "0.250"            # MFMA busy fraction
    assert cells[2] == f"{2e6 * 512 / 1e9:.2f}"  # executed MFMA GFLOP
    assert cells[3] == "0.25"             # wave time waiting to issue
    assert cells[4] == "3.50"             # LDS instructions, millions
