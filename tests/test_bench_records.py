"""Host logic of the bench's per-case records: the case list and the merge of
rocprofv3 counter CSVs of --counter-pass runs (dispatches of the library's
products grouped by the idle gaps between cases, setup kernels ignored,
FETCH_SIZE scaled by the closing 256 MiB copy)."""
import csv
import os

import pytest

import bench
import synth


def test_record_cases_cover_every_matrix():
    cases = bench.record_cases(synth)
    ones = [(w.cfg_id, i) for w, i, n in cases if n == 1]
    want = [(w.cfg_id, i) for w in (synth.CFG1, synth.CFG2, synth.CFG3, synth.CFG4, synth.CFG5, synth.CFG6)
            for i in range(len(w.tensors))]
    assert ones == want
    assert [(w.cfg_id, n) for w, i, n in cases if w is synth.CFG5 and n > 1] == [(5, 8)] * 3 + [(5, 128)] * 3
    assert len(cases) == len(set((w.cfg_id, i, n) for w, i, n in cases))


def _write(path, dispatches):
    cols = ["Correlation_Id", "Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp",
            "End_Timestamp"]
    with open(path, "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=cols)
        wr.writeheader()
        for k, (name, t0, counters) in enumerate(dispatches):
            for c, v in counters.items():
                wr.writerow({"Correlation_Id": k, "Dispatch_Id": k + 1, "Kernel_Name": name, "Counter_Name": c,
                             "Counter_Value": v, "Start_Timestamp": t0, "End_Timestamp": t0 + 1000})


def test_counters_grouped_by_gaps_and_scaled(tmp_path):
    gap = int(bench.COUNTER_GAP_S * 1e9)
    rp = "qg::(anonymous namespace)::repack_q4_0_kernel(unsigned char const*)"
    g1 = "void qg::xs_detail::gemv_xs_kernel<0, 1, 0, 4, 4>(qg::xs_detail::XsParams)"
    g2 = "void qg::prefill_mfma_kernel<0, 1, 1, 4, 8, 1, 0>(qg::PrefillParams)"
    red = "void qg::(anonymous namespace)::prefill_reduce_kernel<1, 4>(float const*)"
    cp = "__amd_rocclr_copyBuffer"
    t = 10 ** 9
    d = [(rp, t, {"FETCH_SIZE": 5.0}), (rp, t + 50, {"FETCH_SIZE": 5.0}),            # setup, ignored
         (g1, t + gap, {"FETCH_SIZE": 100.0}),                                          # case 0
         (g2, t + 2 * gap, {"FETCH_SIZE": 200.0}), (red, t + 2 * gap + 5000, {"FETCH_SIZE": 30.0}),  # case 1
         (g1, t + 3 * gap, {"FETCH_SIZE": 7.0}),                                        # case 2
         (cp, t + 4 * gap, {"FETCH_SIZE": 131072.0})]                                   # half of 256 MiB
    os.makedirs(tmp_path / "a")
    _write(tmp_path / "a" / "run_counter_collection.csv", d)
    d2 = [(g1, t + gap, {"SQ_INSTS_VALU": 10.0, "GRBM_GUI_ACTIVE": 8.0}),
          (g2, t + 2 * gap, {"SQ_INSTS_VALU": 20.0, "GRBM_GUI_ACTIVE": 16.0}),
          (red, t + 2 * gap + 5000, {"SQ_INSTS_VALU": 1.0, "GRBM_GUI_ACTIVE": 8.0}),
          (g1, t + 3 * gap, {"SQ_INSTS_VALU": 3.0, "GRBM_GUI_ACTIVE": 8.0})]
    os.makedirs(tmp_path / "b")
    _write(tmp_path / "b" / "run_counter_collection.csv", d2)
    out = bench.counters_by_case([str(tmp_path / "a"), str(tmp_path / "b")], 3)
    assert out["FETCH_SIZE"] == [100.0 * 2048, 230.0 * 2048, 7.0 * 2048]
    assert out["SQ_INSTS_VALU"] == [10.0, 21.0, 3.0]
    assert out["GRBM_GUI_ACTIVE"] == [8.0, 24.0, 8.0]
    with pytest.raises(RuntimeError):
        bench.counters_by_case([str(tmp_path / "b")], 4)
