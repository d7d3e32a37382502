"""The profile summariser on tiny hand-made rocprofv3 CSV files (CPU only)."""

import json

from exact_attention_state_amd import profsum

TRACE_HEAD = "Kernel_Name,Grid_Size,Start_Timestamp,End_Timestamp\n"


def _write(p, text):
    p.write_text(text)
    return str(p)


def test_trace_table_averages_and_filters(tmp_path):
    rows = [
        '"void lc::a_kernel<1>(lc::Args)",512,1000,3000',      # 2 us
        '"void lc::a_kernel<1>(lc::Args)",512,5000,9000',      # 4 us
        '"void lc::a_kernel<1>(lc::Args)",1024,10000,30000',   # 20 us, another shape
        '"other(int)",64,0,1000',                              # 1 us
    ]
    path = _write(tmp_path / "t.csv", TRACE_HEAD + "\n".join(rows) + "\n")
    t = profsum.trace_table(path)
    assert t[0][0] == "void lc::a_kernel<1>" and t[0][1] == 3 and abs(t[0][2] - 26 / 3) < 1e-9
    assert abs(sum(r[5] for r in t) - 1.0) < 1e-12
    t = profsum.trace_table(path, only=["a_kernel"], max_grid=512)
    assert len(t) == 1 and t[0][1] == 2 and t[0][2] == 3.0 and t[0][3] == 2.0 and t[0][4] == 4.0
    md = profsum.trace_markdown(path, "T", "cmd", only=["a_kernel"], max_grid=512)
    assert "| `void lc::a_kernel<1>` | 2 | 3.00 | 2.00 | 4.00 | 100.0% |" in md and "cmd" in md


def test_traffic_is_scaled_by_the_copy_calibration(tmp_path):
    head = "Kernel_Name,Counter_Value\n"
    cf = _write(tmp_path / "cf.csv", head + '"__amd_rocclr_copyBuffer",1024\n"__amd_rocclr_copyBuffer",1024\n')
    cw = _write(tmp_path / "cw.csv", head + '"__amd_rocclr_copyBuffer",2048\n')
    f = _write(tmp_path / "f.csv", head + '"k(int)",10\n"k(int)",30\n"k(int)",20\n')
    w = _write(tmp_path / "w.csv", head + '"k(int)",4\n')
    r = profsum.traffic(f, w, cf, cw, copy_bytes=2 * 1024 * 1024)
    # the copy's fetch reads 1024 KiB for 2 MiB: factor 2; its write 2048 KiB: factor 1
    assert r["calibration"]["fetch_factor"] == 2.0 and r["calibration"]["write_factor"] == 1.0
    k = r["kernels"]["k"]
    assert k["fetch_bytes_median"] == 20 * 1024 * 2 and k["write_bytes_median"] == 4 * 1024 and k["dispatches"] == 3
    json.dumps(r)
