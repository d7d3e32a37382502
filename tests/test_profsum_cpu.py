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


def test_step_traffic_takes_the_step_grid_and_bench_hashes(tmp_path):
    import bench
    head = "Kernel_Name,Grid_Size,Counter_Value\n"
    cf = _write(tmp_path / "cf.csv", head + '"__amd_rocclr_copyBuffer",64,1024\n')
    cw = _write(tmp_path / "cw.csv", head + '"__amd_rocclr_copyBuffer",64,2048\n')
    # three step launches of the skinny projection (grid 131072), refresh-shaped
    # launches (more of them, another grid) and three attention launches; a
    # prep kernel launched once (the refresh's) is left out
    sk = '"void lc::qkv_skinny_fused_kernel<128, 2, 8>(lc::QkvArgs)"'
    at = '"void lc::attn_ab_kernel<half, unsigned short, 128, 32>(lc::SeqArgs, lc::AttnArgs, int)"'
    rows = [f"{sk},131072,100", f"{sk},131072,300", f"{sk},131072,200"] + [f"{sk},4096,9999"] * 5 + \
           [f"{at},122880,50"] * 3 + ['"void lc::qkv_prep_kernel<8>(lc::PrepArgs)",49152,77']
    f = _write(tmp_path / "f.csv", head + "\n".join(rows) + "\n")
    w = _write(tmp_path / "w.csv", head + "\n".join(r.rsplit(",", 1)[0] + ",8" for r in rows) + "\n")
    r = profsum.step_traffic("llada8b", f, w, cf, cw, copy_bytes=2 * 1024 * 1024)
    q = r["kernels"]["qkv_gemm"]
    assert q["grid_size"] == 131072 and q["launches"] == 3 and q["fetch_size_kib"] == 200.0
    assert q["hbm_fetch_bytes"] == 200 * 1024 * 2 and q["hbm_write_bytes"] == 8 * 1024
    assert q["hbm_bytes_per_launch"] == q["hbm_fetch_bytes"] + q["hbm_write_bytes"]
    assert q["source_sha256"] == bench.kernel_source_hash("qkv_gemm")
    assert q["algorithmic_bytes"] == bench.step_accounting(__import__("exact_attention_state_amd.synth").synth.WORKLOADS["llada8b"])["kernels"]["qkv_gemm"]["bytes"]
    assert set(r["kernels"]) == {"qkv_gemm", "attn"}
    assert profsum.step_class("lc::merge_kernel<half, unsigned short, 128>") == "merge"
    assert profsum.step_class("lc::qkv_prep_kernel<8>") == "qkv_prep"
