"""The rocprofv3 summaries (host only): symbol names map to the library's profiler names, and
the traffic record scales each kernel's counters by the calibration copy's."""
import csv

from hierarchical_top_sparse_amd import profiling


def _write(path, rows):
    cols = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=cols)
        w.writeheader()
        for r in rows:
            w.writerow(dict(zip(cols, r)))


def test_profile_names():
    assert profiling.profile_name("llsa::bwd_key_kernel<2>(llsa::BwdArgs)")[0] == \
        "bwd_key_overflow_kernel"
    assert profiling.profile_name("void llsa::select_pool_next_kernel<8>(a, b)")[0] == \
        "select_pool_kernel"
    assert profiling.profile_name("llsa::pool_next_kernel<16>(x)") == ("pool_next_kernel",
                                                                       "pool.hip")
    # kernels templated on the head width as well
    assert profiling.profile_name("void llsa::bwd_key_kernel<2, 64>(llsa::BwdArgs)")[0] == \
        "bwd_key_overflow_kernel"
    assert profiling.profile_name("llsa::bwd_key_kernel<0, 128>(llsa::BwdArgs)")[0] == \
        "bwd_key_kernel"
    assert profiling.profile_name("void llsa::csc_radix_kernel(llsa::CscArgs)") == \
        ("csc_radix_kernel", "transpose.hip")
    assert profiling.profile_name("at::native::elementwise_kernel<128, 4>(...)") is None


def test_traffic_record_scales_by_the_copy(tmp_path):
    T = 96 * 2 ** 20
    _write(tmp_path / "f.csv", [(1, "llsa::reorder_kernel(x)", "FETCH_SIZE", T / 2048),
                                (2, "llsa::attn_fwd_kernel<true, 4>(a)", "FETCH_SIZE", 1000.0),
                                (3, "llsa::attn_fwd_kernel<true, 4>(a)", "FETCH_SIZE", 3000.0)])
    _write(tmp_path / "w.csv", [(1, "llsa::reorder_kernel(x)", "WRITE_SIZE", T / 1024),
                                (2, "llsa::attn_fwd_kernel<true, 4>(a)", "WRITE_SIZE", 500.0),
                                (3, "llsa::attn_fwd_kernel<true, 4>(a)", "WRITE_SIZE", 500.0)])
    rec = profiling.traffic_record(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), T,
                                   "test", ["cmd"])
    assert rec["fetch_scale"] == 2.0 and rec["write_scale"] == 1.0
    k = rec["kernels"]["attn_fwd_kernel"]
    assert k["dispatches"] == 2
    assert k["hbm_read_bytes_per_launch"] == 2000 * 2 * 1024
    assert k["hbm_write_bytes_per_launch"] == 500 * 1024
    assert k["source"].endswith("attn_fwd.hip") and len(k["source_sha256"]) == 64


def test_step_timelines_split_at_the_first_kernel(tmp_path):
    cols = ["Kernel_Name", "Queue_Id", "Start_Timestamp", "End_Timestamp"]
    rows = []
    for step, t0 in enumerate((1000, 9000, 20000)):   # ns; the third step is cut short
        rows.append(("void llsa::pool12_bf16_kernel<64>(a)", 1, t0, t0 + 1000))
        rows.append(("llsa::copy_kernel(x)", 1, t0 + 1100, t0 + 1200))   # calibration: skipped
        if step < 2:
            rows.append(("void llsa::attn_fwd_kernel<true, 4, 64>(a)", 1, t0 + 1500, t0 + 5000))
            rows.append(("llsa::csc_radix_kernel(a)", 4, t0 + 1600, t0 + 3000))
    path = tmp_path / "k_kernel_trace.csv"
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=cols)
        w.writeheader()
        for r in rows:
            w.writerow(dict(zip(cols, r)))
    steps = profiling.step_timelines(str(path), last_steps=3)
    assert len(steps) == 2   # the short one is left out
    assert steps[1] == [("pool12_kernel", 1, 0.0, 1.0), ("attn_fwd_kernel", 1, 1.5, 5.0),
                        ("csc_radix_kernel", 4, 1.6, 3.0)]


def test_sq_rows_derive_busy_flops_and_per_wave_counts(tmp_path):
    gui = 8 * 1000.0   # summed over the 8 XCDs: 1000 cycles
    p1 = [(1, "void llsa::attn_fwd_kernel<true, 4, 64>(a)", n, v) for n, v in
          (("GRBM_GUI_ACTIVE", gui), ("SQ_WAVES", 100.0),
           ("SQ_VALU_MFMA_BUSY_CYCLES", 1024 * 250.0), ("SQ_INSTS_VALU_MFMA_MOPS_BF16", 2e6))]
    p2 = [(1, "void llsa::attn_fwd_kernel<true, 4, 64>(a)", n, v) for n, v in
          (("GRBM_GUI_ACTIVE", gui), ("SQ_INSTS_VALU", 5000.0), ("SQ_INSTS_MFMA", 300.0),
           ("SQ_INSTS_LDS", 700.0), ("SQ_LDS_IDX_ACTIVE", 256 * 500.0),
           ("SQ_LDS_BANK_CONFLICT", 256 * 100.0))]
    _write(tmp_path / "p1.csv", p1)
    _write(tmp_path / "p2.csv", p2)
    (r,) = profiling.sq_rows([str(tmp_path / "p1.csv"), str(tmp_path / "p2.csv")],
                             ["attn_fwd_kernel"])
    assert r["gui_cycles"] == 1000.0
    assert r["mfma_busy"] == 0.25 and r["mfma_gflop"] == 2e6 * 512 / 1e9
    assert (r["valu_per_wave"], r["mfma_per_wave"], r["lds_per_wave"]) == (50.0, 3.0, 7.0)
    assert r["lds_active"] == 0.5 and r["bank_conflict_share"] == 0.2


def test_sweep_tables_read_the_bench_lines(tmp_path):
    import json
    r = {"side": 64, "tokens": 4096, "dense_fwd_ms": 0.085, "llsa_fwd_ms": 0.05,
         "speedup_fwd": 1.7, "b64_fwd_ms": 0.0438, "b64_speedup_fwd": 1.94,
         "dense_train_ms": 0.306, "llsa_train_ms": 0.1154, "speedup_train": 2.65,
         "b64_train_ms": 0.1245, "b64_speedup_train": 2.46, "llsa_select_ms": 0.0223,
         "single_level_select_ms": 0.0528, "single_level_top32_train_ms": 0.176,
         "speedup_vs_single_level": 1.52, "single_level_bwd_csc_ms": 0.0969,
         "single_level_bwd_mask_ms": 0.0737, "key_pass_csc_block_pairs_per_s": 1.46e9,
         "key_pass_mask_block_pairs_per_s": 1.45e9, "key_pass_block_pairs_per_s": None}
    path = tmp_path / "sweep.jsonl"
    path.write_text("a progress line\n" + json.dumps(r) + "\n")
    md = profiling.sweep_tables(str(path))
    assert "| 64 | 4096 | 0.085 | 0.0500 | 1.7x |" in md
    assert "| 64 | 0.0223 | 0.0528 | 0.1154 | 0.1760 | 1.52x |" in md
    assert "| 64 | 0.0969 | 0.0737 | 1.46 G | 1.45 G | - |" in md
