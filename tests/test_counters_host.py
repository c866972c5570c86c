"""Host logic of the counter reduction (video_diffusion_transformer_step_amd.counters) on synthetic
rocprofv3 CSV folders: launch labelling by position inside a block, copy calibration of the byte
counters, the MFMA-busy ratio against the probe, kernel-trace durations and the markdown table."""
import csv
import json

from video_diffusion_transformer_step_amd import counters as C

# kernel names as the block launches them (fragments are what the labeller matches)
BLOCK = [("mod_combine_kernel", "mod_combine"), ("ln_mod_kernel", "ln1"), ("attn_prologue_kernel", "attn_prologue"),
         ("gemm_lds_kernel<EpiQKV>", "qkv_gemm"), ("qk_rms_kernel", "qk_rms"),
         ("attention_pp_kernel<bf16>", "self_attn"), ("gemm_lds_kernel<EpiResidual>", "o_gemm"),
         ("ln_mod_kernel", "ln3"), ("gemm_lds_kernel<EpiStore>", "cross_q_gemm"),
         ("attention_kernel<bf16,1>", "cross_attn"), ("gemm_lds_kernel<EpiResidual>", "cross_o_gemm"),
         ("ln_mod_kernel", "ln2"), ("gemm_lds_kernel<EpiStore>", "ffn1_gemm"),
         ("gemm_lds_kernel<EpiResidual>", "ffn2_gemm")]


def _write(folder, rows, fields, name):
    folder.mkdir(parents=True, exist_ok=True)
    with open(folder / name, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=fields)
        w.writeheader()
        for r in rows:
            w.writerow(r)


def _pmc_rows(values):
    """values: list of (kernel name, {counter: value}) in dispatch order."""
    rows = []
    for i, (name, cnt) in enumerate(values):
        for c, v in cnt.items():
            rows.append({"Dispatch_Id": i + 1, "Kernel_Name": name, "Grid_Size": 1, "Counter_Name": c,
                         "Counter_Value": v})
    return rows


def test_labels_calibration_and_markdown(tmp_path):
    copy_bytes = 1 << 20
    # a small copy first (the runtime's), the calibration copy, the probe, then two blocks
    seq = [("__amd_rocclr_copyBuffer", {"FETCH_SIZE": 10.0, "WRITE_SIZE": 5.0}),
           ("__amd_rocclr_copyBuffer", {"FETCH_SIZE": 2048.0, "WRITE_SIZE": 1024.0}),  # 1 MiB copy: x0.5 / x1
           ("mfma_peak_kernel<0>", {"SQ_VALU_MFMA_BUSY_CYCLES": 400.0, "GRBM_GUI_ACTIVE": 4.0})]
    seq.append(("wan::patchify_kernel(float const*)", {"FETCH_SIZE": 8.0, "WRITE_SIZE": 16.0}))
    for blk in range(2):
        for i, (name, label) in enumerate(BLOCK):
            seq.append((name, {"FETCH_SIZE": 100.0 * (i + 1) + blk, "WRITE_SIZE": 10.0 * (i + 1),
                               "SQ_VALU_MFMA_BUSY_CYCLES": 50.0 * (i + 1), "GRBM_GUI_ACTIVE": 2.0,
                               "SQ_ACTIVE_INST_VALU": 6.0}))
    fields = ["Dispatch_Id", "Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"]
    seq.append(("wan::unpatchify_kernel(float const*)", {"FETCH_SIZE": 4.0, "WRITE_SIZE": 16.0}))
    seq.append(("wan::euler_kernel(float*)", {"FETCH_SIZE": 32.0, "WRITE_SIZE": 16.0}))
    _write(tmp_path / "pmc", _pmc_rows(seq), fields, "p_counter_collection.csv")
    trace = [{"Dispatch_Id": i + 1, "Kernel_Name": n, "Start_Timestamp": 1000 * i,
              "End_Timestamp": 1000 * i + 500 + 10 * i} for i, (n, _) in enumerate(seq)]
    _write(tmp_path / "kt", trace, ["Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp"],
           "k_kernel_trace.csv")

    labelled = C.label_dispatches(C.read_dispatches(str(tmp_path / "pmc")))
    labels = [lab for lab, _ in labelled]
    assert labels.count("copy") == 2 and labels.count("mfma_probe") == 1
    assert [lab for lab in labels if lab not in ("copy", "mfma_probe")] == (["patchify"] + [b for _, b in BLOCK] * 2 +
                                                                          ["unpatchify", "euler"])

    res = C.derive(C.reduce([str(tmp_path / "pmc")]), copy_bytes)
    assert abs(res["meta"]["fetch_scale"] - 0.5) < 1e-12 and abs(res["meta"]["write_scale"] - 1.0) < 1e-12
    k = res["kernels"]
    # o_gemm is the 7th launch of each block: FETCH 700 / 701 KiB -> mean 700.5 KiB x 0.5, WRITE 70 KiB
    assert abs(k["o_gemm"]["fetch_bytes"] - 700.5 * 1024 * 0.5) < 1e-6
    assert abs(k["o_gemm"]["write_bytes"] - 70 * 1024) < 1e-6
    # MFMA busy per GUI cycle 350 / 2 against the probe's 100
    assert abs(k["o_gemm"]["mfma_busy_vs_probe"] - 1.75) < 1e-12
    assert abs(k["ln1"]["SQ_ACTIVE_INST_VALU_per_gui_cycle"] - 3.0) < 1e-12
    # once-per-step kernels: "unpatchify" must not be taken for "patchify"
    assert abs(k["euler"]["hbm_bytes"] - (32 * 1024 * 0.5 + 16 * 1024)) < 1e-6
    assert abs(k["unpatchify"]["fetch_bytes"] - 4 * 1024 * 0.5) < 1e-6

    means = C.trace_means(str(tmp_path / "kt"))
    # self_attn is dispatch 10 (block 0) and 24 (block 1): durations 500 + 10 * (9, 23)
    assert abs(means["self_attn"] - (500 + 10 * 16)) < 1e-9
    out = tmp_path / "c.json"
    md = tmp_path / "c.md"
    assert C.main([str(tmp_path / "pmc"), "--copy-bytes", str(copy_bytes), "--out", str(out), "--trace",
                   str(tmp_path / "kt"), "--md", str(md), "--command", "rocprofv3 ..."]) == 0
    rec = json.loads(out.read_text())
    assert abs(rec["kernels"]["self_attn"]["mean_ns"] - 660.0) < 1e-9
    text = md.read_text()
    assert "| self_attn |" in text and "| ffn2_gemm |" in text and "| euler |" in text and "rocprofv3 ..." in text


def test_by_name_fractions_and_trace(tmp_path):
    """--by-name: per-fragment means over dispatches, SQ fractions of SQ_WAVE_CYCLES, MFMA busy per GUI
    cycle, trace durations; dispatches of other kernels are ignored."""
    fields = ["Dispatch_Id", "Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"]
    seq = [("attention_q8_kernel<128>", {"SQ_WAVE_CYCLES": 100.0, "SQ_WAIT_ANY": 40.0, "GRBM_GUI_ACTIVE": 10.0,
                                         "SQ_VALU_MFMA_BUSY_CYCLES": 300.0}),
           ("ln_mod_kernel", {"SQ_WAVE_CYCLES": 7.0}),
           ("attention_q8_kernel<128>", {"SQ_WAVE_CYCLES": 300.0, "SQ_WAIT_ANY": 200.0, "GRBM_GUI_ACTIVE": 30.0,
                                         "SQ_VALU_MFMA_BUSY_CYCLES": 500.0}),
           ("attention_pp_kernel<bf16>", {"SQ_WAVE_CYCLES": 50.0, "SQ_ACTIVE_INST_VALU": 10.0})]
    _write(tmp_path / "p", _pmc_rows(seq), fields, "p_counter_collection.csv")
    trace = [{"Dispatch_Id": i + 1, "Kernel_Name": n, "Start_Timestamp": 0, "End_Timestamp": 1000 * (i + 1)}
             for i, (n, _) in enumerate(seq)]
    _write(tmp_path / "kt", trace, ["Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp"],
           "k_kernel_trace.csv")
    res = C.by_name([str(tmp_path / "p")], ["attention_q8_kernel", "attention_pp_kernel"], str(tmp_path / "kt"))
    q8 = res["attention_q8_kernel"]
    assert q8["n"] == 2 and abs(q8["mean"]["SQ_WAVE_CYCLES"] - 200.0) < 1e-12
    assert abs(q8["wave_fraction"]["SQ_WAIT_ANY"] - 120.0 / 200.0) < 1e-12
    assert abs(q8["mfma_busy_per_gui"] - 400.0 / 20.0) < 1e-12
    assert abs(q8["mean_ns"] - (1000 + 3000) / 2) < 1e-9 and q8["trace_n"] == 2
    pp = res["attention_pp_kernel"]
    assert abs(pp["wave_fraction"]["SQ_ACTIVE_INST_VALU"] - 0.2) < 1e-12 and "mfma_busy_per_gui" not in pp
    md = tmp_path / "k.md"
    assert C.main([str(tmp_path / "p"), "--by-name", "attention_q8_kernel,attention_pp_kernel", "--out",
                   str(tmp_path / "k.json"), "--md", str(md), "--command", "rocprofv3 ..."]) == 0
    text = md.read_text()
    assert "| SQ_WAIT_ANY / SQ_WAVE_CYCLES | 0.600 |" in text and "rocprofv3 ..." in text
