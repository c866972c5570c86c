"""Reduce rocprofv3 hardware-counter runs of bench.py to per-kernel figures of one DiT block.

Measurement tooling, not part of the compute path.  Input: the output folders of several
`rocprofv3 --pmc ... --output-format csv -d DIR -- python3 bench.py ...` runs (one counter set per
run) of the same workload.  Each dispatch is labelled by its kernel name and its position inside a
block (a block starts with the modulation-combine launch, and the block's launches come in a fixed
order: LN1, V^T tail, Q/K/V product, QK norm + RoPE, self-attention, O product, LN3, cross-q product,
cross-attention, cross-O product, LN2, FFN1, FFN2).  Counter values are averaged per label.

Derived figures:
  * HBM bytes per launch: FETCH_SIZE and WRITE_SIZE (KiB per dispatch) scaled by what the same counter
    reads for a plain device copy of known size in the same run (the `--copy-bytes` dispatch);
  * MFMA FLOPs per launch: SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512;
  * MFMA busy: SQ_VALU_MFMA_BUSY_CYCLES / GRBM_GUI_ACTIVE, relative to the same ratio of the
    register-only MFMA probe in the same run (a kernel that issues nothing but MFMAs);
  * VALU and LDS activity: SQ_ACTIVE_INST_VALU, SQ_ACTIVE_INST_LDS per GRBM_GUI_ACTIVE cycle and wave,
    and SQ_LDS_BANK_CONFLICT against SQ_INSTS_LDS.

Usage: python -m video_diffusion_transformer_step_amd.counters DIR [DIR ...] --out JSON
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import sys

# Order of the launches of one bf16 block (no attention cache, no quantised path).
BLOCK_ORDER = ["mod_combine", "ln1", "vt_tail", "qkv_gemm", "qk_norm_rope", "self_attn", "o_gemm", "ln3",
               "cross_q_gemm", "cross_attn", "cross_o_gemm", "ln2", "ffn1_gemm", "ffn2_gemm"]
# kernel-name fragment -> the labels its launches take, in their order inside a block
BY_NAME = [("mod_combine", ["mod_combine"]),
           ("ln_mod", ["ln1", "ln3", "ln2"]),
           ("vt_tail_zero", ["vt_tail"]),
           ("EpiQKV", ["qkv_gemm"]),
           ("qk_norm_rope", ["qk_norm_rope"]),
           ("attention_pp_kernel", ["self_attn"]),
           ("EpiResidual", ["o_gemm", "cross_o_gemm", "ffn2_gemm"]),
           ("EpiStore", ["cross_q_gemm", "ffn1_gemm"]),
           ("attention_kernel", ["cross_attn"])]
COPY_NAME = "copyBuffer"
PROBE_NAME = "mfma_peak_kernel<0>"  # the bf16 register-only MFMA probe
SOURCES = ["attention.hip", "gemm.hip", "norm.hip", "layout.hip"]


def _col(row, *names):
    for n in names:
        if n in row and row[n] != "":
            return row[n]
    return None


def read_dispatches(folder):
    """{dispatch id: {"name", "grid", "counters": {name: value}}} from one rocprofv3 output folder."""
    out = {}
    files = glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True)
    for path in files:
        with open(path, newline="") as fh:
            for row in csv.DictReader(fh):
                did = int(_col(row, "Dispatch_Id", "Dispatch_ID", "Correlation_Id"))
                d = out.setdefault(did, {"name": _col(row, "Kernel_Name", "Kernel-Name") or "",
                                         "grid": _col(row, "Grid_Size", "Grid_Size_X") or "",
                                         "counters": {}})
                cname = _col(row, "Counter_Name", "Counter-Name")
                val = float(_col(row, "Counter_Value", "Counter-Value"))
                d["counters"][cname] = d["counters"].get(cname, 0.0) + val
    return out


def label_dispatches(disp):
    """[(label, dispatch)] for block launches, plus the copy and probe dispatches."""
    labelled = []
    seen = {}
    in_block = False
    for did in sorted(disp):
        d = disp[did]
        name = d["name"]
        if COPY_NAME in name:
            labelled.append(("copy", d))
            continue
        if PROBE_NAME in name:
            labelled.append(("mfma_probe", d))
            continue
        if "mod_combine" in name:
            seen = {}
            in_block = True
        if not in_block:
            continue
        for frag, labels in BY_NAME:
            if frag in name:
                k = seen.get(frag, 0)
                seen[frag] = k + 1
                if k < len(labels):
                    labelled.append((labels[k], d))
                    if labels[k] == "ffn2_gemm":
                        in_block = False
                break
    return labelled


def reduce(folders):
    per = {}
    for f in folders:
        for label, d in label_dispatches(read_dispatches(f)):
            e = per.setdefault(label, {"name": d["name"], "counters": {}})
            for c, v in d["counters"].items():
                e["counters"].setdefault(c, []).append(v)
    res = {}
    for label, e in per.items():
        res[label] = {"kernel": e["name"], "n": {c: len(v) for c, v in e["counters"].items()},
                      "mean": {c: sum(v) / len(v) for c, v in e["counters"].items()},
                      "max": {c: max(v) for c, v in e["counters"].items()}}
    return res


def derive(res, copy_bytes):
    out = {}
    # the calibration copy is the largest device copy of the run (the runtime also copies small buffers)
    cp = res.get("copy", {}).get("max", {})
    fscale = (copy_bytes / 1024.0) / cp["FETCH_SIZE"] if cp.get("FETCH_SIZE") else None
    wscale = (copy_bytes / 1024.0) / cp["WRITE_SIZE"] if cp.get("WRITE_SIZE") else None
    probe = res.get("mfma_probe", {}).get("mean", {})
    probe_busy = (probe["SQ_VALU_MFMA_BUSY_CYCLES"] / probe["GRBM_GUI_ACTIVE"]
                  if probe.get("SQ_VALU_MFMA_BUSY_CYCLES") and probe.get("GRBM_GUI_ACTIVE") else None)
    for label in BLOCK_ORDER:
        if label not in res:
            continue
        m = res[label]["mean"]
        e = {"kernel": res[label]["kernel"]}
        if fscale and "FETCH_SIZE" in m:
            e["fetch_bytes"] = m["FETCH_SIZE"] * 1024.0 * fscale
        if wscale and "WRITE_SIZE" in m:
            e["write_bytes"] = m["WRITE_SIZE"] * 1024.0 * wscale
        if "fetch_bytes" in e and "write_bytes" in e:
            e["hbm_bytes"] = e["fetch_bytes"] + e["write_bytes"]
        if "SQ_INSTS_VALU_MFMA_MOPS_BF16" in m:
            e["mfma_flops"] = m["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512.0
        gui = m.get("GRBM_GUI_ACTIVE")
        if gui and "SQ_VALU_MFMA_BUSY_CYCLES" in m and probe_busy:
            e["mfma_busy_vs_probe"] = m["SQ_VALU_MFMA_BUSY_CYCLES"] / gui / probe_busy
        if "SQ_INSTS_LDS" in m and "SQ_LDS_BANK_CONFLICT" in m:
            e["lds_bank_conflict_cycles_per_lds_inst"] = m["SQ_LDS_BANK_CONFLICT"] / max(m["SQ_INSTS_LDS"], 1.0)
        for c in ("SQ_INSTS_VALU", "SQ_INSTS_VALU_TRANS_F32", "SQ_INSTS_LDS", "SQ_INSTS_MFMA", "SQ_WAVES"):
            if c in m:
                e[c] = m[c]
        if gui:
            e["gui_active_cycles"] = gui
            for c in ("SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_LDS", "SQ_WAIT_INST_LDS", "SQ_VALU_MFMA_COEXEC_CYCLES",
                      "SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_ANY", "SQ_BUSY_CYCLES", "SQ_WAVE_CYCLES"):
                if c in m:
                    e[c + "_per_gui_cycle"] = m[c] / gui
        out[label] = e
    meta = {"fetch_scale": fscale, "write_scale": wscale, "copy_bytes": copy_bytes,
            "probe_mfma_busy_per_gui_cycle": probe_busy,
            "source_sha256": {s: _sha(s) for s in SOURCES}}
    return {"meta": meta, "kernels": out}


def _sha(src):
    p = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc", src)
    return hashlib.sha256(open(p, "rb").read()).hexdigest()


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("folders", nargs="+")
    ap.add_argument("--copy-bytes", type=int, default=1 << 30)
    ap.add_argument("--out", required=True)
    a = ap.parse_args(argv)
    res = derive(reduce(a.folders), a.copy_bytes)
    with open(a.out, "w") as fh:
        json.dump(res, fh, indent=1, sort_keys=True)
    print(json.dumps(res, indent=1, sort_keys=True))
    return 0


if __name__ == "__main__":
    sys.exit(main())
