"""Reduce rocprofv3 hardware-counter runs of bench.py to per-kernel figures of one DiT block (and of
the once-per-step layout kernels: patchify, unpatchify, the Euler update, the I2V input).

Measurement tooling, not part of the compute path.  Input: the output folders of several
`rocprofv3 --pmc ... --output-format csv -d DIR -- python3 bench.py ...` runs (one counter set per
run) of the same workload.  Each dispatch is labelled by its kernel name and its position inside a
block (a block starts with the modulation-combine launch, and the block's launches come in a fixed
order: LN1, attention prologue, Q/K/V product, QK RMS finish, self-attention, O product, LN3,
cross-q product, cross-attention, cross-O product, LN2, FFN1, FFN2).  Counter values are averaged per
label.

Derived figures:
  * HBM bytes per launch: FETCH_SIZE and WRITE_SIZE (KiB per dispatch) scaled by what the same counter
    reads for a plain device copy of known size in the same run (the `--copy-bytes` dispatch);
  * MFMA FLOPs per launch: SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512;
  * MFMA busy: SQ_VALU_MFMA_BUSY_CYCLES / GRBM_GUI_ACTIVE, relative to the same ratio of the
    register-only MFMA probe in the same run (a kernel that issues nothing but MFMAs);
  * VALU and LDS activity: SQ_ACTIVE_INST_VALU, SQ_ACTIVE_INST_LDS per GRBM_GUI_ACTIVE cycle and wave,
    and SQ_LDS_BANK_CONFLICT against SQ_INSTS_LDS.

With --trace DIR (a `rocprofv3 --kernel-trace --output-format csv` folder of the same workload) the
launches are labelled the same way and their mean durations added; with --md FILE a table of the
figures is written as markdown.

With --by-name FRAG[,FRAG...] the dispatches are grouped by kernel-name fragment instead (any workload):
per fragment, the mean of every counter over its dispatches, the SQ activity and wait counters as
fractions of SQ_WAVE_CYCLES, MFMA busy per GRBM_GUI_ACTIVE cycle, and the kernel-trace mean duration.

Usage: python -m video_diffusion_transformer_step_amd.counters DIR [DIR ...] --out JSON [--trace DIR]
       [--md FILE] [--command TEXT] [--by-name FRAG[,FRAG...]]
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import sys

# Order of the launches of one bf16 block (no attention cache, no quantised path).
BLOCK_ORDER = ["mod_combine", "ln1", "attn_prologue", "qkv_gemm", "qk_rms", "self_attn", "o_gemm", "ln3",
               "cross_q_gemm", "cross_attn", "cross_o_gemm", "ln2", "ffn1_gemm", "ffn2_gemm"]
# kernel-name fragment -> the labels its launches take, in their order inside a block
BY_NAME = [("mod_combine", ["mod_combine"]),
           ("ln_mod", ["ln1", "ln3", "ln2"]),
           ("attn_prologue", ["attn_prologue"]),
           ("EpiQKV", ["qkv_gemm"]),
           ("qk_rms", ["qk_rms"]),
           ("attention_pp_kernel", ["self_attn"]),
           ("EpiResidual", ["o_gemm", "cross_o_gemm", "ffn2_gemm"]),
           ("EpiStore", ["cross_q_gemm", "ffn1_gemm"]),
           ("attention_kernel", ["cross_attn"])]
# once-per-step kernels outside the blocks (name fragment -> label; the first match wins)
STEP_KERNELS = [("unpatchify_kernel", "unpatchify"), ("patchify_kernel", "patchify"), ("euler_kernel", "euler"),
                ("i2v_input_kernel", "i2v_input")]
STEP_ORDER = ["i2v_input", "patchify", "unpatchify", "euler"]
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


# launches that mark a block as not the plain bf16 one (quantised attention, E4M3 products, cache modes)
FOREIGN = ("EpiScaled", "q8", "quant", "e4m3", "cache")


def label_dispatches(disp):
    """[(label, dispatch)] for the launches of complete bf16 blocks, plus the copy and probe dispatches.
    A block's launches are kept only once its last launch (FFN2) is seen and none of its launches
    belongs to another block variant."""
    labelled = []
    seen = {}
    cur = None  # the current block's labelled launches, or None outside a block
    for did in sorted(disp):
        d = disp[did]
        name = d["name"]
        if COPY_NAME in name:
            labelled.append(("copy", d))
            continue
        if PROBE_NAME in name:
            labelled.append(("mfma_probe", d))
            continue
        step = next((lab for frag, lab in STEP_KERNELS if frag in name), None)
        if step is not None:
            labelled.append((step, d))
            continue
        if "mod_combine" in name:
            seen = {}
            cur = []
        if cur is None:
            continue
        if any(f in name for f in FOREIGN):
            cur = None
            continue
        for frag, labels in BY_NAME:
            if frag in name:
                k = seen.get(frag, 0)
                seen[frag] = k + 1
                if k < len(labels):
                    cur.append((labels[k], d))
                    if labels[k] == "ffn2_gemm":
                        labelled.extend(cur)
                        cur = None
                break
    return labelled


def read_trace(folder):
    """{dispatch id: {"name", "ns"}} from one rocprofv3 kernel-trace output folder."""
    out = {}
    for path in glob.glob(os.path.join(folder, "**", "*kernel_trace.csv"), recursive=True):
        with open(path, newline="") as fh:
            for row in csv.DictReader(fh):
                did = int(_col(row, "Dispatch_Id", "Dispatch_ID", "Correlation_Id"))
                ns = int(_col(row, "End_Timestamp")) - int(_col(row, "Start_Timestamp"))
                out[did] = {"name": _col(row, "Kernel_Name", "Kernel-Name") or "", "ns": ns}
    return out


def trace_means(folder):
    """{label: mean duration in ns} of the block launches in a kernel trace."""
    acc = {}
    for label, d in label_dispatches(read_trace(folder)):
        acc.setdefault(label, []).append(d["ns"])
    return {k: sum(v) / len(v) for k, v in acc.items()}


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
    for label in BLOCK_ORDER + STEP_ORDER:
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


def short_name(kernel):
    """The kernel's base name (and the GEMM epilogue, if any) from a mangled or demangled name."""
    m = re.search(r"_GLOBAL__N_1(\d+)", kernel)
    if m:  # mangled: <length><identifier> follows the anonymous namespace
        n = int(m.group(1))
        base = kernel[m.end():m.end() + n]
    else:
        base = re.sub(r"^void |wan::|\(anonymous namespace\)::", "", kernel)
        base = re.split(r"[<(]", base, maxsplit=1)[0]
    epi = re.findall(r"Epi(?:Scaled|QKV|Residual|Store)", kernel)
    return base + (" / " + ", ".join(dict.fromkeys(epi)) if epi else "")


def markdown(res, command=None):
    """A table of the per-launch figures (one row per block launch, in block order)."""
    meta = res["meta"]
    lines = ["# Per-launch hardware counters of one DiT block and the step's layout kernels", ""]
    if command:
        lines += ["Command (one rocprofv3 run per counter set, then this reduction):", "", "```", command, "```", ""]
    lines += [f"Byte counters scaled by the plain-copy calibration: FETCH_SIZE x {meta['fetch_scale']:.3f}, "
              f"WRITE_SIZE x {meta['write_scale']:.3f} (a {meta['copy_bytes'] / 2**30:.0f} GiB device copy in the "
              "same run). MFMA busy is SQ_VALU_MFMA_BUSY_CYCLES per GRBM_GUI_ACTIVE cycle relative to the "
              "register-only MFMA probe's ratio in the same run. VALU / LDS activity: SQ_ACTIVE_INST_VALU and "
              "SQ_ACTIVE_INST_LDS per GUI cycle (summed over the chip). Sources hashed in the JSON beside this "
              "file; the figures hold for those sources only.", "",
              "| launch | kernel | mean us | HBM bytes (fetch + write) | GB/s | MFMA busy vs probe | "
              "VALU active / GUI cycle | LDS active / GUI cycle | LDS bank-conflict cycles per LDS instr |",
              "|---|---|---|---|---|---|---|---|---|"]
    for label in BLOCK_ORDER + STEP_ORDER:
        e = res["kernels"].get(label)
        if e is None:
            continue
        ns = e.get("mean_ns")
        hb = e.get("hbm_bytes")
        gbs = hb / ns if (hb is not None and ns) else None  # bytes per ns = GB/s
        name = short_name(e["kernel"])

        def f(v, fmt):
            return "-" if v is None else format(v, fmt)
        lines.append(f"| {label} | `{name}` | {f(ns / 1e3 if ns else None, '.1f')} | {f(hb, '.3e')} | {f(gbs, '.0f')} | "
                     f"{f(e.get('mfma_busy_vs_probe'), '.3f')} | {f(e.get('SQ_ACTIVE_INST_VALU_per_gui_cycle'), '.2f')} | "
                     f"{f(e.get('SQ_ACTIVE_INST_LDS_per_gui_cycle'), '.2f')} | "
                     f"{f(e.get('lds_bank_conflict_cycles_per_lds_inst'), '.3f')} |")
    return "\n".join(lines) + "\n"


def _sha(src):
    p = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc", src)
    return hashlib.sha256(open(p, "rb").read()).hexdigest()


# SQ counters reported as fractions of a wave's lifetime (SQ_WAVE_CYCLES) in --by-name mode
WAVE_FRACTIONS = ["SQ_ACTIVE_INST_ANY", "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_LDS", "SQ_ACTIVE_INST_SCA",
                  "SQ_ACTIVE_INST_MISC", "SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_WAIT_INST_LDS"]


def by_name(folders, fragments, trace=None):
    """{fragment: {"n", "mean": {counter: value}, "wave_fraction": {...}, "mfma_busy_per_gui", "mean_ns"}}:
    every dispatch whose kernel name contains the fragment, averaged per counter over the folders."""
    acc = {f: {} for f in fragments}
    for folder in folders:
        for d in read_dispatches(folder).values():
            frag = next((f for f in fragments if f in d["name"]), None)
            if frag is None:
                continue
            for c, v in d["counters"].items():
                acc[frag].setdefault(c, []).append(v)
    res = {}
    for frag, cnt in acc.items():
        mean = {c: sum(v) / len(v) for c, v in cnt.items()}
        e = {"n": min((len(v) for v in cnt.values()), default=0), "mean": mean}
        wc = mean.get("SQ_WAVE_CYCLES")
        if wc:
            e["wave_fraction"] = {c: mean[c] / wc for c in WAVE_FRACTIONS if c in mean}
        gui = mean.get("GRBM_GUI_ACTIVE")
        if gui and "SQ_VALU_MFMA_BUSY_CYCLES" in mean:
            e["mfma_busy_per_gui"] = mean["SQ_VALU_MFMA_BUSY_CYCLES"] / gui
        res[frag] = e
    if trace:
        durs = {}
        for d in read_trace(trace).values():
            frag = next((f for f in fragments if f in d["name"]), None)
            if frag is not None:
                durs.setdefault(frag, []).append(d["ns"])
        for frag, v in durs.items():
            res[frag]["mean_ns"] = sum(v) / len(v)
            res[frag]["trace_n"] = len(v)
    return res


def by_name_markdown(res, command=None):
    lines = ["# Hardware counters per kernel", ""]
    if command:
        lines += ["Command:", "", "```", command, "```", ""]
    frags = list(res)
    lines += ["| counter | " + " | ".join(f"`{f}`" for f in frags) + " |",
              "|---|" + "---:|" * len(frags)]
    lines.append("| dispatches per counter / in the trace | " +
                 " | ".join(f"{res[f]['n']} / {res[f].get('trace_n', 0)}" for f in frags) + " |")
    lines.append("| mean duration, trace (ms) | " +
                 " | ".join(f"{res[f]['mean_ns'] / 1e6:.4f}" if "mean_ns" in res[f] else "—" for f in frags) + " |")
    counters = sorted({c for f in frags for c in res[f]["mean"]})
    for c in counters:
        lines.append(f"| {c} | " + " | ".join(f"{res[f]['mean'][c]:.4e}" if c in res[f]["mean"] else "—"
                                              for f in frags) + " |")
    for c in WAVE_FRACTIONS:
        if any(c in res[f].get("wave_fraction", {}) for f in frags):
            lines.append(f"| {c} / SQ_WAVE_CYCLES | " +
                         " | ".join(f"{res[f]['wave_fraction'][c]:.3f}" if c in res[f].get("wave_fraction", {})
                                    else "—" for f in frags) + " |")
    if any("mfma_busy_per_gui" in res[f] for f in frags):
        lines.append("| SQ_VALU_MFMA_BUSY_CYCLES / GRBM_GUI_ACTIVE | " +
                     " | ".join(f"{res[f]['mfma_busy_per_gui']:.1f}" if "mfma_busy_per_gui" in res[f] else "—"
                                for f in frags) + " |")
    return "\n".join(lines) + "\n"


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("folders", nargs="+")
    ap.add_argument("--copy-bytes", type=int, default=1 << 30)
    ap.add_argument("--out", required=True)
    ap.add_argument("--trace", help="kernel-trace folder of the same workload (mean durations per launch)")
    ap.add_argument("--md", help="also write a markdown table here")
    ap.add_argument("--command", help="the profiling command, quoted in the markdown")
    ap.add_argument("--by-name", help="comma-separated kernel-name fragments: group dispatches by kernel")
    a = ap.parse_args(argv)
    if a.by_name:
        res = by_name(a.folders, [f for f in a.by_name.split(",") if f], a.trace)
        if a.md:
            with open(a.md, "w") as fh:
                fh.write(by_name_markdown(res, a.command))
        with open(a.out, "w") as fh:
            json.dump(res, fh, indent=1, sort_keys=True)
        print(json.dumps(res, indent=1, sort_keys=True))
        return 0
    res = derive(reduce(a.folders), a.copy_bytes)
    if a.trace:
        for label, ns in trace_means(a.trace).items():
            if label in res["kernels"]:
                res["kernels"][label]["mean_ns"] = ns
    if a.md:
        with open(a.md, "w") as fh:
            fh.write(markdown(res, a.command))
    with open(a.out, "w") as fh:
        json.dump(res, fh, indent=1, sort_keys=True)
    print(json.dumps(res, indent=1, sort_keys=True))
    return 0


if __name__ == "__main__":
    sys.exit(main())
