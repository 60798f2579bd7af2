"""Profile the decode launch with rocprofv3 and write the summaries kept under profiles/.

    python -m gated_deltanet_linear_decode_amd.build && python -m gated_deltanet_linear_decode_amd.build --trace
    python -m gated_deltanet_linear_decode_amd.profiling run --raw gpurun_out/prof
    python -m gated_deltanet_linear_decode_amd.profiling summarize --raw gpurun_out/prof --profiles profiles

    python -m gated_deltanet_linear_decode_amd.profiling run --raw gpurun_out/prof --verify 1x4,4x4
    python -m gated_deltanet_linear_decode_amd.profiling summarize --raw gpurun_out/prof --verify 1x4,4x4

    python -m gated_deltanet_linear_decode_amd.profiling same-code --rev <git revision> [--restamp]

`run` profiles bench.py (a child process per profile; this process never touches the GPU)
for each workload in WORKLOADS: a kernel trace with statistics; the HBM byte counters
FETCH_SIZE and WRITE_SIZE, one pass each; one pass of matrix-core counters; and the
in-kernel timeline of the profiling build. It also profiles a plain 256 MiB device copy,
whose counter readings scale FETCH_SIZE and WRITE_SIZE to bytes. `summarize` turns the
CSV files into one markdown summary per workload and profile, and profiles/hbm_traffic.json
(bytes per launch, which bench.py reports as roofline.traffic while the kernel source is
unchanged). With `--verify SxT,...` both take only kernel traces of verify steps (S sequences
of T tokens on the headline shape) instead. `same-code` assembles the kernel source as it
was at a git revision (which must be the source the summaries were taken from) and as it
is now, and compares the gfx950 assembly of every kernel the kernel-trace summaries name,
instruction for instruction (branch-label numbers and comments removed); with `--restamp`,
when all are the same, it writes the current source hash into the summaries (on the CPU).
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
KERNEL_SOURCE = os.path.join(ROOT, "gated_deltanet_linear_decode_amd", "csrc", "gdn_block.hip")
HBM_PEAK_GBS = 8000.0

# (workload, rows): the headline, the f32-state and dense workloads at their largest row
# counts, MXFP4 at 8 and 16 rows, MXFP6 at the pages' 2 rows, the normed and out_proj-fold
# variants at 8 rows
WORKLOADS = [("tp8_rank_bf16_state_layer0", 8), ("tp8_rank_f32_state_pads", 16), ("dense_full_width", 8),
             ("tp8_rank_mxfp4", 8), ("tp8_rank_mxfp4", 16), ("tp8_rank_mxfp6", 2),
             ("tp8_rank_bf16_state_normed_input", 8), ("tp8_rank_bf16_state_out_proj", 8)]
# raw counters, then rocprofv3's derived utilisation (busy cycles summed over the SIMDs over
# the busiest instance's active cycles times the SIMD count): the CSV sums a counter over
# its instances (GRBM_GUI_ACTIVE over the 8 XCDs), which the derived expression takes apart
MFMA_COUNTERS = ["SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_MFMA", "SQ_INSTS_VALU_MFMA_MOPS_BF16",
                 "SQ_INSTS_VALU_MFMA_MOPS_F6F4", "GRBM_GUI_ACTIVE", "MfmaUtil"]
COPY_MIB = 256
BENCH_ARGS = ["--sweep-rows", "", "--workloads", "", "--verify", "", "--no-cpu-baseline"]


def kernel_source_hash() -> str:
    with open(KERNEL_SOURCE, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def tag(cfg: str, rows: int) -> str:
    return f"{cfg}_rows{rows}"


def bench_cmd(cfg: str, rows: int, steps: int, warmup: int) -> list:
    return ["python3", os.path.join(ROOT, "bench.py"), "--config", cfg, "--rows", str(rows), "--steps", str(steps),
            "--warmup", str(warmup), *BENCH_ARGS]


def commands(raw: str, workloads=None):
    """(name, argv, timeout seconds) of every profile, in the order `run` takes them."""
    workloads = WORKLOADS if workloads is None else workloads
    out = []
    for cfg, rows in workloads:
        t = tag(cfg, rows)
        out.append((f"kt_{t}", ["rocprofv3", "--kernel-trace", "--stats", "--output-format", "csv", "-d",
                                 os.path.join(raw, f"kt_{t}"), "-o", "run", "--", *bench_cmd(cfg, rows, 960, 96)], 400))
        for ctr in ("FETCH_SIZE", "WRITE_SIZE"):
            out.append((f"pmc_{ctr}_{t}", ["rocprofv3", "--pmc", ctr, "--output-format", "csv", "-d",
                                           os.path.join(raw, f"pmc_{ctr}_{t}"), "-o", "run", "--",
                                           *bench_cmd(cfg, rows, 96, 48)], 300))
        out.append((f"mfma_{t}", ["rocprofv3", "--pmc", *MFMA_COUNTERS, "--output-format", "csv", "-d",
                                  os.path.join(raw, f"mfma_{t}"), "-o", "run", "--", *bench_cmd(cfg, rows, 96, 48)], 300))
    for ctr in ("FETCH_SIZE", "WRITE_SIZE"):
        out.append((f"pmc_{ctr}_copy", ["rocprofv3", "--pmc", ctr, "--output-format", "csv", "-d",
                                        os.path.join(raw, f"pmc_{ctr}_copy"), "-o", "run", "--", "python3",
                                        os.path.join(ROOT, "bench.py"), "--copy-calibration", str(COPY_MIB),
                                        "--steps", "4"], 120))
    for cfg, rows in workloads:
        out.append((f"timeline_{tag(cfg, rows)}", ["python3", "-m", "gated_deltanet_linear_decode_amd.timeline",
                                                    "--config", cfg, "--rows", str(rows)], 300))
    return out


VERIFY_CONFIG = "tp8_rank_bf16_state_layer0"


def verify_commands(raw: str, steps):
    """(name, argv, timeout seconds) of a kernel trace per verify step (seqs, tokens): bench.py
    times the step as in its verify sweep, after a short headline run."""
    out = []
    for seqs, tokens in steps:
        argv = ["python3", os.path.join(ROOT, "bench.py"), "--config", VERIFY_CONFIG, "--rows", "1", "--steps", "48",
                "--warmup", "8", "--sweep-rows", "", "--workloads", "", "--verify", f"{seqs}x{tokens}",
                "--sweep-steps", "960", "--no-cpu-baseline"]
        name = f"kt_verify_{seqs}x{tokens}"
        out.append((name, ["rocprofv3", "--kernel-trace", "--stats", "--output-format", "csv", "-d",
                           os.path.join(raw, name), "-o", "run", "--", *argv], 400))
    return out


def run(raw: str, workloads=None, verify=None) -> None:
    os.makedirs(raw, exist_ok=True)
    env = dict(os.environ, TMPDIR="/tmp")
    for name, argv, limit in (verify_commands(raw, verify) if verify else commands(raw, workloads)):
        print(f"[profiling] {name}", flush=True)
        log = os.path.join(raw, f"{name}.log")
        with open(log, "w") as f:
            rc = subprocess.run(["timeout", "-k", "10", str(limit), *argv], cwd="/tmp" if argv[0] == "rocprofv3" else ROOT,
                                env=env, stdout=f, stderr=subprocess.STDOUT).returncode
        if rc != 0:
            print(open(log).read()[-3000:], flush=True)
            raise SystemExit(f"[profiling] {name} failed with exit status {rc}")


def _rows(path):
    with open(path) as f:
        return list(csv.DictReader(f))


def _short(name: str) -> str:
    return name.replace("void (anonymous namespace)::", "").replace("(anonymous namespace)::", "").split("(")[0]


def _counter(raw, name, counter, kernel):
    vals = [float(r["Counter_Value"]) for r in _rows(os.path.join(raw, name, "run_counter_collection.csv"))
            if kernel in r["Kernel_Name"] and r["Counter_Name"] == counter]
    return vals


def _cmd_text(argv) -> str:
    return " ".join(a if a and " " not in a else f'"{a}"' for a in argv).replace(ROOT, "<repo>")


def summarize(raw: str, profiles: str, workloads=None) -> None:
    sys.path.insert(0, ROOT)
    from gated_deltanet_linear_decode_amd import configs
    h = kernel_source_hash()
    workloads = WORKLOADS if workloads is None else workloads
    cmds = {name: argv for name, argv, _ in commands(raw, workloads)}
    copy_kib = COPY_MIB * 1024
    cf = _counter(raw, "pmc_FETCH_SIZE_copy", "FETCH_SIZE", "copyBuffer")
    cw = _counter(raw, "pmc_WRITE_SIZE_copy", "WRITE_SIZE", "copyBuffer")
    fscale, wscale = copy_kib / (sum(cf) / len(cf)), copy_kib / (sum(cw) / len(cw))
    traffic = {"kernel_source_hash": h, "fetch_scale": round(fscale, 4), "write_scale": round(wscale, 4)}
    foot = f"Kernel source hash (sha256 of gdn_block.hip, first 16 hex digits): {h}.\n"
    for cfg, rows in workloads:
        t = tag(cfg, rows)
        shape = configs.ALL[cfg]
        valid = rows  # bench.py's timed launches have no pad rows
        algo = configs.algorithmic_bytes(shape, rows, valid)
        # kernel trace
        st = _rows(os.path.join(raw, f"kt_{t}", "run_kernel_stats.csv"))
        dec = next(float(r["AverageNs"]) for r in st if "decode_kernel" in r["Name"])
        lines = [f"# decode_kernel, {cfg}, {rows} rows: kernel trace", "",
                 "Command (run from /tmp with TMPDIR=/tmp; <repo> is the repository root):", "", "```",
                 _cmd_text(cmds[f"kt_{t}"]), "```", "",
                 "| kernel | calls | average ns | min ns | max ns | share of GPU time |", "|---|---|---|---|---|---|"]
        for r in st:
            lines.append(f"| `{_short(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']):.0f} | {r['MinNs']} | "
                         f"{r['MaxNs']} | {float(r['Percentage']):.2f} % |")
        gbs = algo / (dec * 1e-9) / 1e9
        lines += ["", f"decode_kernel: {dec / 1000:.2f} µs on average per launch; algorithmic bytes per launch "
                      f"{algo:,} ({valid} valid rows), so {gbs:.0f} GB/s = {gbs / HBM_PEAK_GBS:.3f} of 8 TB/s."]
        rs = [float(r["AverageNs"]) for r in st if _short(r["Name"]) == "read_stream_kernel"]
        if rs:
            sgbs = ((algo + 15) // 16 * 16) / (rs[0] * 1e-9) / 1e9
            lines.append(f"read_stream_kernel: the plain read of the same bytes that bench.py times beside the "
                         f"block, {rs[0] / 1000:.2f} µs ({sgbs:.0f} GB/s = {sgbs / HBM_PEAK_GBS:.3f} of 8 TB/s); the "
                         f"block runs at {gbs / sgbs:.3f} of it.")
        lines += ["The other kernels are set-up work (weight copies and the tiled-weight pack) outside the timed "
                  "graphs.", foot]
        with open(os.path.join(profiles, f"decode_kernel_{t}_kernel_trace.md"), "w") as f:
            f.write("\n".join(lines))
        # HBM counters
        df = _counter(raw, f"pmc_FETCH_SIZE_{t}", "FETCH_SIZE", "decode_kernel")
        dw = _counter(raw, f"pmc_WRITE_SIZE_{t}", "WRITE_SIZE", "decode_kernel")
        fk, wk = sum(df) / len(df), sum(dw) / len(dw)
        rb, wb = int(round(fk * 1024 * fscale)), int(round(wk * 1024 * wscale))
        traffic.setdefault(cfg, {})[str(rows)] = {
            "bytes_per_launch": rb + wb, "read_bytes": rb, "write_bytes": wb, "fetch_kib_raw": round(fk, 2),
            "write_kib_raw": round(wk, 2), "dispatches": len(df), "algo_bytes": algo,
            "kernel_trace_avg_ns": round(dec, 1)}
        lines = [f"# decode_kernel, {cfg}, {rows} rows: HBM bytes from FETCH_SIZE and WRITE_SIZE", "",
                 "Commands (run from /tmp with TMPDIR=/tmp), one counter per run:", "", "```",
                 _cmd_text(cmds[f"pmc_FETCH_SIZE_{t}"]), _cmd_text(cmds[f"pmc_WRITE_SIZE_{t}"]),
                 _cmd_text(cmds["pmc_FETCH_SIZE_copy"]), _cmd_text(cmds["pmc_WRITE_SIZE_copy"]), "```", "",
                 f"Scale: a {COPY_MIB} MiB device-to-device copy reads FETCH_SIZE {sum(cf) / len(cf):.1f} and "
                 f"WRITE_SIZE {sum(cw) / len(cw):.1f} KiB per dispatch, so FETCH_SIZE is scaled by {fscale:.4f} "
                 f"and WRITE_SIZE by {wscale:.4f}.", "",
                 "| counter | KiB per dispatch | bytes per launch (scaled) | dispatches |", "|---|---|---|---|",
                 f"| FETCH_SIZE | {fk:.2f} | {rb:,} | {len(df)} |", f"| WRITE_SIZE | {wk:.2f} | {wb:,} | {len(dw)} |",
                 f"| total | | {rb + wb:,} | |", "",
                 f"Algorithmic bytes per launch: {algo:,}; measured / algorithmic = {(rb + wb) / algo:.3f}.", foot]
        with open(os.path.join(profiles, f"decode_kernel_{t}_hbm_counters.md"), "w") as f:
            f.write("\n".join(lines))
        # matrix-core counters
        c = {k: _counter(raw, f"mfma_{t}", k, "decode_kernel") for k in MFMA_COUNTERS}
        avg = {k: (sum(v) / len(v) if v else float("nan")) for k, v in c.items()}
        util = avg["MfmaUtil"]
        # 16x16x32 bf16 and 16x16x128 f8f6f4 MFMAs: 16 weight rows x 16 decode rows each
        inst = avg["SQ_INSTS_MFMA"]
        lines = [f"# decode_kernel, {cfg}, {rows} rows: matrix-core counters", "",
                 "Command (run from /tmp with TMPDIR=/tmp):", "", "```", _cmd_text(cmds[f"mfma_{t}"]), "```", "",
                 "| counter | per dispatch (average) |", "|---|---|"]
        lines += [f"| {k} | {v:,.2f} |" if k == "MfmaUtil" else f"| {k} | {v:,.0f} |" for k, v in avg.items()]
        lines += ["", f"Matrix cores busy {util:.2f} % of the launch (MfmaUtil), for {inst:,.0f} MFMA instructions "
                      "per launch. The projections multiply at most 16 decode rows per weight row, so they are "
                      "bound by the weight stream, not the matrix cores, and a low figure is expected: the "
                      "matrix cores are used because one instruction consumes a whole 1 KiB weight load of a "
                      "wave (the activations are the instruction's other operand).", foot]
        with open(os.path.join(profiles, f"decode_kernel_{t}_mfma_counters.md"), "w") as f:
            f.write("\n".join(lines))
        # timeline
        with open(os.path.join(raw, f"timeline_{t}.log")) as f:
            body = [ln for ln in f.read().splitlines() if "amdgpu.ids" not in ln]
        lines = [f"# decode_kernel, {cfg}, {rows} rows: in-kernel timeline (profiling build)", "",
                 "Commands (from the repository root):", "", "```",
                 "python3 -m gated_deltanet_linear_decode_amd.build --trace", _cmd_text(cmds[f"timeline_{t}"]), "```",
                 "", "Per role and point: minimum, median and maximum microseconds after the first workgroup "
                     "started, for the last of 48 launches that rotate over layer copies. Each stamp reads the "
                     "clock through the scalar memory path and waits for it, so stamps close together (the "
                     "recurrence) inflate the sections between them.", "", "```", *body, "```", foot]
        with open(os.path.join(profiles, f"decode_kernel_{t}_timeline.md"), "w") as f:
            f.write("\n".join(lines))
    with open(os.path.join(profiles, "hbm_traffic.json"), "w") as f:
        json.dump(traffic, f, indent=1)


def summarize_verify(raw: str, profiles: str, steps) -> None:
    sys.path.insert(0, ROOT)
    from gated_deltanet_linear_decode_amd import configs
    shape = configs.ALL[VERIFY_CONFIG]
    foot = f"Kernel source hash (sha256 of gdn_block.hip, first 16 hex digits): {kernel_source_hash()}.\n"
    cmds = {name: argv for name, argv, _ in verify_commands(raw, steps)}
    for seqs, tokens in steps:
        name = f"kt_verify_{seqs}x{tokens}"
        st = _rows(os.path.join(raw, name, "run_kernel_stats.csv"))
        # decode_kernel<PACKED, FMT, DK, ST, FOLD, MULTI, DST>: the verify step's instantiation
        # has MULTI set (or DST, for one token at head dim 128); the headline run's has neither
        ver = [r for r in st if "decode_kernel" in r["Name"] and not _short(r["Name"]).endswith("false, false>")]
        assert len(ver) == 1, [r["Name"] for r in st]
        us = float(ver[0]["AverageNs"]) / 1000
        algo = configs.algorithmic_bytes_verify(shape, seqs, tokens)
        gbs = algo / (us * 1e-6) / 1e9
        lines = [f"# decode_kernel, verify step of {seqs} x {tokens} tokens ({VERIFY_CONFIG}): kernel trace", "",
                 "Command (run from /tmp with TMPDIR=/tmp; <repo> is the repository root):", "", "```",
                 _cmd_text(cmds[name]), "```", "",
                 "| kernel | calls | average ns | min ns | max ns | share of GPU time |", "|---|---|---|---|---|---|"]
        for r in st:
            lines.append(f"| `{_short(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']):.0f} | {r['MinNs']} | "
                         f"{r['MaxNs']} | {float(r['Percentage']):.2f} % |")
        lines += ["", f"The verify launch (`{_short(ver[0]['Name'])}`): {us:.2f} µs on average; algorithmic bytes "
                      f"per launch {algo:,}, so {gbs:.0f} GB/s = {gbs / HBM_PEAK_GBS:.3f} of 8 TB/s. The decode "
                      "launches with MULTI and DST unset are the short headline run before the verify sweep, and "
                      "read_stream_kernel the plain read of the headline's bytes that bench.py times beside it; the "
                      "other kernels are set-up work outside the timed graphs.", foot]
        with open(os.path.join(profiles, f"decode_kernel_verify_{seqs}x{tokens}_kernel_trace.md"), "w") as f:
            f.write("\n".join(lines))


def _kernel_asm(src: str, work: str) -> dict:
    """{demangled kernel name (no parameter list): its gfx950 assembly, branch-label numbers
    and comments removed} of one source file."""
    import re

    from gated_deltanet_linear_decode_amd import build
    out = os.path.join(work, os.path.basename(src) + ".s")
    flags = [f for f in build.FLAGS if f not in ("-shared", "-fPIC")]
    subprocess.run([build.HIPCC, *flags, "--cuda-device-only", "-S", "-I", os.path.join(ROOT, "include"), src,
                    "-o", out], check=True, capture_output=True, text=True)
    txt = open(out).read()
    funcs = {m.group(1): m.group(2) for m in re.finditer(r"^(_Z\w+):\s.*?\n(.*?)\n\s*s_endpgm", txt, re.S | re.M)}
    import shutil
    filt = shutil.which("c++filt") or shutil.which("llvm-cxxfilt")
    names = subprocess.run([filt], input="\n".join(funcs), capture_output=True, text=True, check=True).stdout.split("\n")
    norm = lambda body: "\n".join(ln.split(";")[0].rstrip() for ln in re.sub(r"BB\d+_", "BB_", body).split("\n"))  # noqa: E731
    return {_short(n): norm(b) for n, b in zip(names, funcs.values())}


def same_code(rev: str, profiles: str, restamp: bool) -> bool:
    import glob
    import re
    import tempfile
    with open(os.path.join(profiles, "hbm_traffic.json")) as f:
        recorded = json.load(f)["kernel_source_hash"]
    rel = os.path.relpath(KERNEL_SOURCE, ROOT)
    with tempfile.TemporaryDirectory() as work:
        old = os.path.join(work, "old", os.path.basename(KERNEL_SOURCE))
        os.makedirs(os.path.dirname(old))
        with open(old, "wb") as f:
            f.write(subprocess.run(["git", "show", f"{rev}:{rel}"], cwd=ROOT, check=True, capture_output=True).stdout)
        with open(old, "rb") as f:
            old_hash = hashlib.sha256(f.read()).hexdigest()[:16]
        if old_hash != recorded:
            print(f"[same-code] {rev}:{rel} has hash {old_hash}, the summaries {recorded}: not their source")
            return False
        a, b = _kernel_asm(old, work), _kernel_asm(KERNEL_SOURCE, work)
    names = set()
    for path in glob.glob(os.path.join(profiles, "*_kernel_trace.md")):
        names |= set(re.findall(r"^\| `((?:decode|read_stream)_kernel[^`]*)` \|", open(path).read(), re.M))
    diff = sorted(n for n in names if n not in a or a[n] != b.get(n))
    for n in sorted(names):
        print(f"[same-code] {'different' if n in diff else 'same     '} {n}")
    if diff or not restamp:
        return not diff
    new = kernel_source_hash()
    for path in glob.glob(os.path.join(profiles, "*")):
        text = open(path).read()
        if recorded in text:
            with open(path, "w") as f:
                f.write(text.replace(recorded, new))
    print(f"[same-code] summaries stamped {new}")
    return True


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("action", choices=["run", "summarize", "same-code"])
    ap.add_argument("--raw", default=os.path.join(ROOT, "gpurun_out", "prof"))
    ap.add_argument("--profiles", default=os.path.join(ROOT, "profiles"))
    ap.add_argument("--only", default="", help="comma-separated workload:rows pairs (default: every workload)")
    ap.add_argument("--verify", default="", help="comma-separated verify steps SxT: kernel traces of these only")
    ap.add_argument("--rev", default="HEAD", help="same-code: the git revision the summaries were taken from")
    ap.add_argument("--restamp", action="store_true", help="same-code: stamp the current hash when all are the same")
    a = ap.parse_args()
    if a.action == "same-code":
        raise SystemExit(0 if same_code(a.rev, os.path.abspath(a.profiles), a.restamp) else 1)
    wl = [(w.split(":")[0], int(w.split(":")[1])) for w in a.only.split(",") if w] or None
    ver = [tuple(int(v) for v in p.split("x")) for p in a.verify.split(",") if p]
    if a.action == "run":
        run(os.path.abspath(a.raw), wl, ver)
    elif ver:
        summarize_verify(os.path.abspath(a.raw), os.path.abspath(a.profiles), ver)
    else:
        summarize(os.path.abspath(a.raw), os.path.abspath(a.profiles), wl)


if __name__ == "__main__":
    main()
