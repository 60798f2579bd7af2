#!/usr/bin/env python3
"""Time the GDN decode block on one MI355X.

A step is one decode launch of the whole block over one batch of rows. The
timed launches are captured in HIP graphs that rotate over `layers` copies of
the weights, each copy with its own conv and SSM state pools, so the 256 MB
MALL cannot keep a layer resident between its launches (the method of "vLLM PR
#60833", Validation / Per launch: graphs of 46 launches, weights rotated past
the MALL). Time comes from HIP events on the stream the block is launched on.

Prints one JSON line: µs per launch at the headline row count, the roofline
(algorithmic HBM bytes per launch / launch time against 8 TB/s), a sweep over
row counts, and the CPU oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "GDN block µs/launch at 1-16 rows; achieved HBM GB/s vs peak"
HBM_PEAK_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")
KERNEL_SOURCES = [os.path.join(ROOT, "gated_deltanet_linear_decode_amd", "csrc", "gdn_block.hip")]


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


class Rotation:
    """`layers` copies of one layer's weights and state pools on the device."""

    def __init__(self, shape, layers, max_rows, seed=0, pads=False):
        import torch

        from gated_deltanet_linear_decode_amd import synth
        from gated_deltanet_linear_decode_amd.block import GdnBlock

        dev = torch.device("cuda:0")
        self.shape, self.dev = shape, dev
        self.blk = GdnBlock(shape, max_rows=max_rows, device=dev)
        self.w_cpu = synth.make_weights(shape, seed)
        self.call_cpu = synth.make_call(shape, max_rows, seed, pads=pads)
        self.copies = []
        for i in range(layers):
            w = synth.GdnWeights(**{k: (v.to(dev).clone() if v is not None else None)
                                    for k, v in self.w_cpu.__dict__.items()})
            packed = self.blk.pack(w)
            c = dict(
                w=w, ws=self.blk.weights_struct(w), packed=packed, wsp=self.blk.packed_struct(w, packed),
                x=self.call_cpu.x.to(dev).clone(), res=self.call_cpu.residual.to(dev).clone(),
                conv=self.call_cpu.conv_state.to(dev).clone(), ssm=self.call_cpu.ssm_state.to(dev).clone(),
                idx=self.call_cpu.state_idx.to(dev).clone(),
                core=torch.empty(max_rows, shape.value_dim, dtype=torch.bfloat16, device=dev),
                out=(torch.empty(max_rows, shape.hidden, dtype=torch.bfloat16, device=dev)
                     if shape.fold_out_proj else None))
            self.copies.append(c)
        torch.cuda.synchronize()

    def launch(self, i, rows, packed):
        c = self.copies[i % len(self.copies)]
        self.blk.decode(c["x"][:rows], c["res"][:rows], None, c["conv"], c["ssm"], c["idx"][:rows],
                        c["core"][:rows], weights_struct=c["wsp"] if packed else c["ws"],
                        out=c["out"][:rows] if c["out"] is not None else None)

    def graph(self, n, rows, packed):
        import torch
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            for i in range(len(self.copies)):
                self.launch(i, rows, packed)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(n):
                self.launch(i, rows, packed)
        return g

    def time(self, rows, steps, warmup, packed=True):
        """Average µs per launch over exactly `steps` launches (after `warmup`)."""
        import torch
        per = 4 * len(self.copies)           # launches per graph: whole rotations, >= 46 at 12 copies
        while per < 46:
            per += len(self.copies)
        g = self.graph(per, rows, packed)
        rem = steps % per
        g_rem = self.graph(rem, rows, packed) if rem else None
        for _ in range(max(1, warmup // per)):
            g.replay()
        torch.cuda.synchronize()
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record()
        for _ in range(steps // per):
            g.replay()
        if g_rem is not None:
            g_rem.replay()
        end.record()
        torch.cuda.synchronize()
        err = self.blk.check()
        if err:
            raise RuntimeError(f"a wait inside the decode gave up (error word {err:#x})")
        return start.elapsed_time(end) * 1000.0 / steps


    def valid_rows(self, rows):
        return int((self.call_cpu.state_idx[:rows] > 0).sum())

    def close(self):
        import torch
        self.copies.clear()
        self.blk.close()
        torch.cuda.synchronize()
        torch.cuda.empty_cache()


class VerifyRotation(Rotation):
    """`layers` copies of a layer set up for verify steps of `seqs` sequences of `tokens`
    tokens: every copy reads its sources and writes all of its snapshots into slots
    disjoint from them, so every replay does the same work."""

    def __init__(self, shape, layers, seqs, tokens, seed=0):
        import numpy as np
        import torch

        from gated_deltanet_linear_decode_amd import synth
        from gated_deltanet_linear_decode_amd.block import GdnBlock

        dev = torch.device("cuda:0")
        self.shape, self.dev, self.tokens = shape, dev, tokens
        rows = seqs * tokens
        self.blk = GdnBlock(shape, max_rows=rows, device=dev)
        self.w_cpu = synth.make_weights(shape, seed)
        self.call_cpu = synth.make_call(shape, rows, seed)
        rng = np.random.Generator(np.random.PCG64(seed + 5))
        perm = (rng.permutation(shape.num_state_slots - 1)[:seqs + rows] + 1).astype(np.int32)
        src, dst = torch.from_numpy(perm[:seqs].copy()), torch.from_numpy(perm[seqs:].reshape(seqs, tokens).copy())
        self.copies = []
        for i in range(layers):
            w = synth.GdnWeights(**{k: (v.to(dev).clone() if v is not None else None)
                                    for k, v in self.w_cpu.__dict__.items()})
            packed = self.blk.pack(w)
            self.copies.append(dict(
                w=w, ws=self.blk.weights_struct(w), packed=packed, wsp=self.blk.packed_struct(w, packed),
                x=self.call_cpu.x.to(dev).clone(), res=self.call_cpu.residual.to(dev).clone(),
                conv=self.call_cpu.conv_state.to(dev).clone(), ssm=self.call_cpu.ssm_state.to(dev).clone(),
                src=src.to(dev), dst=dst.to(dev),
                core=torch.empty(rows, shape.value_dim, dtype=torch.bfloat16, device=dev)))
        torch.cuda.synchronize()

    def launch(self, i, rows, packed):
        c = self.copies[i % len(self.copies)]
        self.blk.verify(c["x"], c["res"], None, c["conv"], c["ssm"], c["src"], c["dst"], c["core"],
                        weights_struct=c["wsp"] if packed else c["ws"])


def time_read_stream(nbytes, copies, steps, warmup):
    """µs per launch of the plain read stream (gdn_read_stream) over `nbytes`, timed like the
    block: graphs of launches rotating over `copies` buffers of that size (past the MALL)."""
    import torch

    from gated_deltanet_linear_decode_amd import abi
    n = (nbytes + 15) // 16 * 16
    bufs = [torch.randint(0, 256, (n,), dtype=torch.uint8, device="cuda:0") for _ in range(copies)]
    sinks = torch.empty(copies, (n + 32767) // 32768, dtype=torch.int32, device="cuda:0")

    def launch(i):
        abi.gdn_read_stream(bufs[i % copies].data_ptr(), n, sinks[i % copies].data_ptr(),
                            torch.cuda.current_stream().cuda_stream)

    per = 4 * copies
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for i in range(copies):
            launch(i)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(per):
            launch(i)
    reps = max(1, steps // per)
    for _ in range(max(1, warmup // per)):
        g.replay()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(reps):
        g.replay()
    end.record()
    torch.cuda.synchronize()
    us = start.elapsed_time(end) * 1000.0 / (reps * per)
    del bufs, sinks, g
    torch.cuda.empty_cache()
    return n, us


def sweep_verify(shape, pairs, steps):
    """µs per verify launch for each (sequences, tokens) pair."""
    out = {}
    for seqs, tokens in pairs:
        rot = VerifyRotation(shape, shape.layers, seqs, tokens)
        t = rot.time(seqs * tokens, steps, steps // 4)
        b = configs_mod().algorithmic_bytes_verify(shape, seqs, tokens)
        out[f"{seqs}x{tokens}"] = dict(us=round(t, 3), algo_bytes=b, gbs=round(b / (t * 1e-6) / 1e9, 1),
                                       frac=round(b / (t * 1e-6) / 1e9 / HBM_PEAK_GBS, 4))
        log(f"verify {shape.name} {seqs} sequences x {tokens} tokens: {t:.2f} us/launch")
        rot.close()
    return out


def sweep_workload(shape, rows_list, steps, packed=True):
    """µs per launch of `shape` (its own layer count, pad rows as the workload has them)."""
    rot = Rotation(shape, shape.layers, max(rows_list), pads=shape.pad_rows)
    out = {}
    for r in rows_list:
        t = rot.time(r, steps, steps // 4, packed=packed)
        b = configs_mod().algorithmic_bytes(shape, r, rot.valid_rows(r))
        out[str(r)] = dict(us=round(t, 3), valid_rows=rot.valid_rows(r), algo_bytes=b,
                           gbs=round(b / (t * 1e-6) / 1e9, 1), frac=round(b / (t * 1e-6) / 1e9 / HBM_PEAK_GBS, 4))
        log(f"{shape.name} rows {r}: {t:.2f} us/launch")
    rot.close()
    return out


def configs_mod():
    from gated_deltanet_linear_decode_amd import configs
    return configs


def cpu_baseline(shape, rot, rows, seconds, single_thread=False):
    """The oracle on the same workload (same bytes), timed for about `seconds`, on all the
    BLAS threads numpy has, or on one."""
    import contextlib

    import numpy as np
    import torch

    import oracle
    limit = contextlib.nullcontext()
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
        if single_thread:
            limit, threads = threadpool_limits(limits=1), 1
    except Exception:
        threads = 1
    bits = lambda t: t.contiguous().view(torch.int16).numpy().view(np.uint16).copy()  # noqa: E731
    cfg = dict(hidden=shape.hidden, num_k_heads=shape.num_k_heads, head_k_dim=shape.head_k_dim,
               num_v_heads=shape.num_v_heads, head_v_dim=shape.head_v_dim, conv_width=shape.conv_width,
               ssm_state_dtype=shape.ssm_state_dtype, has_residual=shape.has_residual,
               qkvz_format=shape.qkvz_format, norm_eps=shape.norm_eps,
               gated_norm_eps=shape.gated_norm_eps, l2norm_eps=shape.l2norm_eps,
               mx_scale_rule=shape.mx_scale_rule)
    w = {k: (bits(v) if v.dtype == torch.bfloat16 else v.numpy()) for k, v in rot.w_cpu.tensors().items()}
    c = rot.call_cpu
    x, res = bits(c.x[:rows]), bits(c.residual[:rows])
    conv = bits(c.conv_state)
    ssm = bits(c.ssm_state) if c.ssm_state.dtype == torch.bfloat16 else c.ssm_state.numpy()
    idx = c.state_idx[:rows].numpy()
    n, t0 = 0, time.perf_counter()
    with limit:
        while True:
            oracle.decode_block(cfg, w, x, res, conv, ssm, idx)
            n += 1
            el = time.perf_counter() - t0
            if el >= seconds:
                break
    return dict(value=el / n * 1e6, unit="µs/launch", cores=threads, kind="oracle",
                sample=f"{n} oracle decode calls of the {rows}-row step of {shape.name} "
                       f"(float64 numpy, {threads} BLAS thread{'s' if threads != 1 else ''}), {el:.1f} s")


def main():
    from gated_deltanet_linear_decode_amd import configs

    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=4800)
    ap.add_argument("--warmup", type=int, default=480)
    ap.add_argument("--config", default=configs.TP8_RANK_BF16.name, choices=sorted(configs.ALL))
    ap.add_argument("--rows", type=int, default=8)
    ap.add_argument("--sweep-rows", default="1,2,4,8,12,16")
    ap.add_argument("--sweep-steps", type=int, default=960)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--workloads", default="tp8_rank_f32_state_pads,dense_full_width,tp8_rank_mxfp4,tp8_rank_mxfp6,"
                    "tp8_rank_bf16_state_normed_input,tp8_rank_mxfp4_normed_input,tp8_rank_bf16_state_out_proj",
                    help="other workloads to sweep (tiled weights) after the headline; '' for none")
    ap.add_argument("--verify", default="1x2,1x4,2x4,4x4,8x2",
                    help="verify steps (sequences x tokens) to time on the headline shape; '' for none")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run device-to-device copies of MIB MiB (HBM counter calibration) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the block shards by heads with no exchange inside it; see the design notes)", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy_calibration:
        # a plain copy of known size, for scaling the HBM byte counters of a profiler run
        n = args.copy_calibration << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(max(1, args.steps)):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "copies": max(1, args.steps)}))
        return

    shape = configs.ALL[args.config]
    sweep_rows = [int(r) for r in args.sweep_rows.split(",") if r]
    max_rows = max([args.rows] + sweep_rows)
    assert max_rows <= 16
    log(f"setting up {shape.layers} layer copies of {shape.name} (max_rows {max_rows})")
    rot = Rotation(shape, shape.layers, max_rows)
    log(f"timing {args.steps} launches at {args.rows} rows")
    torch.cuda.synchronize()
    us = rot.time(args.rows, args.steps, args.warmup)
    algo = configs.algorithmic_bytes(shape, args.rows)
    gbs = algo / (us * 1e-6) / 1e9
    sweep = {"tiled_weights": {}, "row_major_weights": {}}
    for r in sweep_rows:
        b = configs.algorithmic_bytes(shape, r)
        for key, packed in (("tiled_weights", True), ("row_major_weights", False)):
            t = rot.time(r, args.sweep_steps, args.sweep_steps // 4, packed=packed)
            sweep[key][str(r)] = dict(us=round(t, 3), algo_bytes=b, gbs=round(b / (t * 1e-6) / 1e9, 1),
                                      frac=round(b / (t * 1e-6) / 1e9 / HBM_PEAK_GBS, 4))
            log(f"rows {r} {key}: {t:.2f} us/launch")

    workloads = {}
    for name in [n for n in args.workloads.split(",") if n]:
        wl = configs.ALL[name]
        rows_list = [r for r in (1, 2, 4, 8, 12, 16) if r <= wl.max_rows] if wl.max_rows >= 8 else list(wl.rows)
        rows_list = sorted(set(rows_list) | set(wl.rows) if len(wl.rows) <= 8 else rows_list)
        log(f"sweeping {name}: rows {rows_list}, {wl.layers} layer copies")
        workloads[name] = sweep_workload(wl, rows_list, args.sweep_steps)

    pairs = [tuple(int(v) for v in p.split("x")) for p in args.verify.split(",") if p]
    verify = sweep_verify(shape, pairs, args.sweep_steps) if pairs else {}

    stream_bytes, stream_us = time_read_stream(algo, shape.layers, args.sweep_steps, args.sweep_steps // 4)
    stream_gbs = stream_bytes / (stream_us * 1e-6) / 1e9
    log(f"read stream of {stream_bytes} bytes: {stream_us:.2f} us/launch, {stream_gbs:.0f} GB/s")

    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as f:
            tr = json.load(f)
        entry = tr.get(shape.name, {}).get(str(args.rows))
        if tr.get("kernel_source_hash") == kernel_source_hash() and entry:
            traffic = entry["bytes_per_launch"]

    cpu = cpu1 = None
    if not args.no_cpu_baseline:
        log(f"timing the CPU oracle for ~{args.cpu_seconds:.0f} s, then on one thread")
        cpu = cpu_baseline(shape, rot, args.rows, args.cpu_seconds)
        cpu1 = cpu_baseline(shape, rot, args.rows, args.cpu_seconds / 2, single_thread=True)

    out = {
        "metric": METRIC,
        "value": round(us, 3),
        "unit": "µs/launch",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(us / 1000.0, 6),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": shape.name, "rows": args.rows, "hidden": shape.hidden,
            "key_heads": f"{shape.num_k_heads}x{shape.head_k_dim}",
            "value_heads": f"{shape.num_v_heads}x{shape.head_v_dim}",
            "ssm_state": shape.ssm_state_dtype, "in_proj_qkvz": shape.qkvz_format,
            "has_residual": shape.has_residual, "layers_rotated": shape.layers,
            "state_slots": shape.num_state_slots, "projection_weights": "tiled copy (gdn_block_pack_weights)",
        },
        "roofline": {
            "bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic,
            "algo_bytes_per_launch": algo, "kernel": "decode_kernel (the whole block, one launch)",
        },
        "read_stream": {
            "bytes": stream_bytes, "us": round(stream_us, 3), "gbs": round(stream_gbs, 1),
            "frac_of_peak": round(stream_gbs / HBM_PEAK_GBS, 4), "decode_frac_of_stream": round(gbs / stream_gbs, 4),
            "kernel": "read_stream_kernel (gdn_read_stream: one plain read of the launch's algorithmic bytes)",
        },
        "sweep": sweep,
        "workloads": workloads,
        "verify": verify,
        "cpu_baseline": cpu,
        "cpu_baseline_single_thread": cpu1,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
