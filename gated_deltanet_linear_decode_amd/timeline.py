"""Per-workgroup timeline of the decode launch, from the profiling build.

    python -m gated_deltanet_linear_decode_amd.build --trace
    python -m gated_deltanet_linear_decode_amd.timeline --config tp8_rank_bf16_state_layer0 --rows 8
    python -m gated_deltanet_linear_decode_amd.timeline --verify 1x4   (a verify step instead)

The profiling build (libgdn_block_trace.so, compiled with GDN_TRACE) has thread 0 of every
workgroup stamp the 100 MHz wall clock at fixed points of its role; this tool runs launches
that rotate over layer copies (as the bench does), copies the stamps of the last launch and
prints, per role and point, the minimum / median / maximum time in microseconds after the
first workgroup started, then where the projection workgroups ran (XCD, and how many shared
a CU) against when their matrix-core work ended. In a verify step the recurrence points
inside the token loop are those of the last token. The stamps themselves cost time (each is a
scalar memory read of the clock and a store), so the points are a guide to where the time
goes, not a measurement of the plain kernel's duration.
"""
from __future__ import annotations

import argparse
import ctypes
import os
from collections import Counter, defaultdict

import numpy as np

SLOTS = 16
BLOCKS = 8192

# the point each stamp slot marks, per role (slot 15 of a projection workgroup is its hardware id)
POINTS = {
    "norm": {0: "start", 1: "row sum done", 2: "rstd (or xn + MXFP4 image) stored", 3: "residual rewritten"},
    "proj": {0: "start", 1: "activations staged", 2: "matrix-core work done", 3: "partials published"},
    "rec": {0: "start", 1: "waits done", 5: "partials loaded", 8: "gates computed", 9: "barrier",
            2: "conv done", 10: "state pass", 6: "row-group butterfly", 11: "d and o", 7: "state update issued",
            12: "gated-norm sum", 3: "core row stored", 4: "end", 13: "token outputs: loads issued",
            14: "token loop start"},
    "oproj": {0: "start", 1: "core rows seen", 2: "matrix-core work done", 3: "out rows stored"},
}
ORDER = {"rec": [0, 1, 13, 14, 5, 8, 9, 2, 10, 6, 11, 7, 12, 3, 4]}
# a verify step of more than one token at head dim 128 (the chunked recurrence)
VERIFY_REC = {0: "start", 1: "waits done", 14: "token outputs loaded", 2: "conv of all tokens done",
              11: "S0^T k, S0^T q, tables, d_t, o_t", 12: "core rows stored", 3: "state snapshots issued"}
VERIFY_ORDER = [0, 1, 14, 2, 11, 12, 3]


def main():
    import torch  # noqa: F401  (the HIP runtime torch loads is the one the library binds to)

    from . import abi, configs, synth
    from .block import GdnBlock
    from .build import TRACE_LIB

    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--config", default=configs.TP8_RANK_BF16.name, choices=sorted(configs.ALL))
    ap.add_argument("--rows", type=int, default=8)
    ap.add_argument("--launches", type=int, default=48)
    ap.add_argument("--verify", default="", help="sequences x tokens (e.g. 1x4): time verify steps instead")
    args = ap.parse_args()
    if not os.path.exists(TRACE_LIB):
        raise SystemExit(f"{TRACE_LIB} is not built: python -m gated_deltanet_linear_decode_amd.build --trace")
    abi.LIB_PATH = TRACE_LIB
    lib = abi.load()
    copy = lib.gdn_block_trace_copy
    copy.argtypes = [ctypes.c_void_p, ctypes.c_size_t]
    copy.restype = ctypes.c_int

    shape = configs.ALL[args.config]
    seqs, tokens = (int(v) for v in args.verify.split("x")) if args.verify else (args.rows, 1)
    R = seqs * tokens
    dev = torch.device("cuda:0")
    blk = GdnBlock(shape, max_rows=R, device=dev)
    w_cpu = synth.make_weights(shape, 0)
    c_cpu = synth.make_call(shape, R, 0, pads=shape.pad_rows and not args.verify)
    # verify: sources and destination slots all distinct, as the bench draws them
    perm = (np.random.Generator(np.random.PCG64(5)).permutation(shape.num_state_slots - 1)[:seqs + R] + 1)
    src = torch.from_numpy(perm[:seqs].astype(np.int32)).to(dev)
    dst = torch.from_numpy(perm[seqs:].astype(np.int32).reshape(seqs, tokens)).to(dev)
    copies = []
    for _ in range(min(shape.layers, 12)):
        w = synth.GdnWeights(**{k: (v.to(dev).clone() if v is not None else None) for k, v in w_cpu.__dict__.items()})
        packed = blk.pack(w)
        copies.append(dict(w=w, packed=packed, ws=blk.packed_struct(w, packed), x=c_cpu.x.to(dev), res=c_cpu.residual.to(dev),
                           conv=c_cpu.conv_state.to(dev), ssm=c_cpu.ssm_state.to(dev), idx=c_cpu.state_idx.to(dev),
                           core=torch.empty(R, shape.value_dim, dtype=torch.bfloat16, device=dev),
                           out=(torch.empty(R, shape.hidden, dtype=torch.bfloat16, device=dev)
                                if shape.fold_out_proj else None)))
    for i in range(args.launches):
        c = copies[i % len(copies)]
        if args.verify:
            blk.verify(c["x"], c["res"], None, c["conv"], c["ssm"], src, dst, c["core"], weights_struct=c["ws"])
        else:
            blk.decode(c["x"], c["res"], None, c["conv"], c["ssm"], c["idx"], c["core"], weights_struct=c["ws"],
                       out=c["out"])
    torch.cuda.synchronize()
    assert blk.check() == 0, "a wait inside the decode gave up"
    buf = np.zeros(BLOCKS * SLOTS, dtype=np.uint64)
    assert copy(buf.ctypes.data, BLOCKS) == 0
    t = buf.reshape(BLOCKS, SLOTS).astype(np.int64)

    # the grid: norm workgroups, projection workgroups, recurrence workgroups, out_proj ones
    p_mx = -(-shape.hidden // 2048)  # MXFP4 image workgroups per row
    if shape.input_normed:
        P = p_mx if shape.qkvz_format == "mxfp4" and R > 2 else 0
    else:
        P = p_mx if shape.qkvz_format == "mxfp4" else 1
    unit = 128 if shape.qkvz_format == "bf16" else 512  # K ranges: whole units up to 1024
    S = shape.hidden // max(k for k in range(unit, 1025, unit) if shape.hidden % k == 0)
    G = (shape.n_qkvz // 64 + -(-shape.n_ba // 16)) * S
    nn, nrec = R * P, seqs * shape.num_v_heads
    nout = shape.hidden // 64 if shape.fold_out_proj else 0
    roles = {"norm": range(0, nn), "proj": range(nn, nn + G), "rec": range(nn + G, nn + G + nrec),
             "oproj": range(nn + G + nrec, nn + G + nrec + nout)}
    t0 = min(t[i, 0] for r in roles.values() for i in r if t[i, 0] > 0)
    last = max(t[i, s] for r in roles.values() for i in r for s in range(SLOTS - 1) if t[i, s] > 0)
    what = f"verify {seqs}x{tokens}" if args.verify else f"{R} rows"
    print(f"{shape.name}, {what}: {nn} norm, {G} projection, {nrec} recurrence, {nout} out_proj workgroups; "
          f"last stamp {(last - t0) * 0.01:.2f} us after the first start")
    chunked = args.verify and tokens > 1 and shape.head_k_dim == 128
    points = dict(POINTS, rec=VERIFY_REC) if chunked else POINTS
    order = dict(ORDER, rec=VERIFY_ORDER) if chunked else ORDER
    for name, rng in roles.items():
        if not len(rng):
            continue
        print(f"  {name}")
        for slot in order.get(name, sorted(points[name])):
            v = np.array([t[i, slot] for i in rng if t[i, slot] > 0], dtype=np.int64)
            if len(v) == 0:
                continue
            r = (v - t0) * 0.01
            print(f"    {points[name].get(slot, f'point {slot}'):36s} {r.min():7.2f} {np.median(r):7.2f} {r.max():7.2f}")
    hw = buf.reshape(BLOCKS, SLOTS)[list(roles["proj"]), SLOTS - 1].astype(np.uint64)
    xcc = ((hw >> np.uint64(32)) & np.uint64(0xF)).astype(int)
    hwid = hw & np.uint64(0xFFFFFFFF)
    cu = ((hwid >> np.uint64(8)) & np.uint64(0xF)).astype(int)
    sh = ((hwid >> np.uint64(12)) & np.uint64(1)).astype(int)
    se = ((hwid >> np.uint64(13)) & np.uint64(0x7)).astype(int)
    key = list(zip(xcc, se, sh, cu))
    per_cu = Counter(key)
    done = (t[list(roles["proj"]), 2] - t0) * 0.01
    by = defaultdict(list)
    for k, d in zip(key, done):
        by[per_cu[k]].append(d)
    print(f"  projection workgroups on {len(per_cu)} CUs, workgroups per CU: {dict(Counter(per_cu.values()))}")
    for n in sorted(by):
        v = np.array(by[n])
        print(f"    on CUs holding {n}: {len(v)} workgroups, matrix-core work done {v.min():.2f} / "
              f"{np.median(v):.2f} / {v.max():.2f} us")
    blk.close()


if __name__ == "__main__":
    main()
