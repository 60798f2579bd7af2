"""Shared pieces of the GPU tests: moving a synthetic call to the device,
running the HIP block through the C ABI, and the parity rule.

Parity rule for floating-point outputs (bf16 core, conv state, out_proj partial, SSM
state), over the written elements of each tensor, with scale = max(|oracle value|, the
tensor's rms):
  outer floor (every tensor): |gpu - oracle| <= max(2e-2, one bf16 ulp of the oracle
    value) element by element, and cosine >= 0.9999;
  bf16 tensors: |gpu - oracle| <= 4 bf16 ulps of the scale, and
    ||gpu - oracle|| / ||oracle|| <= 4e-3;
  the f32 SSM state: |gpu - oracle| <= 1.5e-2 * scale, and
    ||gpu - oracle|| / ||oracle|| <= 3e-4.
The tight bounds are set with a margin of 2-4 over the largest errors measured on
MI355X over every GPU test case (2 ulps at scale and 1.4e-3 for the bf16 tensors; 5.6e-3
at scale and 7.2e-5 for the f32 state): a correct kernel differs from the oracle by the
f32-versus-f64 rounding of its sums, and where that moves a bf16 value by one ulp
(projection outputs, conv outputs, o) the change spreads through the rest of the head.
A uniform relative error of 1 % fails the norm bounds of both. The residual, pad rows and
untouched slots are compared bit for bit.
"""
import json
import os
import sys

import numpy as np
import torch

from gated_deltanet_linear_decode_amd.block import GdnBlock
from gated_deltanet_linear_decode_amd.synth import GdnCall, GdnWeights
from oracle import gdn as og
from tests.helpers import oracle_state, run_oracle, u16

ABS_TOL = 2e-2
COS_MIN = 0.9999
ULPS_AT_SCALE = 4         # bf16 tensors: element bound in bf16 ulps of max(|oracle|, rms)
REL_NORM_BF16 = 4e-3      # bf16 tensors: ||gpu - oracle|| / ||oracle||
REL_AT_SCALE_F32 = 1.5e-2  # f32 state: element bound relative to max(|oracle|, rms)
REL_NORM_F32 = 3e-4       # f32 state: ||gpu - oracle|| / ||oracle||
FLIP_NORM_FACTOR = 10     # the norm bounds under the MXFP4 code-flip allowance


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def record(label, stats):
    """Append one case's measured errors to the JSON-lines file named by the environment
    variable GDN_PARITY_STATS, when it is set (the bounds of the parity rule are derived
    from these measurements)."""
    path = os.environ.get("GDN_PARITY_STATS")
    if path:
        with open(path, "a") as f:
            f.write(json.dumps({"case": label, "stats": stats}) + "\n")


def weights_to(w: GdnWeights, dev) -> GdnWeights:
    return GdnWeights(**{k: (v.to(dev) if v is not None else None) for k, v in w.__dict__.items()})


def call_to(c: GdnCall, dev) -> GdnCall:
    return GdnCall(**{k: v.to(dev).contiguous() for k, v in c.__dict__.items()})


def run_gpu(blk: GdnBlock, shape, wd: GdnWeights, cd: GdnCall, rows=None, packed=None, check=True, noalloc=False):
    """Run one decode on copies of the device inputs; returns CPU tensors.

    `packed`: None streams the row-major weights; a tensor from blk.pack() streams
    the tiled copy. With `check`, the handle's sticky error word must stay 0. With
    `noalloc`, the decode goes through gdn_block_decode_noalloc."""
    R = cd.x.shape[0] if rows is None else rows
    res = cd.residual.clone()
    conv = cd.conv_state.clone()
    ssm = cd.ssm_state.clone()
    core = torch.full((R, shape.value_dim), float("nan"), dtype=torch.bfloat16, device=cd.x.device)
    out = (torch.full((R, shape.hidden), float("nan"), dtype=torch.bfloat16, device=cd.x.device)
           if shape.fold_out_proj else None)
    ws = blk.packed_struct(wd, packed) if packed is not None else blk.weights_struct(wd)
    blk.decode(cd.x, res, None, conv, ssm, cd.state_idx, core, weights_struct=ws, out=out, noalloc=noalloc)
    torch.cuda.synchronize()
    if check:
        assert blk.check() == 0, "a wait inside the decode gave up"
    r = dict(core=core.cpu(), residual=res.cpu(), conv_state=conv.cpu(), ssm_state=ssm.cpu())
    if out is not None:
        r["out"] = out.cpu()
    return r


def same_bits(a: dict, b: dict):
    for k in a:
        x, y = a[k], b[k]
        if x.dtype == torch.bfloat16:
            x, y = x.view(torch.int16), y.view(torch.int16)
        assert torch.equal(x, y), f"{k} differs between the two weight layouts"


def _ulp_bf16(r):
    a = np.maximum(np.abs(r), 2.0 ** -126)
    return np.exp2(np.floor(np.log2(a)) - 7)


def error_stats(g, r, bf16):
    """Measured error of one tensor: max abs; for bf16 the largest error in units of the
    oracle value's bf16 ulp and the fraction of elements whose bits differ; for f32 the
    largest relative error (elements above 1e-3 of the tensor's rms) and the fraction
    above 1e-5 relative; and ||gpu - oracle|| / ||oracle|| over the whole tensor."""
    err = np.abs(g - r)
    nr = np.linalg.norm(r)
    rms = nr / np.sqrt(r.size) if r.size else 0.0
    scale = np.maximum(np.abs(r), rms)  # an element's magnitude, at least the tensor's rms
    st = {"max_abs": float(err.max()), "rel_norm": float(np.linalg.norm(g - r) / nr) if nr > 0 else 0.0}
    if bf16:
        st["max_ulp"] = float((err / _ulp_bf16(r)).max())
        st["ulp_at_scale"] = float((err / _ulp_bf16(scale)).max()) if rms > 0 else 0.0
        st["frac_diff"] = float((err > 0).mean())
    else:
        st["rel_at_scale"] = float((err / scale).max()) if rms > 0 else 0.0
        big = np.abs(r) > 1e-3 * rms
        rel = err[big] / np.abs(r[big]) if big.any() else np.zeros(1)
        st["max_rel"] = float(rel.max())
        st["frac_rel_1e-5"] = float((rel > 1e-5).mean())
    return st


def close(name, got, ref, bf16=True, flips=None):
    """Assert the parity rule (see the module docstring); returns the tensor's measured
    error (error_stats) with the counts above ABS_TOL ("n_abs") and outside either element
    bound ("n_bad").

    `flips` = (fraction, cap) relaxes the element rules for outputs downstream of the
    MXFP4 activation quantiser: up to `fraction` of the elements may leave the bounds, each
    by at most `cap`, and the norm bound is FLIP_NORM_FACTOR times wider (see
    tests/test_gpu_mxfp4.py for why); the cosine rule still holds."""
    g = og.bf16_to_f64(got) if bf16 else np.asarray(got, np.float64)
    r = og.bf16_to_f64(ref) if bf16 else np.asarray(ref, np.float64)
    g, r = g.reshape(-1), r.reshape(-1)
    if g.size == 0:
        return {}
    assert np.all(np.isfinite(g)), f"{name}: non-finite values"
    err = np.abs(g - r)
    nr = np.linalg.norm(r)
    scale = np.maximum(np.abs(r), nr / np.sqrt(r.size))
    if bf16:
        bound = np.minimum(np.maximum(ABS_TOL, _ulp_bf16(r)), ULPS_AT_SCALE * _ulp_bf16(scale))
        norm_bound = REL_NORM_BF16
    else:
        bound = np.minimum(ABS_TOL, REL_AT_SCALE_F32 * scale)
        norm_bound = REL_NORM_F32
    bad = err > bound
    worst = (f"worst err {err.max():.4g} at {np.argmax(err)} (gpu {g[np.argmax(err)]}, "
             f"oracle {r[np.argmax(err)]})")
    if flips is None:
        assert not bad.any(), f"{name}: {bad.sum()} of {err.size} outside the bound; {worst}"
    else:
        frac, cap = flips
        assert bad.sum() <= frac * err.size, f"{name}: {bad.sum()} of {err.size} outside the bound; {worst}"
        assert err.max() <= cap, f"{name}: an error above the cap {cap}; {worst}"
    ng = np.linalg.norm(g)
    if nr > 0:
        cos = float(g @ r / (nr * ng))
        assert cos >= COS_MIN, f"{name}: cosine {cos}"
        rel = float(np.linalg.norm(g - r) / nr)
        nb = norm_bound * (FLIP_NORM_FACTOR if flips is not None else 1)
        assert rel <= nb, f"{name}: ||gpu - oracle|| / ||oracle|| = {rel:.3g} above {nb:.3g}"
    st = error_stats(g, r, bf16)
    st["n_abs"], st["n_bad"] = int((err > ABS_TOL).sum()), int(bad.sum())
    return st


def check_parity(shape, w, call, out, label="", flips=None):
    """Compare one GPU decode's outputs with the oracle's (`flips`: see close())."""
    ref = run_oracle(shape, w, call)
    idx = call.state_idx.numpy()
    valid = (idx > 0) & (idx < shape.num_state_slots)  # an index past the pool is a pad row
    core = u16(out["core"])
    # residual: bit for bit (a normed input leaves it untouched)
    want = u16(call.residual) if ref["residual"] is None else ref["residual"]
    assert np.array_equal(u16(out["residual"]), want), f"{label}: residual differs"
    # pad rows: all +0.0
    assert np.all(core[~valid] == 0), f"{label}: pad row core not +0"
    stats = {}
    stats["core"] = close(f"{label} core", core[valid], ref["core"][valid], flips=flips)
    slots = idx[valid]
    conv_g, conv_r = u16(out["conv_state"]), ref["conv_state"]
    bf16_state = shape.ssm_state_dtype == "bf16"
    ssm_g, ssm_r = oracle_state(out["ssm_state"]), ref["ssm_state"]
    untouched = np.setdiff1d(np.arange(shape.num_state_slots), slots)
    assert np.array_equal(conv_g[untouched], u16(call.conv_state)[untouched]), f"{label}: untouched conv slot changed"
    assert np.array_equal(ssm_g[untouched], oracle_state(call.ssm_state)[untouched]), \
        f"{label}: untouched ssm slot changed"
    if shape.fold_out_proj:  # the out_proj partial: pad rows are zero
        og_ = u16(out["out"])
        assert np.all((og_[~valid] & 0x7FFF) == 0), f"{label}: pad row out_proj partial not zero"
        stats["out"] = close(f"{label} out_proj", og_[valid], ref["out"][valid], flips=flips)
    if len(slots):
        stats["conv"] = close(f"{label} conv_state", conv_g[slots], conv_r[slots], flips=flips)
        stats["ssm"] = close(f"{label} ssm_state", ssm_g[slots], ssm_r[slots], bf16=bf16_state, flips=flips)
    record(label, stats)
    return stats


def parity_case(shape, rows, seed, *, pads=None, all_pad=False, stress=False, max_rows=None,
                weights=None, call=None, flips=None, dev="cuda:0"):
    """One decode of `shape` on seeded inputs (or the given weights / call), with the
    row-major and the tiled weights (which must agree bit for bit), against the oracle."""
    from gated_deltanet_linear_decode_amd import synth
    note(f"case {shape.name} rows={rows} seed={seed} pads={pads} all_pad={all_pad} stress={stress}")
    w = weights if weights is not None else synth.make_weights(shape, seed, gated_norm_stress=stress)
    c = call if call is not None else synth.make_call(shape, rows, seed, pads=pads, all_pad=all_pad)
    blk = GdnBlock(shape, max_rows=max_rows or max(rows, shape.max_rows), device=dev)
    wd, cd = weights_to(w, dev), call_to(c, dev)
    out = run_gpu(blk, shape, wd, cd)
    same_bits(out, run_gpu(blk, shape, wd, cd, packed=blk.pack(wd)))
    blk.close()
    stats = check_parity(shape, w, c, out, label=f"{shape.name}/r{rows}/s{seed}" + ("/wg1" if stress else ""),
                         flips=flips)
    note(f"  ok {stats}")
    return stats
