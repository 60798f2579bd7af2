"""GPU-against-GPU properties that hold exactly ("sgl-amd-mono PR #89", Kernel
checks): batch invariance, the bf16 state being the f32 state rounded, graph
replay equal to eager, run-to-run determinism; plus the decode call's host-side
argument checks with a live handle."""
import ctypes

import numpy as np
import pytest
import torch

from gated_deltanet_linear_decode_amd import abi, configs, synth
from gated_deltanet_linear_decode_amd.block import GdnBlock
from tests.gpu_util import call_to, note, run_gpu, weights_to
from tests.helpers import u16

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _bits(t):
    return u16(t) if t.dtype == torch.bfloat16 else t.numpy().view(np.uint32)


@pytest.mark.parametrize("name", ["tiny", "tp8_rank_f32_state_pads", "tp8_rank_mxfp4",
                                  "tp8_rank_mxfp4_normed_input", "tp8_rank_bf16_state_out_proj",
                                  "tp8_rank_mxfp6"])
def test_batch_invariance(name):
    """A probe row's outputs do not change with the other rows or the width."""
    shape = configs.ALL[name].with_(num_state_slots=40, rows=(16,), pad_rows=False)
    w = weights_to(synth.make_weights(shape, 21), DEV)
    blk = GdnBlock(shape, max_rows=16, device=DEV)
    base = synth.make_call(shape, 16, 21)
    probe_slot = int(base.state_idx[0])
    ref = None
    for width in (1, 2, 5, 8, 9, 16):
        for pos in sorted({0, width - 1, width // 2}):
            note(f"batch invariance {name} width={width} pos={pos}")
            other = synth.make_call(shape, width, 1000 + width * 17 + pos)
            idx = other.state_idx.clone()
            idx[idx == probe_slot] = int(base.state_idx[1])   # keep slots distinct
            idx[pos] = probe_slot
            x, res = other.x.clone(), other.residual.clone()
            x[pos], res[pos] = base.x[0], base.residual[0]
            call = synth.GdnCall(x, res, base.conv_state, base.ssm_state, idx)
            out = run_gpu(blk, shape, w, call_to(call, DEV))
            got = (u16(out["core"][pos]), u16(out["residual"][pos]), u16(out["conv_state"][probe_slot]),
                   _bits(out["ssm_state"][probe_slot])) + ((u16(out["out"][pos]),) if "out" in out else ())
            if ref is None:
                ref = got
            for a, b in zip(ref, got):
                assert np.array_equal(a, b), f"width {width} pos {pos}"
    blk.close()


@pytest.mark.parametrize("name", ["tiny", "tp8_rank_bf16_state_layer0"])
def test_bf16_state_is_f32_state_rounded(name):
    shape_b = configs.ALL[name].with_(ssm_state_dtype="bf16", pad_rows=True, rows=(8,), num_state_slots=16)
    shape_f = shape_b.with_(ssm_state_dtype="f32")
    rows = min(8, shape_b.num_state_slots - 1)
    w = weights_to(synth.make_weights(shape_b, 22), DEV)
    call_b = synth.make_call(shape_b, rows, 22)
    call_f = synth.GdnCall(call_b.x, call_b.residual, call_b.conv_state, call_b.ssm_state.float(),
                           call_b.state_idx)
    bb = GdnBlock(shape_b, max_rows=8, device=DEV)
    bf = GdnBlock(shape_f, max_rows=8, device=DEV)
    out_b = run_gpu(bb, shape_b, w, call_to(call_b, DEV))
    out_f = run_gpu(bf, shape_f, w, call_to(call_f, DEV))
    assert np.array_equal(u16(out_b["core"]), u16(out_f["core"]))
    assert np.array_equal(u16(out_b["conv_state"]), u16(out_f["conv_state"]))
    assert np.array_equal(u16(out_b["ssm_state"]), u16(out_f["ssm_state"].to(torch.bfloat16)))
    bb.close()
    bf.close()


def test_determinism():
    shape = configs.TP8_RANK_F32
    w = weights_to(synth.make_weights(shape, 23), DEV)
    cd = call_to(synth.make_call(shape, 16, 23), DEV)
    blk = GdnBlock(shape, device=DEV)
    a = run_gpu(blk, shape, w, cd)
    b = run_gpu(blk, shape, w, cd)
    for k in a:
        assert torch.equal(a[k].view(torch.int16) if a[k].dtype == torch.bfloat16 else a[k],
                           b[k].view(torch.int16) if b[k].dtype == torch.bfloat16 else b[k]), k
    blk.close()


def test_graph_replay_equals_eager():
    """Widths 8, 1, 3, 8, 2, 5 in one graph on one state pool, replayed 200 times."""
    shape = configs.TP8_RANK_BF16.with_(num_state_slots=32, rows=(8,), has_residual=True, pad_rows=True)
    w = weights_to(synth.make_weights(shape, 24), DEV)
    blk = GdnBlock(shape, max_rows=8, device=DEV)
    packed = blk.pack(w)
    ws = blk.packed_struct(w, packed)
    widths = (8, 1, 3, 8, 2, 5)
    calls = [call_to(synth.make_call(shape, r, 300 + i), DEV) for i, r in enumerate(widths)]
    conv0, ssm0 = calls[0].conv_state.clone(), calls[0].ssm_state.clone()
    conv, ssm = conv0.clone(), ssm0.clone()
    res = [c.residual.clone() for c in calls]
    cores = [torch.zeros(r, shape.value_dim, dtype=torch.bfloat16, device=DEV) for r in widths]

    def step_all():
        for i, c in enumerate(calls):
            blk.decode(c.x, res[i], None, conv, ssm, c.state_idx, cores[i], weights_struct=ws)

    def reset():
        conv.copy_(conv0)
        ssm.copy_(ssm0)
        for i, c in enumerate(calls):
            res[i].copy_(c.residual)

    reset()
    step_all()
    torch.cuda.synchronize()
    eager = [conv.clone(), ssm.clone()] + [r.clone() for r in res] + [c.clone() for c in cores]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        reset()
        step_all()            # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step_all()
    mismatches = 0
    for rep in range(200):
        reset()
        for c in cores:
            c.fill_(1.0)
        g.replay()
        torch.cuda.synchronize()
        got = [conv, ssm] + res + cores
        for a, b in zip(eager, got):
            if not torch.equal(a.view(torch.int16), b.view(torch.int16)):
                mismatches += 1
        if rep % 50 == 0:
            note(f"graph replay {rep}: mismatches so far {mismatches}")
    assert mismatches == 0
    assert blk.check() == 0
    blk.close()


def test_graph_replay_fold_and_verify():
    """One graph mixing out_proj-fold decodes (8 and 1 rows) and verify steps (2 x 4 and 1 x 3
    tokens) on two handles, replayed 60 times: every replay equals the eager run bit for bit
    (the fold's and verify's counters are cleared by the launches themselves)."""
    import numpy as np
    fold_shape = configs.TP8_RANK_BF16_OUT.with_(num_state_slots=48, rows=(8,))
    ver_shape = configs.TP8_RANK_BF16.with_(num_state_slots=48, rows=(8,))
    wf = weights_to(synth.make_weights(fold_shape, 25), DEV)
    wv = weights_to(synth.make_weights(ver_shape, 25), DEV)
    bf = GdnBlock(fold_shape, max_rows=8, device=DEV)
    bv = GdnBlock(ver_shape, max_rows=8, device=DEV)
    packed_f, packed_v = bf.pack(wf), bv.pack(wv)  # kept alive: the structs hold raw pointers
    wsf, wsv = bf.packed_struct(wf, packed_f), bv.packed_struct(wv, packed_v)
    dcalls = [call_to(synth.make_call(fold_shape, r, 400 + r), DEV) for r in (8, 1)]
    vcalls = [call_to(synth.make_call(ver_shape, s_ * t, 410 + t), DEV) for s_, t in ((2, 4), (1, 3))]
    src = [torch.tensor([3, 7], dtype=torch.int32, device=DEV), torch.tensor([11], dtype=torch.int32, device=DEV)]
    dst = [torch.tensor([[20, 21, 22, 3], [23, 0, 24, 25]], dtype=torch.int32, device=DEV),
           torch.tensor([[30, 31, 32]], dtype=torch.int32, device=DEV)]
    conv0f, ssm0f = dcalls[0].conv_state.clone(), dcalls[0].ssm_state.clone()
    conv0v, ssm0v = vcalls[0].conv_state.clone(), vcalls[0].ssm_state.clone()
    convf, ssmf, convv, ssmv = conv0f.clone(), ssm0f.clone(), conv0v.clone(), ssm0v.clone()
    resd = [c.residual.clone() for c in dcalls]
    resv = [c.residual.clone() for c in vcalls]
    cored = [torch.zeros(c.x.shape[0], fold_shape.value_dim, dtype=torch.bfloat16, device=DEV) for c in dcalls]
    outs = [torch.zeros(c.x.shape[0], fold_shape.hidden, dtype=torch.bfloat16, device=DEV) for c in dcalls]
    corev = [torch.zeros(c.x.shape[0], ver_shape.value_dim, dtype=torch.bfloat16, device=DEV) for c in vcalls]

    def step_all():
        for i in range(2):
            bf.decode(dcalls[i].x, resd[i], None, convf, ssmf, dcalls[i].state_idx, cored[i], weights_struct=wsf,
                      out=outs[i])
            bv.verify(vcalls[i].x, resv[i], None, convv, ssmv, src[i], dst[i], corev[i], weights_struct=wsv)

    def reset():
        convf.copy_(conv0f)
        ssmf.copy_(ssm0f)
        convv.copy_(conv0v)
        ssmv.copy_(ssm0v)
        for i in range(2):
            resd[i].copy_(dcalls[i].residual)
            resv[i].copy_(vcalls[i].residual)

    def state():
        return [convf, ssmf, convv, ssmv] + resd + resv + cored + outs + corev

    names = ["conv fold", "ssm fold", "conv verify", "ssm verify", "residual fold 8", "residual fold 1",
             "residual verify 2x4", "residual verify 1x3", "core fold 8", "core fold 1", "out fold 8",
             "out fold 1", "core verify 2x4", "core verify 1x3"]

    reset()
    step_all()
    torch.cuda.synchronize()
    eager = [t.clone() for t in state()]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        reset()
        step_all()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step_all()
    mismatches = 0
    for rep in range(60):
        reset()
        for t in cored + outs + corev:
            t.fill_(1.0)
        g.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(names, eager, state()):
            bits = (lambda t: t.view(torch.int16)) if a.dtype == torch.bfloat16 else (lambda t: t)
            if not torch.equal(bits(a), bits(b)):
                mismatches += 1
                if rep == 0:
                    note(f"  replay 0: {name} differs from the eager run")
        if rep % 20 == 0:
            note(f"fold/verify graph replay {rep}: mismatches so far {mismatches}")
    assert mismatches == 0
    assert bf.check() == 0 and bv.check() == 0
    bf.close()
    bv.close()


def test_decode_rejects_bad_arguments_on_the_host():
    shape = configs.TINY
    w = weights_to(synth.make_weights(shape, 25), DEV)
    cd = call_to(synth.make_call(shape, 1, 25), DEV)
    blk = GdnBlock(shape, device=DEV)
    ws = blk.weights_struct(w)
    core = torch.zeros(1, shape.value_dim, dtype=torch.bfloat16, device=DEV)
    lib = abi.load()
    p = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    args = [p(cd.x), p(cd.residual), ctypes.byref(ws), p(cd.conv_state), p(cd.ssm_state), p(cd.state_idx)]

    def call(rows, *, x=None, core_ptr=None):
        a = list(args)
        if x is not None:
            a[0] = x
        return lib.gdn_block_decode(blk.handle, *a, rows, core_ptr if core_ptr is not None else p(core), None)

    assert call(2) == abi.GDN_E_INVALID_ARG and "rows" in abi.gdn_block_last_error(blk.handle)
    assert call(-1) == abi.GDN_E_INVALID_ARG
    assert call(1, x=ctypes.c_void_p(0)) == abi.GDN_E_INVALID_ARG and "x is NULL" in abi.gdn_block_last_error(blk.handle)
    assert call(1, x=ctypes.c_void_p(cd.x.data_ptr() + 2)) == abi.GDN_E_INVALID_ARG
    assert "aligned" in abi.gdn_block_last_error(blk.handle)
    torch.cuda.synchronize()
    before = core.clone()
    assert call(0) == abi.GDN_OK        # an empty call enqueues nothing
    torch.cuda.synchronize()
    assert torch.equal(core, before)
    assert call(1) == abi.GDN_OK
    torch.cuda.synchronize()
    blk.close()


def test_pack_rejects_bad_arguments():
    shape = configs.TINY
    w = weights_to(synth.make_weights(shape, 26), DEV)
    blk = GdnBlock(shape, device=DEV)
    ws = blk.weights_struct(w)
    lib = abi.load()
    assert abi.gdn_block_packed_weight_bytes(blk.handle) == (shape.n_qkvz // 16 + 1) * 16 * shape.hidden * 2
    assert lib.gdn_block_pack_weights(blk.handle, ctypes.byref(ws), None, None) == abi.GDN_E_INVALID_ARG
    out = torch.empty(abi.gdn_block_packed_weight_bytes(blk.handle) + 16, dtype=torch.uint8, device=DEV)
    assert lib.gdn_block_pack_weights(blk.handle, ctypes.byref(ws), ctypes.c_void_p(out.data_ptr() + 8),
                                      None) == abi.GDN_E_INVALID_ARG
    blk.close()


def test_repeated_decodes_keep_counters_consistent():
    """Many back-to-back launches of varying width and pad mix on one handle: every
    launch must find its hand-off counters cleared by the previous one."""
    shape = configs.TP8_RANK_F32.with_(num_state_slots=40)
    w = weights_to(synth.make_weights(shape, 27), DEV)
    blk = GdnBlock(shape, device=DEV)
    packed = blk.pack(w)
    for i, rows in enumerate((16, 1, 7, 16, 3, 1, 12)):
        cd = call_to(synth.make_call(shape, rows, 400 + i, all_pad=(i == 5)), DEV)
        a = run_gpu(blk, shape, w, cd, packed=packed)
        b = run_gpu(blk, shape, w, cd)
        for k in a:
            x, y = a[k], b[k]
            if x.dtype == torch.bfloat16:
                x, y = x.view(torch.int16), y.view(torch.int16)
            assert torch.equal(x, y), (rows, k)
    blk.close()
