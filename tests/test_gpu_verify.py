"""GPU parity of the verify step (gdn_block_verify): R sequences of T tokens each, the
state after every token stored into its own slot so a caller can continue from whichever
draft is accepted (the follow-up "sgl-amd-mono PR #89", Modifications, and "vLLM PR
#60833", Limitations, leave open).

* Against the oracle's verify_block: core rows, the residual (bitwise), every written
  snapshot (conv window and SSM state) by the parity rule, every other slot bitwise
  unchanged, pad sequences' core rows +0; row-major and tiled weights bit for bit.
* GPU against GPU: one token with destination = source is gdn_block_decode bit for bit;
  with an f32 pool, T tokens in one step end where T decode steps end, bit for bit where
  the step runs its tokens one after the other (head dim below 128: the f32 state
  round-trips exactly, and projections are batch invariant) and within the parity rule in
  the chunked form (head dim 128); a sequence's results do not depend on the other
  sequences of the step.
"""
import numpy as np
import pytest
import torch

from gated_deltanet_linear_decode_amd import configs, synth
from gated_deltanet_linear_decode_amd.block import GdnBlock
from oracle import gdn as og
from tests.gpu_util import call_to, close, note, record, weights_to
from tests.helpers import oracle_cfg, oracle_state, oracle_weights, u16

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

TINY_V = configs.TINY.with_(name="tiny_verify", num_state_slots=64, rows=(16,))


def verify_indices(shape, R, T, seed, *, pad=True, skip=True, in_place=True):
    """Source slots (one pad sequence when R > 1), distinct destination slots disjoint from
    the sources, one snapshot not kept, and one sequence whose last snapshot goes back to
    its source slot."""
    rng = np.random.Generator(np.random.PCG64(seed + 31337))
    need = R + R * T
    assert need <= shape.num_state_slots - 1
    perm = (rng.permutation(shape.num_state_slots - 1)[:need] + 1).astype(np.int32)
    src, dst = perm[:R].copy(), perm[R:].reshape(R, T).copy()
    if pad and R > 1:
        src[1] = -1 if seed % 2 else 0
    if skip and R > 2:
        dst[2, rng.integers(0, T)] = 0
    if in_place:
        dst[0, T - 1] = src[0]
    return src, dst


def run_verify(blk, shape, wd, cd, src, dst, packed=None):
    R, T = dst.shape
    res = cd.residual.clone()
    conv = cd.conv_state.clone()
    ssm = cd.ssm_state.clone()
    core = torch.full((R * T, shape.value_dim), float("nan"), dtype=torch.bfloat16, device=cd.x.device)
    ws = blk.packed_struct(wd, packed) if packed is not None else blk.weights_struct(wd)
    blk.verify(cd.x, res, None, conv, ssm, torch.from_numpy(src).to(cd.x.device),
               torch.from_numpy(dst).to(cd.x.device), core, weights_struct=ws)
    torch.cuda.synchronize()
    assert blk.check() == 0, "a wait inside the verify step gave up"
    return dict(core=core.cpu(), residual=res.cpu(), conv_state=conv.cpu(), ssm_state=ssm.cpu())


def _same(a, b, keys=("core", "residual", "conv_state", "ssm_state")):
    for k in keys:
        x, y = a[k], b[k]
        if x.dtype == torch.bfloat16:
            x, y = x.view(torch.int16), y.view(torch.int16)
        assert torch.equal(x, y), k


def verify_case(shape, R, T, seed, flips=None, stress=False, **kw):
    note(f"verify {shape.name} R={R} T={T} seed={seed} stress={stress} {kw}")
    w = synth.make_weights(shape, seed, gated_norm_stress=stress)
    c = synth.make_call(shape, R * T, seed)
    src, dst = verify_indices(shape, R, T, seed, **kw)
    blk = GdnBlock(shape, max_rows=R * T, device=DEV)
    wd, cd = weights_to(w, DEV), call_to(c, DEV)
    out = run_verify(blk, shape, wd, cd, src, dst)
    _same(out, run_verify(blk, shape, wd, cd, src, dst, packed=blk.pack(wd)))
    blk.close()
    ref = og.verify_block(oracle_cfg(shape), oracle_weights(w), u16(c.x), u16(c.residual), u16(c.conv_state),
                          oracle_state(c.ssm_state), src, dst)
    label = f"{shape.name}/R{R}T{T}/s{seed}" + ("/wg1" if stress else "")
    want_res = u16(c.residual) if ref["residual"] is None else ref["residual"]
    assert np.array_equal(u16(out["residual"]), want_res), f"{label}: residual differs"
    core = u16(out["core"])
    live = np.repeat((src > 0) & (src < shape.num_state_slots), T)
    assert np.all(core[~live] == 0), f"{label}: pad sequence core not +0"
    stats = {"core": close(f"{label} core", core[live], ref["core"][live], flips=flips)}
    written = np.array(sorted(set(int(s) for s, ok in zip(dst.reshape(-1), live)
                                  if ok and 0 < s < shape.num_state_slots)), dtype=np.int64)
    others = np.setdiff1d(np.arange(shape.num_state_slots), written)
    conv_g, ssm_g = u16(out["conv_state"]), oracle_state(out["ssm_state"])
    assert np.array_equal(conv_g[others], u16(c.conv_state)[others]), f"{label}: an unwritten conv slot changed"
    assert np.array_equal(ssm_g[others], oracle_state(c.ssm_state)[others]), f"{label}: an unwritten ssm slot changed"
    if len(written):
        stats["conv"] = close(f"{label} conv", conv_g[written], ref["conv_state"][written], flips=flips)
        stats["ssm"] = close(f"{label} ssm", ssm_g[written], ref["ssm_state"][written],
                             bf16=shape.ssm_state_dtype == "bf16", flips=flips)
    record(label, stats)
    note(f"  ok {stats}")


@pytest.mark.parametrize("R,T", [(1, 2), (3, 3), (4, 4), (2, 8), (1, 16)])
@pytest.mark.parametrize("state", ["f32", "bf16"])
def test_tiny_verify(R, T, state):
    verify_case(TINY_V.with_(ssm_state_dtype=state), R, T, 600 + 10 * R + T)


@pytest.mark.parametrize("R,T", [(4, 4), (2, 3), (8, 2), (5, 3), (1, 16), (2, 7), (16, 1)])
def test_tp8_rank_verify(R, T):
    """Up to the most tokens a step takes (16) and an odd count in the chunked form, and 16
    one-token sequences (the single-token verify launch at its largest)."""
    verify_case(configs.TP8_RANK_BF16, R, T, 700 + 10 * R + T)


def test_dense_verify():
    """The full-width layer: three value heads per key head (two of them hand the key head's
    old q|k conv rows over to the third) and a K range of 1024 over H = 5120."""
    verify_case(configs.DENSE_FULL, 2, 4, 731)


@pytest.mark.parametrize("R,T", [(5, 3), (1, 16)])
def test_tp8_rank_f32_residual_verify(R, T):
    verify_case(configs.TP8_RANK_F32, R, T, 711 + 10 * R + T)


@pytest.mark.parametrize("R,T", [(4, 2), (1, 16)])
def test_tp8_rank_mxfp4_verify(R, T):
    verify_case(configs.TP8_RANK_MXFP4, R, T, 712 + 10 * R + T, flips=(0.02, 0.15))


def test_tp8_rank_mxfp6_verify():
    """MXFP6 weights with a residual input (the rstd hand-off)."""
    verify_case(configs.TP8_RANK_MXFP6, 2, 4, 714)


@pytest.mark.parametrize("R,T", [(1, 2), (3, 4)])
def test_tp8_rank_mxfp4_normed_verify(R, T):
    """A normed input with MXFP4: at 2 token rows each projection workgroup quantises its
    K range itself, past 2 the quantiser workgroups make the image once per row."""
    verify_case(configs.TP8_RANK_MXFP4_NORMED, R, T, 716 + R)


def test_tp8_rank_mxfp6_normed_verify():
    verify_case(configs.TP8_RANK_MXFP6.with_(name="mx6_normed", input_normed=True, has_residual=False), 2, 4, 713)


@pytest.mark.parametrize("name", ["tiny", "tp8_rank_bf16_state_layer0", "tp8_rank_f32_state_pads"])
def test_verify_gated_norm_weight_near_one(name):
    """The w_g = 1 + N(0, 0.02) draw, so the core values are O(1) and the element bound
    bites on them."""
    shape = TINY_V if name == "tiny" else configs.ALL[name]
    verify_case(shape, 3, 4, 714, stress=True)


def test_tp8_rank_mxfp4_verify_gated_norm_weight_near_one():
    verify_case(configs.TP8_RANK_MXFP4, 2, 4, 715, flips=(0.02, 0.15), stress=True)


def _decode(blk, shape, wd, x, res, conv, ssm, idx):
    core = torch.empty(x.shape[0], shape.value_dim, dtype=torch.bfloat16, device=DEV)
    blk.decode(x, res, wd, conv, ssm, idx, core)
    return core


def test_one_token_verify_is_decode():
    shape = configs.TP8_RANK_F32
    R = 8
    w, c = synth.make_weights(shape, 720), synth.make_call(shape, R, 720, pads=True)
    wd, cd = weights_to(w, DEV), call_to(c, DEV)
    blk = GdnBlock(shape, max_rows=R, device=DEV)
    src = c.state_idx.numpy().copy()
    ver = run_verify(blk, shape, wd, cd, src, src[:, None].copy())
    res, conv, ssm = cd.residual.clone(), cd.conv_state.clone(), cd.ssm_state.clone()
    core = _decode(blk, shape, wd, cd.x, res, conv, ssm, cd.state_idx)
    torch.cuda.synchronize()
    blk.close()
    _same(ver, dict(core=core.cpu(), residual=res.cpu(), conv_state=conv.cpu(), ssm_state=ssm.cpu()))


@pytest.mark.parametrize("name", ["tiny", "tp8_rank_f32"])
def test_verify_equals_decode_chain_with_f32_state(name):
    """With an f32 pool, T tokens of one verify step end where T decode steps end: bit for
    bit where the verify step runs its tokens one after the other (head dim below 128),
    within the parity rule at head dim 128, where it takes the chunked form (the same
    arithmetic in another rounding order). The conv windows are copies: bit for bit."""
    shape = TINY_V if name == "tiny" else configs.TP8_RANK_F32
    exact = shape.head_k_dim < 128
    R, T = 3, 4
    w, c = synth.make_weights(shape, 721), synth.make_call(shape, R * T, 721)
    src, dst = verify_indices(shape, R, T, 721, pad=False, skip=False, in_place=False)
    wd, cd = weights_to(w, DEV), call_to(c, DEV)
    blk = GdnBlock(shape, max_rows=R * T, device=DEV)
    ver = run_verify(blk, shape, wd, cd, src, dst)
    conv, ssm = cd.conv_state.clone(), cd.ssm_state.clone()
    slots = torch.from_numpy(src).to(DEV)
    for t in range(T):
        rows = torch.arange(R, device=DEV) * T + t
        res = cd.residual[rows].clone()
        core = _decode(blk, shape, wd, cd.x[rows].contiguous(), res, conv, ssm, slots)
        torch.cuda.synchronize()
        got = u16(ver["core"])[rows.cpu().numpy()]
        if exact:
            assert np.array_equal(u16(core), got), f"token {t}: core differs"
        else:
            close(f"{name} chain token {t} core", got, u16(core))
        nxt = torch.from_numpy(dst[:, t].copy()).to(DEV)
        conv[nxt.long()] = conv[slots.long()]
        ssm[nxt.long()] = ssm[slots.long()]
        slots = nxt
    blk.close()
    # each decode step ran in place on the previous snapshot's slot, so only the last
    # snapshot survives in the chain's pools
    d = torch.from_numpy(dst[:, T - 1].astype(np.int64))
    if exact:
        assert torch.equal(ver["ssm_state"][d], ssm.cpu()[d]), "final snapshot differs"
    else:
        close(f"{name} chain final ssm", oracle_state(ver["ssm_state"][d]), oracle_state(ssm.cpu()[d]), bf16=False)
    assert torch.equal(ver["conv_state"][d].view(torch.int16), conv.cpu()[d].view(torch.int16))


def test_verify_batch_invariance():
    """A sequence's core rows and snapshots are the same alone and among others."""
    shape = configs.TP8_RANK_BF16
    R, T = 4, 3
    w, c = synth.make_weights(shape, 722), synth.make_call(shape, R * T, 722)
    src, dst = verify_indices(shape, R, T, 722, pad=False, skip=False, in_place=False)
    wd, cd = weights_to(w, DEV), call_to(c, DEV)
    blk = GdnBlock(shape, max_rows=R * T, device=DEV)
    full = run_verify(blk, shape, wd, cd, src, dst)
    one = synth.GdnCall(c.x[3:6].clone(), c.residual[3:6].clone(), c.conv_state, c.ssm_state, c.state_idx[:1])
    alone = run_verify(blk, shape, wd, call_to(one, DEV), src[1:2].copy(), dst[1:2].copy())
    blk.close()
    assert torch.equal(full["core"][3:6].view(torch.int16), alone["core"].view(torch.int16))
    d = torch.from_numpy(dst[1].astype(np.int64))
    assert torch.equal(full["ssm_state"][d].view(torch.int16), alone["ssm_state"][d].view(torch.int16))
    assert torch.equal(full["conv_state"][d].view(torch.int16), alone["conv_state"][d].view(torch.int16))
