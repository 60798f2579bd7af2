"""Whole-block properties of the CPU oracle.

The pages print no end-to-end values for the block, so beyond the per-step
pins these check properties that hold for any correct implementation: the
pad-row rule ("sgl-amd-mono PR #89", Kernel checks: a pad row writes a zero
core row and no state, and no other slot changes), the layer-0 residual, row
independence (batch invariance, same section), the bf16 state being the f32
state rounded, and equivariance under a permutation of the key heads (which
catches a wrong value-head -> key-head mapping or a mixed-up channel index).
"""
import numpy as np
import pytest

from gated_deltanet_linear_decode_amd import configs, synth
from oracle import gdn as og
from tests.helpers import from_u16, oracle_cfg, oracle_state, oracle_weights, run_oracle, u16


def test_pad_rows_write_nothing_but_the_residual():
    shape = configs.TINY.with_(num_state_slots=8, pad_rows=True)
    w = synth.make_weights(shape, 0)
    call = synth.make_call(shape, 6, 0)
    idx = call.state_idx.numpy()
    assert (idx <= 0).sum() == 1
    out = run_oracle(shape, w, call)
    for row, slot in enumerate(idx):
        if slot <= 0:
            assert np.all(out["core"][row] == 0)
    touched = set(int(s) for s in idx if s > 0)
    cs0, ss0 = u16(call.conv_state), oracle_state(call.ssm_state)
    for slot in range(shape.num_state_slots):
        if slot not in touched:
            assert np.array_equal(out["conv_state"][slot], cs0[slot])
            assert np.array_equal(out["ssm_state"][slot], ss0[slot])
        else:
            assert not np.array_equal(out["conv_state"][slot], cs0[slot])


def test_all_pad_call():
    shape = configs.TINY
    w = synth.make_weights(shape, 1)
    call = synth.make_call(shape, 1, 1, all_pad=True)
    out = run_oracle(shape, w, call)
    assert np.all(out["core"] == 0)
    assert np.array_equal(out["ssm_state"], oracle_state(call.ssm_state))
    assert np.array_equal(out["conv_state"], u16(call.conv_state))


def test_layer0_residual_is_x():
    shape = configs.TINY.with_(has_residual=False)
    w = synth.make_weights(shape, 2)
    call = synth.make_call(shape, 1, 2)
    out = run_oracle(shape, w, call)
    assert np.array_equal(out["residual"], u16(call.x))


def test_rows_are_independent():
    shape = configs.TINY.with_(num_state_slots=8)
    w = synth.make_weights(shape, 3)
    call = synth.make_call(shape, 5, 3, pads=False)
    full = run_oracle(shape, w, call)
    for row in range(5):
        one = synth.GdnCall(call.x[row:row + 1], call.residual[row:row + 1], call.conv_state,
                            call.ssm_state, call.state_idx[row:row + 1])
        alone = run_oracle(shape, w, one)
        assert np.array_equal(alone["core"][0], full["core"][row])
        slot = int(call.state_idx[row])
        assert np.array_equal(alone["ssm_state"][slot], full["ssm_state"][slot])


def test_bf16_state_is_the_f32_state_rounded():
    shape = configs.TINY.with_(ssm_state_dtype="bf16")
    w = synth.make_weights(shape, 4)
    call = synth.make_call(shape, 1, 4)
    out_b = run_oracle(shape, w, call)
    wide = synth.GdnCall(call.x, call.residual, call.conv_state, call.ssm_state.float(), call.state_idx)
    out_f = run_oracle(shape.with_(ssm_state_dtype="f32"), w, wide)
    assert np.array_equal(out_b["core"], out_f["core"])
    assert np.array_equal(out_b["conv_state"], out_f["conv_state"])
    slot = int(call.state_idx[0])
    rb = og.bf16_to_f64(out_b["ssm_state"][slot])
    rf = og.bf16_to_f64(og.f64_to_bf16(out_f["ssm_state"][slot].astype(np.float64)))
    # one rounding from f64 vs one through f32: equal except at rare double-rounding ties
    assert np.mean(rb == rf) > 0.999
    ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(rf), 1e-30))) - 7)
    assert np.all(np.abs(rb - rf) <= ulp)


def _permute_groups(shape, w, call, perm):
    """Relabel key heads g -> perm[g] (value heads, weights, states follow)."""
    nk, dk, nv, dv, r = shape.num_k_heads, shape.head_k_dim, shape.num_v_heads, shape.head_v_dim, \
        shape.heads_per_group
    inv = np.argsort(perm)                           # new group j holds old group inv[j]
    vh = np.concatenate([np.arange(r) + r * g for g in inv])          # new value head -> old
    W = oracle_weights(w)
    qkvz = W["w_qkvz"].reshape(nk, shape.group_width, -1)[inv].reshape(W["w_qkvz"].shape)
    ba = W["w_ba"].reshape(nk, 2 * r, -1)[inv].reshape(W["w_ba"].shape)
    qc = np.arange(nk * dk).reshape(nk, dk)[inv].reshape(-1)
    vc = np.arange(nv * dv).reshape(nv, dv)[vh].reshape(-1)
    ch = np.concatenate([qc, nk * dk + qc, 2 * nk * dk + vc])
    W2 = dict(W, w_qkvz=qkvz, w_ba=ba, conv_w=W["conv_w"][ch], A_log=W["A_log"][vh],
              dt_bias=W["dt_bias"][vh])
    cs = u16(call.conv_state)[:, :, ch]
    ss = oracle_state(call.ssm_state)[:, vh]
    return W2, cs, ss, vh, ch


def test_key_head_permutation_equivariance():
    shape = configs.TINY.with_(num_state_slots=8)
    w = synth.make_weights(shape, 5)
    call = synth.make_call(shape, 3, 5, pads=False)
    base = run_oracle(shape, w, call)
    perm = np.array([1, 0])
    W2, cs, ss, vh, ch = _permute_groups(shape, w, call, perm)
    out = og.decode_block(oracle_cfg(shape), W2, u16(call.x), u16(call.residual), cs, ss,
                          call.state_idx.numpy())
    dv = shape.head_v_dim
    core_b = base["core"].reshape(3, shape.num_v_heads, dv)[:, vh].reshape(3, -1)
    assert np.array_equal(out["core"], core_b)
    assert np.array_equal(out["ssm_state"], base["ssm_state"][:, vh])
    assert np.array_equal(out["conv_state"], base["conv_state"][:, :, ch])


def _library_block(shape, w, call):
    """The block composed from torch float64 library routines, written from the
    step list independently of the oracle's code: rms_norm, matmul, conv1d,
    softplus, sigmoid, normalize. Rounding to bf16 uses the (separately pinned)
    oracle rounding only where the stock chain stores bf16."""
    import torch
    import torch.nn.functional as F
    rb = lambda t: torch.from_numpy(og.bf16_to_f64(og.f64_to_bf16(t.numpy())))  # noqa: E731
    d = lambda t: t.double()                                                    # noqa: E731
    nk, dk, nv, dv, r = shape.num_k_heads, shape.head_k_dim, shape.num_v_heads, shape.head_v_dim, \
        shape.heads_per_group
    h = rb(d(call.x) + d(call.residual)) if shape.has_residual else d(call.x)
    xn = rb(F.rms_norm(h, (shape.hidden,), weight=1 + d(w.norm_w), eps=shape.norm_eps))
    yq = rb(xn @ d(w.w_qkvz).T).reshape(-1, nk, shape.group_width)
    yb = rb(xn @ d(w.w_ba).T).reshape(-1, nk, 2 * r)
    q, k = yq[..., :dk], yq[..., dk:2 * dk]
    v = yq[..., 2 * dk:2 * dk + r * dv].reshape(-1, nv, dv)
    z = yq[..., 2 * dk + r * dv:].reshape(-1, nv, dv)
    b, a = yb[..., :r].reshape(-1, nv), yb[..., r:].reshape(-1, nv)
    qkv = torch.cat([q.reshape(-1, nk * dk), k.reshape(-1, nk * dk), v.reshape(-1, nv * dv)], -1)
    S_all = d(call.ssm_state).clone()
    C_all = d(call.conv_state).clone()
    core = torch.zeros(len(call.state_idx), nv * dv, dtype=torch.float64)
    for row, slot in enumerate(call.state_idx.tolist()):
        if slot <= 0:
            continue
        seq = torch.cat([C_all[slot], qkv[row:row + 1]], 0)            # [W, Cd]
        conv = F.conv1d(seq.T[None], d(w.conv_w)[:, None, :], groups=shape.conv_dim)[0, :, -1]
        c = rb(F.silu(conv))
        C_all[slot] = seq[1:]
        cq = F.normalize(c[:nk * dk].reshape(nk, dk), dim=-1, eps=0) \
            * (c[:nk * dk].reshape(nk, dk).square().sum(-1, keepdim=True)
               / (c[:nk * dk].reshape(nk, dk).square().sum(-1, keepdim=True) + shape.l2norm_eps)).sqrt()
        ck_raw = c[nk * dk:2 * nk * dk].reshape(nk, dk)
        ck = ck_raw / (ck_raw.square().sum(-1, keepdim=True) + shape.l2norm_eps).sqrt()
        cv = c[2 * nk * dk:].reshape(nv, dv)
        g = -torch.exp(d(w.A_log)) * F.softplus(a[row] + d(w.dt_bias))
        beta = torch.sigmoid(b[row])
        for hv in range(nv):
            kk, qq = ck[hv // r], cq[hv // r] / dk ** 0.5
            S = torch.exp(g[hv]) * S_all[slot, hv]
            S = S + torch.outer(kk, beta[hv] * (cv[hv] - S.T @ kk))
            S_all[slot, hv] = S
            o = rb(S.T @ qq)
            core[row, hv * dv:(hv + 1) * dv] = rb(
                F.rms_norm(o, (dv,), weight=d(w.gated_norm_w), eps=shape.gated_norm_eps) * F.silu(z[row, hv]))
    return core, S_all, C_all, h


@pytest.mark.parametrize("bf16_state", [False, True])
def test_block_against_library_composition(bf16_state):
    shape = configs.TINY.with_(num_state_slots=8, pad_rows=True,
                               ssm_state_dtype="bf16" if bf16_state else "f32")
    w = synth.make_weights(shape, 6)
    call = synth.make_call(shape, 4, 6)
    out = run_oracle(shape, w, call)
    core, S_all, C_all, h = _library_block(shape, w, call)
    assert np.array_equal(og.bf16_to_f64(out["core"]), core.numpy())
    assert np.array_equal(og.bf16_to_f64(out["residual"]), h.numpy())
    assert np.array_equal(og.bf16_to_f64(out["conv_state"]), C_all.numpy())
    got_S = og.bf16_to_f64(out["ssm_state"]) if bf16_state else out["ssm_state"].astype(np.float64)
    ref_S = og.bf16_to_f64(og.f64_to_bf16(S_all.numpy())) if bf16_state \
        else S_all.numpy().astype(np.float32).astype(np.float64)
    assert np.allclose(got_S, ref_S, rtol=0, atol=1e-7 if not bf16_state else 0)


def test_normed_input_equals_the_block_from_its_norm_output():
    """The "normed" variant ("SGLang PR #43558", Modifications): fed the xn the full block
    computes from (x, residual), it gives the same core and state bit for bit, and
    returns no residual."""
    shape = configs.TINY.with_(num_state_slots=12, pad_rows=True, rows=(6,))
    w = synth.make_weights(shape, 90)
    call = synth.make_call(shape, 6, 90)
    full = run_oracle(shape, w, call)
    normed_call = synth.GdnCall(from_u16(full["xn"]), call.residual, call.conv_state, call.ssm_state,
                                call.state_idx)
    normed = run_oracle(shape.with_(input_normed=True, has_residual=False), w, normed_call)
    assert normed["residual"] is None
    for k in ("core", "conv_state", "ssm_state", "y_qkvz", "y_ba"):
        assert np.array_equal(normed[k], full[k]), k


# ----------------------------------------------------------------------------------------
# verify: several tokens per sequence, the state after each kept


def _verify_inputs(shape, R, T, seed):
    """R sequences of T tokens: sources 1..R (sequence 1 a pad), destinations from a
    disjoint range, one snapshot not kept, and sequence 0 continuing in its own slot."""
    call = synth.make_call(shape, R * T, seed)
    src = np.arange(1, R + 1, dtype=np.int32)
    src[1] = -1
    dst = (R + 1 + np.arange(R * T, dtype=np.int32)).reshape(R, T)
    dst[0, T - 1] = src[0]
    dst[2, 0] = 0
    return call, src, dst


def _library_verify(shape, w, call, src, dst):
    """Verify composed from torch float64 library routines: the front row by row as in
    _library_block, then per sequence conv1d over [old window; the tokens] at once and the
    delta rule carried across the tokens unrounded."""
    import torch
    import torch.nn.functional as F
    rb = lambda t: torch.from_numpy(og.bf16_to_f64(og.f64_to_bf16(t.numpy())))  # noqa: E731
    d = lambda t: t.double()                                                    # noqa: E731
    nk, dk, nv, dv, r = shape.num_k_heads, shape.head_k_dim, shape.num_v_heads, shape.head_v_dim, \
        shape.heads_per_group
    R, T = dst.shape
    h = rb(d(call.x) + d(call.residual)) if shape.has_residual else d(call.x)
    xn = rb(F.rms_norm(h, (shape.hidden,), weight=1 + d(w.norm_w), eps=shape.norm_eps))
    yq = rb(xn @ d(w.w_qkvz).T).reshape(-1, nk, shape.group_width)
    yb = rb(xn @ d(w.w_ba).T).reshape(-1, nk, 2 * r)
    q, k = yq[..., :dk], yq[..., dk:2 * dk]
    v = yq[..., 2 * dk:2 * dk + r * dv].reshape(-1, nv, dv)
    z = yq[..., 2 * dk + r * dv:].reshape(-1, nv, dv)
    b, a = yb[..., :r].reshape(-1, nv), yb[..., r:].reshape(-1, nv)
    qkv = torch.cat([q.reshape(-1, nk * dk), k.reshape(-1, nk * dk), v.reshape(-1, nv * dv)], -1)
    S_pool = d(call.ssm_state).clone()
    C_pool = d(call.conv_state).clone()
    core = torch.zeros(R * T, nv * dv, dtype=torch.float64)
    bf16_state = shape.ssm_state_dtype == "bf16"
    for s_, slot in enumerate(src.tolist()):
        if slot <= 0:
            continue
        rows = slice(s_ * T, (s_ + 1) * T)
        seq = torch.cat([d(call.conv_state)[slot], qkv[rows]], 0)           # [W-1+T, Cd]
        conv = F.conv1d(seq.T[None], d(w.conv_w)[:, None, :], groups=shape.conv_dim)[0].T   # [T, Cd]
        c = rb(F.silu(conv))
        S = d(call.ssm_state)[slot].clone()                                  # [nv, dk, dv]
        for t in range(T):
            row = s_ * T + t
            cq_raw = c[t, :nk * dk].reshape(nk, dk)
            ck_raw = c[t, nk * dk:2 * nk * dk].reshape(nk, dk)
            cq = cq_raw / (cq_raw.square().sum(-1, keepdim=True) + shape.l2norm_eps).sqrt() / dk ** 0.5
            ck = ck_raw / (ck_raw.square().sum(-1, keepdim=True) + shape.l2norm_eps).sqrt()
            cv = c[t, 2 * nk * dk:].reshape(nv, dv)
            g = -torch.exp(d(w.A_log)) * F.softplus(a[row] + d(w.dt_bias))
            beta = torch.sigmoid(b[row])
            for hv in range(nv):
                kk, qq = ck[hv // r], cq[hv // r]
                Sh = torch.exp(g[hv]) * S[hv]
                S[hv] = Sh + torch.outer(kk, beta[hv] * (cv[hv] - Sh.T @ kk))
                o = rb(S[hv].T @ qq)
                core[row, hv * dv:(hv + 1) * dv] = rb(
                    F.rms_norm(o, (dv,), weight=d(w.gated_norm_w), eps=shape.gated_norm_eps) * F.silu(z[row, hv]))
            dslot = int(dst[s_, t])
            if 0 < dslot < shape.num_state_slots:
                C_pool[dslot] = seq[t + 1:t + shape.conv_width]
                S_pool[dslot] = rb(S) if bf16_state else S.float().double()
    return core, S_pool, C_pool


@pytest.mark.parametrize("bf16_state", [False, True])
def test_verify_against_library_composition(bf16_state):
    shape = configs.TINY.with_(num_state_slots=24, ssm_state_dtype="bf16" if bf16_state else "f32")
    R, T = 4, 3
    w = synth.make_weights(shape, 12)
    call, src, dst = _verify_inputs(shape, R, T, 12)
    out = og.verify_block(oracle_cfg(shape), oracle_weights(w), u16(call.x), u16(call.residual),
                          u16(call.conv_state), oracle_state(call.ssm_state), src, dst)
    core, S_pool, C_pool = _library_verify(shape, w, call, src, dst)
    assert np.array_equal(og.bf16_to_f64(out["core"]), core.numpy())
    assert np.array_equal(og.bf16_to_f64(out["conv_state"]), C_pool.numpy())
    got_S = og.bf16_to_f64(out["ssm_state"]) if bf16_state else out["ssm_state"].astype(np.float64)
    assert np.allclose(got_S, S_pool.numpy(), rtol=0, atol=1e-7 if not bf16_state else 0)


def test_verify_one_token_is_a_decode_step():
    """tokens = 1 with each sequence's destination its own source is decode_block, bit for bit."""
    shape = configs.TINY.with_(num_state_slots=10, pad_rows=True)
    w = synth.make_weights(shape, 13)
    call = synth.make_call(shape, 5, 13)
    src = call.state_idx.numpy().copy()
    dec = run_oracle(shape, w, call)
    ver = og.verify_block(oracle_cfg(shape), oracle_weights(w), u16(call.x), u16(call.residual),
                          u16(call.conv_state), oracle_state(call.ssm_state), src, src[:, None])
    for k in ("core", "residual", "conv_state", "ssm_state"):
        assert np.array_equal(ver[k], dec[k]), k


def test_verify_keeps_only_the_named_snapshots():
    """Pad sequences and unkept snapshots write nothing; every slot not named as a valid
    destination keeps its bits; a pad sequence's core rows are +0."""
    shape = configs.TINY.with_(num_state_slots=24)
    R, T = 4, 3
    w = synth.make_weights(shape, 14)
    call, src, dst = _verify_inputs(shape, R, T, 14)
    out = og.verify_block(oracle_cfg(shape), oracle_weights(w), u16(call.x), u16(call.residual),
                          u16(call.conv_state), oracle_state(call.ssm_state), src, dst)
    written = set(int(s) for s in dst.reshape(-1) if 0 < s < shape.num_state_slots)
    for slot in range(shape.num_state_slots):
        if slot not in written:
            assert np.array_equal(out["conv_state"][slot], u16(call.conv_state)[slot]), slot
            assert np.array_equal(out["ssm_state"][slot], oracle_state(call.ssm_state)[slot]), slot
    assert np.all(out["core"][1 * T:2 * T] == 0)
    assert np.any(out["core"][0] != 0)


def test_verify_chain_of_decodes_with_f32_state():
    """With an f32 pool, T tokens in one verify step end where T decode steps end (the
    state is carried unrounded inside the step, rounded to f32 between decode steps)."""
    shape = configs.TINY.with_(num_state_slots=24)
    R, T = 3, 4
    w = synth.make_weights(shape, 15)
    call, src, dst = _verify_inputs(shape, R, T, 15)
    src[1] = 2  # no pad here
    dst[2, 0] = R + 1 + 2 * T
    ver = og.verify_block(oracle_cfg(shape), oracle_weights(w), u16(call.x), u16(call.residual),
                          u16(call.conv_state), oracle_state(call.ssm_state), src, dst)
    conv, ssm = u16(call.conv_state), oracle_state(call.ssm_state)
    slots = src.copy()
    for t in range(T):
        rows = np.arange(R) * T + t
        dec = og.decode_block(oracle_cfg(shape), oracle_weights(w), u16(call.x)[rows], u16(call.residual)[rows],
                              conv, ssm, slots)
        assert np.array_equal(dec["core"], ver["core"][rows]), t
        conv, ssm = dec["conv_state"], dec["ssm_state"]
        for s_ in range(R):   # move each sequence's state to its destination slot
            conv[dst[s_, t]] = conv[slots[s_]]
            ssm[dst[s_, t]] = ssm[slots[s_]]
        slots = dst[:, t].copy()
    for s_ in range(R):
        assert np.array_equal(ver["conv_state"][dst[s_, T - 1]], conv[dst[s_, T - 1]])
        assert np.allclose(ver["ssm_state"][dst[s_, T - 1]], ssm[dst[s_, T - 1]], rtol=0, atol=1e-6)
