"""Pins of the CPU oracle against things other than itself.

Each test checks an oracle step against an independent fact: a library
routine on a special case (torch's bf16 cast, rms_norm, conv1d, softplus),
exact integer arithmetic, a closed form, a brute-force unrolled product, or a
hand-worked fixture under tests/golden/. They are chosen so that a plausible
slip in the oracle (a dropped term, a wrong sign or index, a transposed
operand, a rounding taken twice) fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import gdn as og
from tests.helpers import from_u16, u16

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ----------------------------------------------------------------------------------------
# bf16 storage


def test_bf16_rounding_matches_torch_on_f32_inputs():
    rng = np.random.default_rng(0)
    v = np.concatenate([
        rng.normal(0, 1, 20000),
        rng.normal(0, 1, 5000) * np.exp2(rng.integers(-140, 120, 5000)),
        [0.0, -0.0, 1.0, -1.0, 2.0 ** -126, 2.0 ** -130, -(2.0 ** -133), 3.0e38],
    ]).astype(np.float32)
    expect = u16(torch.from_numpy(v).to(torch.bfloat16))
    got = og.f64_to_bf16(v.astype(np.float64))
    assert np.array_equal(got, expect)


def test_bf16_ties_to_even_and_single_rounding():
    one = 1.0
    ulp = 2.0 ** -7
    # exactly halfway: ties go to the even significand
    assert og.f64_to_bf16(one + ulp / 2) == 0x3F80           # -> 1.0
    assert og.f64_to_bf16(one + 3 * ulp / 2) == 0x3F82       # -> 1 + 2 ulp
    # just above halfway in f64 but below f32's resolution: a detour through
    # f32 would land on the tie and round down; one rounding goes up
    v = one + ulp / 2 + 2.0 ** -30
    assert np.float32(v) == np.float32(one + ulp / 2)
    assert og.f64_to_bf16(v) == 0x3F81
    assert og.f64_to_bf16(-(one + ulp / 2 + 2.0 ** -30)) == 0xBF81


def test_bf16_widening_known_patterns():
    got = og.bf16_to_f64(np.array([0x3F80, 0xC000, 0x0001, 0x7F7F, 0x8000], dtype=np.uint16))
    assert got[0] == 1.0 and got[1] == -2.0 and got[2] == 2.0 ** -133
    assert got[3] == (2 - 2.0 ** -7) * 2.0 ** 127
    assert got[4] == 0.0 and math.copysign(1, got[4]) < 0


# ----------------------------------------------------------------------------------------
# residual add and Gemma RMSNorm


def test_residual_add_equals_bf16_sum():
    rng = np.random.default_rng(1)
    x = torch.from_numpy(rng.normal(0, 1, (3, 512)).astype(np.float32)).to(torch.bfloat16)
    r = torch.from_numpy(rng.normal(0, 3, (3, 512)).astype(np.float32)).to(torch.bfloat16)
    expect = u16((x.float() + r.float()).to(torch.bfloat16))
    assert np.array_equal(og.residual_add(u16(x), u16(r), True), expect)
    # the layer without a residual input passes x through
    assert np.array_equal(og.residual_add(u16(x), u16(r), False), u16(x))


def test_gemma_norm_reduces_to_rms_norm_when_weight_is_zero():
    rng = np.random.default_rng(2)
    h = torch.from_numpy(rng.normal(0, 1, (4, 384)).astype(np.float32)).to(torch.bfloat16)
    w0 = torch.zeros(384, dtype=torch.bfloat16)
    got = og.gemma_rmsnorm(u16(h), u16(w0), 1e-6)
    ref = F.rms_norm(h.double(), (384,), eps=1e-6).numpy()
    assert np.array_equal(got, og.f64_to_bf16(ref))


def test_gemma_norm_scales_by_one_plus_weight():
    rng = np.random.default_rng(3)
    h = torch.from_numpy(rng.normal(0, 1, (2, 256)).astype(np.float32)).to(torch.bfloat16)
    base = og.bf16_to_f64(og.gemma_rmsnorm(u16(h), u16(torch.zeros(256, dtype=torch.bfloat16)), 1e-6))
    ones = og.bf16_to_f64(og.gemma_rmsnorm(u16(h), u16(torch.ones(256, dtype=torch.bfloat16)), 1e-6))
    assert np.array_equal(ones, 2.0 * base)          # (1 + 1) doubles exactly
    neg = og.bf16_to_f64(og.gemma_rmsnorm(u16(h), u16(-torch.ones(256, dtype=torch.bfloat16)), 1e-6))
    assert np.all(neg == 0.0)                          # (1 - 1) zeroes


def test_gemma_norm_constant_row_closed_form():
    for c in (0.5, -3.0, 1e-3):
        h = torch.full((1, 64), c).to(torch.bfloat16)
        cb = float(h[0, 0])
        got = og.bf16_to_f64(og.gemma_rmsnorm(u16(h), u16(torch.zeros(64, dtype=torch.bfloat16)), 1e-6))
        expect = og.bf16_to_f64(og.f64_to_bf16(np.sign(cb) / math.sqrt(1 + 1e-6 / cb ** 2)))
        assert np.all(got == expect)


# ----------------------------------------------------------------------------------------
# projections


def test_bf16_projection_exact_on_small_integers():
    rng = np.random.default_rng(4)
    W = rng.integers(-2, 3, (40, 64))
    X = rng.integers(-2, 3, (3, 64))
    Wb = u16(torch.from_numpy(W.astype(np.float32)).to(torch.bfloat16))
    Xb = u16(torch.from_numpy(X.astype(np.float32)).to(torch.bfloat16))
    got = og.bf16_to_f64(og.project_bf16(Wb, Xb))
    assert got.shape == (3, 40)
    assert np.array_equal(got, (X @ W.T).astype(np.float64))   # |sum| <= 256: exact in bf16


def test_bf16_projection_one_hot_rows_select_inputs():
    rng = np.random.default_rng(5)
    H, N = 128, 24
    cols = rng.integers(0, H, N)
    W = np.zeros((N, H), dtype=np.float32)
    W[np.arange(N), cols] = 1.0
    X = torch.from_numpy(rng.normal(0, 1, (2, H)).astype(np.float32)).to(torch.bfloat16)
    got = og.project_bf16(u16(torch.from_numpy(W).to(torch.bfloat16)), u16(X))
    assert np.array_equal(got, u16(X)[:, cols])


def test_bf16_projection_single_rounding_of_exact_sum():
    # terms whose exact sum needs many more than 24 bits: a large value, its
    # negation and small ones (the pages' "bf16(fp32(exact sum))" check)
    W = np.zeros((1, 64), dtype=np.float32)
    W[0, :4] = 1.0
    X = np.zeros((1, 64), dtype=np.float32)
    X[0, :4] = [2.0 ** 20, 1.0, -(2.0 ** 20), 2.0 ** -10]
    got = og.bf16_to_f64(og.project_bf16(u16(torch.from_numpy(W).to(torch.bfloat16)),
                                         u16(torch.from_numpy(X).to(torch.bfloat16))))
    assert got[0, 0] == 1.0 + 0.0  # 1 + 2^-10 rounds to 1 in bf16


@pytest.mark.parametrize("rule", ["rounded_max", "ceil"])
def test_mxfp4_hand_worked_blocks(rule):
    fx = _golden("mxfp4_blocks.json")["rules"][rule]
    for blk in fx["blocks"]:
        v = np.zeros(32)
        for i, val in blk["values"].items():
            v[int(i)] = val
        codes, scales = og.mxfp4_quantize(v, rule)
        assert int(scales[0]) == blk["scale_byte"], blk["note"]
        want = np.zeros(32, dtype=np.uint8)
        for i, c in blk["codes"].items():
            want[int(i)] = c
        assert np.array_equal(codes, want), blk["note"]


def test_mxfp4_scale_rules_differ_only_between_1_5_and_1_75():
    """With the block maximum M 2^E (1 <= M < 2): both rules give E - 2 for M <= 1.5 and
    E - 1 for M >= 1.75; between, the rounded maximum stays at E - 2 (its elements round
    down to 6) while the ceiling moves up, so no element passes 6 times the scale."""
    rng = np.random.default_rng(11)
    E = rng.integers(-100, 100, 4000)
    M = np.concatenate([rng.uniform(1.0, 2.0, 3000), [1.0, 1.5, 1.75, 1.9921875] * 250])
    amax = M * np.exp2(E.astype(np.float64))
    er = og.mx_block_exponent(amax, 1, "rounded_max")
    ec = og.mx_block_exponent(amax, 1, "ceil")
    assert np.array_equal(er, E - 2 + (M >= 1.75))
    assert np.array_equal(ec, E - 2 + (M > 1.5))
    assert np.all(amax <= 6.0 * np.exp2(ec.astype(np.float64)))
    assert np.all(amax < 7.0 * np.exp2(er.astype(np.float64)))
    # E2M3's three mantissa bits: a carry exactly from 1.1111b (the MXFP6 weights' rule)
    e3 = og.mx_block_exponent(amax, 3, "rounded_max")
    assert np.array_equal(e3, E - 2 + (M >= 1.9375))


@pytest.mark.parametrize("rule", ["rounded_max", "ceil"])
def test_mxfp4_round_trip_on_representable_blocks(rule):
    rng = np.random.default_rng(6)
    codes = rng.integers(0, 16, (5, 64)).astype(np.uint8)
    codes[:, 0] = 7                                # every block reaches 6 * 2^e
    codes[:, 32] = 15
    codes[codes == 8] = 0                          # -0 quantises to +0
    scales = rng.integers(100, 140, (5, 2)).astype(np.uint8)
    v = og.mxfp4_dequantize(codes, scales)
    c2, s2 = og.mxfp4_quantize(v, rule)
    assert np.array_equal(c2, codes) and np.array_equal(s2, scales)


def test_mxfp4_projection_exact_against_integer_arithmetic():
    rng = np.random.default_rng(7)
    N, H = 6, 64
    wcodes = rng.integers(0, 16, (N, H)).astype(np.uint8)
    wscales = np.full((N, H // 32), 127, dtype=np.uint8)       # scale 1
    packed = (wcodes[:, 0::2] | (wcodes[:, 1::2] << 4)).astype(np.uint8)
    # activations already on the e2m1 grid with block max 6: quantisation is the identity
    acodes = rng.integers(0, 16, (2, H)).astype(np.uint8)
    acodes[:, 0] = 7
    acodes[:, 32] = 7
    acodes[acodes == 8] = 0
    xa = og.mxfp4_dequantize(acodes, np.full((2, 2), 127, np.uint8))
    xb = u16(torch.from_numpy(xa.astype(np.float32)).to(torch.bfloat16))
    got = og.bf16_to_f64(og.project_mxfp4(packed, wscales, xb))
    # integer reference: e2m1 values are multiples of 1/2
    tab2 = np.array([0, 1, 2, 3, 4, 6, 8, 12])
    wi = np.where(wcodes & 8, -1, 1) * tab2[wcodes & 7]
    ai = np.where(acodes & 8, -1, 1) * tab2[acodes & 7]
    exact = (ai @ wi.T) / 4.0
    assert np.array_equal(got, og.bf16_to_f64(og.f64_to_bf16(exact)))


def test_e2m3_table_ocp_facts():
    """OCP E2M3: largest magnitude 7.5 (code 0x1F), smallest subnormal 1/8 (0x01), smallest
    normal 1 (0x08), steps 1/8 below 2, 1/4 below 4, 1/2 up to 7.5, sign at bit 5."""
    t = og.E2M3_VALUES
    assert len(t) == 32 and t[0x1F] == 7.5 and t[0x01] == 0.125 and t[0x08] == 1.0
    assert np.all(np.diff(t) > 0)
    assert np.all(np.diff(t[:17]) == 0.125) and np.all(np.diff(t[16:25]) == 0.25) and np.all(np.diff(t[24:]) == 0.5)
    v = og.mxfp6_dequantize(np.array([0x21, 0x3F, 0x20, 0x08], np.uint8).repeat(8), np.array([127], np.uint8))
    assert v[0] == -0.125 and v[8] == -7.5 and v[16] == 0.0 and v[24] == 1.0


def test_mxfp6_hand_worked_blocks():
    fx = _golden("mxfp6_blocks.json")
    for blk in fx["blocks"]:
        v = np.zeros(32)
        for i, val in blk["values"].items():
            v[int(i)] = float.fromhex(val) if isinstance(val, str) else val
        codes, scales = og.mxfp6_round(v)
        assert int(scales[0]) == blk["scale_byte"], blk["note"]
        want = np.zeros(32, dtype=np.uint8)
        for i, c in blk["codes"].items():
            want[int(i)] = c
        assert np.array_equal(codes, want), blk["note"]


def test_mxfp6_round_trip_on_representable_blocks():
    """A block whose largest magnitude lies in the top binade (4 .. 7.5 times its scale)
    rounds back to itself: the scale is recovered and every value is on the grid."""
    rng = np.random.default_rng(16)
    codes = rng.integers(0, 64, (6, 96)).astype(np.uint8)
    codes[:, [0, 32, 64]] = rng.integers(24, 32, (6, 3))    # a top-binade maximum per block
    codes[:, 1:32] &= 0x37                                   # the others at most 3.75 ... 7.5
    codes[codes == 0x20] = 0                                 # -0 rounds to +0
    scales = rng.integers(100, 140, (6, 3)).astype(np.uint8)
    v = og.mxfp6_dequantize(codes, scales)
    c2, s2 = og.mxfp6_round(v)
    assert np.array_equal(s2, scales) and np.array_equal(c2, codes)


def test_e2m3_packing_bit_positions():
    """Code i of a block sits at bits 6i .. 6i+5 of its 24 bytes, little-endian."""
    c = np.zeros(32, np.uint8)
    c[0] = 1
    assert og.pack_e2m3(c)[0].tolist() == [1] + [0] * 23
    c[:] = 0
    c[1] = 1                       # bit 6
    assert og.pack_e2m3(c)[0].tolist() == [0x40] + [0] * 23
    c[:] = 0
    c[31] = 63                     # bits 186 .. 191: the top 6 bits of byte 23
    assert og.pack_e2m3(c)[0].tolist() == [0] * 23 + [0xFC]
    c[:] = 0
    c[4] = 0x2B                    # bits 24 .. 29: byte 3 = 0x2B
    c[5] = 0x15                    # bits 30 .. 35: 0b010101 -> byte 3 bits 6,7 = 01, byte 4 = 0101
    p = og.pack_e2m3(c)[0]
    assert p[3] == (0x2B | (0x1 << 6)) and p[4] == 0x5
    rng = np.random.default_rng(3)
    codes = rng.integers(0, 64, (4, 128)).astype(np.uint8)
    assert np.array_equal(og.unpack_e2m3(og.pack_e2m3(codes)), codes)


def test_mxfp6_projection_exact_against_integer_arithmetic():
    """E2M3 values are multiples of 1/8: with scale 2^0 and small integer activations the
    projection is an integer sum divided by 8, rounded once."""
    rng = np.random.default_rng(17)
    N, H = 5, 96
    wcodes = rng.integers(0, 64, (N, H)).astype(np.uint8)
    wscales = np.full((N, H // 32), 127, dtype=np.uint8)
    xi = rng.integers(-8, 9, (3, H))
    xb = og.f64_to_bf16(xi.astype(np.float64))
    got = og.bf16_to_f64(og.project_mxfp6(og.pack_e2m3(wcodes), wscales, xb))
    mag8 = np.array([m for m in range(8)] + [(8 + m) << (e - 1) for e in range(1, 4) for m in range(8)])
    wi = np.where(wcodes & 32, -1, 1) * mag8[wcodes & 31]
    exact = (xi @ wi.T) / 8.0
    assert np.array_equal(got, og.bf16_to_f64(og.f64_to_bf16(exact)))
    # a scale byte b multiplies by 2^(b - 127), per block of 32
    ws2 = wscales.copy()
    ws2[:, 1] = 130
    got2 = og.bf16_to_f64(og.project_mxfp6(og.pack_e2m3(wcodes), ws2, xb))
    f = np.ones(H)
    f[32:64] = 8.0
    exact2 = (xi @ (wi * f).T) / 8.0
    assert np.array_equal(got2, og.bf16_to_f64(og.f64_to_bf16(exact2)))


# ----------------------------------------------------------------------------------------
# split


def test_split_layout_fixture():
    fx = _golden("split_tiny.json")
    s = fx["shape"]
    q, k, v, z = og.split_qkvz(np.array(fx["y_qkvz"]), s["nk"], s["dk"], s["nv"], s["dv"])
    assert np.array_equal(q, fx["q"]) and np.array_equal(k, fx["k"])
    assert np.array_equal(v, fx["v"]) and np.array_equal(z, fx["z"])
    b, a = og.split_ba(np.array(fx["y_ba"]), s["nk"], s["nv"])
    assert np.array_equal(b, fx["b"]) and np.array_equal(a, fx["a"])


# ----------------------------------------------------------------------------------------
# conv


def _bf(a):
    return u16(torch.from_numpy(np.asarray(a, dtype=np.float32)).to(torch.bfloat16))


def test_conv_one_hot_taps():
    rng = np.random.default_rng(8)
    C, W = 16, 4
    state = _bf(rng.normal(0, 1, (W - 1, C)))
    new = _bf(rng.normal(0, 1, C))
    w_new = np.zeros((C, W), np.float32)
    w_new[:, W - 1] = 1.0
    out, st = og.conv_update(state, new, _bf(w_new))
    assert np.array_equal(out, og.f64_to_bf16(F.silu(from_u16(new).double()).numpy()))
    w_old = np.zeros((C, W), np.float32)
    w_old[:, 0] = 1.0
    out0, _ = og.conv_update(state, new, _bf(w_old))
    assert np.array_equal(out0, og.f64_to_bf16(F.silu(from_u16(state[0]).double()).numpy()))
    # the state keeps the last W-1 raw inputs, oldest first
    assert np.array_equal(st, np.concatenate([state[1:], new[None]]))


def test_conv_steps_equal_causal_conv1d():
    rng = np.random.default_rng(9)
    C, W, T = 12, 4, 9
    xs = _bf(rng.normal(0, 1, (T, C)))
    w = _bf(rng.normal(0, 0.5, (C, W)))
    state = np.zeros((W - 1, C), np.uint16)
    outs = []
    for t in range(T):
        o, state = og.conv_update(state, xs[t], w)
        outs.append(o)
    xt = from_u16(xs).double().T[None]                       # [1, C, T]
    wt = from_u16(w).double()[:, None, :]                     # [C, 1, W]
    ref = F.conv1d(F.pad(xt, (W - 1, 0)), wt, groups=C)[0].T  # causal, depthwise
    assert np.array_equal(np.array(outs), og.f64_to_bf16(F.silu(ref).numpy()))
    assert np.array_equal(state, xs[-(W - 1):])


# ----------------------------------------------------------------------------------------
# gates and L2 norm


def test_gates_closed_forms_and_library():
    A_log = np.array([0.0, 0.7, 1.9])
    g, beta = og.gates(np.array([0.25, -1.0, 3.0]), np.zeros(3), A_log, np.array([-0.25, 1.0, -3.0]))
    assert np.allclose(g, -np.exp(A_log) * math.log(2.0), rtol=0, atol=1e-15)
    assert np.all(beta == 0.5)
    x = np.linspace(-30, 30, 241)
    assert np.allclose(og.softplus(x), F.softplus(torch.from_numpy(x)).numpy(), rtol=1e-15, atol=0)
    assert np.allclose(og.sigmoid(x), torch.sigmoid(torch.from_numpy(x)).numpy(), rtol=1e-15, atol=0)
    # decay is in (0, 1]: g <= 0 for every input
    gg, _ = og.gates(np.linspace(-40, 40, 50), np.zeros(50), np.full(50, 1.0), np.zeros(50))
    assert np.all(gg <= 0)


def test_l2norm_library_and_eps():
    rng = np.random.default_rng(10)
    x = rng.normal(0, 1, (5, 128))
    assert np.allclose(og.l2norm(x, 0.0), F.normalize(torch.from_numpy(x), dim=-1).numpy(),
                       rtol=0, atol=1e-15)
    assert np.allclose(np.linalg.norm(og.l2norm(x, 1e-6), axis=-1), 1.0, atol=1e-6)
    c = np.full(16, 0.01)
    assert np.allclose(og.l2norm(c, 1e-6), 0.01 / math.sqrt(16 * 1e-4 + 1e-6), rtol=1e-15)


# ----------------------------------------------------------------------------------------
# the gated delta rule


def _unit(v):
    return v / np.linalg.norm(v)


def test_delta_rule_hand_worked_fixture():
    fx = _golden("gated_delta_2x2.json")
    S = np.array(fx["S0"])
    for st in fx["steps"]:
        S, o = og.gated_delta_step(S, np.array(st["q"]), np.array(st["k"]), np.array(st["v"]),
                                   st["g"], st["beta"])
        assert np.allclose(o, st["o"], rtol=0, atol=1e-15)
    assert np.allclose(S, fx["S_final"], rtol=0, atol=1e-15)


def test_delta_rule_identity_when_beta_and_g_are_zero():
    rng = np.random.default_rng(11)
    S = rng.normal(0, 1, (8, 6))
    q, k, v = rng.normal(size=8), _unit(rng.normal(size=8)), rng.normal(size=6)
    S2, o = og.gated_delta_step(S, q, k, v, 0.0, 0.0)
    assert np.array_equal(S2, S)
    assert np.allclose(o, (torch.from_numpy(S).T @ torch.from_numpy(q)).numpy(), rtol=1e-14, atol=1e-14)


def test_delta_rule_full_decay_resets_state():
    rng = np.random.default_rng(12)
    S = rng.normal(0, 1, (8, 6))
    q, k, v = rng.normal(size=8), _unit(rng.normal(size=8)), rng.normal(size=6)
    S2, o = og.gated_delta_step(S, q, k, v, -np.inf, 0.3)
    assert np.allclose(S2, 0.3 * np.outer(k, v), rtol=0, atol=1e-15)
    assert np.allclose(o, 0.3 * v * (k @ q), rtol=0, atol=1e-14)


def test_delta_rule_rank_one_write_on_empty_state():
    rng = np.random.default_rng(13)
    k = _unit(rng.normal(size=6))
    q = rng.normal(size=6)
    S2, o = og.gated_delta_step(np.zeros((6, 6)), q, k, k.copy(), 0.0, 1.0)
    assert np.allclose(S2, np.outer(k, k), rtol=0, atol=1e-15)
    assert np.allclose(o, k * (k @ q), rtol=0, atol=1e-15)


def test_delta_rule_write_property():
    # with a unit key, the updated state reads back (1-beta) of the decayed
    # state's reading plus beta of the new value
    rng = np.random.default_rng(14)
    for _ in range(20):
        S = rng.normal(0, 1, (7, 5))
        k, q, v = _unit(rng.normal(size=7)), rng.normal(size=7), rng.normal(size=5)
        g, beta = -abs(rng.normal()), rng.uniform()
        S2, _ = og.gated_delta_step(S, q, k, v, g, beta)
        assert np.allclose(S2.T @ k, (1 - beta) * (math.exp(g) * S).T @ k + beta * v, atol=1e-12)


def test_delta_rule_matches_unrolled_products():
    # S_T = A_T..A_1 S_0 + sum_t A_T..A_{t+1} beta_t k_t v_t^T, A_t = e^{g_t} (I - beta_t k_t k_t^T)
    rng = np.random.default_rng(15)
    for dk, dv, T in ((4, 3, 5), (8, 8, 8), (2, 5, 3)):
        S0 = rng.normal(0, 1, (dk, dv))
        ks = [_unit(rng.normal(size=dk)) for _ in range(T)]
        qs = [rng.normal(size=dk) for _ in range(T)]
        vs = [rng.normal(size=dv) for _ in range(T)]
        gs = [-abs(rng.normal()) for _ in range(T)]
        bs = [rng.uniform() for _ in range(T)]
        A = [math.exp(g) * (np.eye(dk) - b * np.outer(k, k)) for g, b, k in zip(gs, bs, ks)]

        def prod(lo, hi):           # A_hi ... A_lo (1-based, inclusive); identity when empty
            P = np.eye(dk)
            for t in range(lo, hi + 1):
                P = A[t - 1] @ P
            return P

        S_T, outs = og.gated_delta_recurrence(S0, qs, ks, vs, gs, bs)
        brute = prod(1, T) @ S0 + sum(prod(t + 1, T) @ (bs[t - 1] * np.outer(ks[t - 1], vs[t - 1]))
                                      for t in range(1, T + 1))
        assert np.allclose(S_T, brute, atol=1e-12)
        for t in range(1, T + 1):
            St = prod(1, t) @ S0 + sum(prod(j + 1, t) @ (bs[j - 1] * np.outer(ks[j - 1], vs[j - 1]))
                                       for j in range(1, t + 1))
            assert np.allclose(outs[t - 1], St.T @ qs[t - 1], atol=1e-12)


# ----------------------------------------------------------------------------------------
# gated RMSNorm


def test_gated_norm_library_special_case():
    rng = np.random.default_rng(16)
    o = _bf(rng.normal(0, 1, (3, 64)))
    z = _bf(rng.normal(0, 1, (3, 64)))
    w = _bf(rng.normal(1, 0.1, 64))
    got = og.gated_rmsnorm(o, z, w, 1e-6)
    ref = F.rms_norm(from_u16(o).double(), (64,), weight=from_u16(w).double(), eps=1e-6) \
        * F.silu(from_u16(z).double())
    assert np.array_equal(got, og.f64_to_bf16(ref.numpy()))


def test_gated_norm_constant_head_and_zero_gate():
    z = _bf(np.linspace(-2, 2, 32))
    w = _bf(np.full(32, 0.5))
    o = _bf(np.full(32, -0.75))
    got = og.bf16_to_f64(og.gated_rmsnorm(o, z, w, 1e-6))
    zf = og.bf16_to_f64(z)
    expect = og.bf16_to_f64(og.f64_to_bf16(-1.0 / math.sqrt(1 + 1e-6 / 0.75 ** 2) * 0.5 * zf / (1 + np.exp(-zf))))
    assert np.array_equal(got, expect)
    zero = og.gated_rmsnorm(_bf(np.linspace(-1, 1, 32)), _bf(np.zeros(32)), w, 1e-6)
    assert np.all(og.bf16_to_f64(zero) == 0.0)


def test_pow2_rows_have_an_exact_norm():
    """The exact-activation rows of the MXFP4 GPU tests: the oracle's norm (weight 0,
    eps 1e-6) returns h * 2^-j bit for bit, and its MXFP4 image is the exact one."""
    from tests.helpers import pow2_rows
    for hidden in (512, 8192):
        x, xn_exact = pow2_rows(hidden, 3, 5)
        bits = og.f64_to_bf16(x)
        assert np.array_equal(og.bf16_to_f64(bits), x)  # representable in bf16
        xn = og.gemma_rmsnorm(bits, og.f64_to_bf16(np.zeros(hidden)), 1e-6)
        assert np.array_equal(og.bf16_to_f64(xn), xn_exact)
        codes, scales = og.mxfp4_quantize(xn_exact)
        # powers of two at most 4 steps below the block maximum are exact in e2m1 (0.25 x
        # the maximum's code value rounds to 0 as a tie to even)
        deq = og.mxfp4_dequantize(codes, scales)
        blocks = np.abs(xn_exact).reshape(3, -1, 32).max(axis=-1)
        small = np.abs(xn_exact) < np.repeat(blocks, 32, axis=-1) / 8
        assert np.array_equal(deq[~small], xn_exact[~small])
