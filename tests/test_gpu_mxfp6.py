"""GPU parity of the MXFP6 E2M3 in_proj_qkvz path (W6A16: "vLLM PR #60833", a reviewer's
comment proposing MXFP6 for the GDN projections; E2M3 weights with one e8m0 scale per 32
along K, converted to bf16 exactly and multiplied with the bf16 activations).

* The weight rounding alone (gdn_mxfp6_round_weights) against the oracle's mxfp6_round,
  bit for bit, on blocks built to hit its cases: the carry of the block maximum into the
  next binade, ties in every binade, the exponent clamp, zero, negative-zero and subnormal
  blocks, one-ulp neighbours of every rounding boundary, random bit patterns.
* Whole decodes. The activations are not quantised, so GPU and oracle multiply the same
  weight values by xn and the strict element rule applies; row-major and tiled weights
  agree bit for bit (parity_case).
* Weights made on the device from bf16 by the pages' recipe, then decoded.
"""
import numpy as np
import pytest
import torch

from gated_deltanet_linear_decode_amd import abi, configs, synth
from oracle import gdn as og
from tests.gpu_util import note, parity_case
from tests.helpers import from_u16

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

TINY_MX6 = configs.GdnShape(
    "tiny_mxfp6", hidden=512, num_k_heads=2, head_k_dim=32, num_v_heads=4, head_v_dim=32,
    num_state_slots=24, ssm_state_dtype="f32", has_residual=True, qkvz_format="mxfp6",
    rows=(16,), pad_rows=True)


def _rounding_inputs(cols, seed):
    """bf16 bit patterns [8, cols] covering the weight rounding's cases."""
    rng = np.random.Generator(np.random.PCG64(seed))
    nb = cols // 32
    rows = [og.f64_to_bf16(rng.normal(0, 0.02, cols))]
    scale = np.repeat(np.exp2(rng.integers(-135, 120, nb).astype(np.float64)), 32)
    rows.append(og.f64_to_bf16(rng.normal(0, 1, cols) * scale))
    # ties in every binade, each block anchored at 7.5 * 2^e (scale 2^e)
    mids = np.array([0.0625, 0.1875, 0.4375, 0.9375, 1.0625, 1.4375, 1.9375, 2.125, 2.625, 3.875,
                     4.25, 5.75, 7.25, 1.0, 3.0, 6.0])
    t = rng.choice(mids, size=(nb, 32)) * rng.choice([-1.0, 1.0], size=(nb, 32))
    t[:, 0] = 7.5
    e = rng.integers(-120, 120, nb).astype(np.float64)
    rows.append(og.f64_to_bf16((t * np.exp2(e)[:, None]).reshape(-1)))
    # block maxima at the carry boundary: mantissa bits 1111xxx carry, 1110111 does not
    z = np.clip(rng.normal(0, 0.3, (nb, 32)), -0.9, 0.9)
    zb = og.f64_to_bf16(z.reshape(-1)).reshape(nb, 32)
    ex = rng.integers(100, 140, nb).astype(np.uint16)
    mant = rng.choice(np.array([0x78, 0x77, 0x7F, 0x70, 0x00, 0x7C], np.uint16), nb)
    zb[:, 0] = (ex << 7) | mant | (rng.integers(0, 2, nb).astype(np.uint16) << 15)
    zb[:, 1:] = og.f64_to_bf16(og.bf16_to_f64(zb[:, 1:]) * np.exp2(ex.astype(np.float64) - 127)[:, None])
    rows.append(zb.reshape(-1))
    # zero, negative-zero and subnormal blocks
    q = rng.normal(0, 1, (nb, 32))
    q[0::4] = 0.0
    q[1::4] = -0.0
    qb = og.f64_to_bf16(q.reshape(-1)).reshape(nb, 32)
    qb[2::4] = (rng.integers(1, 128, (len(qb[2::4]), 32)).astype(np.uint16)
                | (rng.integers(0, 2, (len(qb[2::4]), 32)).astype(np.uint16) << 15))
    rows.append(qb.reshape(-1))
    # random finite bit patterns
    bits = rng.integers(0, 1 << 16, cols).astype(np.uint16)
    rows.append(np.where((bits & 0x7F80) == 0x7F80, bits & 0xBFFF, bits).astype(np.uint16))
    # one bf16 ulp either side of the rounding boundaries, scale 2^1 after the anchor
    b = rng.choice(mids[:13], size=(nb, 32)) * 2.0
    bb = (og.f64_to_bf16(b).astype(np.int32) + rng.integers(-1, 2, size=(nb, 32))).astype(np.uint16)
    bb[:, 0] = og.f64_to_bf16(np.array([15.0]))[0]
    rows.append(bb.reshape(-1))
    # tiny normal values: the scale clamps at 2^-126
    rows.append(og.f64_to_bf16(rng.normal(0, 1, cols) * 2.0 ** -124))
    return np.stack(rows).astype(np.uint16)


@pytest.mark.parametrize("cols", [32, 1120, 8192])
def test_weight_rounding_bit_exact(cols):
    x = _rounding_inputs(cols, 80 + cols)
    R = x.shape[0]
    note(f"mxfp6 rounding rows={R} cols={cols}")
    xd = from_u16(x).to(DEV)
    codes = torch.zeros(R, cols // 32, 24, dtype=torch.uint8, device=DEV)
    scales = torch.zeros(R, cols // 32, dtype=torch.uint8, device=DEV)
    abi.gdn_mxfp6_round_weights(xd.data_ptr(), R, cols, codes.data_ptr(), scales.data_ptr(),
                                torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    ref_codes, ref_scales = og.mxfp6_round(og.bf16_to_f64(x))
    got_s = scales.cpu().numpy()
    assert np.array_equal(got_s, ref_scales), np.argwhere(got_s != ref_scales)[:5]
    got_c = og.unpack_e2m3(codes.cpu().numpy())
    bad = np.argwhere(got_c != ref_codes)
    assert bad.size == 0, f"{len(bad)} codes differ, first at {bad[:5].tolist()}"
    assert np.array_equal(codes.cpu().numpy(), og.pack_e2m3(ref_codes))


@pytest.mark.parametrize("rows", [1, 4, 7, 16])
@pytest.mark.parametrize("state", ["f32", "bf16"])
def test_tiny_mxfp6(rows, state):
    parity_case(TINY_MX6.with_(ssm_state_dtype=state), rows, 400 + rows, dev=DEV)


@pytest.mark.parametrize("hidden,dk", [(1536, 32), (2048, 128), (4096, 64)])
def test_mxfp6_shapes(hidden, dk):
    """Hidden sizes with 1, 2 and 2 groups of 512 K per K range (3, 2 and 4 ranges), and
    every head size."""
    shape = TINY_MX6.with_(name=f"mx6_h{hidden}_d{dk}", hidden=hidden, head_k_dim=dk, head_v_dim=dk,
                           num_v_heads=6)
    parity_case(shape, 8, 500 + dk, dev=DEV)


@pytest.mark.parametrize("rows", [1, 2, 5, 8, 13, 16])
def test_tp8_rank_mxfp6(rows):
    parity_case(configs.TP8_RANK_MXFP6, rows, 41, dev=DEV)


@pytest.mark.parametrize("rows", [2, 16])
def test_tp8_rank_mxfp6_gated_norm_weight_near_one(rows):
    parity_case(configs.TP8_RANK_MXFP6, rows, 46, stress=True, dev=DEV)


def test_tp8_rank_mxfp6_all_pad():
    parity_case(configs.TP8_RANK_MXFP6, 3, 42, all_pad=True, dev=DEV)


@pytest.mark.parametrize("rows", [1, 9])
def test_tp8_rank_mxfp6_normed_input(rows):
    parity_case(configs.TP8_RANK_MXFP6.with_(name="tp8_rank_mxfp6_normed_input", input_normed=True,
                                             has_residual=False), rows, 43, dev=DEV)


def test_tp8_rank_mxfp6_out_proj_fold():
    parity_case(configs.TP8_RANK_MXFP6.with_(name="tp8_rank_mxfp6_out_proj", fold_out_proj=True), 6, 44, dev=DEV)


def test_device_rounded_weights_decode():
    """The pages' recipe: bf16 N(0, 0.02) weights rounded to MXFP6 on the device, then
    decoded; the oracle reads the same codes and scales."""
    shape = configs.TP8_RANK_MXFP6
    w = synth.make_weights(shape, 45)
    wb = synth.make_weights(shape.with_(qkvz_format="bf16"), 45).w_qkvz
    N, H = wb.shape
    codes = torch.zeros(N, H // 32, 24, dtype=torch.uint8, device=DEV)
    scales = torch.zeros(N, H // 32, dtype=torch.uint8, device=DEV)
    abi.gdn_mxfp6_round_weights(wb.to(DEV).data_ptr(), N, H, codes.data_ptr(), scales.data_ptr(),
                                torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    w.w_qkvz, w.w_qkvz_scales = codes.cpu(), scales.cpu()
    parity_case(shape, 8, 45, weights=w, dev=DEV)
