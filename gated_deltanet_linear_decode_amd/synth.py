"""Seeded synthetic inputs for the GDN decode block.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic. The same bytes feed the HIP path and the CPU oracle.

Distributions (the workloads of the pages carry random weights in the stock
layouts, "sgl-amd-mono PR #89", Kernel checks):
  bf16 weights (in_proj_qkvz, in_proj_ba, conv, both norm weights, out_proj) ~ N(0, 0.02)
  A_log ~ U(0, 2) f32; dt_bias ~ N(0, 0.1) bf16
  x, residual ~ N(0, 1) bf16; conv state ~ N(0, 1) bf16
  SSM state ~ N(0, 0.1), stored f32 or bf16
Values are drawn in f32 with numpy's PCG64 and rounded to bf16 by torch's
round-to-nearest-even cast.

MXFP4 weights are drawn directly as codes and scales (no quantiser runs
here): a random sign and e2m1 magnitude per element and a random e8m0 block
exponent near the one an N(0, 0.02) block of 32 would get. MXFP6 weights
likewise: a random sign and E2M3 magnitude code per element (32 magnitudes,
smaller ones more likely), packed 32 codes to 24 bytes (code i at bits
6i..6i+5 of the block, little-endian), and a random e8m0 block exponent.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

from .configs import FMT_MXFP4, FMT_MXFP6, SSM_BF16, GdnShape


def _bf16(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)


@dataclass
class GdnWeights:
    norm_w: torch.Tensor          # [H] bf16
    w_qkvz: torch.Tensor          # [Nqkvz, H] bf16, or [Nqkvz, H/2] uint8 e2m1 codes (MXFP4)
    w_qkvz_scales: torch.Tensor | None  # [Nqkvz, H/32] uint8 e8m0 (MXFP4 only)
    w_ba: torch.Tensor            # [2*nv, H] bf16
    conv_w: torch.Tensor          # [Cd, W] bf16
    A_log: torch.Tensor           # [nv] f32
    dt_bias: torch.Tensor         # [nv] bf16
    gated_norm_w: torch.Tensor    # [dv] bf16
    w_out: torch.Tensor | None = None  # [H, nv*dv] bf16 out_proj (its rank's columns), fold only

    def tensors(self):
        return {k: v for k, v in self.__dict__.items() if v is not None}


@dataclass
class GdnCall:
    x: torch.Tensor               # [R, H] bf16
    residual: torch.Tensor        # [R, H] bf16 (ignored as input when the layer has none)
    conv_state: torch.Tensor      # [slots, W-1, Cd] bf16
    ssm_state: torch.Tensor       # [slots, nv, dk, dv] f32 or bf16
    state_idx: torch.Tensor       # [R] int32


# e2m1 magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6 drawn with these probabilities
_E2M1_P = np.array([0.10, 0.18, 0.18, 0.15, 0.13, 0.12, 0.08, 0.06])
# E2M3 magnitude codes 0..31 (0..0.875, 1..1.875, 2..3.75, 4..7.5): weights per code
_E2M3_W = np.array([4.0] * 8 + [3.0] * 8 + [4.0] * 8 + [2.0] * 8)
_E2M3_P = _E2M3_W / _E2M3_W.sum()


def pack_6bit_blocks(codes: np.ndarray) -> np.ndarray:
    """[N, K] 6-bit codes -> [N, K/32, 24] bytes, code i of a block at bits 6i..6i+5."""
    n, k = codes.shape
    bits = ((codes.reshape(n, k // 32, 32, 1) >> np.arange(6, dtype=np.uint8)) & 1).astype(np.uint8)
    return np.packbits(bits.reshape(n, k // 32, 192), axis=-1, bitorder="little")


def make_weights(shape: GdnShape, seed: int, *, gated_norm_stress: bool = False) -> GdnWeights:
    s = shape
    rng = np.random.Generator(np.random.PCG64(seed))
    H = s.hidden
    norm_w = _bf16(rng.normal(0.0, 0.02, H))
    if s.qkvz_format == FMT_MXFP4:
        mag = rng.choice(8, size=(s.n_qkvz, H), p=_E2M1_P).astype(np.uint8)
        sign = rng.integers(0, 2, size=(s.n_qkvz, H), dtype=np.uint8) << 3
        code = mag | sign
        packed = (code[:, 0::2] | (code[:, 1::2] << 4)).astype(np.uint8)
        # an N(0, 0.02) block's maximum is about 0.045, i.e. 6 * 2^-7.1
        scales = (127 - 7 + rng.integers(-1, 1, size=(s.n_qkvz, H // 32))).astype(np.uint8)
        w_qkvz = torch.from_numpy(packed)
        w_scales = torch.from_numpy(scales)
    elif s.qkvz_format == FMT_MXFP6:
        mag = rng.choice(32, size=(s.n_qkvz, H), p=_E2M3_P).astype(np.uint8)
        sign = rng.integers(0, 2, size=(s.n_qkvz, H), dtype=np.uint8) << 5
        w_qkvz = torch.from_numpy(pack_6bit_blocks(mag | sign))
        # an N(0, 0.02) block's maximum is about 0.045 = 5.8 * 2^-7: scale 2^-7 or 2^-6
        w_scales = torch.from_numpy((127 - 7 + rng.integers(0, 2, size=(s.n_qkvz, H // 32))).astype(np.uint8))
    else:
        w_qkvz = _bf16(rng.normal(0.0, 0.02, (s.n_qkvz, H)).astype(np.float32))
        w_scales = None
    w_ba = _bf16(rng.normal(0.0, 0.02, (s.n_ba, H)))
    conv_w = _bf16(rng.normal(0.0, 0.02, (s.conv_dim, s.conv_width)))
    A_log = torch.from_numpy(rng.uniform(0.0, 2.0, s.num_v_heads).astype(np.float32))
    dt_bias = _bf16(rng.normal(0.0, 0.1, s.num_v_heads))
    g = rng.normal(0.0, 0.02, s.head_v_dim)
    gated_norm_w = _bf16(1.0 + g if gated_norm_stress else g)
    w_out = _bf16(rng.normal(0.0, 0.02, (H, s.value_dim))) if s.fold_out_proj else None
    return GdnWeights(norm_w, w_qkvz, w_scales, w_ba, conv_w, A_log, dt_bias, gated_norm_w, w_out)


def make_state_idx(shape: GdnShape, rows: int, seed: int, *, pads: bool | None = None,
                   all_pad: bool = False) -> torch.Tensor:
    """Distinct valid slots in 1..slots-1; pad rows carry 0 or -1.

    With pads, floor(rows/4) rows (rows >= 2) at seeded positions are pads,
    alternating index 0 and -1.
    """
    rng = np.random.Generator(np.random.PCG64(seed + 7919))
    if all_pad:
        idx = np.array([0 if i % 2 == 0 else -1 for i in range(rows)], dtype=np.int32)
        return torch.from_numpy(idx)
    assert rows <= shape.num_state_slots - 1, "not enough distinct valid slots"
    idx = (rng.permutation(shape.num_state_slots - 1)[:rows] + 1).astype(np.int32)
    use_pads = shape.pad_rows if pads is None else pads
    if use_pads and rows >= 2:
        where = np.sort(rng.choice(rows, size=rows // 4, replace=False))
        for j, p in enumerate(where):
            idx[p] = 0 if j % 2 == 0 else -1
    return torch.from_numpy(idx)


def make_call(shape: GdnShape, rows: int, seed: int, *, pads: bool | None = None,
              all_pad: bool = False) -> GdnCall:
    s = shape
    rng = np.random.Generator(np.random.PCG64(seed + 104729))
    H = s.hidden
    x = _bf16(rng.normal(0.0, 1.0, (rows, H)))
    residual = _bf16(rng.normal(0.0, 1.0, (rows, H)))
    conv_state = _bf16(rng.normal(0.0, 1.0, (s.num_state_slots, s.conv_width - 1, s.conv_dim)))
    ssm = rng.normal(0.0, 0.1, (s.num_state_slots, s.num_v_heads, s.head_k_dim, s.head_v_dim)
                     ).astype(np.float32)
    ssm_state = _bf16(ssm) if s.ssm_state_dtype == SSM_BF16 else torch.from_numpy(ssm)
    state_idx = make_state_idx(s, rows, seed, pads=pads, all_pad=all_pad)
    return GdnCall(x, residual, conv_state, ssm_state, state_idx)
