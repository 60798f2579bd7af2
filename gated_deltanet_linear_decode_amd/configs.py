"""Shapes and workloads of the Gated DeltaNet decode block.

Plain data: no arithmetic of the method lives here.

The shapes follow the pages:
  * "sgl-amd-mono PR #89" (Modifications, Kernel checks): one tensor-parallel
    rank's share of a large MoE model's GDN layer, with a bf16 or f32 SSM state
    and a layer-0 variant that has no residual input;
  * "vLLM PR #60833" (Per launch table): the same share with an MXFP4
    in_proj_qkvz, timed at 1 to 16 rows with weights rotated past the MALL;
  * "SGLang PR #43558" (Modifications, K1 at TP1): the full-width dense layer,
    hidden 5120 with 16 key and 48 value heads of 128;
  * "vLLM PR #60833" (a reviewer's comment proposing MXFP6): the TP8 share with
    an MXFP6 E2M3 in_proj_qkvz read by K1 with bf16 activations, timed at 2 rows.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace

SSM_F32 = "f32"
SSM_BF16 = "bf16"
FMT_BF16 = "bf16"
FMT_MXFP4 = "mxfp4"
FMT_MXFP6 = "mxfp6"
# scale rules of the MXFP4 activation quantiser: the block maximum rounded at e2m1's
# mantissa, exponent - 2 (the default); or the smallest power of two with max <= 6 * scale
MX_SCALE_ROUNDED_MAX = "rounded_max"
MX_SCALE_CEIL = "ceil"


@dataclass(frozen=True)
class GdnShape:
    name: str
    hidden: int
    num_k_heads: int
    head_k_dim: int
    num_v_heads: int
    head_v_dim: int
    conv_width: int = 4
    num_state_slots: int = 4
    ssm_state_dtype: str = SSM_F32
    has_residual: bool = True
    qkvz_format: str = FMT_BF16
    norm_eps: float = 1e-6
    gated_norm_eps: float = 1e-6
    l2norm_eps: float = 1e-6
    input_normed: bool = False   # x is already the norm's output (no residual add, no norm)
    fold_out_proj: bool = False  # also write the out_proj partial [R, H] from the core rows
    mx_scale_rule: str = MX_SCALE_ROUNDED_MAX  # MXFP4 activation scale rule
    # workload fields: the row counts this shape is exercised at, whether pad
    # rows are mixed in, and how many layer copies a timing run rotates over
    rows: tuple = (1,)
    pad_rows: bool = False
    layers: int = 1
    description: str = field(default="", compare=False)

    # derived sizes -----------------------------------------------------------
    @property
    def heads_per_group(self) -> int:  # value heads per key head
        return self.num_v_heads // self.num_k_heads

    @property
    def key_dim(self) -> int:
        return self.num_k_heads * self.head_k_dim

    @property
    def value_dim(self) -> int:
        return self.num_v_heads * self.head_v_dim

    @property
    def conv_dim(self) -> int:  # channels of the depthwise conv: q | k | v
        return 2 * self.key_dim + self.value_dim

    @property
    def n_qkvz(self) -> int:
        return 2 * self.key_dim + 2 * self.value_dim

    @property
    def n_ba(self) -> int:
        return 2 * self.num_v_heads

    @property
    def group_width(self) -> int:  # in_proj_qkvz outputs per key head
        return 2 * self.head_k_dim + 2 * self.heads_per_group * self.head_v_dim

    @property
    def max_rows(self) -> int:
        return max(self.rows)

    def with_(self, **kw) -> "GdnShape":
        return replace(self, **kw)


TINY = GdnShape(
    name="tiny",
    hidden=256, num_k_heads=2, head_k_dim=32, num_v_heads=4, head_v_dim=32,
    num_state_slots=4, ssm_state_dtype=SSM_F32, has_residual=True,
    rows=(1,), description="tiny block, 1 row, f32 state, residual input",
)

TP8_RANK_BF16 = GdnShape(
    name="tp8_rank_bf16_state_layer0",
    hidden=8192, num_k_heads=4, head_k_dim=128, num_v_heads=8, head_v_dim=128,
    num_state_slots=256, ssm_state_dtype=SSM_BF16, has_residual=False,
    rows=(1, 2, 4, 8), layers=12,
    description="one TP8 rank's share, bf16 SSM state, layer-0 variant",
)

TP8_RANK_F32 = GdnShape(
    name="tp8_rank_f32_state_pads",
    hidden=8192, num_k_heads=4, head_k_dim=128, num_v_heads=8, head_v_dim=128,
    num_state_slots=256, ssm_state_dtype=SSM_F32, has_residual=True,
    rows=(1, 5, 8, 9, 12, 16), pad_rows=True, layers=12,
    description="one TP8 rank's share, f32 SSM state, pad rows",
)

DENSE_FULL = GdnShape(
    name="dense_full_width",
    hidden=5120, num_k_heads=16, head_k_dim=128, num_v_heads=48, head_v_dim=128,
    num_state_slots=32, ssm_state_dtype=SSM_BF16, has_residual=True,
    rows=(1, 2, 3, 4, 5, 6, 7, 8), layers=48,
    description="full-width dense GDN layer on one GPU, bf16 state",
)

TP8_RANK_MXFP4 = GdnShape(
    name="tp8_rank_mxfp4",
    hidden=8192, num_k_heads=4, head_k_dim=128, num_v_heads=8, head_v_dim=128,
    num_state_slots=256, ssm_state_dtype=SSM_BF16, has_residual=True,
    qkvz_format=FMT_MXFP4, rows=tuple(range(1, 17)), pad_rows=True, layers=69,
    description="one TP8 rank's share, MXFP4 in_proj_qkvz, bf16 state, pad rows",
)

# MXFP6 E2M3 in_proj_qkvz with bf16 activations; 19.7 MB of weights a layer, so 32 layer
# copies (630 MB) keep the MALL from holding a layer between its launches
TP8_RANK_MXFP6 = TP8_RANK_MXFP4.with_(
    name="tp8_rank_mxfp6", qkvz_format=FMT_MXFP6, layers=32,
    description="one TP8 rank's share, MXFP6 E2M3 in_proj_qkvz (W6A16), bf16 state, pad rows")

# the "normed" variant: the block starts from the norm's output ("SGLang PR #43558",
# Modifications: K1Build.normed)
TP8_RANK_BF16_NORMED = TP8_RANK_BF16.with_(
    name="tp8_rank_bf16_state_normed_input", input_normed=True, rows=(1, 2, 4, 8, 12, 16),
    description="one TP8 rank's share, bf16 state, input already normed")
TP8_RANK_MXFP4_NORMED = TP8_RANK_MXFP4.with_(
    name="tp8_rank_mxfp4_normed_input", input_normed=True, has_residual=False,
    description="one TP8 rank's share, MXFP4 in_proj_qkvz, input already normed")

# out_proj folded in: the launch also writes the rank's out_proj partial ("SGLang PR
# #43558", Modifications: K1 with the out_proj fold)
TP8_RANK_BF16_OUT = TP8_RANK_BF16.with_(
    name="tp8_rank_bf16_state_out_proj", fold_out_proj=True, rows=(1, 2, 4, 8, 12, 16),
    description="one TP8 rank's share, bf16 state, out_proj partial folded in")

ALL = {s.name: s for s in (TINY, TP8_RANK_BF16, TP8_RANK_F32, DENSE_FULL, TP8_RANK_MXFP4,
                           TP8_RANK_MXFP6, TP8_RANK_BF16_NORMED, TP8_RANK_MXFP4_NORMED, TP8_RANK_BF16_OUT)}


def algorithmic_bytes(shape: GdnShape, rows: int, valid_rows: int | None = None) -> int:
    """Bytes one launch must move between HBM and the chip, counted once each.

    Weights (every launch streams them) + per row the input x, the residual in
    (when present) and out, and the core output + per valid row the SSM and
    conv state rows read and written. Scratch is not counted.
    """
    s = shape
    v = rows if valid_rows is None else valid_rows
    H = s.hidden
    if s.qkvz_format == FMT_MXFP4:
        w_qkvz = H * s.n_qkvz // 2 + H * s.n_qkvz // 32
    elif s.qkvz_format == FMT_MXFP6:
        w_qkvz = H * s.n_qkvz * 3 // 4 + H * s.n_qkvz // 32
    else:
        w_qkvz = 2 * H * s.n_qkvz
    w_other = 2 * H * s.n_ba + 2 * H + 2 * s.conv_dim * s.conv_width + 4 * s.num_v_heads \
        + 2 * s.num_v_heads + 2 * s.head_v_dim
    if s.input_normed:  # x read, no residual, no norm weight
        w_other -= 2 * H
        per_row = 2 * H + 2 * s.value_dim
    else:
        per_row = 2 * H + (2 * H if s.has_residual else 0) + 2 * H + 2 * s.value_dim
    if s.fold_out_proj:  # W_out [H, nv*dv] bf16, and the partial [R, H] bf16 written
        w_other += 2 * H * s.value_dim
        per_row += 2 * H
    ssm_elem = 4 if s.ssm_state_dtype == SSM_F32 else 2
    ssm_slot = ssm_elem * s.num_v_heads * s.head_k_dim * s.head_v_dim
    conv_slot = 2 * (s.conv_width - 1) * s.conv_dim
    return w_qkvz + w_other + rows * per_row + v * 2 * (ssm_slot + conv_slot)


def algorithmic_bytes_verify(shape: GdnShape, seqs: int, tokens: int, kept: int | None = None) -> int:
    """Bytes one verify launch must move: the weights once, every token row's input, residual
    and core as in a decode row, each sequence's source state read once, and each kept
    snapshot (the state and conv window after a token) written once."""
    s = shape
    ssm_elem = 4 if s.ssm_state_dtype == SSM_F32 else 2
    slot = ssm_elem * s.num_v_heads * s.head_k_dim * s.head_v_dim + 2 * (s.conv_width - 1) * s.conv_dim
    no_state = algorithmic_bytes(s, seqs * tokens, 0)
    return no_state + seqs * slot + (seqs * tokens if kept is None else kept) * slot
