"""GPU parity: the HIP block against the CPU oracle, element by element, on the
same seeded inputs, at the tiny shape (many seeds, ragged row counts) and at
the full sizes of each workload (all rows, pad rows, all-pad calls)."""
import pytest
import torch

from gated_deltanet_linear_decode_amd import configs
from tests.gpu_util import parity_case

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _case(shape, rows, seed, **kw):
    return parity_case(shape, rows, seed, dev=DEV, **kw)


@pytest.mark.parametrize("seed", range(8))
@pytest.mark.parametrize("state", ["f32", "bf16"])
def test_tiny_one_row(seed, state):
    _case(configs.TINY.with_(ssm_state_dtype=state), 1, seed)


@pytest.mark.parametrize("rows", [1, 2, 3, 7, 13, 16])
@pytest.mark.parametrize("has_res", [True, False])
def test_tiny_ragged_rows_with_pads(rows, has_res):
    shape = configs.TINY.with_(num_state_slots=24, pad_rows=True, has_residual=has_res, rows=(16,))
    _case(shape, rows, 100 + rows)


@pytest.mark.parametrize("dk", [32, 64, 128])
def test_head_dims(dk):
    shape = configs.GdnShape("heads", hidden=512, num_k_heads=2, head_k_dim=dk, num_v_heads=6,
                             head_v_dim=dk, num_state_slots=12, pad_rows=True, rows=(8,))
    _case(shape, 8, 7)


def test_largest_hidden():
    shape = configs.GdnShape("wide", hidden=16384, num_k_heads=1, head_k_dim=64, num_v_heads=2,
                             head_v_dim=64, num_state_slots=20, rows=(16,), pad_rows=True)
    _case(shape, 16, 3)


@pytest.mark.parametrize("rows", configs.TP8_RANK_BF16.rows)
def test_tp8_rank_bf16_state_layer0(rows):
    _case(configs.TP8_RANK_BF16, rows, 11)


@pytest.mark.parametrize("rows", configs.TP8_RANK_F32.rows)
def test_tp8_rank_f32_state_pads(rows):
    _case(configs.TP8_RANK_F32, rows, 12)


def test_tp8_rank_all_pad():
    _case(configs.TP8_RANK_F32, 1, 13, all_pad=True)
    _case(configs.TP8_RANK_F32, 4, 14, all_pad=True)


@pytest.mark.parametrize("rows", [1, 4, 8])
def test_dense_full_width(rows):
    _case(configs.DENSE_FULL, rows, 15)


@pytest.mark.parametrize("name", ["tiny", "tp8_rank_bf16_state_layer0", "dense_full_width"])
def test_gated_norm_weight_near_one(name):
    shape = configs.ALL[name]
    _case(shape, min(4, shape.max_rows), 16, stress=True, pads=False)


@pytest.mark.parametrize("rows", [1, 7, 16])
def test_tiny_normed_input(rows):
    """The block started from the norm's output ("SGLang PR #43558", Modifications)."""
    shape = configs.TINY.with_(name="tiny_normed", input_normed=True, has_residual=False,
                               num_state_slots=24, pad_rows=True, rows=(16,))
    _case(shape, rows, 400 + rows)


@pytest.mark.parametrize("rows", [1, 5, 16])
def test_tp8_rank_normed_input(rows):
    _case(configs.TP8_RANK_BF16_NORMED.with_(pad_rows=True), rows, 41)


@pytest.mark.parametrize("rows", [1, 7, 16])
def test_tiny_out_proj_fold(rows):
    """The rank's out_proj partial written by the same launch ("SGLang PR #43558",
    Modifications: K1 with the out_proj fold)."""
    shape = configs.TINY.with_(name="tiny_out_proj", fold_out_proj=True, num_state_slots=24, pad_rows=True,
                               rows=(16,))
    _case(shape, rows, 500 + rows)


@pytest.mark.parametrize("rows", [1, 8, 16])
def test_tp8_rank_out_proj_fold(rows):
    _case(configs.TP8_RANK_BF16_OUT.with_(pad_rows=True), rows, 61)


def test_tp8_rank_mxfp4_normed_out_proj_fold():
    _case(configs.TP8_RANK_MXFP4_NORMED.with_(fold_out_proj=True), 9, 62)
