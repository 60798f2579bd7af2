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


@pytest.mark.parametrize("name", ["tiny", "tp8_rank_bf16_state_layer0", "tp8_rank_f32_state_pads",
                                  "dense_full_width"])
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


@pytest.mark.parametrize("state", ["f32", "bf16"])
def test_tiny_256_seeds(state):
    """The tiny one-row config over 256 seeds (one handle, row-major and tiled weights)."""
    from gated_deltanet_linear_decode_amd import synth
    from gated_deltanet_linear_decode_amd.block import GdnBlock
    from tests.gpu_util import call_to, check_parity, note, run_gpu, same_bits, weights_to
    shape = configs.TINY.with_(ssm_state_dtype=state)
    blk = GdnBlock(shape, device=DEV)
    worst = {}
    for seed in range(256):
        w, c = synth.make_weights(shape, 1000 + seed), synth.make_call(shape, 1, 1000 + seed)
        wd, cd = weights_to(w, DEV), call_to(c, DEV)
        out = run_gpu(blk, shape, wd, cd)
        same_bits(out, run_gpu(blk, shape, wd, cd, packed=blk.pack(wd)))
        st = check_parity(shape, w, c, out, label=f"tiny/{state}/s{1000 + seed}")
        for t, d in st.items():
            for k, v in d.items():
                worst[(t, k)] = max(worst.get((t, k), 0), v)
    blk.close()
    note(f"  256 seeds ok; worst {worst}")


@pytest.mark.parametrize("state", ["f32", "bf16"])
def test_index_past_the_pool_is_a_pad_row(state):
    """An index >= num_state_slots is handled like a pad row: zero core, no state access
    (include/gdn_block.h, gdn_block_decode)."""
    from gated_deltanet_linear_decode_amd import synth
    shape = configs.TINY.with_(name="tiny_oob", ssm_state_dtype=state, num_state_slots=12, rows=(8,))
    c = synth.make_call(shape, 8, 801)
    c.state_idx = torch.tensor([3, 12, 5, 1000, -1, 7, 2 ** 31 - 1, 11], dtype=torch.int32)
    _case(shape, 8, 801, call=c)


@pytest.mark.parametrize("rows", [8, 16])
def test_partials_of_two_groups_never_share_a_line(rows):
    """nk = 4, nv = 12, dk = 128 at H = 8192: with unpadded partial rows (16,480 bytes) a
    128-byte line would hold channels of two key-head groups, or of two rows, read by
    recurrence workgroups on one XCD; the padded layout keeps every group on lines of its
    own."""
    shape = configs.GdnShape("g4v12", hidden=8192, num_k_heads=4, head_k_dim=128, num_v_heads=12,
                             head_v_dim=128, num_state_slots=24, ssm_state_dtype="bf16", has_residual=True,
                             rows=(16,), pad_rows=True)
    _case(shape, rows, 802 + rows)


@pytest.mark.parametrize("nv,rows", [(3, 1), (3, 3), (5, 7)])
def test_odd_value_head_count(nv, rows):
    """An odd nv gives 2 nv b|a channels (2 mod 4): the partial rows stay whole lines."""
    shape = configs.GdnShape(f"odd_nv{nv}", hidden=5120, num_k_heads=1, head_k_dim=128, num_v_heads=nv,
                             head_v_dim=128, num_state_slots=12, ssm_state_dtype="f32", has_residual=True,
                             rows=(8,), pad_rows=True)
    _case(shape, rows, 810 + nv + rows)


@pytest.mark.parametrize("name,rows", [("tp8_rank_bf16_state_layer0", 8), ("tp8_rank_f32_state_pads", 16),
                                       ("dense_full_width", 8), ("tp8_rank_bf16_state_out_proj", 16),
                                       ("tp8_rank_bf16_state_normed_input", 12)])
def test_gated_norm_weight_near_one_full_size(name, rows):
    """The w_g = 1 + N(0, 0.02) draw at the full sizes: core values are O(1), so the
    element bound is not vacuous on them."""
    shape = configs.ALL[name]
    _case(shape, rows, 820 + rows, stress=True)


def test_give_up_path_reports_and_recovers():
    """A spin limit of 0 makes every wait that is not already complete give up at once
    (forced from the host; every workgroup still exits): the error word is set, and
    gdn_block_check clears it and the hand-off counters, so the next decode is correct."""
    from gated_deltanet_linear_decode_amd import synth
    from gated_deltanet_linear_decode_amd.block import GdnBlock
    from tests.gpu_util import call_to, check_parity, note, run_gpu, weights_to
    shape = configs.TP8_RANK_BF16
    w, c = synth.make_weights(shape, 830), synth.make_call(shape, 8, 830)
    blk = GdnBlock(shape, max_rows=8, device=DEV)
    wd, cd = weights_to(w, DEV), call_to(c, DEV)
    packed = blk.pack(wd)
    blk.set_spin_limit(0)
    run_gpu(blk, shape, wd, cd, packed=packed, check=False)
    word = blk.check()
    note(f"  error word after a give-up: {word:#x}")
    assert word != 0, "a wait with spin limit 0 should have given up"
    assert blk.check() == 0, "the check clears the word"
    blk.set_spin_limit(1 << 20)
    out = run_gpu(blk, shape, wd, cd, packed=packed)
    blk.close()
    check_parity(shape, w, c, out, label="after give-up")
