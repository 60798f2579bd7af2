"""gdn_block_decode_noalloc (the entry point for callers that cannot allocate: its
scratch is the library's fixed per-GPU array) against gdn_block_decode on the same
inputs: the same bits in every output, and the oracle's parity rule. Two calls in a row
on one handle, the second with fewer rows; calls of handles of other shapes in between
share the array."""
import pytest
import torch

from gated_deltanet_linear_decode_amd import abi, configs, synth
from gated_deltanet_linear_decode_amd.block import GdnBlock
from tests.gpu_util import call_to, check_parity, note, run_gpu, same_bits, weights_to

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

TINY_MX = configs.GdnShape(
    "tiny_mxfp4_noalloc", hidden=512, num_k_heads=2, head_k_dim=32, num_v_heads=4, head_v_dim=32,
    num_state_slots=24, ssm_state_dtype="f32", has_residual=True, qkvz_format="mxfp4", rows=(16,), pad_rows=True)


def _pair(blk, shape, w, c, packed):
    """One call of each entry point on fresh copies of the inputs; the outputs must agree
    bit for bit, and the no-alloc one must meet the parity rule against the oracle."""
    wd, cd = weights_to(w, DEV), call_to(c, DEV)
    pk = blk.pack(wd) if packed else None
    ref = run_gpu(blk, shape, wd, cd, packed=pk)
    got = run_gpu(blk, shape, wd, cd, packed=pk, noalloc=True)
    same_bits(got, ref)
    rows = c.x.shape[0]
    flips = (0.02, 0.15) if shape.qkvz_format == "mxfp4" else None  # see tests/test_gpu_mxfp4.py
    st = check_parity(shape, w, c, got, label=f"noalloc {shape.name}/r{rows}", flips=flips)
    note(f"  noalloc {shape.name} rows {rows} packed {packed}: same bits as gdn_block_decode; {st}")


@pytest.mark.parametrize("packed", [True, False])
def test_noalloc_equals_decode_two_calls_smaller_second(packed):
    shape = configs.TP8_RANK_F32
    blk = GdnBlock(shape, max_rows=16, device=DEV)
    for rows, seed in ((12, 901), (5, 902)):
        _pair(blk, shape, synth.make_weights(shape, seed), synth.make_call(shape, rows, seed), packed)
    blk.close()


def test_noalloc_handles_of_other_shapes_share_the_array():
    a_shape, b_shape = configs.TP8_RANK_BF16, TINY_MX
    a = GdnBlock(a_shape, max_rows=8, device=DEV)
    b = GdnBlock(b_shape, max_rows=16, device=DEV)
    _pair(a, a_shape, synth.make_weights(a_shape, 903), synth.make_call(a_shape, 8, 903), True)
    _pair(b, b_shape, synth.make_weights(b_shape, 904), synth.make_call(b_shape, 16, 904), True)
    _pair(a, a_shape, synth.make_weights(a_shape, 905), synth.make_call(a_shape, 3, 905), True)
    _pair(b, b_shape, synth.make_weights(b_shape, 906), synth.make_call(b_shape, 7, 906), False)
    a.close()
    b.close()


def test_noalloc_refuses_a_handle_whose_scratch_does_not_fit():
    shape = configs.GdnShape("huge", hidden=16384, num_k_heads=16, head_k_dim=128, num_v_heads=64,
                             head_v_dim=128, num_state_slots=2, rows=(16,))
    blk = GdnBlock(shape, max_rows=16, device=DEV)
    lib = abi.load()
    fake = 1 << 20  # never dereferenced: the call is refused before anything is enqueued
    ws = abi.GdnBlockWeights()
    rc = lib.gdn_block_decode_noalloc(blk.handle, fake, fake, ws, fake, fake, fake, 1, fake, None)
    msg = abi.gdn_block_last_error(blk.handle)
    blk.close()
    assert rc == abi.GDN_E_UNSUPPORTED and "static scratch" in msg, (rc, msg)
