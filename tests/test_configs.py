"""Algorithmic bytes per launch against the figures worked out by hand from the shapes
(weights + per row x, residual in/out, core + per valid row the state and conv slots
read and written; the roofline's byte count, in MB of 10^6 bytes)."""
import pytest

from gated_deltanet_linear_decode_amd import configs

# (shape, rows, valid rows, MB): hand arithmetic from H, the head counts and dtypes
CASES = [
    (configs.TP8_RANK_BF16, 1, 1, 51.21), (configs.TP8_RANK_BF16, 2, 2, 51.79),
    (configs.TP8_RANK_BF16, 4, 4, 52.96), (configs.TP8_RANK_BF16, 8, 8, 55.30),
    (configs.TP8_RANK_F32, 1, 1, 51.75), (configs.TP8_RANK_F32, 5, 5, 56.25),
    (configs.TP8_RANK_F32, 8, 8, 59.62), (configs.TP8_RANK_F32, 16, 16, 68.62),
    (configs.DENSE_FULL, 1, 1, 172.16), (configs.DENSE_FULL, 8, 8, 195.34),
    (configs.TP8_RANK_MXFP4, 1, 1, 14.27), (configs.TP8_RANK_MXFP4, 16, 16, 23.27),
]


@pytest.mark.parametrize("shape,rows,valid,mb", CASES, ids=lambda v: getattr(v, "name", str(v)))
def test_algorithmic_bytes(shape, rows, valid, mb):
    assert configs.algorithmic_bytes(shape, rows, valid) / 1e6 == pytest.approx(mb, abs=0.006 * max(1, mb / 50))


def test_weight_bytes_by_format():
    """The in_proj_qkvz bytes alone: bf16 2 B, MXFP4 0.5 B + 1/32 B, MXFP6 0.75 B + 1/32 B
    per weight; H = 8192, Nqkvz = 3072."""
    H, N = 8192, 3072
    base = configs.algorithmic_bytes(configs.TP8_RANK_BF16, 1) - 2 * H * N
    mx4 = configs.TP8_RANK_BF16.with_(qkvz_format="mxfp4")
    mx6 = configs.TP8_RANK_BF16.with_(qkvz_format="mxfp6")
    assert configs.algorithmic_bytes(mx4, 1) - base == H * N // 2 + H * N // 32
    assert configs.algorithmic_bytes(mx6, 1) - base == H * N * 3 // 4 + H * N // 32


def test_pad_rows_move_no_state():
    s = configs.TP8_RANK_F32
    slot = 4 * s.num_v_heads * s.head_k_dim * s.head_v_dim + 2 * 3 * s.conv_dim
    assert configs.algorithmic_bytes(s, 8, 8) - configs.algorithmic_bytes(s, 8, 6) == 2 * 2 * slot


def test_verify_bytes():
    """A verify step reads each source state once and writes every kept snapshot."""
    s = configs.TP8_RANK_BF16
    slot = 2 * s.num_v_heads * s.head_k_dim * s.head_v_dim + 2 * 3 * s.conv_dim
    v = configs.algorithmic_bytes_verify(s, 2, 4)
    assert v == configs.algorithmic_bytes(s, 8, 0) + 2 * slot + 8 * slot
    assert configs.algorithmic_bytes_verify(s, 3, 1) == configs.algorithmic_bytes(s, 3, 3)


def test_partial_rows_keep_every_hand_off_on_lines_of_its_own():
    """The split partials' layout (the decode kernel's [S, R, PW] f32 scratch): for every
    head shape the library accepts, each key-head group's channels and the b|a block start
    on a 128-byte line and a row is whole lines, so no line holds partials of two
    hand-offs (two groups, a group and the b|a block, or two rows)."""
    for dk in (32, 64, 128):
        for nk in (1, 2, 3, 4, 8, 16):
            for r in range(1, 17):
                nv = nk * r
                gw = 2 * dk + 2 * r * dk                 # channels of one key-head group
                nq, nb = nk * gw, 2 * nv
                pw = nq + -(-nb // 32) * 32              # b|a padded to whole lines
                assert (gw * 4) % 128 == 0, (dk, nk, r)
                assert (nq * 4) % 128 == 0 and (pw * 4) % 128 == 0 and pw % 4 == 0, (dk, nk, r)
                starts = [g * gw for g in range(nk)] + [nq]
                assert all((4 * c) % 128 == 0 for c in starts)
