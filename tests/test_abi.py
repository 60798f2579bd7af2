"""Host-side checks of the C ABI: the library loads, exports every function
include/gdn_block.h declares, its structs match the header, and create()
refuses bad configurations (listing every reason) without touching a device."""
import ctypes
import os
import re

import pytest

from gated_deltanet_linear_decode_amd import abi, configs
from gated_deltanet_linear_decode_amd.block import make_config

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn_block.h")


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_\w+)\s*\(", src)))


def test_library_exports_every_declared_function():
    lib = abi.load()
    declared = _declared_functions()
    assert declared == sorted(abi.EXPORTED)
    for name in declared:
        assert hasattr(lib, name), name


def test_struct_layout_matches_header():
    src = open(HEADER).read()
    body = re.search(r"typedef struct gdn_block_config \{(.*?)\} gdn_block_config;", src, re.S).group(1)
    fields = re.findall(r"(int32_t|float)\s+([\w ,]+);", re.sub(r"/\*.*?\*/", "", body, flags=re.S))
    names = [n.strip() for _, group in fields for n in group.split(",")]
    assert names == [f[0] for f in abi.GdnBlockConfig._fields_]
    assert ctypes.sizeof(abi.GdnBlockConfig) == 4 * len(names)
    wbody = re.search(r"typedef struct gdn_block_weights \{(.*?)\} gdn_block_weights;", src, re.S).group(1)
    wnames = re.findall(r"\*\s*(\w+);", wbody)
    assert wnames == [f[0] for f in abi.GdnBlockWeights._fields_]


def _cfg(**kw):
    c = make_config(configs.TINY)
    for k, v in kw.items():
        setattr(c, k, v)
    return c


@pytest.mark.parametrize("field,value,needle", [
    ("hidden", 100, "hidden"),
    ("hidden", 15872, "K ranges"),   # 31 x 512: no K range of a multiple of 128 up to 1024 in 16
    ("num_v_heads", 3, "num_v_heads"),
    ("head_k_dim", 48, "head_k_dim"),
    ("head_v_dim", 64, "head_v_dim"),
    ("conv_width", 3, "conv_width"),
    ("num_state_slots", 1, "num_state_slots"),
    ("max_rows", 17, "max_rows"),
    ("max_rows", 0, "max_rows"),
    ("qkvz_format", 9, "qkvz_format"),
    ("ssm_state_dtype", 2, "ssm_state_dtype"),
    ("has_residual", 2, "has_residual"),
    ("norm_eps", 0.0, "eps"),
    ("mx_scale_rule", 2, "mx_scale_rule"),
])
def test_create_refuses_each_bad_field(field, value, needle):
    with pytest.raises(abi.GdnError) as e:
        abi.gdn_block_create(_cfg(**{field: value}))
    assert e.value.code == abi.GDN_E_UNSUPPORTED
    assert needle in str(e.value)


def test_normed_input_refuses_a_residual_input():
    with pytest.raises(abi.GdnError) as e:
        abi.gdn_block_create(_cfg(input_normed=1, has_residual=1))
    assert e.value.code == abi.GDN_E_UNSUPPORTED and "input_normed" in str(e.value)


def test_out_proj_fold_needs_one_k_range():
    with pytest.raises(abi.GdnError) as e:
        abi.gdn_block_create(_cfg(fold_out_proj=1, num_v_heads=64, head_v_dim=32, head_k_dim=32))
    assert e.value.code == abi.GDN_E_UNSUPPORTED and "fold_out_proj" in str(e.value)


def test_create_lists_every_reason():
    with pytest.raises(abi.GdnError) as e:
        abi.gdn_block_create(_cfg(hidden=100, conv_width=5, max_rows=40, has_residual=3))
    msg = str(e.value)
    for needle in ("hidden", "conv_width", "max_rows", "has_residual"):
        assert needle in msg


def test_mxfp4_needs_hidden_multiple_of_512():
    with pytest.raises(abi.GdnError) as e:
        abi.gdn_block_create(_cfg(qkvz_format=abi.GDN_FMT_MXFP4))  # the tiny shape has H = 256
    assert e.value.code == abi.GDN_E_UNSUPPORTED and "512" in str(e.value)


def test_mxfp6_needs_hidden_multiple_of_512():
    with pytest.raises(abi.GdnError) as e:
        abi.gdn_block_create(_cfg(qkvz_format=abi.GDN_FMT_MXFP6))  # the tiny shape has H = 256
    assert e.value.code == abi.GDN_E_UNSUPPORTED and "MXFP6" in str(e.value) and "512" in str(e.value)


def test_mxfp6_rounding_arguments_are_checked_on_the_host():
    lib = abi.load()
    fake = 1 << 20  # an aligned address that is never dereferenced: every call below is refused
    for rows, cols, w, codes, scales, needle in [
        (1, 48, fake, fake, fake, "multiple of 32"),
        (-1, 32, fake, fake, fake, "rows"),
        (1, 0, fake, fake, fake, "cols"),
        (1, 32, fake, None, fake, "NULL"),
        (1, 32, fake + 8, fake, fake, "aligned"),
        (1, 32, fake, fake + 4, fake, "aligned"),
    ]:
        assert lib.gdn_mxfp6_round_weights(w, rows, cols, codes, scales, None) == abi.GDN_E_INVALID_ARG
        assert needle in abi.gdn_block_last_error(None)
    assert lib.gdn_mxfp6_round_weights(fake, 0, 32, fake, fake, None) == abi.GDN_OK  # nothing to do


def test_quantize_arguments_are_checked_on_the_host():
    lib = abi.load()
    fake = 1 << 20  # an aligned address that is never dereferenced: every call below is refused
    for rows, cols, x, codes, scales, needle in [
        (1, 48, fake, fake, fake, "multiple of 32"),
        (-1, 32, fake, fake, fake, "rows"),
        (1, 0, fake, fake, fake, "cols"),
        (1, 32, None, fake, fake, "NULL"),
        (1, 32, fake + 8, fake, fake, "aligned"),
        (1, 32, fake, fake + 2, fake, "aligned"),
    ]:
        assert lib.gdn_mxfp4_quantize(x, rows, cols, codes, scales, 0, None) == abi.GDN_E_INVALID_ARG
        assert needle in abi.gdn_block_last_error(None)
    assert lib.gdn_mxfp4_quantize(fake, 1, 32, fake, fake, 2, None) == abi.GDN_E_INVALID_ARG
    assert "scale_rule" in abi.gdn_block_last_error(None)
    for rule in (abi.GDN_MXSCALE_ROUNDED_MAX, abi.GDN_MXSCALE_CEIL):
        assert lib.gdn_mxfp4_quantize(fake, 0, 32, fake, fake, rule, None) == abi.GDN_OK  # nothing to do


def test_read_stream_arguments_are_checked_on_the_host():
    lib = abi.load()
    fake = 1 << 20  # an aligned address that is never dereferenced: every call below is refused
    for src, nbytes, sink, needle in [
        (None, 64, fake, "NULL"),
        (fake, 64, None, "NULL"),
        (fake, 0, fake, "multiple of 16"),
        (fake, 40, fake, "multiple of 16"),
        (fake + 8, 64, fake, "aligned"),
        (fake, 64, fake + 2, "aligned"),
    ]:
        assert lib.gdn_read_stream(src, nbytes, sink, None) == abi.GDN_E_INVALID_ARG
        assert needle in abi.gdn_block_last_error(None)


def test_null_arguments_are_rejected_on_the_host():
    lib = abi.load()
    assert lib.gdn_block_create(None, None) == abi.GDN_E_INVALID_ARG
    assert "NULL" in abi.gdn_block_last_error(None)
    assert lib.gdn_block_decode(None, None, None, None, None, None, None, 1, None, None) == abi.GDN_E_INVALID_ARG
    assert lib.gdn_block_set_spin_limit(None, 5) == abi.GDN_E_INVALID_ARG
    lib.gdn_block_destroy(None)  # a no-op
