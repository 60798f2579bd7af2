"""ctypes binding of the C ABI in include/gdn_block.h, function for function.

Argument marshalling only: every step of the block runs in the HIP library.
Loading fails loudly when the library is not built; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_char_p, c_float, c_int, c_int32, c_size_t, c_uint32, c_void_p

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgdn_block.so")

GDN_OK = 0
GDN_E_INVALID_ARG = -1
GDN_E_UNSUPPORTED = -2
GDN_E_HIP = -3
GDN_FMT_BF16 = 0
GDN_FMT_MXFP4 = 1
GDN_FMT_MXFP6 = 2
GDN_STATE_F32 = 0
GDN_STATE_BF16 = 1
GDN_MXSCALE_ROUNDED_MAX = 0
GDN_MXSCALE_CEIL = 1
GDN_MAX_ROWS = 16

EXPORTED = ("gdn_block_create", "gdn_block_decode", "gdn_block_destroy", "gdn_block_last_error",
            "gdn_block_packed_weight_bytes", "gdn_block_pack_weights", "gdn_block_check",
            "gdn_mxfp4_quantize", "gdn_block_decode_with_out_proj", "gdn_mxfp6_round_weights",
            "gdn_block_verify", "gdn_block_set_spin_limit", "gdn_block_decode_noalloc", "gdn_read_stream")


class GdnBlockConfig(ctypes.Structure):
    _fields_ = [
        ("hidden", c_int32), ("num_k_heads", c_int32), ("head_k_dim", c_int32),
        ("num_v_heads", c_int32), ("head_v_dim", c_int32), ("conv_width", c_int32),
        ("num_state_slots", c_int32), ("max_rows", c_int32), ("qkvz_format", c_int32),
        ("ssm_state_dtype", c_int32), ("has_residual", c_int32),
        ("norm_eps", c_float), ("gated_norm_eps", c_float), ("l2norm_eps", c_float),
        ("input_normed", c_int32), ("fold_out_proj", c_int32), ("mx_scale_rule", c_int32),
    ]


class GdnBlockWeights(ctypes.Structure):
    _fields_ = [
        ("norm_w", c_void_p), ("w_qkvz", c_void_p), ("w_qkvz_scales", c_void_p), ("w_ba", c_void_p),
        ("conv_w", c_void_p), ("A_log", c_void_p), ("dt_bias", c_void_p), ("gated_norm_w", c_void_p),
        ("w_proj_packed", c_void_p), ("w_out", c_void_p),
    ]


class GdnError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"[{code}] {msg}")
        self.code = code


_lib = None


def load() -> ctypes.CDLL:
    """Load libgdn_block.so (built in-tree by gated_deltanet_linear_decode_amd.build).

    In a process that also uses torch, import torch first, so that the library binds
    to the HIP runtime torch has loaded rather than bringing up a second one."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run `python -m gated_deltanet_linear_decode_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        lib.gdn_block_create.argtypes = [POINTER(GdnBlockConfig), POINTER(c_void_p)]
        lib.gdn_block_create.restype = c_int
        lib.gdn_block_decode.argtypes = [c_void_p, c_void_p, c_void_p, POINTER(GdnBlockWeights), c_void_p,
                                         c_void_p, c_void_p, c_int32, c_void_p, c_void_p]
        lib.gdn_block_decode.restype = c_int
        lib.gdn_block_decode_noalloc.argtypes = [c_void_p, c_void_p, c_void_p, POINTER(GdnBlockWeights), c_void_p,
                                                 c_void_p, c_void_p, c_int32, c_void_p, c_void_p]
        lib.gdn_block_decode_noalloc.restype = c_int
        lib.gdn_block_destroy.argtypes = [c_void_p]
        lib.gdn_block_destroy.restype = None
        lib.gdn_block_last_error.argtypes = [c_void_p]
        lib.gdn_block_last_error.restype = c_char_p
        lib.gdn_block_packed_weight_bytes.argtypes = [c_void_p]
        lib.gdn_block_packed_weight_bytes.restype = c_size_t
        lib.gdn_block_pack_weights.argtypes = [c_void_p, POINTER(GdnBlockWeights), c_void_p, c_void_p]
        lib.gdn_block_pack_weights.restype = c_int
        lib.gdn_block_check.argtypes = [c_void_p, POINTER(c_uint32)]
        lib.gdn_block_check.restype = c_int
        lib.gdn_block_set_spin_limit.argtypes = [c_void_p, c_int32]
        lib.gdn_block_set_spin_limit.restype = c_int
        lib.gdn_block_decode_with_out_proj.argtypes = [c_void_p, c_void_p, c_void_p, POINTER(GdnBlockWeights),
                                                       c_void_p, c_void_p, c_void_p, c_int32, c_void_p, c_void_p,
                                                       c_void_p]
        lib.gdn_block_decode_with_out_proj.restype = c_int
        lib.gdn_mxfp4_quantize.argtypes = [c_void_p, c_int32, c_int32, c_void_p, c_void_p, c_int32, c_void_p]
        lib.gdn_mxfp4_quantize.restype = c_int
        lib.gdn_mxfp6_round_weights.argtypes = [c_void_p, c_int32, c_int32, c_void_p, c_void_p, c_void_p]
        lib.gdn_mxfp6_round_weights.restype = c_int
        lib.gdn_block_verify.argtypes = [c_void_p, c_void_p, c_void_p, POINTER(GdnBlockWeights), c_void_p, c_void_p,
                                         c_void_p, c_void_p, c_int32, c_int32, c_void_p, c_void_p]
        lib.gdn_block_verify.restype = c_int
        lib.gdn_read_stream.argtypes = [c_void_p, c_size_t, c_void_p, c_void_p]
        lib.gdn_read_stream.restype = c_int
        _lib = lib
    return _lib


def gdn_block_last_error(handle) -> str:
    return load().gdn_block_last_error(handle).decode()


def gdn_block_create(cfg: GdnBlockConfig) -> c_void_p:
    h = c_void_p()
    rc = load().gdn_block_create(ctypes.byref(cfg), ctypes.byref(h))
    if rc != GDN_OK:
        raise GdnError(rc, gdn_block_last_error(None))
    return h


def gdn_block_decode(handle, x: int, residual: int, weights: GdnBlockWeights, conv_state: int,
                     ssm_state: int, state_idx: int, rows: int, core_out: int, stream: int) -> None:
    rc = load().gdn_block_decode(handle, x, residual, ctypes.byref(weights), conv_state, ssm_state,
                                 state_idx, rows, core_out, stream)
    if rc != GDN_OK:
        raise GdnError(rc, gdn_block_last_error(handle))


def gdn_block_decode_noalloc(handle, x: int, residual: int, weights: GdnBlockWeights, conv_state: int,
                             ssm_state: int, state_idx: int, rows: int, core_out: int, stream: int) -> None:
    rc = load().gdn_block_decode_noalloc(handle, x, residual, ctypes.byref(weights), conv_state, ssm_state,
                                         state_idx, rows, core_out, stream)
    if rc != GDN_OK:
        raise GdnError(rc, gdn_block_last_error(handle))


def gdn_block_decode_with_out_proj(handle, x: int, residual: int, weights: GdnBlockWeights, conv_state: int,
                                   ssm_state: int, state_idx: int, rows: int, core_out: int, out: int,
                                   stream: int) -> None:
    rc = load().gdn_block_decode_with_out_proj(handle, x, residual, ctypes.byref(weights), conv_state, ssm_state,
                                               state_idx, rows, core_out, out, stream)
    if rc != GDN_OK:
        raise GdnError(rc, gdn_block_last_error(handle))


def gdn_block_verify(handle, x: int, residual: int, weights: GdnBlockWeights, conv_state: int, ssm_state: int,
                     src_idx: int, dst_idx: int, rows: int, tokens: int, core_out: int, stream: int) -> None:
    rc = load().gdn_block_verify(handle, x, residual, ctypes.byref(weights), conv_state, ssm_state, src_idx,
                                 dst_idx, rows, tokens, core_out, stream)
    if rc != GDN_OK:
        raise GdnError(rc, gdn_block_last_error(handle))


def gdn_block_packed_weight_bytes(handle) -> int:
    return int(load().gdn_block_packed_weight_bytes(handle))


def gdn_block_pack_weights(handle, weights: GdnBlockWeights, packed: int, stream: int) -> None:
    rc = load().gdn_block_pack_weights(handle, ctypes.byref(weights), packed, stream)
    if rc != GDN_OK:
        raise GdnError(rc, gdn_block_last_error(handle))


def gdn_block_check(handle) -> int:
    """The sticky error word of the handle's decodes (read and cleared; synchronous)."""
    word = c_uint32(0)
    rc = load().gdn_block_check(handle, ctypes.byref(word))
    if rc != GDN_OK:
        raise GdnError(rc, gdn_block_last_error(handle))
    return int(word.value)


def gdn_mxfp4_quantize(x: int, rows: int, cols: int, codes: int, scales: int, scale_rule: int,
                       stream: int) -> None:
    rc = load().gdn_mxfp4_quantize(x, rows, cols, codes, scales, scale_rule, stream)
    if rc != GDN_OK:
        raise GdnError(rc, gdn_block_last_error(None))


def gdn_block_set_spin_limit(handle, polls: int) -> None:
    rc = load().gdn_block_set_spin_limit(handle, polls)
    if rc != GDN_OK:
        raise GdnError(rc, gdn_block_last_error(handle))


def gdn_mxfp6_round_weights(w: int, rows: int, cols: int, codes: int, scales: int, stream: int) -> None:
    rc = load().gdn_mxfp6_round_weights(w, rows, cols, codes, scales, stream)
    if rc != GDN_OK:
        raise GdnError(rc, gdn_block_last_error(None))


def gdn_read_stream(src: int, nbytes: int, sink: int, stream: int) -> None:
    rc = load().gdn_read_stream(src, nbytes, sink, stream)
    if rc != GDN_OK:
        raise GdnError(rc, gdn_block_last_error(None))


def gdn_block_destroy(handle) -> None:
    if handle:
        load().gdn_block_destroy(handle)
