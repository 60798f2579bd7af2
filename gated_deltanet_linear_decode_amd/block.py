"""GdnBlock: the C ABI driven with torch device tensors.

torch provides device memory and the stream; this module checks dtypes,
shapes and devices and passes raw pointers through the ctypes binding.
"""
from __future__ import annotations

import torch

from . import abi
from .configs import FMT_MXFP4, FMT_MXFP6, MX_SCALE_CEIL, SSM_BF16, GdnShape

_FMT = {FMT_MXFP4: abi.GDN_FMT_MXFP4, FMT_MXFP6: abi.GDN_FMT_MXFP6}


def make_config(shape: GdnShape, max_rows: int | None = None) -> abi.GdnBlockConfig:
    s = shape
    return abi.GdnBlockConfig(
        hidden=s.hidden, num_k_heads=s.num_k_heads, head_k_dim=s.head_k_dim,
        num_v_heads=s.num_v_heads, head_v_dim=s.head_v_dim, conv_width=s.conv_width,
        num_state_slots=s.num_state_slots, max_rows=s.max_rows if max_rows is None else max_rows,
        qkvz_format=_FMT.get(s.qkvz_format, abi.GDN_FMT_BF16),
        ssm_state_dtype=abi.GDN_STATE_BF16 if s.ssm_state_dtype == SSM_BF16 else abi.GDN_STATE_F32,
        has_residual=1 if s.has_residual else 0,
        norm_eps=s.norm_eps, gated_norm_eps=s.gated_norm_eps, l2norm_eps=s.l2norm_eps,
        input_normed=1 if s.input_normed else 0, fold_out_proj=1 if s.fold_out_proj else 0,
        mx_scale_rule=abi.GDN_MXSCALE_CEIL if s.mx_scale_rule == MX_SCALE_CEIL else abi.GDN_MXSCALE_ROUNDED_MAX)


def _check(t: torch.Tensor, name: str, dtype, shape, device):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


class GdnBlock:
    """One handle of the HIP decode block for a fixed shape."""

    def __init__(self, shape: GdnShape, max_rows: int | None = None, device=None):
        self.shape = shape
        self.device = torch.device(device) if device is not None else torch.device("cuda", torch.cuda.current_device())
        with torch.cuda.device(self.device):
            self.handle = abi.gdn_block_create(make_config(shape, max_rows))
        self.max_rows = shape.max_rows if max_rows is None else max_rows

    def close(self):
        if getattr(self, "handle", None):
            abi.gdn_block_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def weights_struct(self, w) -> abi.GdnBlockWeights:
        """Pointers of a GdnWeights whose tensors already live on the device (checked)."""
        s, d = self.shape, self.device
        H = s.hidden
        st = abi.GdnBlockWeights()
        st.norm_w = None if s.input_normed else _check(w.norm_w, "norm_w", torch.bfloat16, (H,), d)
        if s.qkvz_format == FMT_MXFP4:
            st.w_qkvz = _check(w.w_qkvz, "w_qkvz", torch.uint8, (s.n_qkvz, H // 2), d)
            st.w_qkvz_scales = _check(w.w_qkvz_scales, "w_qkvz_scales", torch.uint8, (s.n_qkvz, H // 32), d)
        elif s.qkvz_format == FMT_MXFP6:
            st.w_qkvz = _check(w.w_qkvz, "w_qkvz", torch.uint8, (s.n_qkvz, H // 32, 24), d)
            st.w_qkvz_scales = _check(w.w_qkvz_scales, "w_qkvz_scales", torch.uint8, (s.n_qkvz, H // 32), d)
        else:
            st.w_qkvz = _check(w.w_qkvz, "w_qkvz", torch.bfloat16, (s.n_qkvz, H), d)
            st.w_qkvz_scales = None
        st.w_ba = _check(w.w_ba, "w_ba", torch.bfloat16, (s.n_ba, H), d)
        st.conv_w = _check(w.conv_w, "conv_w", torch.bfloat16, (s.conv_dim, s.conv_width), d)
        st.A_log = _check(w.A_log, "A_log", torch.float32, (s.num_v_heads,), d)
        st.dt_bias = _check(w.dt_bias, "dt_bias", torch.bfloat16, (s.num_v_heads,), d)
        st.gated_norm_w = _check(w.gated_norm_w, "gated_norm_w", torch.bfloat16, (s.head_v_dim,), d)
        st.w_proj_packed = None
        st.w_out = _check(w.w_out, "w_out", torch.bfloat16, (H, s.value_dim), d) if s.fold_out_proj else None
        return st

    def pack(self, w, stream=None) -> torch.Tensor:
        """The tiled projection copy of `w` (a new device tensor), enqueued on `stream`."""
        st = self.weights_struct(w)
        out = torch.empty(abi.gdn_block_packed_weight_bytes(self.handle), dtype=torch.uint8, device=self.device)
        if stream is None:
            stream = torch.cuda.current_stream(self.device).cuda_stream
        abi.gdn_block_pack_weights(self.handle, st, out.data_ptr(), stream)
        return out

    def packed_struct(self, w, packed: torch.Tensor) -> abi.GdnBlockWeights:
        """Weights struct that streams `packed` (from pack()) for the projections. The struct
        holds raw device pointers: keep `packed` (and the weights) alive while it is used."""
        st = self.weights_struct(w)
        _check(packed, "packed", torch.uint8, (abi.gdn_block_packed_weight_bytes(self.handle),), self.device)
        st.w_proj_packed = packed.data_ptr()
        return st

    def set_spin_limit(self, polls: int) -> None:
        """Poll limit of the bounded waits of later decodes (see the header)."""
        abi.gdn_block_set_spin_limit(self.handle, polls)

    def check(self) -> int:
        """Sticky error word of this handle's decodes (0 = every wait completed)."""
        return abi.gdn_block_check(self.handle)

    def decode(self, x, residual, weights, conv_state, ssm_state, state_idx, core_out, rows=None,
               stream=None, weights_struct=None, out=None, noalloc=False):
        """Enqueue one decode step on `stream` (default: torch's current stream).

        With a shape that folds out_proj, `out` ([R, H] bf16) receives the rank's out_proj
        partial. With `noalloc` the step runs through gdn_block_decode_noalloc (the
        library's fixed per-GPU scratch instead of the handle's).

        `weights` is a GdnWeights on the device, or pass a prepared
        `weights_struct` (from weights_struct()) to skip re-checking."""
        s, d = self.shape, self.device
        R = x.shape[0] if rows is None else rows
        H = s.hidden
        ws = weights_struct if weights_struct is not None else self.weights_struct(weights)
        ssm_dtype = torch.bfloat16 if s.ssm_state_dtype == SSM_BF16 else torch.float32
        px = _check(x, "x", torch.bfloat16, (R, H), d)
        pr = None if s.input_normed else _check(residual, "residual", torch.bfloat16, (R, H), d)
        pc = _check(conv_state, "conv_state", torch.bfloat16,
                    (s.num_state_slots, s.conv_width - 1, s.conv_dim), d)
        ps = _check(ssm_state, "ssm_state", ssm_dtype,
                    (s.num_state_slots, s.num_v_heads, s.head_k_dim, s.head_v_dim), d)
        pi = _check(state_idx, "state_idx", torch.int32, (R,), d)
        po = _check(core_out, "core_out", torch.bfloat16, (R, s.value_dim), d)
        if stream is None:
            stream = torch.cuda.current_stream(d).cuda_stream
        if s.fold_out_proj:
            pout = _check(out, "out", torch.bfloat16, (R, H), d)
            abi.gdn_block_decode_with_out_proj(self.handle, px, pr, ws, pc, ps, pi, R, po, pout, stream)
        elif noalloc:
            abi.gdn_block_decode_noalloc(self.handle, px, pr, ws, pc, ps, pi, R, po, stream)
        else:
            abi.gdn_block_decode(self.handle, px, pr, ws, pc, ps, pi, R, po, stream)

    def verify(self, x, residual, weights, conv_state, ssm_state, src_idx, dst_idx, core_out,
               stream=None, weights_struct=None):
        """Enqueue one verify step: `rows` sequences of `tokens` tokens (dst_idx is
        [rows, tokens] int32; x, residual and core_out have rows * tokens rows, token t
        of sequence r at row r * tokens + t). See gdn_block_verify in the header."""
        s, d = self.shape, self.device
        rows, tokens = dst_idx.shape
        R = rows * tokens
        H = s.hidden
        ws = weights_struct if weights_struct is not None else self.weights_struct(weights)
        ssm_dtype = torch.bfloat16 if s.ssm_state_dtype == SSM_BF16 else torch.float32
        px = _check(x, "x", torch.bfloat16, (R, H), d)
        pr = None if s.input_normed else _check(residual, "residual", torch.bfloat16, (R, H), d)
        pc = _check(conv_state, "conv_state", torch.bfloat16,
                    (s.num_state_slots, s.conv_width - 1, s.conv_dim), d)
        ps = _check(ssm_state, "ssm_state", ssm_dtype,
                    (s.num_state_slots, s.num_v_heads, s.head_k_dim, s.head_v_dim), d)
        pi = _check(src_idx, "src_idx", torch.int32, (rows,), d)
        pd = _check(dst_idx, "dst_idx", torch.int32, (rows, tokens), d)
        po = _check(core_out, "core_out", torch.bfloat16, (R, s.value_dim), d)
        if stream is None:
            stream = torch.cuda.current_stream(d).cuda_stream
        abi.gdn_block_verify(self.handle, px, pr, ws, pc, ps, pi, pd, rows, tokens, po, stream)
