"""Small test helpers: views of bf16 tensors as numpy bit patterns, and the
oracle's view of a synthetic call."""
import numpy as np
import torch


def u16(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> numpy uint16 bit patterns (a copy, on the CPU)."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16).copy()


def from_u16(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16)).view(torch.bfloat16)


def oracle_cfg(shape) -> dict:
    return dict(hidden=shape.hidden, num_k_heads=shape.num_k_heads, head_k_dim=shape.head_k_dim,
                num_v_heads=shape.num_v_heads, head_v_dim=shape.head_v_dim,
                conv_width=shape.conv_width, ssm_state_dtype=shape.ssm_state_dtype,
                has_residual=shape.has_residual, qkvz_format=shape.qkvz_format,
                norm_eps=shape.norm_eps, gated_norm_eps=shape.gated_norm_eps,
                l2norm_eps=shape.l2norm_eps)


def oracle_weights(w) -> dict:
    out = {}
    for k, v in w.tensors().items():
        if v.dtype == torch.bfloat16:
            out[k] = u16(v)
        else:
            out[k] = v.numpy().copy()
    return out


def oracle_state(t: torch.Tensor) -> np.ndarray:
    return u16(t) if t.dtype == torch.bfloat16 else t.detach().cpu().numpy().copy()


def run_oracle(shape, weights, call):
    import oracle
    return oracle.decode_block(oracle_cfg(shape), oracle_weights(weights), u16(call.x),
                               u16(call.residual), u16(call.conv_state),
                               oracle_state(call.ssm_state), call.state_idx.numpy().copy())
