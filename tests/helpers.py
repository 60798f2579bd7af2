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
                l2norm_eps=shape.l2norm_eps, input_normed=shape.input_normed,
                mx_scale_rule=shape.mx_scale_rule)


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


def pow2_rows(hidden: int, rows: int, seed: int):
    """Rows whose Gemma RMSNorm (weight 0) is exact on any hardware, and the exact norm.

    Every element is 0 or +-2^p (p in -4..1); the last 64 elements fill the row's sum of
    squares up to hidden * 4^j for the smallest such j (base-4 digits of the remainder),
    so mean(h^2) = 4^j exactly, rstd = 2^-j (1 - delta) with delta <= 5e-7 for eps = 1e-6,
    and bf16(h * rstd) = h * 2^-j exactly: far from any bf16 rounding boundary. Sums of
    these squares are exact in f32 up to hidden = 8192. Returns (x [rows, H] float64,
    xn [rows, H] float64)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    body = hidden - 64
    x = np.zeros((rows, hidden))
    xn = np.zeros((rows, hidden))
    for r in range(rows):
        p = rng.integers(-4, 2, size=body)
        v = np.where(rng.random(body) < 0.1, 0.0, rng.choice([-1.0, 1.0], size=body) * np.exp2(p))
        ss = float(np.sum(v * v))
        j = 0
        while hidden * 4.0 ** j < ss:
            j += 1
        rem = int(round((hidden * 4.0 ** j - ss) * 256))  # 256 * (sum the filler must add)
        fill, m = [], 0
        while rem:
            fill += [2.0 ** (m - 4)] * (rem % 4)  # (2^(m-4))^2 = 4^m / 256
            rem //= 4
            m += 1
        assert len(fill) <= 64
        fill = np.array(fill + [0.0] * (64 - len(fill))) * rng.choice([-1.0, 1.0], size=64)
        x[r] = np.concatenate([v, fill])
        assert float(np.sum(x[r] * x[r])) == hidden * 4.0 ** j
        xn[r] = x[r] * 2.0 ** -j
    return x, xn
