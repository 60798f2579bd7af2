"""Float64 CPU oracle of the Gated DeltaNet (GDN) decode block.

TEST INFRASTRUCTURE: imported only by tests/, __graft_entry__.smoke() and the
bench's cpu_baseline leg. Never by the HIP path.

What the block computes, per decode row (the step list of "sgl-amd-mono PR #89",
Modifications: residual add and input norm, in_proj_qkvz and in_proj_ba, conv
update, gated delta rule, gated norm; the same list in "vLLM PR #60833",
Details / Launches):

  1. h = bf16(x + residual) (or h = x for the layer with no residual input);
     the residual buffer receives h.
  2. Gemma RMSNorm: xn = bf16(h * rstd * (1 + w)), rstd = (mean(h^2) + eps)^-1/2
     ("SGLang PR #43558", Modifications: rstd as 1 / sqrt(sum / n + eps)).
  3. y = bf16(W xn) for in_proj_qkvz and in_proj_ba (exact sum, one rounding:
     "SGLang PR #43558", Accuracy, stock GEMM == bf16(fp32(exact sum))).
     MXFP4 in_proj_qkvz: xn is quantised per 32-element block first
     ("vLLM PR #60833", Details / MoE: dynamic MXFP4, 1x32 blocks; Details /
     MXFP4 layouts: two scale roundings), with either scale rule.
  4. split y into q, k, v, z, b, a (grouped per key head).
  5. pad row (state index <= 0, or past the pool): core row = +0, no state written.
  6. depthwise causal conv update, width 4, no bias, SiLU; the conv state
     keeps the last W-1 raw inputs.
  7. g = -exp(A_log) * softplus(a + dt_bias), beta = sigmoid(b).
  8. q, k L2-normalised over the head dim, q scaled by dk^-1/2.
  9. S <- exp(g) S;  S <- S + k (beta (v - S^T k))^T;  o = S^T q
     (S in R^{dk x dv}), stored back as f32 or as RNE bf16
     ("sgl-amd-mono PR #89", Kernel checks: the bf16 state is the f32 result
     rounded to bf16).
 10. RMSNormGated over the head, norm before gate:
     core = bf16(bf16(o) * rstd * w * SiLU(z)).

Readings taken where the pages are silent are listed in the design doc's readings
table (layouts, eps values, softplus threshold, rounding points).

Arrays: bf16 tensors are numpy uint16 bit patterns, f32 tensors float32,
indices int32. All arithmetic is float64.
"""
from __future__ import annotations

import numpy as np

# --------------------------------------------------------------------------------------
# storage types


def bf16_to_f64(bits) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to float64 (exact)."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


_BF16_MIN_NORMAL = 2.0 ** -126
_BF16_SUB_ULP = 2.0 ** -133       # spacing of bf16 subnormals


def f64_to_bf16(v) -> np.ndarray:
    """Round float64 values to the nearest bf16, ties to even; uint16 bit patterns.

    The rounding is done once, from the float64 value (no detour through f32):
    the 52-bit f64 fraction is cut to bf16's 7 bits by adding half an ulp
    minus one plus the kept lsb, then masking, which carries into the exponent
    like any round-to-nearest-even. bf16 subnormals (|v| < 2^-126) are rounded
    on their fixed 2^-133 grid. Inputs are finite and below bf16's maximum.
    """
    v = np.asarray(v, dtype=np.float64)
    bits = v.view(np.uint64)
    keep_lsb = (bits >> np.uint64(45)) & np.uint64(1)
    rounded = (bits + np.uint64((1 << 44) - 1) + keep_lsb) & ~np.uint64((1 << 45) - 1)
    r = rounded.view(np.float64)
    small = np.abs(v) < _BF16_MIN_NORMAL
    if np.any(small):
        r = np.where(small, np.rint(v / _BF16_SUB_ULP) * _BF16_SUB_ULP, r)
        r = np.where(small & (v < 0) & (r == 0), -0.0, r)   # keep the sign of zero
    out = (r.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    return out


def _round_bf16(v) -> np.ndarray:
    """bf16 rounding, returned as the float64 value it stands for."""
    return bf16_to_f64(f64_to_bf16(v))


# --------------------------------------------------------------------------------------
# elementwise functions (float64)


def silu(x):
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(over="ignore"):
        return x / (1.0 + np.exp(-x))


def sigmoid(x):
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-x))


def softplus(x):
    """log(1 + e^x), returning x itself above 20 (the usual threshold)."""
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(over="ignore"):
        return np.where(x > 20.0, x, np.log1p(np.exp(np.minimum(x, 20.0))))


# --------------------------------------------------------------------------------------
# step 1-2: residual add and Gemma RMSNorm ("sgl-amd-mono PR #89", Kernels before
# and after: _gemma_fused_add_rmsnorm_kernel, and _gemma_rmsnorm_kernel on layer 0)


def residual_add(x_bits, res_bits, has_residual: bool):
    """h = bf16(x + residual); for the layer without a residual input, h = x.

    The residual buffer is written with h for every row, pad rows included.
    """
    if not has_residual:
        return np.array(x_bits, dtype=np.uint16, copy=True)
    return f64_to_bf16(bf16_to_f64(x_bits) + bf16_to_f64(res_bits))


def gemma_rmsnorm(h_bits, w_bits, eps: float):
    """xn = bf16(h * rstd * (1 + w)), rstd = 1 / sqrt(mean(h^2) + eps), per row.

    "Gemma" RMSNorm scales by (1 + w); the rstd formula follows "SGLang PR
    #43558", Modifications (the dense FFN kernel's norm description).
    """
    h = bf16_to_f64(h_bits)
    w = bf16_to_f64(w_bits)
    rstd = 1.0 / np.sqrt(np.mean(h * h, axis=-1, keepdims=True) + eps)
    return f64_to_bf16(h * rstd * (1.0 + w))


# --------------------------------------------------------------------------------------
# step 3: projections


def project_bf16(w_bits, xn_bits):
    """y = bf16(W xn): W is [N, H] (output rows, K contiguous), xn is [..., H].

    The float64 sum of bf16 products is exact to 2^-53 relative: one rounding
    of (nearly) the exact sum, as "SGLang PR #43558", Accuracy, describes the
    stock GEMM.
    """
    w = bf16_to_f64(w_bits)
    xn = bf16_to_f64(xn_bits)
    return f64_to_bf16(xn @ w.T)


E2M1_VALUES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


MX_SCALE_ROUNDED_MAX = "rounded_max"
MX_SCALE_CEIL = "ceil"


def mx_block_exponent(amax, mant_bits: int, rule: str = MX_SCALE_ROUNDED_MAX):
    """Block scale exponent e (scale 2^e) of an MX block with maximum magnitude amax.

    rounded_max: the rule "vLLM PR #60833" (a reviewer's comment proposing MXFP6, how
    to make the weights, step 2) gives for AITER's dynamic_mxfp4_quant: the block
    maximum is rounded at the element format's mantissa width (half up, a carry moving
    into the exponent) and the scale is 2 to the exponent of that rounded maximum minus
    2. With amax = M 2^E (1 <= M < 2) and m mantissa bits, M rounds up to 2 exactly when
    floor(M 2^m + 1/2) = 2^(m+1).
    ceil: the smallest e with amax <= 6 2^e (E2M1's largest magnitude is 6), the literal
    round-up of amax / 6 to a power of two ("RCEIL"); no element saturates.
    Both clamp e to [-126, 127]; an all-zero block keeps 2^-126, a normal scale (the
    all-zero handling of the same page's rounding of step 2, so no 0 / 0).
    """
    amax = np.asarray(amax, dtype=np.float64)
    nz = amax > 0
    safe = np.where(nz, amax, 1.0)
    if rule == MX_SCALE_ROUNDED_MAX:
        mant, ex = np.frexp(safe)                      # safe = mant 2^ex, mant in [0.5, 1)
        M, E = 2.0 * mant, (ex - 1).astype(np.int64)   # safe = M 2^E, M in [1, 2)
        carry = np.floor(M * 2.0 ** mant_bits + 0.5) >= 2.0 ** (mant_bits + 1)
        e = E + carry.astype(np.int64) - 2
    elif rule == MX_SCALE_CEIL:
        _, p = np.frexp(safe / 6.0)                    # a first guess, adjusted exactly below
        e = p.astype(np.int64)
        for _ in range(3):                             # exact comparisons against 6 * 2^e
            e = np.where(safe > 6.0 * np.exp2(e.astype(np.float64)), e + 1, e)
            e = np.where(safe <= 6.0 * np.exp2((e - 1).astype(np.float64)), e - 1, e)
    else:
        raise ValueError(f"unknown MX scale rule {rule!r}")
    return np.clip(np.where(nz, e, -126), -126, 127)


def mxfp4_quantize(v, rule: str = MX_SCALE_ROUNDED_MAX):
    """Quantise values to OCP MXFP4: e2m1 codes with one e8m0 scale per 32.

    "vLLM PR #60833", Details / MoE: dynamic MXFP4 with 1x32 blocks; the same page
    (Details / MXFP4 layouts) names two roundings of the scale, one per FP4 GEMM
    family. `rule` picks the block exponent e (mx_block_exponent, with E2M1's one
    mantissa bit). Each v / 2^e is rounded to the nearest e2m1 value
    {0, .5, 1, 1.5, 2, 3, 4, 6}, ties to the even code; values past 6 (the
    rounded-max rule allows up to 7) take 6, the nearest.

    Returns (codes uint8 [..., K], 4-bit sign|magnitude; scale bytes uint8
    [..., K/32] = e + 127).
    """
    v = np.asarray(v, dtype=np.float64)
    blocks = v.reshape(v.shape[:-1] + (v.shape[-1] // 32, 32))
    amax = np.abs(blocks).max(axis=-1)
    e = mx_block_exponent(amax, 1, rule)
    scaled = np.abs(blocks) / np.exp2(e.astype(np.float64))[..., None]
    # nearest e2m1 magnitude, ties to the even code
    d = np.abs(scaled[..., None] - E2M1_VALUES)
    best = np.argmin(d, axis=-1)                 # lowest code among equals
    dmin = np.take_along_axis(d, best[..., None], axis=-1)[..., 0]
    nxt = np.minimum(best + 1, 7)
    dn = np.take_along_axis(d, nxt[..., None], axis=-1)[..., 0]
    tie = (nxt != best) & (dn == dmin)
    best = np.where(tie & (best % 2 == 1), nxt, best)
    sign = (blocks < 0) & (best > 0)
    codes = (best | (sign.astype(np.int64) << 3)).astype(np.uint8)
    return codes.reshape(v.shape), (e + 127).astype(np.uint8)


def mxfp4_dequantize(codes, scale_bytes):
    """Values of e2m1 codes (uint8 [..., K]) with e8m0 block scales ([..., K/32])."""
    codes = np.asarray(codes, dtype=np.uint8)
    mag = E2M1_VALUES[codes & 7]
    val = np.where(codes & 8, -mag, mag)
    sc = np.exp2(np.asarray(scale_bytes, dtype=np.float64) - 127.0)
    return val * np.repeat(sc, 32, axis=-1)


def unpack_e2m1(packed):
    """[..., K/2] bytes -> [..., K] codes; the low nibble holds the even element."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & 0x0F
    out[..., 1::2] = p >> 4
    return out


def project_mxfp4(w_packed, w_scales, xn_bits, rule: str = MX_SCALE_ROUNDED_MAX):
    """y = bf16(sum over K of dequant(W) * dequant(quant(xn))) for MXFP4 weights.

    The activation xn (bf16) is quantised per row and 32-block by
    mxfp4_quantize with the scale rule `rule`; both operands' products are exact
    and summed in float64.
    """
    w = mxfp4_dequantize(unpack_e2m1(w_packed), w_scales)
    xq_codes, xq_scales = mxfp4_quantize(bf16_to_f64(xn_bits), rule)
    xq = mxfp4_dequantize(xq_codes, xq_scales)
    return f64_to_bf16(xq @ w.T)


# MXFP6 E2M3 weights with bf16 activations (W6A16): "vLLM PR #60833", a reviewer's
# comment proposing MXFP6 for the GDN projections (how to make the weights, and their
# packing for the kernels).
#
# OCP E2M3: a 6-bit code sign | 2 exponent bits | 3 mantissa bits, exponent bias 1; a zero
# exponent field is subnormal (m / 8), otherwise (1 + m / 8) * 2^(exp - 1); the largest
# magnitude is 7.5. One e8m0 byte scales each block of 32 along K by 2^(byte - 127).

E2M3_VALUES = np.array([m / 8.0 for m in range(8)] +
                       [(1.0 + m / 8.0) * 2.0 ** (e - 1) for e in range(1, 4) for m in range(8)])


def mxfp6_round(v):
    """The pages' rounding of weights onto MXFP6 E2M3, one block of 32 along K at a time.

    The block scale is the rounded-maximum rule of mx_block_exponent with E2M3's 3
    mantissa bits (the same page names it as AITER's dynamic_mxfp4_quant with the E2M3
    maximum of 7.5): the block maximum is rounded to 3 mantissa bits (half up, a carry
    moving into the exponent), and with E the exponent of that rounded maximum the scale
    is 2^(E - 2), clamped to 2^[-126, 127] (an all-zero block keeps 2^-126, a normal
    scale). Each |v| / scale is rounded to the nearest E2M3 magnitude, ties to the even
    code (steps of 1/8 below 2, 1/4 below 4, 1/2 above), saturating at 7.5. A zero code
    carries no sign.

    Returns (codes uint8 [..., K] with the sign at bit 5, scale bytes uint8 [..., K/32]).
    """
    v = np.asarray(v, dtype=np.float64)
    blocks = v.reshape(v.shape[:-1] + (v.shape[-1] // 32, 32))
    amax = np.abs(blocks).max(axis=-1)
    e = mx_block_exponent(amax, 3, MX_SCALE_ROUNDED_MAX)
    a = np.abs(blocks) / np.exp2(e.astype(np.float64))[..., None]
    step = np.where(a < 2.0, 0.125, np.where(a < 4.0, 0.25, 0.5))
    q = np.minimum(np.round(a / step) * step, 7.5)       # np.round: half to even
    mag = np.searchsorted(E2M3_VALUES, q)
    assert np.all(E2M3_VALUES[mag] == q)
    sign = (blocks < 0) & (mag > 0)
    codes = (mag | (sign.astype(np.int64) << 5)).astype(np.uint8)
    return codes.reshape(v.shape), (e + 127).astype(np.uint8)


def mxfp6_dequantize(codes, scale_bytes):
    """Values of E2M3 codes (uint8 [..., K]) with e8m0 block scales ([..., K/32])."""
    codes = np.asarray(codes, dtype=np.uint8)
    mag = E2M3_VALUES[codes & 31]
    val = np.where(codes & 32, -mag, mag)
    sc = np.exp2(np.asarray(scale_bytes, dtype=np.float64) - 127.0)
    return val * np.repeat(sc, 32, axis=-1)


def pack_e2m3(codes):
    """[..., K] codes -> [..., K/32, 24] bytes: code i of a block at bits 6i .. 6i+5 of
    the block's 24 bytes read as one little-endian 192-bit number."""
    c = np.asarray(codes, dtype=np.uint8)
    blk = c.reshape(c.shape[:-1] + (c.shape[-1] // 32, 32)).astype(np.uint64)
    out = np.zeros(blk.shape[:-1] + (24,), dtype=np.uint8)
    for i in range(32):
        for b in range(6):
            bit = 6 * i + b
            out[..., bit // 8] |= (((blk[..., i] >> np.uint64(b)) & np.uint64(1)) << np.uint64(bit % 8)).astype(np.uint8)
    return out


def unpack_e2m3(packed):
    """[..., K/32, 24] bytes (or [..., K*3/4]) -> [..., K] codes (inverse of pack_e2m3)."""
    p = np.asarray(packed, dtype=np.uint8)
    p = p.reshape(p.shape[:-1] + (p.shape[-1] // 24, 24)) if p.shape[-1] != 24 else p
    bits = np.unpackbits(p, axis=-1, bitorder="little")          # [..., nb, 192]
    bits = bits.reshape(bits.shape[:-1] + (32, 6)).astype(np.uint8)
    codes = (bits * (1 << np.arange(6, dtype=np.uint8))).sum(axis=-1).astype(np.uint8)
    return codes.reshape(codes.shape[:-2] + (codes.shape[-2] * 32,))


def project_mxfp6(w_packed, w_scales, xn_bits):
    """y = bf16(sum over K of dequant(W) * xn) for MXFP6 E2M3 weights and bf16 activations
    (W6A16: the activations are not quantised). An E2M3 value times a power of two is a
    bf16 value, and the sum is exact in float64 before the one rounding."""
    w = mxfp6_dequantize(unpack_e2m3(w_packed), w_scales)
    return f64_to_bf16(bf16_to_f64(xn_bits) @ w.T)


# --------------------------------------------------------------------------------------
# step 4: split of the projection outputs (the stock chain's separate split kernel,
# "sgl-amd-mono PR #89", Kernels before and after). Grouped per key head:
# qkvz group g = [q_g (dk) | k_g (dk) | v_g (r*dv) | z_g (r*dv)], ba group g = [b_g (r) | a_g (r)].


def split_qkvz(y, nk: int, dk: int, nv: int, dv: int):
    r = nv // nk
    g = np.asarray(y).reshape(nk, 2 * dk + 2 * r * dv)
    q = g[:, :dk]
    k = g[:, dk:2 * dk]
    v = g[:, 2 * dk:2 * dk + r * dv].reshape(nv, dv)
    z = g[:, 2 * dk + r * dv:].reshape(nv, dv)
    return q, k, v, z


def split_ba(y, nk: int, nv: int):
    r = nv // nk
    g = np.asarray(y).reshape(nk, 2 * r)
    return g[:, :r].reshape(nv), g[:, r:].reshape(nv)


# --------------------------------------------------------------------------------------
# step 6: causal depthwise conv update ("sgl-amd-mono PR #89", Refusals: a conv with
# no bias and with SiLU; the state is bf16)


def conv_update(state_bits, new_bits, w_bits):
    """One decode step of a causal depthwise conv of width W over C channels.

    state_bits: [W-1, C] the W-1 previous raw inputs, oldest first.
    new_bits:   [C] this step's raw input.
    w_bits:     [C, W]; tap W-1 multiplies the newest input.
    Returns (out bf16 [C] = bf16(SiLU(sum_j w[:, j] * window[j])),
             new state [W-1, C] = the last W-1 raw inputs).
    """
    window = np.concatenate([np.asarray(state_bits, np.uint16),
                             np.asarray(new_bits, np.uint16)[None, :]], axis=0)   # [W, C]
    wf = bf16_to_f64(window)
    acc = np.sum(bf16_to_f64(w_bits).T * wf, axis=0)
    return f64_to_bf16(silu(acc)), window[1:].copy()


# --------------------------------------------------------------------------------------
# step 7-10: gates, L2 norm, gated delta rule, gated RMSNorm


def gates(a, b, A_log, dt_bias):
    """g = -exp(A_log) * softplus(a + dt_bias);  beta = sigmoid(b)  (per value head)."""
    g = -np.exp(np.asarray(A_log, np.float64)) * softplus(np.asarray(a, np.float64)
                                                         + np.asarray(dt_bias, np.float64))
    return g, sigmoid(b)


def l2norm(x, eps: float):
    """x / sqrt(sum(x^2) + eps) over the last axis."""
    x = np.asarray(x, np.float64)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)


def gated_delta_step(S, q_hat, k_hat, v, g, beta):
    """One step of the gated delta rule on S in R^{dk x dv}.

    Decay first, then the delta write against the decayed state, then the
    read-out from the updated state:
        S <- exp(g) S;  u = S^T k;  S <- S + k (beta (v - u))^T;  o = S^T q.
    Returns (S_new, o).
    """
    S = np.exp(g) * np.asarray(S, np.float64)
    u = S.T @ k_hat
    delta = beta * (np.asarray(v, np.float64) - u)
    S = S + np.outer(k_hat, delta)
    return S, S.T @ q_hat


def gated_delta_recurrence(S0, qs, ks, vs, gs, betas):
    """Run gated_delta_step over T steps; returns (S_T, outputs [T, dv])."""
    S = np.asarray(S0, np.float64)
    outs = []
    for q, k, v, g, b in zip(qs, ks, vs, gs, betas):
        S, o = gated_delta_step(S, q, k, v, g, b)
        outs.append(o)
    return S, np.array(outs)


def gated_rmsnorm(o_bits, z_bits, w_bits, eps: float):
    """core = bf16(o * rstd * w * SiLU(z)), rstd = (mean(o^2) + eps)^-1/2 over the head.

    Norm before gate, plain weight w shared by all heads ("sgl-amd-mono PR #89",
    Refusals: a gated norm over the head with SiLU, norm before the gate).
    """
    o = bf16_to_f64(o_bits)
    rstd = 1.0 / np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + eps)
    return f64_to_bf16(o * rstd * bf16_to_f64(w_bits) * silu(bf16_to_f64(z_bits)))


# --------------------------------------------------------------------------------------
# the whole block


def out_proj(w_out_bits, core_bits):
    """The rank's out_proj partial: out = bf16(core W_out^T), core [R, nv*dv] and W_out
    [H, nv*dv] bf16, the sum exact in float64 and rounded once ("SGLang PR #43558",
    Modifications: K1 with out_proj folded in writes the rank's out_proj partial; the
    stock GEMM's output is bf16(fp32(exact sum)) there). A pad row's core is zero, so its
    partial is zero."""
    return project_bf16(w_out_bits, core_bits)


def decode_block(cfg: dict, weights: dict, x, residual, conv_state, ssm_state, state_idx):
    """One decode step of the GDN block over R rows (inputs are not modified).

    cfg: hidden, num_k_heads, head_k_dim, num_v_heads, head_v_dim, conv_width,
         ssm_state_dtype ('f32'|'bf16'), has_residual, qkvz_format
         ('bf16'|'mxfp4'|'mxfp6'), norm_eps, gated_norm_eps, l2norm_eps, optionally
         mx_scale_rule (the MXFP4 activation scale rule, 'rounded_max' unless given;
         see mx_block_exponent), and optionally
         input_normed: x is already the norm's output xn ("SGLang PR #43558",
         Modifications: the "normed" K1 build starts from input_layernorm's
         output), so the residual add and the norm are skipped and the
         residual is neither read nor returned (None).
    weights: norm_w, w_qkvz (bf16 bits [Nqkvz, H], packed e2m1 [Nqkvz, H/2] or packed
         E2M3 [Nqkvz, H/32, 24]), w_qkvz_scales (MXFP4 and MXFP6 only), w_ba, conv_w, A_log (f32), dt_bias, gated_norm_w.
    x, residual: [R, H] bf16 bits; conv_state [slots, W-1, Cd] bf16 bits;
    ssm_state [slots, nv, dk, dv] f32 or bf16 bits; state_idx [R] int32. A row whose
    index is <= 0 or >= slots is a pad row (an index past the pool names no slot).

    With weights["w_out"] ([H, nv*dv] bf16 bits) the rank's out_proj partial is
    returned too (out [R, H] bf16 bits; else None).

    Returns dict(core [R, nv*dv] bf16 bits, residual [R, H] bf16 bits,
                 conv_state, ssm_state (updated copies), out, y_qkvz, y_ba, xn).
    """
    nk, dk = cfg["num_k_heads"], cfg["head_k_dim"]
    nv, dv = cfg["num_v_heads"], cfg["head_v_dim"]
    r_grp = nv // nk
    R = len(state_idx)
    bf16_state = cfg["ssm_state_dtype"] == "bf16"

    if cfg.get("input_normed", False):
        h, xn = None, np.array(x, dtype=np.uint16, copy=True)
    else:
        h = residual_add(x, residual, cfg["has_residual"])
        xn = gemma_rmsnorm(h, weights["norm_w"], cfg["norm_eps"])
    if cfg["qkvz_format"] == "mxfp4":
        y_qkvz = project_mxfp4(weights["w_qkvz"], weights["w_qkvz_scales"], xn,
                               cfg.get("mx_scale_rule", MX_SCALE_ROUNDED_MAX))
    elif cfg["qkvz_format"] == "mxfp6":
        y_qkvz = project_mxfp6(weights["w_qkvz"], weights["w_qkvz_scales"], xn)
    else:
        y_qkvz = project_bf16(weights["w_qkvz"], xn)
    y_ba = project_bf16(weights["w_ba"], xn)

    core = np.zeros((R, nv * dv), dtype=np.uint16)
    conv_out = np.array(conv_state, copy=True)
    ssm_out = np.array(ssm_state, copy=True)
    A_log = np.asarray(weights["A_log"], np.float64)
    dt_bias = bf16_to_f64(weights["dt_bias"])

    slots = conv_state.shape[0]
    for row in range(R):
        slot = int(state_idx[row])
        if slot <= 0 or slot >= slots:  # pad row: zero core, no state touched
            continue
        q, k, v, z = split_qkvz(y_qkvz[row], nk, dk, nv, dv)
        b, a = split_ba(y_ba[row], nk, nv)
        qkv = np.concatenate([q.reshape(-1), k.reshape(-1), v.reshape(-1)])
        c, new_conv = conv_update(conv_out[slot], qkv, weights["conv_w"])
        conv_out[slot] = new_conv
        cq = bf16_to_f64(c[:nk * dk]).reshape(nk, dk)
        ck = bf16_to_f64(c[nk * dk:2 * nk * dk]).reshape(nk, dk)
        cv = bf16_to_f64(c[2 * nk * dk:]).reshape(nv, dv)
        g, beta = gates(bf16_to_f64(a), bf16_to_f64(b), A_log, dt_bias)
        q_hat = l2norm(cq, cfg["l2norm_eps"]) / np.sqrt(dk)
        k_hat = l2norm(ck, cfg["l2norm_eps"])
        for hv in range(nv):
            kappa = hv // r_grp
            S = bf16_to_f64(ssm_out[slot, hv]) if bf16_state else ssm_out[slot, hv].astype(np.float64)
            S, o = gated_delta_step(S, q_hat[kappa], k_hat[kappa], cv[hv], g[hv], beta[hv])
            ssm_out[slot, hv] = f64_to_bf16(S) if bf16_state else S.astype(np.float32)
            core[row, hv * dv:(hv + 1) * dv] = gated_rmsnorm(
                f64_to_bf16(o), z[hv], weights["gated_norm_w"], cfg["gated_norm_eps"])

    out = None
    if "w_out" in weights and weights["w_out"] is not None:
        out = out_proj(weights["w_out"], core)
    return dict(core=core, residual=h, conv_state=conv_out, ssm_state=ssm_out, out=out,
                y_qkvz=y_qkvz, y_ba=y_ba, xn=xn)


def verify_block(cfg: dict, weights: dict, x, residual, conv_state, ssm_state, src_idx, dst_idx):
    """A verify step of speculative decoding: R sequences of T tokens each (the accepted
    token and its drafts), with the state after every token kept, so that a caller can
    continue from whichever token is accepted ("sgl-amd-mono PR #89", Modifications, and
    "vLLM PR #60833", Limitations: K1 keeps no state per draft token, so a rejected draft
    could not roll back; this is that follow-up).

    x, residual: [R*T, H] bf16 bits, token t of sequence r at row r*T + t; the residual
    add, the norm and the projections are row by row, as in decode_block. src_idx [R]:
    the slot holding each sequence's state (<= 0 or >= slots: a pad sequence, zero core
    rows, no state touched). dst_idx [R, T]: after token t the sequence's conv window and
    SSM state (rounded to the pool's dtype) are written to slot dst_idx[r, t] when that is
    a valid slot, else that snapshot is not kept. Between the tokens of a step the state
    is carried unrounded (in float64 here): only the snapshots are stored values.

    Returns dict(core [R*T, nv*dv], residual, conv_state, ssm_state) like decode_block.
    """
    nk, dk = cfg["num_k_heads"], cfg["head_k_dim"]
    nv, dv = cfg["num_v_heads"], cfg["head_v_dim"]
    r_grp = nv // nk
    dst = np.asarray(dst_idx)
    R, T = dst.shape
    bf16_state = cfg["ssm_state_dtype"] == "bf16"
    slots = conv_state.shape[0]

    if cfg.get("input_normed", False):
        h, xn = None, np.array(x, dtype=np.uint16, copy=True)
    else:
        h = residual_add(x, residual, cfg["has_residual"])
        xn = gemma_rmsnorm(h, weights["norm_w"], cfg["norm_eps"])
    if cfg["qkvz_format"] == "mxfp4":
        y_qkvz = project_mxfp4(weights["w_qkvz"], weights["w_qkvz_scales"], xn,
                               cfg.get("mx_scale_rule", MX_SCALE_ROUNDED_MAX))
    elif cfg["qkvz_format"] == "mxfp6":
        y_qkvz = project_mxfp6(weights["w_qkvz"], weights["w_qkvz_scales"], xn)
    else:
        y_qkvz = project_bf16(weights["w_qkvz"], xn)
    y_ba = project_bf16(weights["w_ba"], xn)

    core = np.zeros((R * T, nv * dv), dtype=np.uint16)
    conv_out = np.array(conv_state, copy=True)
    ssm_out = np.array(ssm_state, copy=True)
    A_log = np.asarray(weights["A_log"], np.float64)
    dt_bias = bf16_to_f64(weights["dt_bias"])

    for seq in range(R):
        src = int(src_idx[seq])
        if src <= 0 or src >= slots:      # pad sequence
            continue
        window = np.array(conv_state[src], copy=True)
        S = [bf16_to_f64(ssm_state[src, hv]) if bf16_state else ssm_state[src, hv].astype(np.float64)
             for hv in range(nv)]
        for t in range(T):
            row = seq * T + t
            q, k, v, z = split_qkvz(y_qkvz[row], nk, dk, nv, dv)
            b, a = split_ba(y_ba[row], nk, nv)
            qkv = np.concatenate([q.reshape(-1), k.reshape(-1), v.reshape(-1)])
            c, window = conv_update(window, qkv, weights["conv_w"])
            cq = bf16_to_f64(c[:nk * dk]).reshape(nk, dk)
            ck = bf16_to_f64(c[nk * dk:2 * nk * dk]).reshape(nk, dk)
            cv = bf16_to_f64(c[2 * nk * dk:]).reshape(nv, dv)
            g, beta = gates(bf16_to_f64(a), bf16_to_f64(b), A_log, dt_bias)
            q_hat = l2norm(cq, cfg["l2norm_eps"]) / np.sqrt(dk)
            k_hat = l2norm(ck, cfg["l2norm_eps"])
            for hv in range(nv):
                kappa = hv // r_grp
                S[hv], o = gated_delta_step(S[hv], q_hat[kappa], k_hat[kappa], cv[hv], g[hv], beta[hv])
                core[row, hv * dv:(hv + 1) * dv] = gated_rmsnorm(
                    f64_to_bf16(o), z[hv], weights["gated_norm_w"], cfg["gated_norm_eps"])
            d = int(dst[seq, t])
            if 0 < d < slots:
                conv_out[d] = window
                for hv in range(nv):
                    ssm_out[d, hv] = f64_to_bf16(S[hv]) if bf16_state else S[hv].astype(np.float32)
    return dict(core=core, residual=h, conv_state=conv_out, ssm_state=ssm_out, y_qkvz=y_qkvz, y_ba=y_ba, xn=xn)
