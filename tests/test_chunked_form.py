"""The chunked form of the gated delta rule that verify steps evaluate at head dim 128,
checked in float64 against the oracle's token-by-token recurrence (CPU).

With k_t, q_t normalised, a_t = exp(g_t), Gm(i..t) = a_i ... a_t (1 when empty) and S0 the
state the step starts from, substituting the update S_t = a_t S_{t-1} + k_t d_t^T into
itself gives, for every token t of the step,
    d_t = beta_t (v_t - Gm(0..t) S0^T k_t - sum_{j<t} Gm(j+1..t) (k_j . k_t) d_j)
    o_t = Gm(0..t) S0^T q_t + sum_{j<=t} Gm(j+1..t) (k_j . q_t) d_j
and the states S_t follow from the d_t one token after another. The kernel computes
exactly these quantities (S0^T k and S0^T q on the matrix cores, the dot products, the
coefficient tables, a forward substitution over the tokens, then the serial update); this
test restates the algebra on its own and holds it to the oracle's gated_delta_recurrence,
so that the reading is pinned independently of the GPU.
"""
import numpy as np
import pytest

from oracle import gdn as og


def _chunked(S0, qs, ks, vs, gs, betas):
    T = len(ks)
    a = np.exp(np.asarray(gs, np.float64))
    K, Q, V = (np.asarray(x, np.float64) for x in (ks, qs, vs))
    U, W = K @ S0, Q @ S0                     # rows: S0^T k_t, S0^T q_t
    KK, QK = K @ K.T, Q @ K.T                 # KK[t, j] = k_t . k_j, QK[t, j] = q_t . k_j

    def gm(i, t):                             # a_i ... a_t, 1 when i > t
        return float(np.prod(a[i:t + 1])) if i <= t else 1.0

    D = np.zeros_like(V)
    O = np.zeros_like(V)
    for t in range(T):
        acc = gm(0, t) * U[t]
        for j in range(t):
            acc = acc + gm(j + 1, t) * KK[t, j] * D[j]
        D[t] = betas[t] * (V[t] - acc)
        o = gm(0, t) * W[t]
        for j in range(t + 1):
            o = o + gm(j + 1, t) * QK[t, j] * D[j]
        O[t] = o
    S = np.array(S0, np.float64)
    states = []
    for t in range(T):
        S = a[t] * S + np.outer(K[t], D[t])
        states.append(S.copy())
    return np.array(states), O


def _draw(rng, T, dk, dv, g_scale):
    S0 = rng.standard_normal((dk, dv)) * 0.3
    ks = rng.standard_normal((T, dk))
    ks /= np.linalg.norm(ks, axis=1, keepdims=True)
    qs = rng.standard_normal((T, dk))
    qs /= np.linalg.norm(qs, axis=1, keepdims=True) * np.sqrt(dk)
    vs = rng.standard_normal((T, dv))
    gs = -np.abs(rng.standard_normal(T)) * g_scale
    betas = rng.uniform(0.0, 1.0, T)
    return S0, qs, ks, vs, gs, betas


@pytest.mark.parametrize("T", [1, 2, 3, 4, 7, 16])
@pytest.mark.parametrize("g_scale", [0.05, 1.0, 30.0])
def test_chunked_form_equals_the_token_by_token_recurrence(T, g_scale):
    rng = np.random.Generator(np.random.PCG64(1000 * T + int(10 * g_scale)))
    dk = dv = 32
    S0, qs, ks, vs, gs, betas = _draw(rng, T, dk, dv, g_scale)
    states, O = _chunked(S0, qs, ks, vs, gs, betas)
    S = S0
    for t in range(T):
        S, o = og.gated_delta_step(S, qs[t], ks[t], vs[t], gs[t], betas[t])
        np.testing.assert_allclose(O[t], o, rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(states[t], S, rtol=1e-10, atol=1e-12)


def test_chunked_form_with_a_decay_that_underflows():
    """A decay of exp(-800) is 0 in float64: the products of decays then vanish instead of
    turning into 0/0 (the kernel multiplies decays directly, never divides them)."""
    rng = np.random.Generator(np.random.PCG64(7))
    S0, qs, ks, vs, gs, betas = _draw(rng, 5, 16, 16, 0.1)
    gs[2] = -800.0
    states, O = _chunked(S0, qs, ks, vs, gs, betas)
    S_ref, O_ref = og.gated_delta_recurrence(S0, qs, ks, vs, gs, betas)
    np.testing.assert_allclose(O, O_ref, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(states[-1], S_ref, rtol=1e-10, atol=1e-12)
    assert np.all(np.isfinite(O))


def test_chunked_form_beta_extremes():
    """beta = 0 leaves only the decayed read-out; beta = 1 writes v exactly along k."""
    rng = np.random.Generator(np.random.PCG64(11))
    S0, qs, ks, vs, gs, betas = _draw(rng, 4, 16, 16, 0.5)
    for b in (0.0, 1.0):
        betas[:] = b
        states, O = _chunked(S0, qs, ks, vs, gs, betas)
        S_ref, O_ref = og.gated_delta_recurrence(S0, qs, ks, vs, gs, betas)
        np.testing.assert_allclose(O, O_ref, rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(states[-1], S_ref, rtol=1e-10, atol=1e-12)
    # beta = 1: the state after token t maps k_t to v_t exactly
    np.testing.assert_allclose(states[-1].T @ ks[-1], vs[-1], rtol=1e-10, atol=1e-10)
