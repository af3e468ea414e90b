"""Pins of the oracle's scalar-decay special case (one decay per token and head).

With a scalar decay the factors commute with every key-space operation, so with
gamma_t = prod_{s<=t} alpha_s the gated rule equals the plain (ungated) delta rule run
on values v_t / gamma_t and rescaled afterwards:  S_t = gamma_t Shat_t, o_t = gamma_t ohat_t.
The plain delta rule is written out here in a few lines of its own, so the identity pins
where the decay enters (before the delta read, on the whole state) independently of the
oracle's code.  A planted mutant (decay applied after the write) must fail it.
"""
import numpy as np
import pytest

from oracle import kda_ref as R


def _plain_delta_rule(q, k, v, beta, S0, scale):
    """DeltaNet without decay, one head: S_t = S + beta k (v - S^T k)^T, o_t = S_t^T (scale q)."""
    S = S0.copy()
    o = np.empty((q.shape[0], v.shape[1]))
    for t in range(q.shape[0]):
        S = S + beta[t] * np.outer(k[t], v[t] - S.T @ k[t])
        o[t] = S.T @ (scale * q[t])
    return o, S


def _inputs(seed, B=2, H=2, T=12, K=5, V=3):
    r = np.random.default_rng(seed)
    q = r.standard_normal((B, H, T, K))
    k = r.standard_normal((B, H, T, K))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = r.standard_normal((B, H, T, V))
    a = r.standard_normal((B, H, T))
    beta = 1 / (1 + np.exp(-r.standard_normal((B, H, T))))
    A_log = np.array([-1.0, 0.3])[:H]
    dt_bias = np.array([0.2, -0.4])[:H]
    S0 = 0.1 * r.standard_normal((B, H, K, V))
    return q, k, v, a, beta, A_log, dt_bias, S0


def _gamma_identity(q, k, v, g, beta, S0, scale):
    """o and S_T from the rescaled plain delta rule."""
    B, H, T, _ = q.shape
    o = np.empty(v.shape)
    S = np.empty(S0.shape)
    for b in range(B):
        for h in range(H):
            gam = np.exp(np.cumsum(g[b, h]))
            oh, Sh = _plain_delta_rule(q[b, h], k[b, h], v[b, h] / gam[:, None], beta[b, h], S0[b, h], scale)
            o[b, h] = gam[:, None] * oh
            S[b, h] = gam[-1] * Sh
    return o, S


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_scalar_decay_equals_rescaled_plain_delta_rule(seed):
    q, k, v, a, beta, A_log, dt_bias, S0 = _inputs(seed)
    g, alpha = R.gate_scalar(a, A_log, dt_bias)
    assert np.all(g <= 0) and np.all((alpha >= 0) & (alpha <= 1))
    o, S = R.recurrent_scalar(q, k, v, g, beta, S0, scale=0.7)
    o_ref, S_ref = _gamma_identity(q, k, v, g, beta, S0, 0.7)
    assert R.rel_err(o, o_ref) < 1e-12 and R.rel_err(S, S_ref) < 1e-12


def test_decay_after_the_write_fails_the_identity():
    """Mutant: S_t = alpha (S + beta k (v - S^T k)^T) (decay applied after the delta
    write).  It is a different rule and must be visibly red against the identity."""
    q, k, v, a, beta, A_log, dt_bias, S0 = _inputs(5)
    g, alpha = R.gate_scalar(a, A_log, dt_bias)
    B, H, T, K = q.shape
    o = np.empty(v.shape)
    for b in range(B):
        for h in range(H):
            S = S0[b, h].copy()
            for t in range(T):
                S = alpha[b, h, t] * (S + beta[b, h, t] * np.outer(k[b, h, t], v[b, h, t] - S.T @ k[b, h, t]))
                o[b, h, t] = S.T @ (0.7 * q[b, h, t])
    o_ref, _ = _gamma_identity(q, k, v, g, beta, S0, 0.7)
    assert R.rel_err(o, o_ref) > 1e-2


def test_scalar_gate_values():
    """Hand values: A_log = 0, bias 0, a = 0 gives g = -log 2; a large negative input gives
    g -> 0 (no decay); the A_log clamp at 20 bounds the multiplier; g stays finite."""
    g, _ = R.gate_scalar(np.zeros((1, 1, 1)), np.zeros(1), None)
    assert abs(g[0, 0, 0] + np.log(2.0)) < 1e-15
    g, alpha = R.gate_scalar(np.full((1, 1, 1), -60.0), np.zeros(1), None)
    assert abs(g[0, 0, 0]) < 1e-25 and alpha[0, 0, 0] == 1.0
    g25, _ = R.gate_scalar(np.ones((1, 1, 1)), np.array([25.0]), None)
    g20, _ = R.gate_scalar(np.ones((1, 1, 1)), np.array([20.0]), None)
    assert g25[0, 0, 0] == g20[0, 0, 0] and np.isfinite(g20).all()
    g, _ = R.gate_scalar(np.full((1, 1, 1), 50.0), np.array([20.0]), None)
    assert np.isfinite(g).all() and g[0, 0, 0] < 0


def test_chunked_form_under_scalar_decay():
    """The chunked WY form with the decay copied to every channel equals the scalar recurrence."""
    q, k, v, a, beta, A_log, dt_bias, S0 = _inputs(7, T=37)
    g, _ = R.gate_scalar(a, A_log, dt_bias)
    o, S = R.recurrent_scalar(q, k, v, g, beta, S0)
    gk = np.broadcast_to(g[..., None], q.shape)
    for chunk in (4, 16):
        oc, Sc = R.chunked(q, k, v, gk, beta, S0, chunk=chunk)
        assert R.rel_err(oc, o) < 1e-12 and R.rel_err(Sc, S) < 1e-12
