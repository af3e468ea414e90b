"""Pins of the f64 oracle's forward to facts that do not come from the oracle itself.

Each test names what fixes the expected value: a value worked by hand
(tests/golden/hand_examples.json), a statement of the pages (kdafix page "Fix 1 --
decay form" and "Fix 2 -- read scale"; the CI page "The numbers"; the adjoint page
section 2), a closed form, or an algebraically different formulation of the same
recurrence.
"""
import json
import os

import numpy as np
import pytest

import kda_synth as ks
from oracle import kda_ref as R

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hand_examples.json")))


def _bh(x):
    """Lift per-head arrays (T,...) to (1,1,T,...)."""
    return np.asarray(x, dtype=np.float64)[None, None]


def _rand(B=1, H=2, T=13, K=4, V=3, seed=0, decay=0.3):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, H, T, K))
    k = rng.standard_normal((B, H, T, K))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, H, T, V))
    g = -decay * rng.random((B, H, T, K))
    beta = rng.random((B, H, T))
    S0 = 0.1 * rng.standard_normal((B, H, K, V))
    return q, k, v, g, beta, S0


# ----------------------------------------------------------------------------- hand examples
@pytest.mark.parametrize("name", ["scalar_ungated", "two_dim_orthogonal_keys"])
def test_hand_examples_ungated(name):
    ex = GOLD[name]
    K, V = ex["K"], ex["V"]
    q = np.array(ex["q"], dtype=np.float64).reshape(-1, K)
    k = np.array(ex["k"], dtype=np.float64).reshape(-1, K)
    v = np.array(ex["v"], dtype=np.float64).reshape(-1, V)
    g = np.array(ex["g"], dtype=np.float64).reshape(-1, K)
    beta = np.array(ex["beta"], dtype=np.float64)
    S0 = np.array(ex["state_in"], dtype=np.float64).reshape(K, V)
    o, S = R.recurrent(_bh(q), _bh(k), _bh(v), _bh(g), _bh(beta), S0[None, None], scale=ex["scale"])
    np.testing.assert_allclose(o[0, 0, :, 0], ex["o"], rtol=0, atol=ex["tol"])
    np.testing.assert_allclose(S[0, 0].ravel(), np.ravel(ex["state_out"]), rtol=0, atol=ex["tol"])


def test_hand_example_decayed_read():
    ex = GOLD["scalar_gated_decayed_read"]
    g = np.log(np.array(ex["alpha"]))[:, None]
    o, S = R.recurrent(_bh(np.array(ex["q"])[:, None]), _bh(np.array(ex["k"])[:, None]),
                       _bh(np.array(ex["v"])[:, None]), _bh(g), _bh(np.array(ex["beta"])),
                       np.array([[[[ex["state_in"]]]]]), scale=ex["scale"])
    np.testing.assert_allclose(o[0, 0, :, 0], ex["o"], rtol=0, atol=ex["tol"])
    assert abs(S[0, 0, 0, 0] - ex["state_out"]) <= ex["tol"]


def test_gate_hand_values():
    cases = GOLD["gate_values"]["cases"]
    tol = GOLD["gate_values"]["tol"]
    for c in cases:
        z = np.full((1, 1, 1, 1), c["z"])
        A = np.array([c["A_log"]])
        dt = np.array([[c["dt_bias"]]])
        _, a = R.gate(z, A, dt)
        if "alpha" in c:
            assert abs(a.item() - c["alpha"]) <= tol, c
            _, ap = R.gate_prefix_form(z, A, dt)
            assert abs(ap.item() - c["alpha_prefix_form"]) <= tol, c
        else:
            _, a_ref = R.gate(z, np.array([c["alpha_equals_A_log"]]), dt)
            assert a.item() == a_ref.item()


# ----------------------------------------------------------------------------- gate facts
def test_gate_forms_agree_only_at_A0():
    """kdafix page, Fix 1: the two forms are different functions that agree at A = 0."""
    z = np.linspace(-10, 10, 161)[None, None, :, None]
    dt = np.zeros((1, 1))
    g0, _ = R.gate(z, np.array([0.0]), dt)
    gp0, _ = R.gate_prefix_form(z, np.array([0.0]), dt)
    assert np.array_equal(g0, gp0)
    for A in (-3.0, -0.5, 0.5, 2.0):
        g, _ = R.gate(z, np.array([A]), dt)
        gp, _ = R.gate_prefix_form(z, np.array([A]), dt)
        assert np.max(np.abs(g - gp)) > 1e-3


def test_gate_order_flips_with_sign_of_A():
    """kdafix page, Fix 1: the order of the two answers flips with the sign of A
    (at A = -3, z = +1 the released form gives the larger alpha)."""
    z = np.linspace(-10, 10, 161)[None, None, :, None]
    dt = np.zeros((1, 1))
    for A in np.linspace(-10, 20, 121):
        if A == 0:
            continue
        _, a = R.gate(z, np.array([A]), dt)
        _, ap = R.gate_prefix_form(z, np.array([A]), dt)
        d = (a - ap).ravel()
        informative = np.abs(d) > 1e-12 * np.maximum(np.abs(a).ravel(), 1e-300)
        if A < 0:
            assert np.all(d[informative] > 0), A
        else:
            assert np.all(d[informative] < 0), A
    _, a = R.gate(np.ones((1, 1, 1, 1)), np.array([-3.0]), dt)
    _, ap = R.gate_prefix_form(np.ones((1, 1, 1, 1)), np.array([-3.0]), dt)
    assert a.item() > ap.item()


def test_gate_nonpositive_and_finite_at_extremes():
    """kdafix page, Fix 1: g <= 0 elementwise, so alpha = exp(g) is never NaN;
    saturation is an underflow of alpha to 0."""
    z = np.linspace(-50, 50, 1001)[None, None, :, None]
    for A in (-10.0, -3.0, 0.0, 5.0, 20.0, 25.0):
        for dt in (-5.0, 0.0, 5.0):
            g, a = R.gate(z, np.array([A]), np.array([[dt]]))
            assert np.all(np.isfinite(g)) and np.all(g <= 0)
            assert np.all((a >= 0) & (a <= 1)) and not np.any(np.isnan(a))
    g, a = R.gate(np.array([[[[50.0]]]]), np.array([20.0]), np.zeros((1, 1)))
    assert a.item() == 0.0


def test_recurrence_finite_with_saturated_gates():
    q, k, v, _, beta, S0 = _rand(T=20)
    z = np.random.default_rng(3).uniform(-50, 50, q.shape)
    o, S = R.forward(q, k, v, z, np.array([20.0, -10.0]), np.zeros((2, 4)), beta, S0)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(S))
    oc, Sc = R.chunked(q, k, v, R.gate(z, np.array([20.0, -10.0]), np.zeros((2, 4)))[0], beta, S0, chunk=8)
    assert np.all(np.isfinite(oc)) and np.all(np.isfinite(Sc))
    assert R.rel_err(oc, o) < 1e-12 and R.rel_err(Sc, S) < 1e-12


# ----------------------------------------------------------------------------- read scale
def test_output_linear_in_scale_state_independent():
    """kdafix page, Fix 2: the scale enters only the read (and the intra-chunk
    scores), never the state update."""
    q, k, v, g, beta, S0 = _rand()
    o1, S1 = R.recurrent(q, k, v, g, beta, S0, scale=1.0)
    for s in (0.0, 0.25, 0.5, 3.0):
        o, S = R.recurrent(q, k, v, g, beta, S0, scale=s)
        assert np.array_equal(S, S1)
        np.testing.assert_allclose(o, s * o1, rtol=1e-14, atol=1e-14)
        oc, Sc = R.chunked(q, k, v, g, beta, S0, scale=s, chunk=4)
        np.testing.assert_allclose(oc, s * o1, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(Sc, S1, rtol=1e-12, atol=1e-12)


def test_scale_ratio_K8_matches_ci_page():
    """CI page, 'The numbers': unscaled / K**-0.5-scaled output is exactly 2.8284 at K = 8."""
    ex = GOLD["read_scale_ratio_K8"]
    wl = ks.WORKLOADS["tiny"]
    x = ks.generate(wl)
    g, _ = R.gate(x["z"], x["A_log"], x["dt_bias"])
    o_unit, _ = R.recurrent(x["q"], x["k"], x["v"], g, x["beta"], x["state_in"], scale=1.0)
    o_def, _ = R.recurrent(x["q"], x["k"], x["v"], g, x["beta"], x["state_in"])
    assert R.read_scale(ex["K"]) == pytest.approx(1 / ex["ratio"], rel=1e-15)
    mask = np.abs(o_def) > 1e-6
    np.testing.assert_allclose(o_unit[mask] / o_def[mask], ex["ratio"], rtol=ex["tol"])


# ----------------------------------------------------------------------------- closed forms
def test_delta_rule_closed_form_beta1_q_eq_k():
    """beta = 1 and q = k with |k| = 1: the memory returns exactly what was written,
    o_t = scale * v_t, whatever the decay (the delta rule's defining property)."""
    q, k, v, g, beta, S0 = _rand(T=17, decay=2.0)
    o, _ = R.recurrent(k, k, v, g, np.ones_like(beta), S0, scale=0.7)
    np.testing.assert_allclose(o, 0.7 * v, rtol=0, atol=1e-12)
    oc, _ = R.chunked(k, k, v, g, np.ones_like(beta), S0, scale=0.7, chunk=8)
    np.testing.assert_allclose(oc, 0.7 * v, rtol=0, atol=1e-12)


def test_pure_decay_closed_form():
    """beta = 0: S_t = diag(prod_{s<=t} alpha_s) S0 and o_t = scale * S_t^T q_t."""
    q, k, v, g, beta, S0 = _rand(T=11)
    o, S = R.recurrent(q, k, v, g, np.zeros_like(beta), S0, scale=0.5)
    gam = np.cumprod(np.exp(g), axis=2)                       # (B,H,T,K)
    S_t = gam[..., :, None] * S0[:, :, None]                  # (B,H,T,K,V)
    o_ref = 0.5 * np.einsum("bhtk,bhtkv->bhtv", q, S_t)
    np.testing.assert_allclose(o, o_ref, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(S, S_t[:, :, -1], rtol=1e-13, atol=1e-14)


def test_transition_matrix_form():
    """The same recurrence written as explicit K x K transitions:
    S_t = (I - beta k k^T) diag(alpha) S_{t-1} + beta k v^T  (generalised Householder form)."""
    q, k, v, g, beta, S0 = _rand(T=9, K=5, V=4)
    o, S = R.recurrent(q, k, v, g, beta, S0, scale=0.3)
    for b in range(q.shape[0]):
        for h in range(q.shape[1]):
            St = S0[b, h].copy()
            for t in range(q.shape[2]):
                kt = k[b, h, t][:, None]
                M = (np.eye(5) - beta[b, h, t] * kt @ kt.T) @ np.diag(np.exp(g[b, h, t]))
                St = M @ St + beta[b, h, t] * kt @ v[b, h, t][None, :]
                np.testing.assert_allclose(o[b, h, t], 0.3 * St.T @ q[b, h, t], rtol=1e-12, atol=1e-13)
            np.testing.assert_allclose(S[b, h], St, rtol=1e-12, atol=1e-13)


def test_ungated_limit_is_plain_delta_rule():
    """z = -60 makes softplus underflow, so alpha = 1 exactly in f64 and the model is
    the plain (ungated) delta rule: compare against g = 0."""
    q, k, v, _, beta, S0 = _rand(T=10)
    z = np.full(q.shape, -60.0)
    o, S = R.forward(q, k, v, z, np.array([0.0, 3.0]), np.zeros((2, 4)), beta, S0)
    o0, S0_ = R.recurrent(q, k, v, np.zeros_like(q), beta, S0)
    assert np.array_equal(o, o0) and np.array_equal(S, S0_)


# ----------------------------------------------------------------------------- chunked == recurrent
@pytest.mark.parametrize("chunk", [1, 4, 8, 16, 32, 5, 7])
def test_chunked_equals_recurrent(chunk):
    """Brute-force equality of the chunk-parallel (WY) and token forms on tiny inputs."""
    for wl_name in ("tiny",):
        x = ks.generate(ks.WORKLOADS[wl_name])
        g, _ = R.gate(x["z"], x["A_log"], x["dt_bias"])
        o1, S1 = R.recurrent(x["q"], x["k"], x["v"], g, x["beta"], x["state_in"])
        o2, S2 = R.chunked(x["q"], x["k"], x["v"], g, x["beta"], x["state_in"], chunk=chunk)
        assert R.rel_err(o2, o1) < 1e-12 and R.rel_err(S2, S1) < 1e-12
    q, k, v, g, beta, S0 = _rand(T=29, K=6, V=5, decay=3.0)
    o1, S1 = R.recurrent(q, k, v, g, beta, S0)
    o2, S2 = R.chunked(q, k, v, g, beta, S0, chunk=chunk)
    assert R.rel_err(o2, o1) < 1e-12 and R.rel_err(S2, S1) < 1e-12


def test_chunked_equals_recurrent_layer_workload_subset():
    """The fp32 single-layer workload (A_log up to 20: alpha underflows to 0 in some
    heads) over its first 96 tokens, chunk 32."""
    wl = ks.WORKLOADS["layer"]
    x = ks.generate(wl, T=96)
    g, _ = R.gate(x["z"], x["A_log"], x["dt_bias"])
    o1, S1 = R.recurrent(x["q"], x["k"], x["v"], g, x["beta"], x["state_in"])
    o2, S2 = R.chunked(x["q"], x["k"], x["v"], g, x["beta"], x["state_in"], chunk=32)
    assert R.rel_err(o2, o1) < 1e-11 and R.rel_err(S2, S1) < 1e-11


# ----------------------------------------------------------------------------- resume / padding
def test_resume_split_equals_whole():
    """state_out of a first call fed as state_in of a second equals one call over both."""
    q, k, v, g, beta, S0 = _rand(T=23)
    o, S = R.recurrent(q, k, v, g, beta, S0)
    for cut in (1, 8, 15):
        oa, Sa = R.recurrent(q[:, :, :cut], k[:, :, :cut], v[:, :, :cut], g[:, :, :cut], beta[:, :, :cut], S0)
        ob, Sb = R.recurrent(q[:, :, cut:], k[:, :, cut:], v[:, :, cut:], g[:, :, cut:], beta[:, :, cut:], Sa)
        assert np.array_equal(np.concatenate([oa, ob], axis=2), o) and np.array_equal(Sb, S)


def test_identity_token_padding():
    """Tokens with g = 0, beta = 0 and q = k = v = 0 leave the state unchanged and read 0."""
    q, k, v, g, beta, S0 = _rand(T=10)
    o, S = R.recurrent(q, k, v, g, beta, S0)
    pad = lambda x: np.concatenate([x, np.zeros(x.shape[:2] + (6,) + x.shape[3:])], axis=2)
    op, Sp = R.recurrent(pad(q), pad(k), pad(v), pad(g), pad(beta), S0)
    assert np.array_equal(Sp, S) and np.array_equal(op[:, :, :10], o) and np.all(op[:, :, 10:] == 0)


def test_decode_step_equals_recurrence():
    """recurrent_step applied token by token equals recurrent()."""
    q, k, v, g, beta, S0 = _rand(T=6)
    o, S = R.recurrent(q, k, v, g, beta, S0, scale=0.4)
    St = S0
    for t in range(6):
        ot, St = R.recurrent_step(q[:, :, t], k[:, :, t], v[:, :, t], g[:, :, t], beta[:, :, t], St, scale=0.4)
        assert np.array_equal(ot, o[:, :, t])
    assert np.array_equal(St, S)


def test_rel_err_definition():
    ref = np.array([1.0, -4.0, 2.0])
    assert R.rel_err(ref + np.array([0.0, 0.4, 0.0]), ref) == pytest.approx(0.1)
    assert R.rel_err(np.zeros(3), np.zeros(3)) == 0.0


# ----------------------------------------------------------------------------- output RMSNorm (reading R20)
def test_rmsnorm_hand_rows():
    """Two hand-worked rows, with and without eps (tests/golden, 'rmsnorm_rows'): the mean
    runs over the V outputs of one token (not over tokens, not a sum), and the weight row
    multiplies after the division."""
    ex = GOLD["rmsnorm_rows"]
    o = np.array(ex["o"])
    w = np.array(ex["weight"])
    for case in ex["cases"]:
        y = R.rmsnorm(o, w, eps=case["eps"])
        assert np.allclose(y, np.array(case["y"]), rtol=0, atol=ex["tol"]), case["derivation"]


def test_rmsnorm_absorbs_the_read_scale_to_eps_over_mean_square():
    """kdafix page, 'Fix 2 -- read scale': the norm after the read absorbs a constant
    factor on o up to O(eps / mean(o^2)).  For o and c o the rows differ by the factor
    sqrt((m + eps) / (m + eps / c^2)) (m = mean(o^2)), which lies in (1, 1 + eps / (2m)];
    with eps = 0 the norm is exactly invariant.  c = 8**0.5 is the page's K = 8 ratio."""
    rng = np.random.default_rng(3)
    o = rng.standard_normal((2, 3, 5, 16)) + 0.5
    w = rng.uniform(0.5, 2.0, (3, 16))
    c = GOLD["read_scale_ratio_K8"]["ratio"]
    eps = 1e-5
    y1, yc = R.rmsnorm(o, w, eps), R.rmsnorm(c * o, w, eps)
    m = np.mean(o * o, axis=-1, keepdims=True)
    ratio = yc / y1
    assert np.allclose(ratio, np.sqrt((m + eps) / (m + eps / c ** 2)), rtol=1e-13, atol=0)
    assert np.all(ratio > 1.0) and np.all(ratio - 1.0 <= eps / (2 * m) * (1 + 1e-9))
    assert np.max(np.abs(yc - y1)) / np.max(np.abs(y1)) < 1e-4        # "~1e-5" at mean(o^2) ~ 1
    assert np.allclose(R.rmsnorm(c * o, w, 0.0), R.rmsnorm(o, w, 0.0), rtol=1e-14, atol=0)


def test_rmsnorm_unit_mean_square_and_per_head_weight():
    """With eps = 0 and no weight every row has mean square 1; a weight row acts on its
    own head only, column by column."""
    rng = np.random.default_rng(4)
    o = rng.standard_normal((2, 3, 7, 8))
    y = R.rmsnorm(o, None, 0.0)
    assert np.allclose(np.mean(y * y, axis=-1), 1.0, rtol=1e-14, atol=0)
    w = np.ones((3, 8))
    w[1, 2] = 3.0
    yw = R.rmsnorm(o, w, 0.0)
    assert np.array_equal(yw[:, [0, 2]], y[:, [0, 2]])
    assert np.allclose(yw[:, 1, :, 2], 3.0 * y[:, 1, :, 2], rtol=1e-15, atol=0)
    assert np.array_equal(np.delete(yw[:, 1], 2, axis=-1), np.delete(y[:, 1], 2, axis=-1))
