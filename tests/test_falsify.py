"""Falsification: plant known mistakes in the oracle (on the CPU) and show that the
pins go red.  This is the adjoint page's section 5b pattern (re-insert the
double-exp carry bug and watch the two-chunk gate fire while the one-chunk gate
stays green) and the kdafix page's mutants (decay form, read scale in the state).

Every mutant is installed with monkeypatch, so the real oracle is restored after
each test with no backup file involved (the page's section 5c lesson).
"""
import json
import os

import numpy as np
import pytest

import kda_synth as ks
from oracle import kda_ref as R

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hand_examples.json")))


def _tiny():
    x = ks.generate(ks.WORKLOADS["tiny"])
    g, _ = R.gate(x["z"], x["A_log"], x["dt_bias"])
    return x, g


def _double_exp_carry(g):
    # the bug of the adjoint page, section 2: the cumsum exponentiated twice
    G = np.cumsum(g, axis=0)
    return np.exp(np.exp(G[-1])[None, :] - G)


def test_double_exp_carry_is_invisible_at_one_chunk_and_red_at_two(monkeypatch):
    x, g = _tiny()
    args = (x["q"], x["k"], x["v"], g, x["beta"], x["state_in"])
    o_ref, S_ref = R.recurrent(*args)
    monkeypatch.setattr(R, "_carry_decay", _double_exp_carry)
    o_mut, S_mut = R.chunked(*args, chunk=16)
    # inside the first chunk the output does not use the carry: green there ...
    assert R.rel_err(o_mut[:, :, :16], o_ref[:, :, :16]) < 1e-12
    # ... the second chunk and the final state see it
    assert R.rel_err(o_mut[:, :, 16:], o_ref[:, :, 16:]) > 1e-2
    assert R.rel_err(S_mut, S_ref) > 1e-2


def _step_undecayed_read(S, q_t, k_t, v_t, alpha_t, beta_t, scale):
    r = np.sum(S * k_t[..., :, None], axis=-2)             # reads S_{t-1}, not diag(alpha) S_{t-1}
    S_new = alpha_t[..., :, None] * S + beta_t[..., None, None] * k_t[..., :, None] * (v_t - r)[..., None, :]
    return S_new, np.sum(S_new * (scale * q_t)[..., :, None], axis=-2)


def test_undecayed_read_mutant_fails_closed_forms(monkeypatch):
    monkeypatch.setattr(R, "_step", _step_undecayed_read)
    ex = GOLD["scalar_gated_decayed_read"]
    g = np.log(np.array(ex["alpha"]))[:, None]
    o, _ = R.recurrent(np.array(ex["q"])[None, None, :, None], np.array(ex["k"])[None, None, :, None],
                       np.array(ex["v"])[None, None, :, None], g[None, None], np.array(ex["beta"])[None, None],
                       np.array([[[[ex["state_in"]]]]]), scale=1.0)
    assert abs(o[0, 0, 0, 0] - ex["o"][0]) > 0.5
    rng = np.random.default_rng(0)
    k = rng.standard_normal((1, 1, 9, 4))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((1, 1, 9, 3))
    o, _ = R.recurrent(k, k, v, -rng.random((1, 1, 9, 4)), np.ones((1, 1, 9)),
                       rng.standard_normal((1, 1, 4, 3)), scale=1.0)
    assert np.max(np.abs(o - v)) > 1e-3


def _step_scale_in_state(S, q_t, k_t, v_t, alpha_t, beta_t, scale):
    # the read scale leaking into the write (the kdafix page's k_scale mutant)
    kk = scale * k_t
    Sd = alpha_t[..., :, None] * S
    r = np.sum(Sd * kk[..., :, None], axis=-2)
    S_new = Sd + beta_t[..., None, None] * kk[..., :, None] * (v_t - r)[..., None, :]
    return S_new, np.sum(S_new * q_t[..., :, None], axis=-2)


def test_scale_in_state_mutant_fails_scale_pins(monkeypatch):
    x, g = _tiny()
    args = (x["q"], x["k"], x["v"], g, x["beta"], x["state_in"])
    monkeypatch.setattr(R, "_step", _step_scale_in_state)
    _, S1 = R.recurrent(*args, scale=1.0)
    _, S2 = R.recurrent(*args, scale=0.5)
    assert not np.array_equal(S1, S2)


def _gate_prefix(z, A_log, dt_bias):
    return R.gate_prefix_form(z, A_log, dt_bias)


def test_prefix_gate_mutant_fails_gate_values_but_not_A0(monkeypatch):
    cases = GOLD["gate_values"]["cases"]
    real = R.gate
    monkeypatch.setattr(R, "gate", _gate_prefix)
    red = []
    for c in cases[:3]:
        z = np.full((1, 1, 1, 1), c["z"])
        _, a = R.gate(z, np.array([c["A_log"]]), np.array([[c["dt_bias"]]]))
        red.append(abs(a.item() - c["alpha"]) > 1e-6)
    assert red == [False, True, False]          # A = 0 cases agree: the page's A=0 control
    monkeypatch.setattr(R, "gate", real)


def _step_adjoint_missing_term(dS, S_prev, S_t, q_t, k_t, v_t, a_t, b_t, do_t, scale):
    dS_prev, (dq, dk, dv, dg, db) = REAL_STEP_ADJOINT(dS, S_prev, S_t, q_t, k_t, v_t, a_t, b_t, do_t, scale)
    # drop the -S' de contribution to dk (a plausible transcription slip)
    Sd = a_t[..., :, None] * S_prev
    dSp = dS + (scale * q_t)[..., :, None] * do_t[..., None, :]
    de = b_t[..., None] * np.sum(dSp * k_t[..., :, None], axis=-2)
    dk = dk + np.sum(Sd * de[..., None, :], axis=-1)
    return dS_prev, (dq, dk, dv, dg, db)


REAL_STEP_ADJOINT = R._step_adjoint


def test_adjoint_mutant_fails_fd(monkeypatch):
    x, g = _tiny()
    args = dict(q=x["q"].astype(np.float64), k=x["k"].astype(np.float64), v=x["v"].astype(np.float64),
                g=g, beta=x["beta"].astype(np.float64), state_in=x["state_in"].astype(np.float64))
    d_o = np.random.default_rng(1).standard_normal(x["v"].shape)
    monkeypatch.setattr(R, "_step_adjoint", _step_adjoint_missing_term)
    grads = R.adjoint(*(args[n] for n in ("q", "k", "v", "g", "beta", "state_in")), d_o)
    d = np.random.default_rng(2).standard_normal(args["k"].shape)

    def fn(kk):
        return R.loss(args["q"], kk, args["v"], args["g"], args["beta"], args["state_in"], d_o)

    fd = R.fd_directional(fn, args["k"], d)
    an = float(np.sum(grads["dk"] * d))
    assert abs(fd - an) / max(abs(an), 1.0) > 1e-3


def _gate_adjoint_sigmoid_of_z(z, A_log, dt_bias, dg):
    # slope taken at z instead of z + dt_bias (a dropped term)
    z = np.asarray(z, dtype=np.float64)
    m = np.exp(np.clip(np.asarray(A_log, dtype=np.float64), R.A_LOG_MIN, R.A_LOG_MAX))[None, :, None, None]
    x = z + np.asarray(dt_bias, dtype=np.float64)[None, :, None, :]
    dz = -m * R.sigmoid(z) * dg
    dA = np.sum(dg * (-m * R.softplus(x)), axis=(0, 2, 3))
    return dz, dA, np.sum(dz, axis=(0, 2))


def _gate_adjoint_no_clamp_mask(z, A_log, dt_bias, dg):
    # the clamp ignored: A_log outside [-10, 20] still receives a gradient
    dz, _, ddb = R.__dict__["_gate_adjoint_real"](z, A_log, dt_bias, dg)
    m = np.exp(np.clip(np.asarray(A_log, dtype=np.float64), R.A_LOG_MIN, R.A_LOG_MAX))[None, :, None, None]
    x = np.asarray(z, dtype=np.float64) + np.asarray(dt_bias, dtype=np.float64)[None, :, None, :]
    return dz, np.sum(dg * (-m * R.softplus(x)), axis=(0, 2, 3)), ddb


@pytest.mark.parametrize("mutant", [_gate_adjoint_sigmoid_of_z, _gate_adjoint_no_clamp_mask])
def test_gate_adjoint_mutants_fail_pins(monkeypatch, mutant):
    import test_oracle_adjoint as TA
    monkeypatch.setattr(R, "_gate_adjoint_real", R.gate_adjoint, raising=False)
    monkeypatch.setattr(R, "gate_adjoint", mutant)
    failed = 0
    for fn, args in ((TA.test_gate_adjoint_matches_central_differences, ("z",)),
                     (TA.test_gate_adjoint_closed_forms, ())):
        try:
            fn(*args)
        except AssertionError:
            failed += 1
    assert failed >= 1


# ----------------------------------------------------------------------------- output RMSNorm mutants
def _rms_sum_not_mean(o, weight=None, eps=1e-6):
    o = np.asarray(o, dtype=np.float64)
    y = o / np.sqrt(np.sum(o * o, axis=-1, keepdims=True) + eps)
    return y if weight is None else y * np.asarray(weight)[None, :, None, :]


def _rms_over_tokens(o, weight=None, eps=1e-6):
    o = np.asarray(o, dtype=np.float64)
    y = o / np.sqrt(np.mean(o * o, axis=-2, keepdims=True) + eps)
    return y if weight is None else y * np.asarray(weight)[None, :, None, :]


def _rms_eps_outside(o, weight=None, eps=1e-6):
    o = np.asarray(o, dtype=np.float64)
    y = o / (np.sqrt(np.mean(o * o, axis=-1, keepdims=True)) + eps)
    return y if weight is None else y * np.asarray(weight)[None, :, None, :]


@pytest.mark.parametrize("mutant", [_rms_sum_not_mean, _rms_over_tokens, _rms_eps_outside])
def test_rmsnorm_mutants_fail_the_hand_rows(monkeypatch, mutant):
    ex = GOLD["rmsnorm_rows"]
    monkeypatch.setattr(R, "rmsnorm", mutant)
    bad = 0
    for case in ex["cases"]:
        y = R.rmsnorm(np.array(ex["o"]), np.array(ex["weight"]), eps=case["eps"])
        bad += not np.allclose(y, np.array(case["y"]), rtol=0, atol=ex["tol"])
    assert bad >= 1
