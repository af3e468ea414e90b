"""Pins of the f64 oracle's adjoint: central finite differences of the pinned forward.

The adjoint page (sections 5a, 5b) keeps an f64 generator that refuses to write a
fixture unless forward-mode derivatives and central differences agree within 1e-9,
and (section 5, 5c-bis) insists on a gate spanning two chunks, where the state
carry is live.  Here every gradient of the reverse-mode oracle is compared against
central differences of `oracle.loss` (which runs the pinned token recurrence) at
one and at two chunks of tokens, plus per-coordinate on a tiny case.
"""
import numpy as np
import pytest

import kda_synth as ks
from oracle import kda_ref as R

BAR = 1e-7          # |fd - analytic| / max(|analytic|, 1) at h = 1e-6 in f64


def _inputs(T, seed=0, K=8, V=8, H=2):
    wl = ks.WORKLOADS["tiny"].with_(T=T, K=K, V=V, H=H)
    x = ks.generate(wl)
    g, _ = R.gate(x["z"], x["A_log"], x["dt_bias"])
    rng = np.random.default_rng(seed)
    d_o = rng.standard_normal(x["v"].shape)
    d_s = rng.standard_normal(x["state_in"].shape)
    args = dict(q=x["q"].astype(np.float64), k=x["k"].astype(np.float64), v=x["v"].astype(np.float64),
                g=g, beta=x["beta"].astype(np.float64), state_in=x["state_in"].astype(np.float64))
    return args, d_o, d_s


GRAD_OF = {"q": "dq", "k": "dk", "v": "dv", "g": "dg", "beta": "dbeta", "state_in": "dstate_in"}


@pytest.mark.parametrize("T", [16, 32])          # one chunk of 16, then two: carry live
@pytest.mark.parametrize("with_state_cotangent", [False, True])
def test_adjoint_matches_central_differences(T, with_state_cotangent):
    args, d_o, d_s = _inputs(T)
    d_s = d_s if with_state_cotangent else None
    grads = R.adjoint(args["q"], args["k"], args["v"], args["g"], args["beta"], args["state_in"],
                      d_o, d_s, segment=5)
    rng = np.random.default_rng(T)
    for name, gname in GRAD_OF.items():
        d = rng.standard_normal(np.shape(args[name]))

        def fn(x, name=name):
            a = dict(args)
            a[name] = x
            return R.loss(a["q"], a["k"], a["v"], a["g"], a["beta"], a["state_in"], d_o, d_s)

        fd = R.fd_directional(fn, args[name], d)
        an = float(np.sum(grads[gname] * d))
        assert abs(fd - an) / max(abs(an), 1.0) < BAR, (name, fd, an)


def test_adjoint_per_coordinate_tiny():
    """Every coordinate of every gradient on K=V=2, T=5 with the carry live."""
    args, d_o, d_s = _inputs(T=5, K=2, V=2, H=1)
    grads = R.adjoint(args["q"], args["k"], args["v"], args["g"], args["beta"], args["state_in"], d_o, d_s)
    for name, gname in GRAD_OF.items():
        x0 = args[name]
        for idx in np.ndindex(np.shape(x0)):
            e = np.zeros(np.shape(x0))
            e[idx] = 1.0

            def fn(x, name=name):
                a = dict(args)
                a[name] = x
                return R.loss(a["q"], a["k"], a["v"], a["g"], a["beta"], a["state_in"], d_o, d_s)

            fd = R.fd_directional(fn, x0, e)
            an = grads[gname][idx]
            assert abs(fd - an) < BAR * max(abs(an), 1.0), (name, idx, fd, an)


def test_adjoint_segment_length_does_not_matter():
    args, d_o, d_s = _inputs(T=32)
    a = R.adjoint(*(args[n] for n in ("q", "k", "v", "g", "beta", "state_in")), d_o, d_s, segment=64)
    b = R.adjoint(*(args[n] for n in ("q", "k", "v", "g", "beta", "state_in")), d_o, d_s, segment=3)
    for n in a:
        assert np.array_equal(a[n], b[n]), n


def test_two_chunk_gradients_differ_from_one_chunk():
    """Adjoint page, section 5c-bis: chunk 1's dk receives state-carry contributions
    chunk 0's does not; a two-token-chunk fixture is a different function."""
    args, d_o, _ = _inputs(T=32)
    g2 = R.adjoint(*(args[n] for n in ("q", "k", "v", "g", "beta", "state_in")), d_o)
    a1 = {n: (x[:, :, :16] if np.ndim(x) == 4 and n != "state_in" else x) for n, x in args.items()}
    a1["beta"] = args["beta"][:, :, :16]
    g1 = R.adjoint(*(a1[n] for n in ("q", "k", "v", "g", "beta", "state_in")), d_o[:, :, :16])
    assert R.rel_err(g2["dk"][:, :, :16], g1["dk"]) > 1e-3


# ---------------------------------------------------------------------------- gate adjoint
def _gate_inputs(seed=3, B=2, H=3, T=5, K=4):
    rng = np.random.default_rng(seed)
    z = rng.standard_normal((B, H, T, K)) * 2.0
    A_log = np.array([-1.5, 0.3, 1.1])[:H]
    dt_bias = rng.standard_normal((H, K)) * 0.5
    dg = rng.standard_normal((B, H, T, K))
    return z, A_log, dt_bias, dg


@pytest.mark.parametrize("wrt", ["z", "A_log", "dt_bias"])
def test_gate_adjoint_matches_central_differences(wrt):
    """dz, dA_log, d dt_bias against central differences of L = sum(dg * g) through
    the pinned gate() (the softplus-outside form of the decay page)."""
    z, A_log, dt_bias, dg = _gate_inputs()
    dz, dA, ddb = R.gate_adjoint(z, A_log, dt_bias, dg)
    vals = dict(z=z, A_log=A_log, dt_bias=dt_bias)
    grads = dict(z=dz, A_log=dA, dt_bias=ddb)
    d = np.random.default_rng(11).standard_normal(np.shape(vals[wrt]))

    def fn(x):
        a = dict(vals)
        a[wrt] = x
        return float(np.sum(dg * R.gate(a["z"], a["A_log"], a["dt_bias"])[0]))

    fd = R.fd_directional(fn, vals[wrt], d)
    an = float(np.sum(grads[wrt] * d))
    assert abs(fd - an) / max(abs(an), 1.0) < BAR, (wrt, fd, an)


def test_gate_adjoint_closed_forms():
    """At x = z + dt_bias = 0 the softplus slope is 1/2: dz = -exp(A_log) dg / 2.  A
    multiplier clamped at either bound passes no gradient to A_log (central
    differences there are exactly 0), and without dt_bias the bias gradient is
    still the per-channel sum of dz."""
    z, A_log, dt_bias, dg = _gate_inputs()
    zc = -np.broadcast_to(dt_bias[None, :, None, :], z.shape).copy()
    dz, _, _ = R.gate_adjoint(zc, A_log, dt_bias, dg)
    want = -np.exp(A_log)[None, :, None, None] * dg / 2.0
    assert np.allclose(dz, want, rtol=1e-14, atol=0.0)

    A_out = np.array([-12.0, 25.0, 0.5])
    _, dA, _ = R.gate_adjoint(z, A_out, dt_bias, dg)
    assert dA[0] == 0.0 and dA[1] == 0.0 and dA[2] != 0.0
    for h in (0, 1):
        e = np.zeros(3)
        e[h] = 1.0
        fd = R.fd_directional(lambda a: float(np.sum(dg * R.gate(z, a, dt_bias)[0])), A_out, e)
        assert fd == 0.0

    dz0, _, ddb0 = R.gate_adjoint(z, A_log, None, dg)
    assert np.allclose(ddb0, dz0.sum(axis=(0, 2)), rtol=1e-14)


def test_gate_adjoint_composes_with_the_recurrence_adjoint():
    """End to end: d/dz of L = sum(o * d_o) through gate() and the token recurrence
    equals gate_adjoint applied to the recurrence adjoint's dg (central differences
    of the whole forward)."""
    wl = ks.WORKLOADS["tiny"].with_(T=12, K=4, V=4, H=2)
    x = ks.generate(wl)
    q, k, v, beta = (x[n].astype(np.float64) for n in ("q", "k", "v", "beta"))
    S0 = x["state_in"].astype(np.float64)
    z, A_log, dt_bias = x["z"].astype(np.float64), x["A_log"], x["dt_bias"]
    d_o = np.random.default_rng(5).standard_normal(v.shape)
    g, _ = R.gate(z, A_log, dt_bias)
    dg = R.adjoint(q, k, v, g, beta, S0, d_o)["dg"]
    dz, dA, ddb = R.gate_adjoint(z, A_log, dt_bias, dg)
    rng = np.random.default_rng(17)
    for name, val, grad in (("z", z, dz), ("A_log", np.asarray(A_log, np.float64), dA),
                            ("dt_bias", np.asarray(dt_bias, np.float64), ddb)):
        d = rng.standard_normal(val.shape)

        def fn(xv, name=name):
            a = dict(z=z, A_log=A_log, dt_bias=dt_bias)
            a[name] = xv
            gg, _ = R.gate(a["z"], a["A_log"], a["dt_bias"])
            return R.loss(q, k, v, gg, beta, S0, d_o)

        fd = R.fd_directional(fn, val, d)
        an = float(np.sum(grad * d))
        assert abs(fd - an) / max(abs(an), 1.0) < BAR, (name, fd, an)
