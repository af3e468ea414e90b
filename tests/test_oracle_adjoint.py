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
