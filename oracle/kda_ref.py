"""Plain float64 CPU oracle for Kimi Delta Attention (KDA): gate, token recurrence,
chunked (WY) form, decode step and reverse-mode adjoint.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or link
this module: only the tests, the package smoke check and the benchmark's CPU
baseline leg use it.  It shares no code with the HIP library.

Sources.  The pages cited are three engineering review notes on the burn-kda
crate:
  [fix]     "kdafix -- the two class-B fixes burn-kda's designed-red gates were
            waiting for"  (sections "Fix 1 -- decay form", "Fix 2 -- read scale")
  [adjoint] "The fused KDA adjoint -- autopsy, and the gate that was missing"
            (sections 2, 3, 5b, 5c-bis)
  [ci]      "kdaoracle red on CI: the platform-drift hypothesis, tested and dead"
            (sections "The numbers", "Why they are red")

What the method computes (per batch b and head h, all in float64):
  gate        g = -exp(clamp(A_log_h, -10, 20)) * softplus(z + dt_bias_h)    [fix, Fix 1]
              alpha = exp(g) <= 1
  read scale  q_hat = scale * q, default scale = K**-0.5                    [fix, Fix 2]
  scalar decay  one pre-activation per token and one bias per head: the same gate,
              the same alpha on every key channel (gate_scalar, recurrent_scalar)
  output norm y = o / sqrt(mean_v(o^2) + eps) * weight_h (rmsnorm; reading R20)
  recurrence  S' = diag(alpha_t) S_{t-1}
              S_t = S' + beta_t k_t (v_t - S'^T k_t)^T
              o_t = S_t^T q_hat_t
  The recurrence itself is not printed on the pages; it is the gated delta rule
  (KDA) whose gate, read scale, head-major layout and chunk carry the pages fix.
  Readings taken where the pages are silent:
    * the delta read S'^T k uses the decayed state S' (the delta rule's defining
      property: with beta=1 and |k|=1 a write of v at key k reads back v);
    * the output reads the state after the write (o_t uses S_t);
    * beta is one scalar per token and head; dt_bias is (H, K); A_log is (H,);
    * softplus(x) = log(1 + e^x) with no threshold.

Pinning.  The tests in tests/test_oracle*.py tie every function here to facts
that do not come from this file: the A=0 agreement of the two gate forms and
their sign-of-A order [fix, Fix 1], g <= 0, linearity of o in the read scale
with the state independent of it [fix, Fix 2; ci, "The numbers"], a hand-worked
scalar example (tests/golden), the delta-rule closed form, the pure-decay closed
form, an explicit transition-matrix form of the recurrence, brute-force equality
of the chunked and token forms, resume splits, and central finite differences
for the adjoint.  No function here is "parity unpinned".
"""
from __future__ import annotations

import numpy as np

A_LOG_MIN = -10.0
A_LOG_MAX = 20.0


# ============================================================================ gate
def softplus(x):
    """log(1 + e^x), evaluated without overflow: max(x, 0) + log1p(e^-|x|)."""
    x = np.asarray(x, dtype=np.float64)
    return np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))


def gate(z, A_log, dt_bias):
    """KDA decay gate, released (FLA) form  [fix, "Fix 1 -- decay form"].

    The softplus is taken first and the -exp(A_h) multiplier applied outside it;
    A_log is clamped to [-10, 20] first (the page keeps that clamp).

    z: (B,H,T,K); A_log: (H,); dt_bias: (H,K).  Returns (g, alpha), float64.
    g <= 0 everywhere, so alpha = exp(g) lies in [0, 1] and cannot be NaN.
    """
    z = np.asarray(z, dtype=np.float64)
    a = np.clip(np.asarray(A_log, dtype=np.float64), A_LOG_MIN, A_LOG_MAX)
    mult = np.exp(a)[None, :, None, None]
    g = -mult * softplus(z + np.asarray(dt_bias, dtype=np.float64)[None, :, None, :])
    return g, np.exp(g)


def gate_prefix_form(z, A_log, dt_bias):
    """The form the page replaced: g = -softplus(exp(A_h) * x), exp(A) INSIDE
    [fix, "Fix 1 -- decay form", the "was" line].  Test-only control: it equals
    gate() exactly at A_log = 0 and differs everywhere else.  dt_bias is added to
    z before the multiplier (the page's control runs at dt_bias = 0)."""
    z = np.asarray(z, dtype=np.float64)
    a = np.clip(np.asarray(A_log, dtype=np.float64), A_LOG_MIN, A_LOG_MAX)
    x = z + np.asarray(dt_bias, dtype=np.float64)[None, :, None, :]
    g = -softplus(np.exp(a)[None, :, None, None] * x)
    return g, np.exp(g)


def read_scale(K):
    """Default read scale K**-0.5, folded into q  [fix, "Fix 2 -- read scale"]."""
    return float(K) ** -0.5


# ============================================================================ token recurrence
def _step(S, q_t, k_t, v_t, alpha_t, beta_t, scale):
    """One token of the gated delta rule for a batch of heads.

    S: (..., K, V); q_t, k_t, alpha_t: (..., K); v_t: (..., V); beta_t: (...).
    Returns (S_t, o_t).
    """
    Sd = alpha_t[..., :, None] * S                       # S' = diag(alpha_t) S_{t-1}
    r = np.sum(Sd * k_t[..., :, None], axis=-2)          # S'^T k_t
    S_new = Sd + beta_t[..., None, None] * k_t[..., :, None] * (v_t - r)[..., None, :]
    o_t = np.sum(S_new * (scale * q_t)[..., :, None], axis=-2)   # S_t^T (scale q_t)
    return S_new, o_t


def recurrent(q, k, v, g, beta, state_in=None, scale=None):
    """Naive per-token KDA forward.  The definition every other form is checked against.

    q,k,g: (B,H,T,K); v: (B,H,T,V); beta: (B,H,T); state_in: (B,H,K,V) or None (zeros);
    scale: None means K**-0.5.  Returns o (B,H,T,V) and the final state (B,H,K,V).
    """
    q, k, v, g, beta = (np.asarray(x, dtype=np.float64) for x in (q, k, v, g, beta))
    B, H, T, K = q.shape
    V = v.shape[-1]
    scale = read_scale(K) if scale is None else float(scale)
    S = np.zeros((B, H, K, V)) if state_in is None else np.array(state_in, dtype=np.float64)
    alpha = np.exp(g)
    o = np.empty((B, H, T, V))
    for t in range(T):
        S, o[:, :, t] = _step(S, q[:, :, t], k[:, :, t], v[:, :, t], alpha[:, :, t],
                              beta[:, :, t], scale)
    return o, S


def forward(q, k, v, z, A_log, dt_bias, beta, state_in=None, scale=None):
    """gate() then recurrent(): the full KDA forward from the gate pre-activation."""
    g, _ = gate(z, A_log, dt_bias)
    return recurrent(q, k, v, g, beta, state_in, scale)


def recurrent_step(q_t, k_t, v_t, g_t, beta_t, state, scale=None):
    """One decode step on (B,H,...) inputs: returns (o_t (B,H,V), new state (B,H,K,V))."""
    q_t, k_t, v_t, g_t, beta_t = (np.asarray(x, dtype=np.float64) for x in (q_t, k_t, v_t, g_t, beta_t))
    K = q_t.shape[-1]
    scale = read_scale(K) if scale is None else float(scale)
    S, o = _step(np.asarray(state, dtype=np.float64), q_t, k_t, v_t, np.exp(g_t), beta_t, scale)
    return o, S


# ============================================================================ scalar-decay special case
def gate_scalar(a, A_log, dt_bias=None):
    """Scalar (per-head) decay: one gate pre-activation a per (b, h, t) and one bias per
    head, so all key channels of a head decay by the same factor.  This is the released
    gate [fix, "Fix 1 -- decay form"] with an input that is constant over the channels:
    g_t = -exp(clamp(A_log_h, -10, 20)) * softplus(a_t + dt_bias_h).

    a: (B,H,T); A_log: (H,); dt_bias: (H,) or None (zeros).  Returns (g, alpha), (B,H,T).
    """
    a = np.asarray(a, dtype=np.float64)
    db = np.zeros(a.shape[1]) if dt_bias is None else np.asarray(dt_bias, dtype=np.float64)
    Al = np.clip(np.asarray(A_log, dtype=np.float64), A_LOG_MIN, A_LOG_MAX)
    g = -np.exp(Al)[None, :, None] * softplus(a + db[None, :, None])
    return g, np.exp(g)


def recurrent_scalar(q, k, v, g, beta, state_in=None, scale=None):
    """The token recurrence under a scalar decay g (B,H,T): alpha_t scales the whole state
    before the delta read.  Defined as the KDA recurrence with g copied to every key channel."""
    g = np.asarray(g, dtype=np.float64)
    return recurrent(q, k, v, np.broadcast_to(g[..., None], np.shape(q)), beta, state_in, scale)


# ============================================================================ chunked (WY) form
def _carry_decay(g):
    """Per-token decay from token i to the chunk end, exp(G_last - G_i) with G the
    inclusive cumulative sum of g: the "decay_last" factor of the chunk carry
    [adjoint, section 2].  Formed as exp(sum_{m>i} g_m), a sum of non-positive
    terms, never as a difference of two cumulative sums."""
    suffix = np.zeros_like(g)
    suffix[:-1] = np.cumsum(g[::-1], axis=0)[::-1][1:]
    return np.exp(suffix)


def _pair_decay_exponents(g):
    """D[i, j, c] = G_ic - G_jc = sum_{m=j+1..i} g_mc for j <= i (0 on the diagonal),
    -inf for j > i.  Summed directly so that no two large cumulative sums are
    subtracted (the gate can reach |g| ~ 1e9 per token at A_log = 20)."""
    n, K = g.shape
    D = np.full((n, n, K), -np.inf)
    for j in range(n):
        D[j, j] = 0.0
        if j + 1 < n:
            D[j + 1:, j] = np.cumsum(g[j + 1:], axis=0)
    return D


def _chunk(S, q, k, v, g, beta, scale):
    """One chunk of n tokens for one head.  S: (K,V) state at the chunk start.

    With G the inclusive cumsum of g, Gamma_i = exp(G_i) and E_ij = exp(G_i - G_j):
      A_ij = beta_i <k_i * E_ij, k_j>   (j < i),   T = (I + A)^-1
      w = T (beta * k * Gamma),  u = T (beta * v),  U = u - w S
      o = (q_hat * Gamma) S + P U,  P_ij = <q_hat_i * E_ij, k_j>  (j <= i)
      S_next = diag(Gamma_n) S + (k * exp(G_n - G))^T U
    Unrolling the recurrence gives these equations exactly; the u_j rows solve a
    unit lower-triangular system.
    """
    n = q.shape[0]
    qh = scale * q
    G = np.cumsum(g, axis=0)                               # (n,K), inclusive
    Gam = np.exp(G)
    lower = np.tril(np.ones((n, n)))
    lower_strict = np.tril(np.ones((n, n)), -1)
    E = np.exp(_pair_decay_exponents(g))                   # (n,n,K); 0 above the diagonal
    A = beta[:, None] * np.einsum("ic,ijc,jc->ij", k, E, k) * lower_strict
    P = np.einsum("ic,ijc,jc->ij", qh, E, k) * lower
    Tm = np.linalg.inv(np.eye(n) + A)
    w = Tm @ (beta[:, None] * k * Gam)
    u = Tm @ (beta[:, None] * v)
    U = u - w @ S
    o = (qh * Gam) @ S + P @ U
    S_next = Gam[-1][:, None] * S + (k * _carry_decay(g)).T @ U
    return o, S_next


def chunked(q, k, v, g, beta, state_in=None, scale=None, chunk=64):
    """Chunk-parallel (WY) KDA forward; equal to recurrent() up to rounding.

    The last chunk may be shorter than `chunk` (a ragged tail).  Same argument
    conventions as recurrent().
    """
    q, k, v, g, beta = (np.asarray(x, dtype=np.float64) for x in (q, k, v, g, beta))
    B, H, T, K = q.shape
    V = v.shape[-1]
    scale = read_scale(K) if scale is None else float(scale)
    S_all = np.zeros((B, H, K, V)) if state_in is None else np.array(state_in, dtype=np.float64)
    o = np.empty((B, H, T, V))
    for b in range(B):
        for h in range(H):
            S = S_all[b, h]
            for t0 in range(0, T, chunk):
                sl = slice(t0, min(T, t0 + chunk))
                o[b, h, sl], S = _chunk(S, q[b, h, sl], k[b, h, sl], v[b, h, sl],
                                        g[b, h, sl], beta[b, h, sl], scale)
            S_all[b, h] = S
    return o, S_all


# ============================================================================ adjoint
def adjoint(q, k, v, g, beta, state_in, d_o, d_state_out=None, scale=None, segment=64):
    """Reverse-mode gradients of  L = sum(o * d_o) + sum(S_T * d_state_out).

    Returns dict(dq, dk, dv, dg, dbeta, dstate_in): gradients w.r.t. the unscaled
    q, k, v, the log-decay g, beta and the initial state.  The page's fixture
    lists the same cotangent (d_out), loss and gradient blocks [adjoint,
    section 3]; its "w" block has no definition on the pages and is not formed.

    Per token t, walking backwards with dS = dL/dS_t:
      dS += q_hat_t do_t^T          dq_t = scale * S_t do_t
      S' = diag(alpha_t) S_{t-1},   e = v_t - S'^T k_t
      dbeta_t = k_t^T dS e          de = beta_t dS^T k_t
      dk_t = beta_t dS e - S' de    dv_t = de
      dS' = dS - k_t de^T           dg_t = alpha_t * rowsum(dS' * S_{t-1})
      dS = diag(alpha_t) dS'
    The states S_t are recomputed per segment of `segment` tokens from stored
    segment-start states (same operations, so bit-identical to the forward).
    """
    q, k, v, g, beta, d_o = (np.asarray(x, dtype=np.float64) for x in (q, k, v, g, beta, d_o))
    B, H, T, K = q.shape
    V = v.shape[-1]
    scale = read_scale(K) if scale is None else float(scale)
    S0 = np.zeros((B, H, K, V)) if state_in is None else np.array(state_in, dtype=np.float64)
    alpha = np.exp(g)

    # forward pass, keeping the state at every segment start
    starts = list(range(0, T, segment))
    ckpt = {}
    S = S0.copy()
    for s0 in starts:
        ckpt[s0] = S.copy()
        for t in range(s0, min(T, s0 + segment)):
            S, _ = _step(S, q[:, :, t], k[:, :, t], v[:, :, t], alpha[:, :, t], beta[:, :, t], scale)

    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    dg = np.zeros_like(g)
    dbeta = np.zeros_like(beta)
    dS = np.zeros((B, H, K, V)) if d_state_out is None else np.array(d_state_out, dtype=np.float64)

    for s0 in reversed(starts):
        s1 = min(T, s0 + segment)
        states = [ckpt[s0]]                      # states[i] = S_{s0+i-1}, i.e. before token s0+i
        S = ckpt[s0]
        for t in range(s0, s1):
            S, _ = _step(S, q[:, :, t], k[:, :, t], v[:, :, t], alpha[:, :, t], beta[:, :, t], scale)
            states.append(S)
        for t in range(s1 - 1, s0 - 1, -1):
            dS, grads = _step_adjoint(dS, states[t - s0], states[t - s0 + 1], q[:, :, t], k[:, :, t],
                                      v[:, :, t], alpha[:, :, t], beta[:, :, t], d_o[:, :, t], scale)
            dq[:, :, t], dk[:, :, t], dv[:, :, t], dg[:, :, t], dbeta[:, :, t] = grads
    return dict(dq=dq, dk=dk, dv=dv, dg=dg, dbeta=dbeta, dstate_in=dS)


def _step_adjoint(dS, S_prev, S_t, q_t, k_t, v_t, a_t, b_t, do_t, scale):
    """Reverse of _step for one token.  dS = dL/dS_t on entry, dL/dS_{t-1} on exit.

    Returns (dS_prev, (dq_t, dk_t, dv_t, dg_t, dbeta_t)).
    """
    dS = dS + (scale * q_t)[..., :, None] * do_t[..., None, :]
    dq_t = scale * np.sum(S_t * do_t[..., None, :], axis=-1)
    Sd = a_t[..., :, None] * S_prev
    e = v_t - np.sum(Sd * k_t[..., :, None], axis=-2)
    dSe = np.sum(dS * e[..., None, :], axis=-1)                      # dS e      (K)
    dbeta_t = np.sum(k_t * dSe, axis=-1)
    de = b_t[..., None] * np.sum(dS * k_t[..., :, None], axis=-2)     # beta dS^T k (V)
    dk_t = b_t[..., None] * dSe - np.sum(Sd * de[..., None, :], axis=-1)
    dv_t = de
    dSd = dS - k_t[..., :, None] * de[..., None, :]
    dg_t = a_t * np.sum(dSd * S_prev, axis=-1)
    return a_t[..., :, None] * dSd, (dq_t, dk_t, dv_t, dg_t, dbeta_t)


def sigmoid(x):
    """1 / (1 + e^-x) = exp(-softplus(-x)): the derivative of softplus, overflow-free."""
    return np.exp(-softplus(-np.asarray(x, dtype=np.float64)))


def gate_adjoint(z, A_log, dt_bias, dg):
    """Reverse mode of gate() for a cotangent dg on g  [fix, "Fix 1 -- decay form"].

    With x = z + dt_bias and m = exp(clamp(A_log, -10, 20)), g = -m * softplus(x):
      dz         = -m * sigmoid(x) * dg        (softplus' = sigmoid)
      d dt_bias  = dz summed over batch and time                  (H, K)
      dA_log     = (dg * g) summed over batch, time and channel,   (H,)
                   where A_log lies in [-10, 20]; 0 outside, where the clamp
                   holds the multiplier constant (at the two bounds the closed
                   interval passes the gradient).
    Returns (dz, dA_log, d_dt_bias), float64.  Steps written out one by one.
    """
    z = np.asarray(z, dtype=np.float64)
    dg = np.asarray(dg, dtype=np.float64)
    A_log = np.asarray(A_log, dtype=np.float64)
    a = np.clip(A_log, A_LOG_MIN, A_LOG_MAX)
    m = np.exp(a)[None, :, None, None]
    x = z + (np.asarray(dt_bias, dtype=np.float64)[None, :, None, :] if dt_bias is not None else 0.0)
    g = -m * softplus(x)
    dz = -m * sigmoid(x) * dg
    inside = (A_log >= A_LOG_MIN) & (A_log <= A_LOG_MAX)
    dA_log = np.where(inside, np.sum(dg * g, axis=(0, 2, 3)), 0.0)
    d_dt_bias = np.sum(dz, axis=(0, 2))
    return dz, dA_log, d_dt_bias


def loss(q, k, v, g, beta, state_in, d_o, d_state_out=None, scale=None):
    """L = sum(o * d_o) + sum(S_T * d_state_out) through recurrent(); for FD checks."""
    o, S = recurrent(q, k, v, g, beta, state_in, scale)
    L = np.sum(o * np.asarray(d_o, dtype=np.float64))
    if d_state_out is not None:
        L += np.sum(S * np.asarray(d_state_out, dtype=np.float64))
    return float(L)


def fd_directional(fn, x, direction, h=1e-6):
    """Central finite difference of a scalar function along `direction`, f64."""
    x = np.asarray(x, dtype=np.float64)
    d = np.asarray(direction, dtype=np.float64)
    return (fn(x + h * d) - fn(x - h * d)) / (2.0 * h)


# ============================================================================ output norm
def rmsnorm(o, weight=None, eps=1e-6):
    """The RMSNorm that follows the read (reading R20: over each head's V outputs of a
    token, one weight row per head, no gate):
        y[b, h, t, :] = o[b, h, t, :] / sqrt(mean_v o[b, h, t, v]^2 + eps) * weight[h, :]
    o (B, H, T, V); weight (H, V) or None (all ones); eps >= 0.  [fix, Fix 2: the module
    normalises the read right after it, so a constant factor on o, such as the read
    scale, changes y only through eps, by O(eps / mean(o^2)).]"""
    o = np.asarray(o, dtype=np.float64)
    ms = np.mean(o * o, axis=-1, keepdims=True)
    y = o / np.sqrt(ms + eps)
    if weight is not None:
        y = y * np.asarray(weight, dtype=np.float64)[None, :, None, :]
    return y


# ============================================================================ metrics
def rel_err(x, ref):
    """max|x - ref| / max|ref| over one output tensor (0 when both are all zero)."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.max(np.abs(ref)) if ref.size else 0.0
    num = np.max(np.abs(x - ref)) if ref.size else 0.0
    if den == 0.0:
        return float(num)
    return float(num / den)
