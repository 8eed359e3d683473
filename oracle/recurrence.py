"""Gated delta-rule recurrence of a Gated DeltaNet layer, in fp64 -- TEST
INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The pages describe the recurrence by its behaviour, not by a formula: every
write overwrites the recurrent state along the current key direction, so the
state is a continually overwritten register rather than an accumulator;
injected noise stays at a flat plateau over 32K tokens and a state impulse is
forgotten within hundreds of steps (bayesiansapien page, "The four-part
mechanism study", third item; nefut page, third bullet; aimodeling page,
"Why the recurrent half survives").  Their gates are the sigmoid write
strength and the softplus/exponential decay of the same study's second item.

Reading taken (the standard gated delta rule those words describe), per value
head h with key head hk(h) = h // (Hv / Hk), state S [d_v, d_k] (row = value
index, column = key index), for t = 0 .. T-1:

    k^ = k_t / sqrt(sum k_t^2 + eps),   q^ = q_t / sqrt(sum q_t^2 + eps)
    alpha = exp(g_t)            g_t <= 0: the decay gate's output
    beta  = beta_t              in (0, 1): the sigmoid gate's output
    S    <- alpha * S                                  decay
    u     = S k^                                       what S holds along k^
    S    <- S + beta * (v_t - u) k^T                   overwrite along k^
    o_t   = S q^

i.e. S_t = alpha_t S_{t-1} (I - beta_t k^ k^T) + beta_t v_t k^T.  eps = 1e-6
(the L2-normalisation convention of Gated DeltaNet implementations).

Inputs are the float values of the GPU's bf16 inputs; everything here is fp64.
"""
import numpy as np

EPS = 1e-6


def l2_normalize(x, eps=EPS):
    """x / sqrt(sum(x^2) + eps) along the last axis, fp64."""
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)


def key_head_of(hv, hk):
    if hv % hk:
        raise ValueError("value heads must be a multiple of key heads")
    return np.arange(hv) // (hv // hk)


def recurrence(q, k, v, beta, g, s_init=None, eps=EPS, return_states=False, return_row_l1=False):
    """Run the gated delta rule.

    q, k  [T, Hk, d_k]; v [T, Hv, d_v]; beta, g [T, Hv]; s_init [Hv, d_v, d_k] or None (zeros).
    Returns (o [T, Hv, d_v], S_final [Hv, d_v, d_k]) and, with return_states, the list of states;
    with return_row_l1 (instead), the row L1 norms sum_j |S_t[h, i, j]| [T, Hv, d_v] after each step.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    T, hk, dk = k.shape
    hv, dv = v.shape[1], v.shape[2]
    kh = key_head_of(hv, hk)
    S = np.zeros((hv, dv, dk)) if s_init is None else np.array(s_init, dtype=np.float64)
    o = np.empty((T, hv, dv))
    states = []
    row_l1 = np.empty((T, hv, dv)) if return_row_l1 else None
    for t in range(T):
        kn = l2_normalize(k[t], eps)[kh]                  # [Hv, d_k]
        qn = l2_normalize(q[t], eps)[kh]
        alpha = np.exp(g[t])[:, None, None]
        S = alpha * S
        u = np.einsum("hij,hj->hi", S, kn)
        S = S + beta[t][:, None, None] * (v[t] - u)[:, :, None] * kn[:, None, :]
        o[t] = np.einsum("hij,hj->hi", S, qn)
        if return_states:
            states.append(S.copy())
        if return_row_l1:
            row_l1[t] = np.sum(np.abs(S), axis=2)
    if return_states:
        return o, S, states
    return (o, S, row_l1) if return_row_l1 else (o, S)


def fp32_tolerance(row_l1, v, s_init=None, out_is_bf16=False, o_ref=None):
    """Per-element bound for an fp32 evaluation of the recurrence, [T, Hv, d_v].

    Each step forms two 128-term dot products of a state row (with a key and a
    query of norm <= 1) and one multiply-add per element; with unit roundoff
    u = 2^-24 the error it adds to row i is at most c u (|S_i|_1 + |v_i|), with
    c = 64 covering the dot-product length's rounding (the key's and query's own
    normalisation errors included), and earlier errors are not amplified
    because every step's map S -> alpha S (I - beta k^ k^T) has norm <= 1.  So
    after t + 1 steps |o_t,i - o~| <= (t + 1) c u max_{tau <= t}(|S_tau,i|_1 + |v_tau,i|),
    plus the state's initial magnitude, plus the bf16 rounding of the output
    when it is bf16 (unit roundoff 2^-8: 8 significand bits, round to nearest).
    """
    u = 2.0 ** -24
    T = row_l1.shape[0]
    m = np.maximum.accumulate(row_l1 + np.abs(np.asarray(v, dtype=np.float64)), axis=0)
    if s_init is not None:
        m = np.maximum(m, np.sum(np.abs(np.asarray(s_init, dtype=np.float64)), axis=2)[None])
    tol = (np.arange(1, T + 1, dtype=np.float64)[:, None, None]) * 64 * u * m
    if out_is_bf16:
        tol = tol + 2.0 ** -8 * (np.abs(o_ref) + tol)
    return tol


def step_matrix_form(S, q, k, v, beta, g, eps=EPS):
    """One step of one head in the explicit matrix form
    S' = alpha S (I - beta k^ k^T) + beta v k^T, o = S' q^ (for pinning the vector form)."""
    S = np.asarray(S, dtype=np.float64)
    kn = l2_normalize(k, eps)
    qn = l2_normalize(q, eps)
    d = kn.shape[0]
    S2 = np.exp(g) * S @ (np.eye(d) - beta * np.outer(kn, kn)) + beta * np.outer(v, kn)
    return S2, S2 @ qn
