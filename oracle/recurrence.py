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


def recurrence(q, k, v, beta, g, s_init=None, eps=EPS, return_states=False):
    """Run the gated delta rule.

    q, k  [T, Hk, d_k]; v [T, Hv, d_v]; beta, g [T, Hv]; s_init [Hv, d_v, d_k] or None (zeros).
    Returns (o [T, Hv, d_v], S_final [Hv, d_v, d_k]) and, with return_states, the list of states.
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
    return (o, S, states) if return_states else (o, S)


def step_matrix_form(S, q, k, v, beta, g, eps=EPS):
    """One step of one head in the explicit matrix form
    S' = alpha S (I - beta k^ k^T) + beta v k^T, o = S' q^ (for pinning the vector form)."""
    S = np.asarray(S, dtype=np.float64)
    kn = l2_normalize(k, eps)
    qn = l2_normalize(q, eps)
    d = kn.shape[0]
    S2 = np.exp(g) * S @ (np.eye(d) - beta * np.outer(kn, kn)) + beta * np.outer(v, kn)
    return S2, S2 @ qn
