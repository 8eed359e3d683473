"""Gated delta-rule recurrence of a Gated DeltaNet layer, in fp64 -- TEST
INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The pages characterise the recurrence by its behaviour, not by a formula:
the delta rule replaces the state's component along the current key instead
of adding to it, which is why, in their measurements, the output error under
injected noise levels off rather than growing with sequence length, and a
disturbance of the state fades after some hundreds of steps
(bayesiansapien page, "The four-part mechanism study", third item; nefut
page, third bullet; aimodeling page, "Why the recurrent half survives").
Their gates are the sigmoid write strength and the softplus/exponential
decay of the same study's second item.

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


def recurrence(q, k, v, beta, g, s_init=None, eps=EPS, return_states=False, return_row_norms=False):
    """Run the gated delta rule.

    q, k  [T, Hk, d_k]; v [T, Hv, d_v]; beta, g [T, Hv]; s_init [Hv, d_v, d_k] or None (zeros).
    Returns (o [T, Hv, d_v], S_final [Hv, d_v, d_k]) and, with return_states, the list of states;
    with return_row_norms (instead), the L2 norms of the state rows, [T + 1, Hv, d_v]: entry 0 for
    the initial state, entry t + 1 after step t.
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
    norms = np.empty((T + 1, hv, dv)) if return_row_norms else None
    if return_row_norms:
        norms[0] = np.linalg.norm(S, axis=2)
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
        if return_row_norms:
            norms[t + 1] = np.linalg.norm(S, axis=2)
    if return_states:
        return o, S, states
    return (o, S, norms) if return_row_norms else (o, S)


U32 = 2.0 ** -24          # unit roundoff of fp32 (round to nearest)
U_BF16 = 2.0 ** -8        # unit roundoff of bf16 (8 significand bits)


def fp32_state_error_bound(row_norms, v, g, d=128):
    """Bound on the error an fp32 evaluation of the recurrence can have in each
    state row: E [T, Hv, d_v], E[t, h, i] >= || S~_t[h, i, :] - S_t[h, i, :] ||_2
    after step t, for any order of the additions inside each step.

    Error analysis of one step (unit roundoff u, row i, a = exp(g_t), state row
    norms N = ||S_{t-1,i}||_2, value v_i; standard bounds: a d-term dot product in
    any summation order is within d u sum|x_j y_j| <= d u ||x|| ||y|| of the exact
    one, and the computed unit key k~ is within (d/2 + 4) u of the exact one,
    the sum of its d squares, the square root and the division included):
      - the state row times the key:        (d + d/2 + 5) u a N
      - decay, write coefficient, the outer product and the add, per element a
        few roundings of terms bounded by a|S_ij| and |v_i - u_i| |k_j|:
                                             3 u (2 a N + |v_i|)
      - the write's direction k~ - k^:      (d/2 + 4) u (|v_i| + a N)
    so the step adds at most c u (a N + |v_i|) with c = 2 d + 20.  The error
    already in the row is carried to the next step by x -> a x (I - beta k^ k^T),
    whose norm is at most a for beta in [0, 1] and a unit key, so
        E_t = a_t E_{t-1} + c u (a_t N_{t-1} + |v_t,i|),   E_{-1} = 0
    (the initial state is given in fp32, exactly).  Norms are those of the exact
    state; the difference to the computed state's is second order and covered by
    a 1% margin."""
    row_norms = np.asarray(row_norms, dtype=np.float64)
    v = np.abs(np.asarray(v, dtype=np.float64))
    a = np.exp(np.asarray(g, dtype=np.float64))[:, :, None]          # [T, Hv, 1]
    c = 2 * d + 20
    T = v.shape[0]
    E = np.empty_like(v)
    e = np.zeros(v.shape[1:])
    for t in range(T):
        e = a[t] * e + c * U32 * (a[t] * row_norms[t] + v[t])
        E[t] = e
    return 1.01 * E


def fp32_tolerance(row_norms, v, g, out_is_bf16=False, o_ref=None, d=128):
    """Per-element bound for the outputs o_t = S_t q^ of an fp32 evaluation, [T, Hv, d_v]:
    the state row's error (fp32_state_error_bound; |q^| <= 1) plus the output dot
    product and the query's normalisation, (d + d/2 + 5) u ||S_t,i||_2, plus, for a
    bf16 output, its rounding (unit roundoff 2^-8)."""
    E = fp32_state_error_bound(row_norms, v, g, d)
    tol = E + 1.01 * (d + d // 2 + 5) * U32 * np.asarray(row_norms, dtype=np.float64)[1:]
    if out_is_bf16:
        tol = tol + U_BF16 * (np.abs(o_ref) + tol)
    return tol


def fp32_state_tolerance(row_norms, v, g, d=128):
    """Per-element bound for the final state of an fp32 evaluation, [Hv, d_v, d_k]
    (an element's error is at most its row's L2 error)."""
    E = fp32_state_error_bound(row_norms, v, g, d)[-1]
    return np.repeat(E[:, :, None], d, axis=2)


def step_matrix_form(S, q, k, v, beta, g, eps=EPS):
    """One step of one head in the explicit matrix form
    S' = alpha S (I - beta k^ k^T) + beta v k^T, o = S' q^ (for pinning the vector form)."""
    S = np.asarray(S, dtype=np.float64)
    kn = l2_normalize(k, eps)
    qn = l2_normalize(q, eps)
    d = kn.shape[0]
    S2 = np.exp(g) * S @ (np.eye(d) - beta * np.outer(kn, kn)) + beta * np.outer(v, kn)
    return S2, S2 @ qn
