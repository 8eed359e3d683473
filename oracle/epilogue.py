"""fp64 epilogues of the fused W4A4 GEMMs -- TEST INFRASTRUCTURE ONLY.

The pages name the gate parameterisations of the Gated DeltaNet block as
sigmoid (write strength) and softplus/exponential (decay), and call them
contractive on error (bayesiansapien page, mechanism study, second item;
nefut page, second bullet; aimodeling page, "four mechanisms").  The MLP half
of the layer is 4-bit too (bayesiansapien page, Figure, node MLP).  The exact
expressions below are the standard ones for these layers:

    silu(z)          = z / (1 + exp(-z))
    silu_mul(g, u)   = silu(g) * u                 (MLP gate/up -> h)
    beta(b)          = 1 / (1 + exp(-b))           (write strength)
    decay(a; A, d)   = -exp(A) * log(1 + exp(a + d))   (log-decay; A = A_log, d = dt_bias)

Each tolerance is the epilogue's Lipschitz constant times the GEMM error
bound T of its input(s), plus an allowance for FP32 evaluation of exp/log on
the GPU (2**-19 relative) and, for bf16 outputs, the bf16 rounding of the
result (unit roundoff 2**-8).
"""
import numpy as np

BF16_U = 2.0 ** -8
EVAL_REL = 2.0 ** -19
SILU_LIPSCHITZ = 1.0998  # max |d silu / dz|, attained near z = 2.4


def silu(z):
    z = np.asarray(z, dtype=np.float64)
    return z / (1.0 + np.exp(-z))


def silu_mul(gate, up):
    return silu(gate) * np.asarray(up, dtype=np.float64)


def sigmoid(b):
    b = np.asarray(b, dtype=np.float64)
    with np.errstate(over="ignore"):          # exp(-b) = inf gives the right limit 0
        return 1.0 / (1.0 + np.exp(-b))


def softplus(x):
    """log(1 + e^x) in float64, as max(x, 0) + log1p(e^-|x|) (the same function,
    written so that e^x cannot overflow)."""
    x = np.asarray(x, dtype=np.float64)
    return np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))


def gdn_decay(a, a_log, dt_bias):
    """-exp(A_log[h]) * softplus(a + dt_bias[h]); a [M, H], a_log/dt_bias [H]."""
    a = np.asarray(a, dtype=np.float64)
    A = np.asarray(a_log, dtype=np.float64)[None, :]
    d = np.asarray(dt_bias, dtype=np.float64)[None, :]
    return -np.exp(A) * softplus(a + d)


def _finish(ref, lip_term, out_is_bf16):
    tol = lip_term + EVAL_REL * np.abs(ref)
    if out_is_bf16:
        tol = tol + BF16_U * (np.abs(ref) + tol)
    return tol


def silu_mul_tolerance(gate, up, t_gate, t_up, out_is_bf16=True):
    """Error allowance of silu(g)*u given GEMM bounds t_gate, t_up on g and u."""
    gate = np.asarray(gate, dtype=np.float64)
    up = np.asarray(up, dtype=np.float64)
    ref = silu_mul(gate, up)
    lip = (SILU_LIPSCHITZ * t_gate * np.abs(up) + np.abs(silu(gate)) * t_up
           + SILU_LIPSCHITZ * t_gate * t_up)
    return _finish(ref, lip, out_is_bf16)


def sigmoid_tolerance(b, t_b, out_is_bf16=True):
    return _finish(sigmoid(b), 0.25 * np.asarray(t_b, dtype=np.float64), out_is_bf16)


def gdn_decay_tolerance(a, a_log, dt_bias, t_a, out_is_bf16=True):
    """|d decay / d a| = exp(A) * sigmoid(a + d) <= exp(A)."""
    ref = gdn_decay(a, a_log, dt_bias)
    lip = np.exp(np.asarray(a_log, dtype=np.float64))[None, :] * np.asarray(t_a, dtype=np.float64)
    return _finish(ref, lip, out_is_bf16)
