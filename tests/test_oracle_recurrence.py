"""Pins of ``oracle/recurrence.py`` (the gated delta rule; bayesiansapien
page, "The four-part mechanism study", third item).  No GPU."""
import numpy as np
import pytest

from oracle import recurrence as R


def test_two_step_hand_worked_example():
    """d = 2, eps = 0 so that keys (3, 4) and (4, -3) normalise exactly.
    step 0: S = 0, k^ = (.6, .8), v = (1, 2), beta = .5, alpha = 1:
            u = 0, S = .5 (1, 2)^T (.6, .8) = [[.3, .4], [.6, .8]]; q^ = (0, 1) -> o = (.4, .8)
    step 1: alpha = .5 -> S = [[.15, .2], [.3, .4]]; k^ = (.8, -.6): u = S k^ = (0, 0);
            beta = 1: S += (1, 0)^T (.8, -.6) = [[.95, -.4], [.3, .4]]; q^ = (1, 0) -> o = (.95, .3)"""
    q = np.array([[[0.0, 2.0]], [[1.0, 0.0]]])
    k = np.array([[[3.0, 4.0]], [[4.0, -3.0]]])
    v = np.array([[[1.0, 2.0]], [[1.0, 0.0]]])
    beta = np.array([[0.5], [1.0]])
    g = np.array([[0.0], [np.log(0.5)]])
    o, S = R.recurrence(q, k, v, beta, g, eps=0.0)
    np.testing.assert_allclose(o[0, 0], [0.4, 0.8], atol=1e-15)
    np.testing.assert_allclose(o[1, 0], [0.95, 0.3], atol=1e-15)
    np.testing.assert_allclose(S[0], [[0.95, -0.4], [0.3, 0.4]], atol=1e-15)


def test_vector_form_equals_matrix_form():
    rng = np.random.default_rng(1)
    d, hv, hk = 8, 6, 2
    S0 = rng.standard_normal((hv, d, d))
    q, k = rng.standard_normal((1, hk, d)), rng.standard_normal((1, hk, d))
    v = rng.standard_normal((1, hv, d))
    beta, g = rng.uniform(0, 1, (1, hv)), -rng.uniform(0, 2, (1, hv))
    o, S = R.recurrence(q, k, v, beta, g, s_init=S0)
    for h in range(hv):
        S2, o2 = R.step_matrix_form(S0[h], q[0, h // 3], k[0, h // 3], v[0, h], beta[0, h], g[0, h])
        np.testing.assert_allclose(S[h], S2, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(o[0, h], o2, rtol=1e-12, atol=1e-12)


def test_zero_write_strength_is_pure_decay():
    rng = np.random.default_rng(2)
    T, d = 20, 16
    S0 = rng.standard_normal((2, d, d))
    q, k = rng.standard_normal((T, 1, d)), rng.standard_normal((T, 1, d))
    v = rng.standard_normal((T, 2, d))
    g = -rng.uniform(0, 0.3, (T, 2))
    o, S = R.recurrence(q, k, v, np.zeros((T, 2)), g, s_init=S0)
    decay = np.exp(np.cumsum(g, axis=0))                         # [T, Hv]
    np.testing.assert_allclose(S, S0 * decay[-1][:, None, None], rtol=1e-12)
    qn = R.l2_normalize(q[:, 0])
    for t in (0, 7, T - 1):
        for h in range(2):
            np.testing.assert_allclose(o[t, h], decay[t, h] * S0[h] @ qn[t], rtol=1e-12, atol=1e-14)


def test_full_write_along_a_basis_key_replaces_one_column():
    rng = np.random.default_rng(3)
    d = 8
    S0 = rng.standard_normal((1, d, d))
    k = np.zeros((1, 1, d))
    k[0, 0, 5] = 2.0
    v = rng.standard_normal((1, 1, d))
    o, S = R.recurrence(rng.standard_normal((1, 1, d)), k, v, np.ones((1, 1)), np.zeros((1, 1)),
                        s_init=S0, eps=0.0)
    np.testing.assert_array_equal(np.delete(S[0], 5, axis=1), np.delete(S0[0], 5, axis=1))
    np.testing.assert_allclose(S[0][:, 5], v[0, 0], rtol=0, atol=1e-15)


@pytest.mark.parametrize("alpha", [1.0, 0.7, 1e-3])
def test_full_write_sets_the_state_along_the_key_to_v(alpha):
    """The overwrite: after a step with beta = 1 (eps = 0), S k^ = v whatever S held before."""
    rng = np.random.default_rng(4)
    d = 32
    S0 = rng.standard_normal((1, d, d)) * 10
    k, v = rng.standard_normal((1, 1, d)), rng.standard_normal((1, 1, d))
    _, S = R.recurrence(rng.standard_normal((1, 1, d)), k, v, np.ones((1, 1)), np.full((1, 1), np.log(alpha)),
                        s_init=S0, eps=0.0)
    np.testing.assert_allclose(S[0] @ R.l2_normalize(k[0, 0], 0.0), v[0, 0], rtol=0, atol=1e-12)


def test_without_writes_the_state_never_grows():
    """v = 0: each step multiplies S by alpha (I - beta k^ k^T), whose spectral norm is <= 1."""
    rng = np.random.default_rng(5)
    T, d = 200, 16
    S0 = rng.standard_normal((3, d, d))
    q, k = rng.standard_normal((T, 1, d)), rng.standard_normal((T, 1, d))
    beta = rng.uniform(0, 1, (T, 3))
    g = -rng.uniform(0, 0.01, (T, 3))
    _, _, states = R.recurrence(q, k, np.zeros((T, 3, d)), beta, g, s_init=S0, return_states=True)
    norms = np.array([np.linalg.norm(s, axis=(1, 2)) for s in [S0] + states])
    assert np.all(np.diff(norms, axis=0) <= 1e-12 * norms[:-1])
    assert np.all(norms[-1] < 0.5 * norms[0])          # and it is forgotten, not just kept


def test_key_head_mapping():
    np.testing.assert_array_equal(R.key_head_of(48, 16)[:7], [0, 0, 0, 1, 1, 1, 2])
    with pytest.raises(ValueError):
        R.key_head_of(10, 4)


def _fp32_recurrence(q, k, v, beta, g, mistake=None):
    """The gated delta rule evaluated in float32 throughout (numpy), written
    independently of the fp64 oracle, optionally with a planted mistake:
    "read_before_decay" takes S k^ on the undecayed state, "bf16_state" keeps the
    state in bf16 between steps."""
    T, hk, d = k.shape
    hv = v.shape[1]
    kh = np.arange(hv) // (hv // hk)
    f = np.float32
    q, k, v, beta, g = (np.asarray(x, dtype=f) for x in (q, k, v, beta, g))
    S = np.zeros((hv, d, d), f)
    o = np.empty((T, hv, d), f)
    eps = f(1e-6)
    for t in range(T):
        kn = (k[t] / np.sqrt(np.sum(k[t] * k[t], axis=-1, keepdims=True) + eps))[kh]
        qn = (q[t] / np.sqrt(np.sum(q[t] * q[t], axis=-1, keepdims=True) + eps))[kh]
        a = np.exp(g[t])[:, None, None]
        if mistake == "read_before_decay":
            u = np.einsum("hij,hj->hi", S, kn)
            S = a * S
        else:
            S = a * S
            u = np.einsum("hij,hj->hi", S, kn)
        S = S + (beta[t][:, None, None] * (v[t] - u)[:, :, None]) * kn[:, None, :]
        if mistake == "bf16_state":
            S = (S.view(np.uint32) + np.uint32(0x7FFF) + ((S.view(np.uint32) >> 16) & 1) & np.uint32(0xFFFF0000)).view(f)
        o[t] = np.einsum("hij,hj->hi", S, qn)
    return o, S


def test_fp32_bound_holds_at_4096_steps_and_rejects_plausible_mistakes():
    """Pin of fp32_tolerance / fp32_state_tolerance: an fp32 evaluation over 4096
    steps (gates drawn as in the recurrence workload) stays inside the bound, with
    the most-used element at more than 1/2000 of its tolerance (the bound takes
    the worst case of every dot product, d u, where rounding errors typically
    cancel to about sqrt(d) u / 2), while two plausible slips -- the key read on
    the undecayed state, and a bf16 state between steps -- exceed it."""
    from nvfp4_w4a4_gemm_quantize_amd import inputs
    T, hk, hv, d = 4096, 1, 3, 128
    raw = inputs.recurrence(T, hk, hv, seed=5)
    f = lambda b: inputs.bf16_bits_to_f32(b).astype(np.float64)
    q, k = f(raw["q"]).reshape(T, hk, d), f(raw["k"]).reshape(T, hk, d)
    v, beta, g = f(raw["v"]).reshape(T, hv, d), f(raw["beta"]), f(raw["g"])
    o, S, nr = R.recurrence(q, k, v, beta, g, return_row_norms=True)
    tol, tol_s = R.fp32_tolerance(nr, v, g), R.fp32_state_tolerance(nr, v, g)
    o32, S32 = _fp32_recurrence(q, k, v, beta, g)
    use = np.abs(o32 - o) / tol
    assert use.max() <= 1.0
    assert use.max() > 1.0 / 2000, use.max()
    assert np.all(np.abs(S32 - S) <= tol_s)
    assert np.linalg.norm(o32 - o) <= 1e-5 * np.linalg.norm(o)
    for mistake in ("read_before_decay", "bf16_state"):
        om, _ = _fp32_recurrence(q, k, v, beta, g, mistake)
        assert np.max(np.abs(om - o) / tol) > 2.0, mistake


def test_fp32_bound_is_decay_damped():
    """With every decay 1/2 an old error is halved each step, so the state bound
    settles at c u (N + |v|) / (1 - 1/2) scale instead of growing with T."""
    T, hv, d = 200, 1, 128
    nr = np.ones((T + 1, hv, 4))
    v = np.ones((T, hv, 4))
    g = np.full((T, hv), np.log(0.5))
    E = R.fp32_state_error_bound(nr, v, g, d)
    c = 2 * d + 20
    np.testing.assert_allclose(E[-1], 1.01 * c * R.U32 * (0.5 + 1) / (1 - 0.5), rtol=1e-12)
    np.testing.assert_allclose(E[0], 1.01 * c * R.U32 * (0.5 + 1), rtol=1e-12)
    # no decay: the bound grows linearly, one step's worth per step
    E1 = R.fp32_state_error_bound(nr, v, np.zeros((T, hv)), d)
    np.testing.assert_allclose(E1[-1], 1.01 * c * R.U32 * 2 * T, rtol=1e-12)
