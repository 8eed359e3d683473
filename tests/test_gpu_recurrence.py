"""GPU parity of the gated delta-rule recurrence (gdn_recurrence) against the
fp64 oracle (bayesiansapien page, "The four-part mechanism study", third
item), and the mechanism measurements that item describes.

Parity: every output element within the fp32 bound of
``oracle.recurrence.fp32_tolerance`` (per-step rounding times the state row's
L2 norm, carried to later steps damped by each step's decay, never amplified
because each step is non-expansive), the output's L2 error within 1e-5 of its
norm (plus the bf16 rounding for bf16 outputs), the final state likewise, ragged chunk tails, one step,
grouped key heads, strided inputs inside a fused in-projection buffer, an
initial state, bf16 output, run-to-run identity, near-total resets in some
chunks (which run the unscaled state update while the rest run the scaled
one); at the full head layout (16 key / 48 value heads) over 4096 tokens.
Mechanism: noise of 10% injected into keys, values and both gates at every
step leaves the output error level (no growth with position) over 32768 tokens; a random
state impulse (values zero) is forgotten, its output falling by 100x within
a few thousand steps even with no decay at all (pure overwriting) and faster
with the decay gates.  The same curves from the oracle over a shorter horizon
match the GPU's.
"""
import numpy as np
import pytest
import torch

from nvfp4_w4a4_gemm_quantize_amd import inputs
from oracle import recurrence as R
from tests.parity import assert_within, dev_bf16, gpu_out_f64, host

pytestmark = pytest.mark.gpu
D = 128


def f(bits):
    return inputs.bf16_bits_to_f32(bits).astype(np.float64)


def oracle_run(d, hk, hv, s_init=None):
    T = d["q"].shape[0]
    o, S, nr = R.recurrence(f(d["q"]).reshape(T, hk, D), f(d["k"]).reshape(T, hk, D), f(d["v"]).reshape(T, hv, D),
                            f(d["beta"]), f(d["g"]), s_init=s_init, return_row_norms=True)
    return o, S, nr


def tolerances(d, nr, hv, bf16_out=False, o_ref=None):
    T = d["q"].shape[0]
    v, g = f(d["v"]).reshape(T, hv, D), f(d["g"])
    return R.fp32_tolerance(nr, v, g, bf16_out, o_ref), R.fp32_state_tolerance(nr, v, g)


def assert_l2(got, ref, bf16_out, what):
    """Aggregate check: ||got - ref||_2 <= (1e-5 [+ 2^-8 for a bf16 output]) ||ref||_2."""
    rel = 1e-5 + (R.U_BF16 if bf16_out else 0.0)
    err, nrm = np.linalg.norm(got - ref), np.linalg.norm(ref)
    assert err <= rel * nrm, "%s: L2 error %.3g of a %.3g norm exceeds %.3g" % (what, err, nrm, rel * nrm)


def gpu_run(lib, d, hk, hv, s_init=None, out_dtype=torch.float32):
    dv = {n: dev_bf16(d[n]) for n in ("q", "k", "v", "beta", "g")}
    si = None if s_init is None else torch.tensor(s_init, dtype=torch.float32, device="cuda").contiguous()
    return lib.gdn_recurrence(dv["q"], dv["k"], dv["v"], dv["beta"], dv["g"], hk, hv, s_init=si,
                              return_state=True, out_dtype=out_dtype)


def _with_resets(d, seed):
    """Near-total resets (g = -12, decay 6e-6) at 2% of the steps: about half of
    the 32-step chunks hold one, so both the scaled and the unscaled state
    update run, in every head, with switches between them."""
    g = f(d["g"])
    hit = np.random.default_rng(seed).uniform(size=g.shape) < 0.02
    out = dict(d)
    out["g"] = inputs.f32_to_bf16_bits(np.where(hit, -12.0, g).astype(np.float32))
    return out


@pytest.mark.parametrize("T,hk,hv,with_init,bf16_out,resets", [
    (300, 2, 6, True, False, False),     # ragged last chunk, grouped key heads, initial state
    (1, 1, 1, False, False, False),      # a single step
    (32, 1, 2, True, True, False),       # half a 64-step chunk (the partial-chunk loop only); bf16 output
    (33, 4, 4, False, False, False),
    (64, 1, 3, True, True, False),       # exactly one chunk
    (65, 2, 2, False, False, False),     # one step into the second chunk
    (640, 2, 6, True, False, True),      # decays outside [2^-12, 2^12] in some chunks
    (301, 1, 3, False, True, True),
])
def test_recurrence_parity_small(gpu_lib, T, hk, hv, with_init, bf16_out, resets):
    d = inputs.recurrence(T, hk, hv, seed=T)
    if resets:
        d = _with_resets(d, T + 1)
    s0 = (np.random.default_rng(T).standard_normal((hv, D, D)) * 0.05).astype(np.float32) if with_init else None
    o, S = gpu_run(gpu_lib, d, hk, hv, s0, torch.bfloat16 if bf16_out else torch.float32)
    o_ref, S_ref, nr = oracle_run(d, hk, hv, s0)
    tol, tol_s = tolerances(d, nr, hv, bf16_out, o_ref)
    got = gpu_out_f64(o).reshape(T, hv, D)
    assert_within(got, o_ref, tol, "recurrence output T=%d" % T)
    assert_within(host(S).astype(np.float64), S_ref, tol_s, "final state")
    assert_l2(got, o_ref, bf16_out, "recurrence output T=%d" % T)
    assert_l2(host(S).astype(np.float64), S_ref, False, "final state T=%d" % T)
    o2, S2 = gpu_run(gpu_lib, d, hk, hv, s0, torch.bfloat16 if bf16_out else torch.float32)
    assert torch.equal(o, o2) and torch.equal(S, S2)


def test_recurrence_reads_a_fused_inprojection_buffer(gpu_lib):
    """q | k | v | z | b | a columns of one bf16 [T, 16480] buffer, passed as strided views."""
    T, hk, hv = 70, 16, 48
    d = inputs.recurrence(T, hk, hv, seed=7)
    offs = np.cumsum([0] + [w for _, w in inputs.GDN_SEGMENTS])
    buf = np.zeros((T, offs[-1]), dtype=np.uint16)
    buf[:, offs[0]:offs[1]], buf[:, offs[1]:offs[2]], buf[:, offs[2]:offs[3]] = d["q"], d["k"], d["v"]
    buf[:, offs[4]:offs[5]], buf[:, offs[5]:offs[6]] = d["beta"], d["g"]
    dbuf = dev_bf16(buf)
    o = gpu_lib.gdn_recurrence(dbuf[:, offs[0]:offs[1]], dbuf[:, offs[1]:offs[2]], dbuf[:, offs[2]:offs[3]],
                               dbuf[:, offs[4]:offs[5]], dbuf[:, offs[5]:offs[6]], hk, hv, out_dtype=torch.bfloat16)
    o_ref, _, nr = oracle_run(d, hk, hv)
    tol, _ = tolerances(d, nr, hv, True, o_ref)
    got = gpu_out_f64(o).reshape(T, hv, D)
    assert_within(got, o_ref, tol, "recurrence on fused buffer")
    assert_l2(got, o_ref, True, "recurrence on fused buffer")


def test_recurrence_full_heads_4096_tokens(gpu_lib):
    T, hk, hv = 4096, 16, 48
    d = inputs.recurrence(T, hk, hv)
    o, S = gpu_run(gpu_lib, d, hk, hv)
    o_ref, S_ref, nr = oracle_run(d, hk, hv)
    tol, tol_s = tolerances(d, nr, hv)
    got = gpu_out_f64(o).reshape(T, hv, D)
    assert_within(got, o_ref, tol, "recurrence 4096 tokens")
    assert_within(host(S).astype(np.float64), S_ref, tol_s, "final state, 4096 tokens")
    assert_l2(got, o_ref, False, "recurrence 4096 tokens")


def _noisy(d, eps, seed):
    """10%-style relative noise on keys, values and both gates (beta kept in [0, 1], g <= 0)."""
    rng = np.random.default_rng(seed)
    out = dict(d)
    for n in ("k", "v"):
        x = f(d[n])
        out[n] = inputs.f32_to_bf16_bits((x * (1 + eps * rng.standard_normal(x.shape))).astype(np.float32))
    b = np.clip(f(d["beta"]) * (1 + eps * rng.standard_normal(d["beta"].shape)), 0.0, 1.0)
    g = np.minimum(f(d["g"]) * (1 + eps * rng.standard_normal(d["g"].shape)), 0.0)
    out["beta"] = inputs.f32_to_bf16_bits(b.astype(np.float32))
    out["g"] = inputs.f32_to_bf16_bits(g.astype(np.float32))
    return out


def _windows(err, ref, w):
    n = err.shape[0] // w
    return np.array([np.linalg.norm(err[i * w:(i + 1) * w]) / np.linalg.norm(ref[i * w:(i + 1) * w])
                     for i in range(n)])


def test_injected_noise_plateaus_over_32k_tokens(gpu_lib):
    T, hk, hv = 32768, 4, 12
    d = inputs.recurrence(T, hk, hv, seed=11)
    dn = _noisy(d, 0.1, 12)
    o, _ = gpu_run(gpu_lib, d, hk, hv)
    on, _ = gpu_run(gpu_lib, dn, hk, hv)
    o, on = gpu_out_f64(o), gpu_out_f64(on)
    rel = _windows(on - o, o, 1024)
    print("\nrelative output error per 1024-token window (noise 10%% on k, v, beta, g):\n%s" %
          np.array2string(rel, precision=4, max_line_width=100))
    late, early = rel[-8:].mean(), rel[1:9].mean()
    assert 0.8 < late / early < 1.25, (early, late)     # flat: no growth with position
    # the oracle's curve over the first 2048 tokens agrees with the GPU's
    To = 2048
    sub = {n: d[n][:To] for n in d}
    subn = {n: dn[n][:To] for n in dn}
    r0, _, _ = oracle_run(sub, hk, hv)
    r1, _, _ = oracle_run(subn, hk, hv)
    ro = _windows((r1 - r0).reshape(To, -1), r0.reshape(To, -1), 1024)
    np.testing.assert_allclose(rel[:2], ro, rtol=1e-3)


@pytest.mark.parametrize("decay", [False, True])
def test_state_impulse_is_forgotten(gpu_lib, decay):
    T, hk, hv = 8192, 4, 12
    d = inputs.recurrence(T, hk, hv, seed=21)
    d["v"] = np.zeros_like(d["v"])
    if not decay:
        d["g"] = np.zeros_like(d["g"])            # alpha = 1: only the overwrites remove the impulse
    s0 = np.random.default_rng(22).standard_normal((hv, D, D)).astype(np.float32)
    o, S = gpu_run(gpu_lib, d, hk, hv, s0)
    amp = np.linalg.norm(gpu_out_f64(o).reshape(T, hv, D), axis=2)       # [T, hv]
    rel = amp / amp[:16].mean(axis=0)
    steps = [int(np.argmax(rel[:, h] < 1e-2)) if (rel[:, h] < 1e-2).any() else T for h in range(hv)]
    print("\nsteps until the impulse's output is below 1%% of its start (%s): median %d, max %d" % (
        "decay gates on" if decay else "no decay, overwrite only", int(np.median(steps)), max(steps)))
    assert max(steps) < T and np.linalg.norm(host(S)) < 1e-2 * np.linalg.norm(s0)
    # oracle agreement on the first 512 steps
    sub = {n: d[n][:512] for n in d}
    o_ref, _, _ = oracle_run(sub, hk, hv, s0)
    amp_ref = np.linalg.norm(o_ref, axis=2)
    np.testing.assert_allclose(amp[:512], amp_ref, rtol=1e-4, atol=1e-6 * amp_ref.max())
