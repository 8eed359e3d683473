"""Seeded synthetic workloads for the NVFP4 W4A4 linear layers.

This module only draws random numbers and rounds them to bf16; it holds none
of the quantizer's or the GEMM's arithmetic.  Tests feed the same bf16 bit
patterns to the HIP library and to the CPU oracle, and the benchmark uses it
to build device inputs.  It imports neither of them.

Workloads (the pages evaluate a 27B hybrid model on public benchmarks; no
dataset or checkpoint is used here, these seeded inputs of the model's
linear-layer shapes stand in for them):

tiny        M=16  N=64    K=128   A ~ N(0,1) with column 7 x100; W ~ N(0, 0.02)
linear      M=2048 N=5120 K=5120  A ~ Student-t(4) with round(0.001 K) outlier
                                  channels x50; W ~ N(0, 1/sqrt(K))
mlp         M=4096 K=5120; gate_up N=2x17408 (gate | up) with SiLU*mul, then
            down N=5120 K=17408; A as 'linear'; W ~ N(0, 1/sqrt(K))
gdn_inproj  M=4096 K=5120; q 2048 | k 2048 | v 6144 | z 6144 | b 48 | a 48;
            module weights N(0, 1/sqrt(K)) * f_s, log2 f_s spread over [0, 3]
            (max/min scale ratio exactly 8); A_log, dt_bias ~ N(0, 0.5) [48]
decode      M in {1, 8, 32, 64}, N=17408, K=5120; A ~ N(0,1) with 5 outlier
            channels x50; W ~ N(0, 1/sqrt(K))
recurrence  gated delta rule over T tokens, 16 key heads / 48 value heads of
            dimension 128 (the in-projection's q | k | v split): q, k, v ~
            N(0, 1); write strength beta ~ U(0, 1); log-decay g = -r with r
            log-uniform on [1e-4, 1e-1] (decay factors 0.905 .. 0.9999, the
            long-memory regime where an accumulating state would grow)

N(mu, sigma) takes sigma as the standard deviation.  Every stream is seeded
by (seed, name) so any tensor can be regenerated on its own.
"""
import zlib

import numpy as np

GDN_SEGMENTS = (("q", 2048), ("k", 2048), ("v", 6144), ("z", 6144), ("b", 48), ("a", 48))
DECODE_M = (1, 8, 32, 64)

SHAPES = {
    "tiny": dict(M=16, N=64, K=128),
    "linear": dict(M=2048, N=5120, K=5120),
    "mlp": dict(M=4096, K=5120, N_gate_up=2 * 17408, N_down=5120, K_down=17408),
    "gdn_inproj": dict(M=4096, K=5120, N=sum(w for _, w in GDN_SEGMENTS)),
    "decode": dict(N=17408, K=5120, M_list=DECODE_M),
}


def rng(name, seed=0):
    """Independent generator for a named sub-stream."""
    return np.random.default_rng(np.random.SeedSequence([seed, zlib.crc32(name.encode())]))


def f32_to_bf16_bits(x):
    """float32 -> bf16 bit patterns, round to nearest even (finite inputs)."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((b + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint16)


def bf16_bits_to_f32(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def normal(shape, sigma, name, seed=0):
    g = rng(name, seed)
    return f32_to_bf16_bits(g.standard_normal(shape, dtype=np.float32) * np.float32(sigma))


def outlier_channels(K, count, name, seed=0):
    return np.sort(rng(name, seed).choice(K, size=count, replace=False))


def student_t_activations(M, K, name, seed=0, outlier_gain=50.0):
    """Student-t(4) activations with round(0.001 K) channels scaled x outlier_gain."""
    a = rng(name, seed).standard_t(4.0, size=(M, K)).astype(np.float32)
    ch = outlier_channels(K, max(1, int(round(0.001 * K))), name + "/outliers", seed)
    a[:, ch] *= np.float32(outlier_gain)
    return f32_to_bf16_bits(a)


def normal_activations(M, K, name, seed=0, n_outliers=5, outlier_gain=50.0):
    a = rng(name, seed).standard_normal((M, K), dtype=np.float32)
    ch = outlier_channels(K, n_outliers, name + "/outliers", seed)
    a[:, ch] *= np.float32(outlier_gain)
    return f32_to_bf16_bits(a)


def tiny(seed=0):
    """A [16,128] N(0,1), column 7 x100; W [64,128] N(0, 0.02)."""
    s = SHAPES["tiny"]
    a = rng("tiny/A", seed).standard_normal((s["M"], s["K"]), dtype=np.float32)
    a[:, 7] *= np.float32(100.0)
    return dict(A=f32_to_bf16_bits(a), W=normal((s["N"], s["K"]), 0.02, "tiny/W", seed))


def linear(seed=0, M=None):
    s = SHAPES["linear"]
    M = s["M"] if M is None else M
    return dict(A=student_t_activations(M, s["K"], "linear/A", seed),
                W=normal((s["N"], s["K"]), 1.0 / np.sqrt(s["K"]), "linear/W", seed))


def mlp(seed=0, M=None, weights=True):
    s = SHAPES["mlp"]
    M = s["M"] if M is None else M
    out = dict(A=student_t_activations(M, s["K"], "mlp/A", seed))
    if weights:
        out["W_gate_up"] = normal((s["N_gate_up"], s["K"]), 1.0 / np.sqrt(s["K"]),
                                  "mlp/W_gate_up", seed)
        out["W_down"] = normal((s["N_down"], s["K_down"]), 1.0 / np.sqrt(s["K_down"]),
                               "mlp/W_down", seed)
    return out


def module_scale_factors(n, name, seed=0, max_ratio=8.0):
    """Per-module weight magnitudes f_s: log2 f_s uniform, mapped so min f = 1, max f = max_ratio."""
    v = rng(name, seed).uniform(0.0, 1.0, size=n)
    v = (v - v.min()) / (v.max() - v.min())
    return np.exp2(v * np.log2(max_ratio))


def gdn_inproj(seed=0, M=None, weights=True):
    s = SHAPES["gdn_inproj"]
    M = s["M"] if M is None else M
    K = s["K"]
    out = dict(A=student_t_activations(M, K, "gdn/A", seed))
    offsets = np.cumsum([0] + [w for _, w in GDN_SEGMENTS]).astype(np.int64)
    out["seg_offsets"] = offsets
    out["seg_names"] = [n for n, _ in GDN_SEGMENTS]
    f = module_scale_factors(len(GDN_SEGMENTS), "gdn/module_scales", seed)
    out["module_factors"] = f
    if weights:
        parts = []
        for (name, width), fs in zip(GDN_SEGMENTS, f):
            w = rng("gdn/W/" + name, seed).standard_normal((width, K), dtype=np.float32)
            parts.append(f32_to_bf16_bits(w * np.float32(fs / np.sqrt(K))))
        out["W"] = np.concatenate(parts, axis=0)
    heads = dict(GDN_SEGMENTS)["a"]
    out["A_log"] = (rng("gdn/A_log", seed).standard_normal(heads) * 0.5).astype(np.float32)
    out["dt_bias"] = (rng("gdn/dt_bias", seed).standard_normal(heads) * 0.5).astype(np.float32)
    return out


def decode(M, seed=0, weights=True):
    s = SHAPES["decode"]
    out = dict(A=normal_activations(M, s["K"], "decode/A%d" % M, seed))
    if weights:
        out["W"] = normal((s["N"], s["K"]), 1.0 / np.sqrt(s["K"]), "decode/W", seed)
    return out


def recurrence(T, hk=16, hv=48, seed=0, d=128):
    """Inputs of the gated delta rule: bf16 bits q, k [T, hk*d], v [T, hv*d], beta, g [T, hv]."""
    out = dict(q=normal((T, hk * d), 1.0, "rec/q", seed), k=normal((T, hk * d), 1.0, "rec/k", seed),
               v=normal((T, hv * d), 1.0, "rec/v", seed))
    out["beta"] = f32_to_bf16_bits(rng("rec/beta", seed).uniform(0.0, 1.0, (T, hv)).astype(np.float32))
    r = np.exp(rng("rec/g", seed).uniform(np.log(1e-4), np.log(1e-1), (T, hv)))
    out["g"] = f32_to_bf16_bits((-r).astype(np.float32))
    return out
