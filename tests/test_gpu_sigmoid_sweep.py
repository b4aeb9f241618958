"""GPU: the sigmoid inside the kernels, swept over every bf16 input.

SwitchGLU's middle step silu(g) * u (MLX issue 4509, moe()) and the shared
expert's gate sigmoid(z) * s (MTPLX PR 558, Summary/Change) are the only
transcendental steps on the path.  The kernels form them in fp32 with the
hardware exponential (and, in the GLU, the hardware reciprocal); the oracle
forms them in float64 and rounds once.  The fp32 steps carry a relative error
of a few units in 2^-24, far below bf16's 2^-8, so each bf16 result may differ
from the oracle's only where the exact value lies next to a rounding boundary,
and then by one bf16 step.  These tests hold every bf16 value of |v| <= 80 to
that: at most one bf16 step from the oracle, and at least 99.9% bit-equal.
Every gate/up route (one-row, few-row, skinny and both tile kernels) applies
the same GLU epilogue to its fp32 g and u, so the decode route stands for all
of them once g and u are exact, which the integer-exact tests establish.
Outside |v| <= 80 the sigmoid saturates: the results are checked against the
limits, 1 for large arguments and 0 (to below 2^-100) for very negative ones.
"""
import numpy as np
import pytest
import torch

import oracle
from helpers import bf, host_bf, i32, triple

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import moe_expert_gathered_amd as m
    m.lib()
    return m


def bf16_values(lo_abs, hi_abs):
    """Every finite bf16 bit pattern with lo_abs <= |v| <= hi_abs (and 0 when lo_abs is 0), both signs."""
    pos = np.arange(0, 0x7F80, dtype=np.uint32).astype(np.uint16)
    mag = oracle.bf16_to_f64(pos)
    pos = pos[(mag >= lo_abs) & (mag <= hi_abs)]
    neg = (pos[pos != 0].astype(np.uint32) | 0x8000).astype(np.uint16)
    return np.concatenate([pos, neg])


def steps_apart(a_u16, b_u16):
    """Distance in bf16 steps between two bf16 bit patterns (+0 and -0 coincide)."""
    def order(u):
        u = u.astype(np.int64)
        return np.where(u & 0x8000, -(u & 0x7FFF), u)
    return np.abs(order(a_u16) - order(b_u16))


def check_sweep(got, want, name):
    d = steps_apart(got, want)
    assert d.max() <= 1, f"{name}: {int((d > 1).sum())} results more than one bf16 step off (max {int(d.max())})"
    exact = float((d == 0).mean())
    assert exact >= 0.999, f"{name}: only {exact:.5f} bit-equal"
    return exact


def test_sigmoid_gate_every_bf16(mg):
    """bf16(sigmoid(z) * s) for every bf16 z in [-80, 80], against s = 1 and
    seven scales of magnitude in [0.5, 2) with random signs (products stay
    normal in fp32 and bf16 at the far end, sigmoid(-80) ~ 1.8e-35)."""
    z = bf16_values(0.0, 80.0)
    T, H = z.size, 8
    g = np.random.default_rng(5)
    sv = np.empty((T, H), dtype=np.float64)
    sv[:, 0] = 1.0
    sv[:, 1:] = g.uniform(0.5, 2.0, (T, H - 1)) * g.choice([-1.0, 1.0], (T, H - 1))
    s = oracle.f64_to_bf16(sv)
    want = oracle.f64_to_bf16(oracle.bf16_to_f64(s) / (1.0 + np.exp(-oracle.bf16_to_f64(z)))[:, None])
    got = host_bf(mg.sigmoid_gate(bf(s), bf(z)))
    exact = check_sweep(got, want, "sigmoid gate")
    print(f"sigmoid gate: {T} gate values x {H}, {exact:.5f} bit-equal")


def test_sigmoid_gate_saturation(mg):
    """Beyond |z| = 80: sigmoid(z) * s is s itself for large z and zero for very negative z."""
    z = bf16_values(80.0 + 1e-9, 3.0e38)
    z = np.concatenate([z, np.array([0x7F80, 0xFF80], dtype=np.uint16)])   # +inf, -inf
    T, H = z.size, 8
    s = oracle.f64_to_bf16(np.random.default_rng(6).uniform(0.5, 2.0, (T, H)))
    got = oracle.bf16_to_f64(host_bf(mg.sigmoid_gate(bf(s), bf(z))))
    zf = oracle.bf16_to_f64(z)
    pos, neg = zf > 0, zf < 0
    assert np.array_equal(got[pos], oracle.bf16_to_f64(s)[pos]), "sigmoid(z) * s != s for z > 80"
    assert np.abs(got[neg]).max() < 2.0 ** -100, "sigmoid(z) * s not ~0 for z < -80"


def glu_probe(mg, v_u16):
    """h[n] = bf16(silu(v[n]) * 1) through the one-token decode gate/up route.

    One token x = (1, 0, ..., 0) and one expert whose gate row n has all codes
    0, scale 0 and bias v[n] in its first group (zero elsewhere), and whose up
    rows have bias 1 in the first group: every route forms g = x . w_gate = v[n]
    and u = 1 exactly, so h isolates the GLU epilogue."""
    N = (v_u16.size + 255) // 256 * 256
    K, gs = 512, 64
    v = np.zeros(N, dtype=np.uint16)
    v[: v_u16.size] = v_u16
    w = np.zeros((1, N, K // 8), dtype=np.uint32)
    zero = np.zeros((1, N, K // gs), dtype=np.uint16)
    gb = zero.copy()
    gb[0, :, 0] = v
    ub = zero.copy()
    ub[0, :, 0] = oracle.f64_to_bf16(np.ones(1))[0]
    x = np.zeros((1, K), dtype=np.uint16)
    x[0, 0] = oracle.f64_to_bf16(np.ones(1))[0]
    h = mg.gather_qmm_glu(bf(x), triple((w, zero, gb)), triple((w, zero, ub)), i32(np.zeros(1)),
                          lhs_div=1, group_size=gs, bits=4)
    return host_bf(h).reshape(-1)[: v_u16.size]


def test_decode_glu_every_bf16(mg):
    """bf16(silu(g) * u) in the decode gate/up kernel for every bf16 g with
    2^-120 <= |g| <= 80 (silu of smaller g is an fp32 subnormal) and g = 0."""
    v = bf16_values(2.0 ** -120, 80.0)
    v = np.concatenate([np.zeros(1, dtype=np.uint16), v])
    got = glu_probe(mg, v)
    want = oracle.f64_to_bf16(oracle.silu(oracle.bf16_to_f64(v)))
    exact = check_sweep(got, want, "decode glu")
    print(f"decode glu: {v.size} gate values, {exact:.5f} bit-equal")


def test_decode_glu_saturation(mg):
    """Beyond |g| = 80: silu(g) is g itself for large g and ~0 for very negative g."""
    v = bf16_values(80.0 + 1e-9, 3.0e38)
    got = oracle.bf16_to_f64(glu_probe(mg, v))
    vf = oracle.bf16_to_f64(v)
    pos, neg = vf > 0, vf < 0
    assert np.array_equal(got[pos], vf[pos]), "silu(g) != g for g > 80"
    assert np.abs(got[neg]).max() < 2.0 ** -100, "silu(g) not ~0 for g < -80"
