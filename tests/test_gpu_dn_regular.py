"""GPU parity of the one-launch dihedral layer between regular-representation
features (eqlinear_d8_regular_forward): x_reg -> group-Fourier transform ->
block products -> inverse transform -> bias + GELU -> y_reg, against the
oracle's chain of pinned steps,
    dn_to_regular(dn_dense_bias_act(dn_to_fourier(x_reg)))
for D_n, n = 2 .. 6 and 12 (one to five 2-D irreps), bf16 and fp16, shapes
with whole and ragged input-channel chunks, ragged output tiles and ragged
token tiles, and the c5 (D8) and d6 (D6) benchmark layers at full size, every
token row.  Same bars as the forward (tests/gpu_util.py).  Inputs from
synthetic.py (seeded); expected values only from oracle/.
"""
import numpy as np
import pytest

import oracle
import synthetic
from gpu_util import Guarded, assert_close, to_dev, to_f64

pytestmark = pytest.mark.gpu

BF16, F16 = synthetic.BF16, synthetic.F16


@pytest.fixture(scope="module")
def eq():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import group_equivariant_linear_amd as eq
    eq.load_library()  # raises if the library was not built: no fallback
    return eq


def _eqdt(eq, dt):
    return {BF16: eq.EQL_BF16, F16: eq.EQL_F16}[dt]


def run_regular(eq, n, C_in, C_out, T, dt, act, with_bias, seed):
    import torch
    G = 2 * n
    d = synthetic.dn_inputs(n, C_in, C_out, T, dt, seed=seed)
    bd, b64 = synthetic.channel_bias(C_out // G, dt, seed=seed + 1)
    plan = eq.eqlinear_dihedral_plan(n, C_in, C_out, _eqdt(eq, dt))
    y = Guarded(T * C_out, dt, (T, C_out))
    eq.eqlinear_d8_regular_forward(plan, to_dev(d["x"], dt).reshape(T, C_in), to_dev(d["w"], dt),
                                   to_dev(bd, dt) if with_bias else None, act, y.t, T=T)
    torch.cuda.synchronize()
    y.check_guards()
    xr = d["x64"].reshape(T, C_in // G, G)  # x read as regular features
    ref = oracle.dn_to_regular(n, oracle.dn_dense_bias_act(n, oracle.dn_to_fourier(n, xr), d["w64"], C_out,
                                                            b64 if with_bias else None, act))
    return to_f64(y.t), ref.reshape(T, C_out)


def _shapes(n):
    G = 2 * n
    # (m_in, m_out, T) in regular channels: whole 32-channel chunks and 32-channel
    # output tiles; a ragged last chunk (40 = 32 + 8) and a ragged output tile
    # (24); one token, a ragged token tile, several tiles
    return [(32, 32, 64), (64, 96, 300), (40, 24, 77), (8, 8, 1), (96, 40, 33)]


@pytest.mark.parametrize("dt", [BF16, F16])
@pytest.mark.parametrize("n", [2, 3, 4, 5, 6, 12])
def test_regular_forward_matches_the_oracle_chain(eq, n, dt):
    G = 2 * n
    for i, (mi, mo, T) in enumerate(_shapes(n)):
        for act, with_bias in [(eq.EQL_ACT_GELU, True), (eq.EQL_ACT_NONE, False), (eq.EQL_ACT_NONE, True)]:
            y, ref = run_regular(eq, n, G * mi, G * mo, T, dt, act, with_bias, seed=10 * n + i)
            assert_close(y, ref, dt, f"D_{n} {dt} m {mi}->{mo} T={T} act={act} bias={with_bias}")


@pytest.mark.parametrize("dt", [BF16, F16])
def test_regular_forward_is_equivariant(eq, dt):
    """Acting with a group element on every input channel (a permutation of its
    G values) acts the same way on every output channel."""
    import torch
    n, m_in, m_out, T = 4, 32, 40, 50
    G = 2 * n
    d = synthetic.dn_inputs(n, G * m_in, G * m_out, T, dt, seed=3)
    bd, _ = synthetic.channel_bias(m_out, dt, seed=4)
    plan = eq.eqlinear_dihedral_plan(n, G * m_in, G * m_out, _eqdt(eq, dt))
    w, b = to_dev(d["w"], dt), to_dev(bd, dt)

    def run(xbits):
        y = torch.empty(T, G * m_out, dtype=w.dtype, device="cuda")
        eq.eqlinear_d8_regular_forward(plan, to_dev(xbits, dt).reshape(T, -1), w, b, eq.EQL_ACT_GELU, y, T=T)
        torch.cuda.synchronize()
        return to_f64(y).reshape(T, m_out, G)

    y0 = run(d["x"])
    xr = d["x"].reshape(T, m_in, G)
    # left multiplication by the generators: element q = a + n b is r^a s^b;
    # r r^a s^b = r^(a+1) s^b, s r^a s^b = r^(-a) s^(1-b)
    q = np.arange(G)
    a, bb = q % n, q // n
    for perm in [((a + 1) % n) + n * bb, ((-a) % n) + n * (1 - bb)]:
        # (g.f)(q) = f(g^-1 q): output element perm[q] takes input element q
        xg = np.empty_like(xr)
        xg[..., perm] = xr
        yg = run(np.ascontiguousarray(xg))
        y0g = np.empty_like(y0)
        y0g[..., perm] = y0
        assert_close(yg, y0g, dt, "equivariance")


@pytest.mark.parametrize("dt", [BF16, F16])
@pytest.mark.parametrize("name", ["c5", "d6"])
def test_regular_forward_workload_full_size(eq, name, dt):
    """The benchmark dihedral layers (D8 width 1280, D6 width 1152, T = 4112)
    with a bias and GELU, regular features in and out, every token row."""
    wl = synthetic.WORKLOADS[name]
    n = wl.N // 2
    y, ref = run_regular(eq, n, wl.C_in, wl.C_out, wl.T, dt, eq.EQL_ACT_GELU, True, seed=0)
    r, m = assert_close(y, ref, dt, f"{name} regular {dt}")
    print(f"{name} regular {dt}: rel-L2 {r:.3e} max/rms {m:.3e} over all {wl.T} tokens")
    for t0 in range(0, wl.T, 32):
        assert_close(y[t0:t0 + 32], ref[t0:t0 + 32], dt, f"{name} tokens {t0}..")


def test_regular_forward_rejections(eq):
    import torch
    plan32 = eq.eqlinear_dihedral_plan(4, 64, 64, eq.EQL_F32)
    x = torch.zeros(64 * 10, device="cuda")
    with pytest.raises(eq.EqlError):  # fp32 plans: not on this path
        eq.eqlinear_d8_regular_forward(plan32, x, torch.zeros(plan32.info["w_hat_elems"], device="cuda"), None,
                                       eq.EQL_ACT_NONE, torch.empty_like(x), T=10)
    plan = eq.eqlinear_dihedral_plan(4, 8 * 12, 8 * 16, eq.EQL_BF16)  # 12 input channels: not a multiple of 8
    xb = torch.zeros(10 * 96, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(eq.EqlError):
        eq.eqlinear_d8_regular_forward(plan, xb, torch.zeros(plan.info["w_hat_elems"], dtype=torch.bfloat16,
                                                             device="cuda"), None, eq.EQL_ACT_NONE,
                                       torch.empty(10 * 128, dtype=torch.bfloat16, device="cuda"), T=10)
