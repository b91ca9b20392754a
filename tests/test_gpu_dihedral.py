"""GPU parity of the dihedral D_n layers (regular n-gon, order 2n) against the fp64 oracle.

The block layer (eqlinear_d8_forward on an eqlinear_dihedral_plan), the
expanded comparator, the fused regular-domain round trip and its two halves
for n = 2, 3, 5, 6, 8, 12 -- odd and even orders, one to five 2-D irreps --
at widths where every block is whole 16-byte pieces (the dedicated bf16
kernel) and where it is not (the row GEMM), both dtypes.  Same bars as the
forward (tests/gpu_util.py).  Inputs from synthetic.py (seeded); expected values
only from oracle/.
"""
import numpy as np
import pytest

import oracle
import synthetic
from gpu_util import Guarded, assert_close, to_dev, to_f64

pytestmark = pytest.mark.gpu

F32, BF16, F16 = synthetic.F32, synthetic.BF16, synthetic.F16
ORDERS = [2, 3, 5, 6, 8, 12]


@pytest.fixture(scope="module")
def eq():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import group_equivariant_linear_amd as eq
    eq.load_library()  # raises if the library was not built: no fallback
    return eq


def _eqdt(eq, dt):
    return {F32: eq.EQL_F32, BF16: eq.EQL_BF16, F16: eq.EQL_F16}[dt]


def _shapes(n):
    G = 2 * n
    # (C_in, C_out, T): blocks of 8-multiples (whole 16-byte bf16 pieces), then ragged ones
    return [(G * 8, G * 16, 300), (G * 3, G * 5, 77), (G, G, 1)]


@pytest.mark.parametrize("dt", [F32, BF16, F16])
@pytest.mark.parametrize("n", ORDERS)
def test_dihedral_forward(eq, n, dt):
    import torch
    for C_in, C_out, T in _shapes(n):
        d = synthetic.dn_inputs(n, C_in, C_out, T, dt, seed=n + C_in)
        plan = eq.eqlinear_dihedral_plan(n, C_in, C_out, _eqdt(eq, dt))
        assert plan.info["w_hat_elems"] == d["w"].size
        y = Guarded(T * C_out, dt, (T, C_out))
        eq.eqlinear_d8_forward(plan, to_dev(d["x"], dt).reshape(T, C_in), to_dev(d["w"], dt), y.t, T=T)
        torch.cuda.synchronize()
        y.check_guards()
        ref = oracle.dn_dense(n, d["x64"], d["w64"], C_out)
        assert_close(to_f64(y.t), ref, dt, f"D_{n} {dt} {C_in}->{C_out} T={T}")


@pytest.mark.parametrize("dt", [BF16, F16])
@pytest.mark.parametrize("n", [3, 6])
def test_dihedral_forward_96_channel_tiles(eq, n, dt):
    """1-D blocks of 96 or 192 output channels take the 64-token x 96-channel
    tile of the matrix-core kernel (the D6 workload's shape at width 1152):
    square and widening layers, ragged token counts."""
    import torch
    G = 2 * n
    for C_in, C_out, T in [(G * 96, G * 96, 130), (G * 48, G * 192, 70)]:
        d = synthetic.dn_inputs(n, C_in, C_out, T, dt, seed=7 * n + C_out)
        plan = eq.eqlinear_dihedral_plan(n, C_in, C_out, _eqdt(eq, dt))
        y = Guarded(T * C_out, dt, (T, C_out))
        eq.eqlinear_d8_forward(plan, to_dev(d["x"], dt).reshape(T, C_in), to_dev(d["w"], dt), y.t, T=T)
        torch.cuda.synchronize()
        y.check_guards()
        ref = oracle.dn_dense(n, d["x64"], d["w64"], C_out)
        assert_close(to_f64(y.t), ref, dt, f"D_{n} {dt} {C_in}->{C_out} T={T}")


@pytest.mark.parametrize("dt", [BF16, F16])
def test_d6_workload_full_size(eq, dt):
    """The D6 benchmark workload (width 1152, T = 4112; bf16 as benchmarked, and
    fp16) in its bench launch, every token row."""
    import torch
    wl = synthetic.WORKLOADS["d6"]
    n = wl.N // 2
    d = synthetic.dn_inputs(n, wl.C_in, wl.C_out, wl.T, dt, seed=0)
    plan = eq.eqlinear_dihedral_plan(n, wl.C_in, wl.C_out, _eqdt(eq, dt))
    y = Guarded(wl.T * wl.C_out, dt, (wl.T, wl.C_out))
    eq.eqlinear_d8_forward(plan, to_dev(d["x"], dt).reshape(wl.T, wl.C_in), to_dev(d["w"], dt), y.t, T=wl.T)
    torch.cuda.synchronize()
    y.check_guards()
    ref = oracle.dn_dense(n, d["x64"], d["w64"], wl.C_out)
    r, m = assert_close(to_f64(y.t), ref, dt, f"d6 {dt}")
    print(f"d6 {dt}: rel-L2 {r:.3e} max/rms {m:.3e} over all {wl.T} tokens")


@pytest.mark.parametrize("dt", [F32, BF16, F16])
@pytest.mark.parametrize("n", [3, 6, 12])
def test_dihedral_comparator(eq, n, dt):
    import torch
    C_in, C_out, T = 2 * n * 4, 2 * n * 6, 50
    d = synthetic.dn_inputs(n, C_in, C_out, T, dt, seed=3)
    plan = eq.eqlinear_dihedral_plan(n, C_in, C_out, _eqdt(eq, dt))
    Wd = Guarded(C_out * C_in, dt, (C_out, C_in))
    eq.eqlinear_expand_dense(plan, to_dev(d["w"], dt), Wd.t)
    y = Guarded(T * C_out, dt, (T, C_out))
    eq.eqlinear_dense_forward(plan, to_dev(d["x"], dt).reshape(T, C_in), Wd.t, y.t, T=T)
    torch.cuda.synchronize()
    Wd.check_guards()
    assert np.array_equal(to_f64(Wd.t), oracle.dn_expand(n, d["w64"], C_in, C_out))  # a copy: exact
    assert_close(to_f64(y.t), oracle.dn_dense(n, d["x64"], d["w64"], C_out), dt, f"D_{n} comparator")


def test_order_four_is_the_d8_layer(eq):
    import torch
    C, T = 64, 100
    d = synthetic.d8_inputs(C, C, T, BF16, seed=1)
    x, w = to_dev(d["x"], BF16).reshape(T, C), to_dev(d["w"], BF16)
    outs = []
    for plan in (eq.eqlinear_d8_plan(C, C, eq.EQL_BF16), eq.eqlinear_dihedral_plan(4, C, C, eq.EQL_BF16)):
        y = torch.empty(T, C, dtype=torch.bfloat16, device="cuda")
        eq.eqlinear_d8_forward(plan, x, w, y, T=T)
        outs.append(y)
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1])


@pytest.mark.parametrize("dt", [F32, BF16, F16])
@pytest.mark.parametrize("n", ORDERS)
def test_dihedral_passes(eq, n, dt):
    import torch
    G = 2 * n
    for C, T in ((G * 3, 41), (G * 8, 130)):
        m = C // G
        plan = eq.eqlinear_dihedral_plan(n, C, C, _eqdt(eq, dt))
        d = synthetic.dn_inputs(n, C, C, T, dt, seed=C + n)
        bd, b64 = synthetic.channel_bias(m, dt, seed=n)
        xin = to_dev(d["x"], dt).reshape(T, C)
        for bias, act in ((True, 1), (False, 1), (True, 0)):
            out = Guarded(T * C, dt, (T, C))
            eq.eqlinear_d8_bias_act(plan, xin, to_dev(bd, dt) if bias else None, act, out.t, T=T)
            torch.cuda.synchronize()
            out.check_guards()
            ref = oracle.dn_bias_act(n, d["x64"], b64 if bias else None, act)
            assert_close(to_f64(out.t), ref, dt, f"D_{n} round trip C={C} bias={bias} act={act}")
        four = Guarded(T * C, dt, (T, C))
        reg = Guarded(T * C, dt, (T, C))
        eq.eqlinear_d8_to_fourier(plan, xin, four.t, T=T)
        eq.eqlinear_d8_to_regular(plan, xin, reg.t, T=T)
        torch.cuda.synchronize()
        four.check_guards()
        reg.check_guards()
        assert_close(to_f64(four.t), oracle.dn_to_fourier(n, d["x64"].reshape(T, m, G)), dt, f"D_{n} to_fourier")
        assert_close(to_f64(reg.t), oracle.dn_to_regular(n, d["x64"]).reshape(T, C), dt, f"D_{n} to_regular")


@pytest.mark.parametrize("n", [3, 6])
def test_dihedral_layer_on_regular_features_with_gelu(eq, n):
    """Regular features -> Fourier layout -> D_n layer -> bias + GELU round trip ->
    regular layout, against the oracle's chain (fp32)."""
    import torch
    G = 2 * n
    C_in, C_out, T = G * 4, G * 6, 120
    d = synthetic.dn_inputs(n, C_in, C_out, T, F32, seed=21)
    bd, b64 = synthetic.channel_bias(C_out // G, F32, seed=22)
    plan = eq.eqlinear_dihedral_plan(n, C_in, C_out, eq.EQL_F32)
    xf = torch.empty(T, C_in, device="cuda")
    yf = torch.empty(T, C_out, device="cuda")
    yr = Guarded(T * C_out, F32, (T, C_out))
    eq.eqlinear_d8_to_fourier(plan, to_dev(d["x"], F32).reshape(T, C_in), xf, T=T)
    eq.eqlinear_d8_forward(plan, xf, to_dev(d["w"], F32), yf, T=T)
    eq.eqlinear_d8_bias_act(plan, yf, to_dev(bd, F32), eq.EQL_ACT_GELU, yf, T=T)
    eq.eqlinear_d8_to_regular(plan, yf, yr.t, T=T)
    torch.cuda.synchronize()
    yr.check_guards()
    xr = d["x64"].reshape(T, C_in // G, G)
    ref = oracle.dn_to_regular(n, oracle.dn_dense_bias_act(n, oracle.dn_to_fourier(n, xr), d["w64"], C_out, b64, 1))
    assert_close(to_f64(yr.t), ref.reshape(T, C_out), F32, f"D_{n} regular chain")
