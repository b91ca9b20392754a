"""GPU parity of the D8 regular-representation passes against the fp64 oracle.

The fused round trip (Fourier -> regular -> act(f + b) -> Fourier) of
eqlinear_d8_bias_act and its two halves, eqlinear_d8_to_fourier and
eqlinear_d8_to_regular, against oracle.d8_bias_act / d8_to_fourier /
d8_to_regular: widths with C/8 a multiple of 4 (vector path) and not (one
channel per thread), both dtypes, ragged token counts, in place and apart;
then the D8 layer with its neighbours, and the D8 layer between
regular-representation features, at the benchmark size on sampled tokens.
Same bars as the forward (tests/gpu_util.py).  Inputs from synthetic.py
(seeded); expected values only from oracle/.
"""
import numpy as np
import pytest

import oracle
import synthetic
from gpu_util import Guarded, assert_close, to_dev, to_f64

pytestmark = pytest.mark.gpu

F32, BF16, F16 = synthetic.F32, synthetic.BF16, synthetic.F16
# C/8 = 1, 3, 4, 12, 160 (LDS-tiled path); 2056 and 2049: rows wider than the
# tiled path stages (more than 2048 16-byte pieces in bf16), one pass per thread
# with four channels (C/8 a multiple of 4) or one
WIDTHS = [8, 24, 32, 96, 1280, 16392, 16448]


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


def _features(T, C, dt, seed):
    """Seeded N(0, 1) features of width C (either layout) and a per-channel bias."""
    d = synthetic.d8_inputs(C, 8, T, dt, seed)
    bd, b64 = synthetic.channel_bias(C // 8, dt, seed + 500)
    return d["x"], d["x64"], bd, b64


@pytest.mark.parametrize("dt", [F32, BF16, F16])
@pytest.mark.parametrize("C", WIDTHS)
def test_round_trip_matches_oracle(eq, C, dt):
    import torch
    plan = eq.eqlinear_d8_plan(8, C, _eqdt(eq, dt))
    for T in (1, 37, 300):
        yd, y64, bd, b64 = _features(T, C, dt, seed=C + T)
        b = to_dev(bd, dt)
        for bias, act in ((True, 1), (False, 1), (True, 0), (False, 0)):
            out = Guarded(T * C, dt, (T, C))
            eq.eqlinear_d8_bias_act(plan, to_dev(yd, dt).reshape(T, C), b if bias else None, act, out.t, T=T)
            torch.cuda.synchronize()
            out.check_guards()
            ref = oracle.d8_bias_act(y64, b64 if bias else None, act)
            assert_close(to_f64(out.t), ref, dt, f"C={C} {dt} T={T} bias={bias} act={act}")


@pytest.mark.parametrize("dt", [F32, BF16, F16])
def test_round_trip_in_place(eq, dt):
    import torch
    C, T = 96, 50
    plan = eq.eqlinear_d8_plan(8, C, _eqdt(eq, dt))
    yd, y64, bd, b64 = _features(T, C, dt, seed=4)
    y = to_dev(yd, dt).reshape(T, C).contiguous()
    eq.eqlinear_d8_bias_act(plan, y, to_dev(bd, dt), eq.EQL_ACT_GELU, y, T=T)
    torch.cuda.synchronize()
    assert_close(to_f64(y), oracle.d8_bias_act(y64, b64, 1), dt, "in place")


@pytest.mark.parametrize("dt", [F32, BF16, F16])
@pytest.mark.parametrize("C", WIDTHS)
def test_transforms_match_oracle(eq, C, dt):
    import torch
    plan = eq.eqlinear_d8_plan(C, C, _eqdt(eq, dt))
    T = 45
    xd, x64, _, _ = _features(T, C, dt, seed=C)
    four = Guarded(T * C, dt, (T, C))
    eq.eqlinear_d8_to_fourier(plan, to_dev(xd, dt).reshape(T, C), four.t, T=T)
    reg = Guarded(T * C, dt, (T, C))
    eq.eqlinear_d8_to_regular(plan, to_dev(xd, dt).reshape(T, C), reg.t, T=T)
    torch.cuda.synchronize()
    four.check_guards()
    reg.check_guards()
    assert_close(to_f64(four.t), oracle.d8_to_fourier(x64.reshape(T, C // 8, 8)), dt, f"to_fourier C={C}")
    assert_close(to_f64(reg.t), oracle.d8_to_regular(x64).reshape(T, C), dt, f"to_regular C={C}")


def test_d8_layer_with_gelu_at_full_size(eq):
    """The c5 layer (D8, width 1280, 4112 tokens, bf16) followed by the fused
    round trip with a bias and GELU: two launches, every token row."""
    import torch
    wl = synthetic.WORKLOADS["c5"]
    d = synthetic.d8_inputs(wl.C_in, wl.C_out, wl.T, wl.dtype, seed=0)
    bd, b64 = synthetic.channel_bias(wl.C_out // 8, wl.dtype, 500)
    plan = eq.eqlinear_d8_plan(wl.C_in, wl.C_out, eq.EQL_BF16)
    y = torch.empty(wl.T, wl.C_out, dtype=torch.bfloat16, device="cuda")
    eq.eqlinear_d8_forward(plan, to_dev(d["x"], wl.dtype).reshape(wl.T, -1), to_dev(d["w"], wl.dtype), y, T=wl.T)
    eq.eqlinear_d8_bias_act(plan, y, to_dev(bd, wl.dtype), eq.EQL_ACT_GELU, y, T=wl.T)
    torch.cuda.synchronize()
    ref = oracle.d8_dense_bias_act(d["x64"], d["w64"], wl.C_out, b64, 1)
    r, m = assert_close(to_f64(y), ref, wl.dtype, "c5 + bias + GELU")
    print(f"c5 bias+GELU: rel-L2 {r:.3e} max/rms {m:.3e} over all {wl.T} tokens")


@pytest.mark.parametrize("dt", [F32, BF16, F16])
def test_d8_layer_on_regular_features(eq, dt):
    """A D8 layer between regular-representation features: to the Fourier
    layout, the block layer, back to the regular layout."""
    import torch
    C_in, C_out, T = 64, 96, 200
    d = synthetic.d8_inputs(C_in, C_out, T, dt, seed=8)
    plan = eq.eqlinear_d8_plan(C_in, C_out, _eqdt(eq, dt))
    tdt = {F32: torch.float32, BF16: torch.bfloat16, F16: torch.float16}[dt]
    xf = torch.empty(T, C_in, dtype=tdt, device="cuda")
    yf = torch.empty(T, C_out, dtype=tdt, device="cuda")
    yr = Guarded(T * C_out, dt, (T, C_out))
    eq.eqlinear_d8_to_fourier(plan, to_dev(d["x"], dt).reshape(T, C_in), xf, T=T)
    eq.eqlinear_d8_forward(plan, xf, to_dev(d["w"], dt), yf, T=T)
    eq.eqlinear_d8_to_regular(plan, yf, yr.t, T=T)
    torch.cuda.synchronize()
    yr.check_guards()
    x_reg = d["x64"].reshape(T, C_in // 8, 8)
    ref = oracle.d8_to_regular(oracle.d8_dense(oracle.d8_to_fourier(x_reg), d["w64"], C_out)).reshape(T, C_out)
    assert_close(to_f64(yr.t), ref, dt, f"regular-feature D8 layer {dt}")
