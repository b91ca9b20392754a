"""The weight gradient without allocation (eqlinear_backward_weight_noalloc),
called through the C ABI, against the entry point with a caller workspace
(eqlinear_backward_weight): same kernels and summation order, so the same bits.
Two calls in a row on each shape, the second with fewer tokens, so the second
runs on scratch memory that still holds the first call's contents."""
import numpy as np
import pytest

import oracle
import synthetic
from gpu_util import assert_close, to_dev, to_f64

pytestmark = pytest.mark.gpu

F32, BF16, F16 = synthetic.F32, synthetic.BF16, synthetic.F16


@pytest.fixture(scope="module")
def eq():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import group_equivariant_linear_amd as eq
    eq.load_library()
    return eq


def _eqdt(eq, dt):
    return {F32: eq.EQL_F32, BF16: eq.EQL_BF16, F16: eq.EQL_F16}[dt]


def _grads(eq, plan, N, C_in, C_out, T, dt, seed):
    import torch
    d = synthetic.cn_inputs(N, C_in, C_out, T, dt, seed)
    g = synthetic.cn_inputs(N, C_out, C_in, T, dt, seed + 1000)
    x, dy = to_dev(d["x"], dt), to_dev(g["x"], dt)
    n = N * C_in * C_out
    dw_ws = torch.full((n,), float("nan"), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(eq.eqlinear_backward_weight_workspace(plan, T), 1), dtype=torch.uint8, device="cuda")
    eq.eqlinear_backward_weight(plan, x, dy, dw_ws, ws, T=T)
    dw_na = torch.full((n,), float("nan"), dtype=torch.float32, device="cuda")
    eq.eqlinear_backward_weight_noalloc(plan, x, dy, dw_na, T=T)
    torch.cuda.synchronize()
    return to_f64(dw_ws).reshape(C_out, C_in, N), to_f64(dw_na).reshape(C_out, C_in, N), d["x64"], g["x64"]


@pytest.mark.parametrize("dt", [F32, BF16, F16])
@pytest.mark.parametrize("N,C_in,C_out,T1,T2", [
    (8, 32, 32, 4096, 1000),     # one-launch path for narrow layers
    (7, 24, 16, 777, 65),
    (8, 96, 96, 1200, 300),      # fp32: planes + per-bin products + reduction;
    (7, 160, 160, 640, 129),     # 16-bit: transforms inside the product kernel
    (6, 100, 24, 900, 17),       # fp32: 64 x 64 product tiles
])
def test_noalloc_matches_the_workspace_entry(eq, N, C_in, C_out, T1, T2, dt):
    plan = eq.eqlinear_plan(N, C_in, C_out, _eqdt(eq, dt))
    for k, T in enumerate((T1, T2)):
        assert eq.eqlinear_backward_weight_workspace(plan, T) <= eq.EQL_NOALLOC_SCRATCH_BYTES
        a, b, x64, dy64 = _grads(eq, plan, N, C_in, C_out, T, dt, seed=10 * k + N)
        assert np.array_equal(a, b), f"call {k + 1} (T={T}): differs from the workspace entry point"
        assert_close(b, oracle.cn_backward_weight(x64, dy64), dt, f"call {k + 1} (T={T}) vs oracle")


def test_noalloc_zero_tokens_writes_zeros(eq):
    import torch
    plan = eq.eqlinear_plan(8, 32, 32, eq.EQL_BF16)
    dw = torch.full((8 * 32 * 32,), 7.0, dtype=torch.float32, device="cuda")
    x = torch.zeros(16, dtype=torch.bfloat16, device="cuda")
    eq.eqlinear_backward_weight_noalloc(plan, x[:0], x[:0], dw, T=0)
    torch.cuda.synchronize()
    assert torch.count_nonzero(dw).item() == 0


def test_noalloc_refuses_shapes_past_its_scratch(eq):
    import torch
    plan = eq.eqlinear_plan(8, 96, 96, eq.EQL_F32)
    T = 12608  # fp32 planes of x and dy: about 80 MiB of workspace
    assert eq.eqlinear_backward_weight_workspace(plan, T) > eq.EQL_NOALLOC_SCRATCH_BYTES
    x = torch.zeros(T * 96 * 8, dtype=torch.float32, device="cuda")
    dw = torch.zeros(8 * 96 * 96, dtype=torch.float32, device="cuda")
    with pytest.raises(eq.EqlError):
        eq.eqlinear_backward_weight_noalloc(plan, x, x, dw, T=T)
