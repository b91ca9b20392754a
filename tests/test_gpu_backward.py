"""GPU parity of the backward pass (input and weight gradients) against the fp64 oracle.

Same bars as the forward (tests/gpu_util.py): rel-L2 <= 1e-5 (fp32 plans),
<= 2e-2 (bf16 plans) or <= 2.5e-3 (fp16 plans) over the whole output, and the
largest element error relative to the output's RMS under 2e-4 / 1e-1 /
1.25e-2.  The weight gradient is fp32 for every plan dtype.  Inputs come from
synthetic.py (seeded); expected values only from oracle/.
"""
import numpy as np
import pytest

import oracle
import synthetic
from gpu_util import Guarded, assert_close, rel_l2, to_dev, to_f64

pytestmark = pytest.mark.gpu

F32, BF16, F16 = synthetic.F32, synthetic.BF16, synthetic.F16


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


def _inputs(N, C_in, C_out, T, dt, seed):
    """x [T][C_in][N], w [C_out][C_in][N] and an upstream gradient dy [T][C_out][N]."""
    d = synthetic.cn_inputs(N, C_in, C_out, T, dt, seed)
    g = synthetic.cn_inputs(N, C_out, C_in, T, dt, seed + 1000)
    d["dy"], d["dy64"] = g["x"], g["x64"]
    return d


def _w_hat(eq, plan, d, N, C_in, C_out, dt):
    wh = Guarded(N * C_out * C_in, dt)
    eq.eqlinear_weight_fft(plan, to_dev(d["w"], dt), wh.t)
    return wh


def run_backward_data(eq, N, C_in, C_out, T, dt, d):
    import torch
    plan = eq.eqlinear_plan(N, C_in, C_out, _eqdt(eq, dt))
    wh = _w_hat(eq, plan, d, N, C_in, C_out, dt)
    adj = Guarded(N * C_out * C_in, dt)
    eq.eqlinear_w_hat_adjoint(plan, wh.t, adj.t)
    dx = Guarded(T * C_in * N, dt, (T, C_in, N))
    eq.eqlinear_backward_data(plan, to_dev(d["dy"], dt), adj.t, dx.t, T=T)
    torch.cuda.synchronize()
    adj.check_guards()
    dx.check_guards()
    return to_f64(dx.t), to_f64(adj.t).reshape(N, C_in, C_out)


def run_backward_weight(eq, N, C_in, C_out, T, dt, d):
    import torch
    plan = eq.eqlinear_plan(N, C_in, C_out, _eqdt(eq, dt))
    nb = eq.eqlinear_backward_weight_workspace(plan, T)
    ws = torch.empty(max(nb, 256), dtype=torch.uint8, device="cuda")
    dw = Guarded(N * C_out * C_in, F32, (C_out, C_in, N))
    eq.eqlinear_backward_weight(plan, to_dev(d["x"], dt), to_dev(d["dy"], dt), dw.t, ws, T=T)
    torch.cuda.synchronize()
    dw.check_guards()
    return to_f64(dw.t)


# --- adjoint spectrum -----------------------------------------------------------------

@pytest.mark.parametrize("dt", [F32, BF16, F16])
@pytest.mark.parametrize("N", [1, 2, 3, 4, 5, 7, 8, 11, 16])
def test_w_hat_adjoint_is_the_spectrum_of_the_adjoint_weight(eq, N, dt):
    C_in, C_out = 37, 21  # ragged 32x32 transpose tiles on both axes
    d = _inputs(N, C_in, C_out, 1, dt, seed=N)
    _, adj = run_backward_data(eq, N, C_in, C_out, 1, dt, d)
    # w'[i][o][m] = w[o][i][(-m) mod N]: the weight of the input gradient layer
    w_adj = np.roll(d["w64"][..., ::-1], 1, axis=-1).transpose(1, 0, 2)
    ref = oracle.cn_weight_dft(w_adj)
    bits = {F32: 24, BF16: 8, F16: 11}[dt]
    _, e = np.frexp(ref)
    half_ulp = np.ldexp(0.5, e - bits)
    if dt == F16:  # fp16 subnormals below 2^-14
        half_ulp = np.maximum(half_ulp, 2.0 ** -25)
    noise = 1e-13 * np.abs(d["w64"]).max()
    assert np.all(np.abs(adj - ref) <= half_ulp * (1 + 1e-9) + noise)


# --- input gradient ---------------------------------------------------------------------

SHAPES = [(5, 7, 37), (32, 48, 150), (8, 24, 64), (96, 40, 97), (3, 130, 29)]


@pytest.mark.parametrize("dt", [F32, BF16, F16])
@pytest.mark.parametrize("N", [1, 2, 3, 4, 5, 7, 8, 12, 16])
def test_backward_data_sweep(eq, N, dt):
    for C_in, C_out, T in SHAPES:
        d = _inputs(N, C_in, C_out, T, dt, seed=7 * N + C_in)
        dx, _ = run_backward_data(eq, N, C_in, C_out, T, dt, d)
        ref = oracle.cn_backward_data(d["dy64"], d["w64"])
        assert_close(dx, ref, dt, f"dx N={N} {dt} {C_in}->{C_out} T={T}")


# --- weight gradient --------------------------------------------------------------------

@pytest.mark.parametrize("dt", [F32, BF16, F16])
@pytest.mark.parametrize("N", [1, 2, 3, 4, 5, 7, 8, 12, 16])
def test_backward_weight_sweep(eq, N, dt):
    for C_in, C_out, T in SHAPES + [(16, 16, 1), (70, 66, 1000)]:
        d = _inputs(N, C_in, C_out, T, dt, seed=11 * N + C_out)
        dw = run_backward_weight(eq, N, C_in, C_out, T, dt, d)
        ref = oracle.cn_backward_weight(d["x64"], d["dy64"])
        # fp32 result for either plan dtype; bf16 inputs round their spectra
        assert_close(dw, ref, dt, f"dw N={N} {dt} {C_in}->{C_out} T={T}")


def test_backward_weight_zero_tokens_writes_zeros(eq):
    import torch
    N, C_in, C_out = 8, 16, 24
    plan = eq.eqlinear_plan(N, C_in, C_out, eq.EQL_F32)
    dw = Guarded(N * C_out * C_in, F32)
    dw.t.fill_(3.0)
    eq.eqlinear_backward_weight(plan, 0, 0, dw.t, torch.empty(256, dtype=torch.uint8, device="cuda"), T=0)
    torch.cuda.synchronize()
    dw.check_guards()
    assert torch.count_nonzero(dw.t).item() == 0


@pytest.mark.parametrize("dt", [F32, BF16, F16])
def test_backward_weight_is_deterministic(eq, dt):
    N, C_in, C_out, T = 7, 40, 72, 3000
    d = _inputs(N, C_in, C_out, T, dt, seed=5)
    a = run_backward_weight(eq, N, C_in, C_out, T, dt, d)
    b = run_backward_weight(eq, N, C_in, C_out, T, dt, d)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("dt", [F32, BF16, F16])
@pytest.mark.parametrize("N,C_in,C_out", [(5, 24, 32), (8, 32, 32), (16, 32, 9)])
def test_backward_weight_small_layers_many_chunks(eq, N, C_in, C_out, dt):
    """Layers with at most 32 channels each way take the one-launch path; at
    T = 20000 every workgroup runs several 16-token chunks (loads of the next
    chunk in flight during the products).  Also deterministic."""
    T = 20000
    d = _inputs(N, C_in, C_out, T, dt, seed=N + C_out)
    dw = run_backward_weight(eq, N, C_in, C_out, T, dt, d)
    ref = oracle.cn_backward_weight(d["x64"], d["dy64"])
    assert_close(dw, ref, dt, f"dw N={N} {dt} {C_in}->{C_out} T={T}")
    assert np.array_equal(dw, run_backward_weight(eq, N, C_in, C_out, T, dt, d))


@pytest.mark.parametrize("dt", [F32, BF16, F16])
@pytest.mark.parametrize("N", [1, 2, 3, 7, 8, 16])
def test_backward_weight_whole_tile_bins(eq, N, dt):
    """Wide layers whose (o, i) tile fits one workgroup of up to 16 waves take the
    per-bin product kernel (one bin, whole tile, range of tokens per workgroup):
    ragged tile edges on both axes (150 -> 140), exact ones (160 -> 160), and
    two tiles along o (96 -> 384) or i (384 -> 96), and a single token (one chunk,
    one range per bin).  Also deterministic."""
    for C_in, C_out, T in [(150, 140, 77), (160, 160, 300), (96, 384, 130), (384, 96, 64), (160, 160, 1)]:
        d = _inputs(N, C_in, C_out, T, dt, seed=3 * N + C_in)
        dw = run_backward_weight(eq, N, C_in, C_out, T, dt, d)
        ref = oracle.cn_backward_weight(d["x64"], d["dy64"])
        assert_close(dw, ref, dt, f"dw N={N} {dt} {C_in}->{C_out} T={T}")
        if C_in == 150:
            assert np.array_equal(dw, run_backward_weight(eq, N, C_in, C_out, T, dt, d))


@pytest.mark.parametrize("dt", [F32, BF16, F16])
@pytest.mark.parametrize("N", [1, 3, 8, 16])
def test_backward_weight_64_tiles(eq, N, dt):
    """At most 32 output channels with more than 32 input channels: no whole tile
    fits the per-bin kernel's load budget, so the 64 x 64 product kernel (all
    bins per workgroup) runs.  Ragged on both axes."""
    for C_in, C_out, T in [(50, 20, 300), (130, 24, 77), (200, 9, 64)]:
        d = _inputs(N, C_in, C_out, T, dt, seed=5 * N + C_in)
        dw = run_backward_weight(eq, N, C_in, C_out, T, dt, d)
        ref = oracle.cn_backward_weight(d["x64"], d["dy64"])
        assert_close(dw, ref, dt, f"dw N={N} {dt} {C_in}->{C_out} T={T}")


@pytest.mark.parametrize("dt", [BF16, F16])
@pytest.mark.parametrize("N,C_in,C_out,T", [
    (8, 37, 45, 101), (6, 65, 33, 1), (4, 65, 33, 77), (2, 33, 70, 95), (8, 64, 64, 32),
    (6, 100, 36, 63), (2, 40, 130, 99), (4, 129, 66, 250), (6, 160, 160, 2000), (8, 96, 200, 1500),
    (8, 1, 200, 33), (2, 3, 130, 29),
])
def test_backward_weight_transforms_in_the_product_kernel(eq, N, C_in, C_out, T, dt):
    """16-bit layers of even order up to 8 with more than 32 channels one way:
    x and dy are transformed inside the product kernel (64 x 64 tiles, 32-token
    chunks, records read by 16-byte windows).  Ragged tiles, token tails, one
    or three input channels (windows that run past the operand's end), a single
    token, and ranges of many chunks.  Also deterministic."""
    d = _inputs(N, C_in, C_out, T, dt, seed=13 * N + C_in + T)
    dw = run_backward_weight(eq, N, C_in, C_out, T, dt, d)
    ref = oracle.cn_backward_weight(d["x64"], d["dy64"])
    assert_close(dw, ref, dt, f"dw N={N} {dt} {C_in}->{C_out} T={T}")
    assert np.array_equal(dw, run_backward_weight(eq, N, C_in, C_out, T, dt, d))


@pytest.mark.parametrize("dt", [F32, BF16, F16])
def test_gradients_satisfy_the_adjoint_identity(eq, dt):
    """<dy, y(x)> = <dx, x> = <dw, w> with all three computed on the GPU."""
    import torch
    N, C_in, C_out, T = 8, 24, 40, 300
    d = _inputs(N, C_in, C_out, T, dt, seed=9)
    plan = eq.eqlinear_plan(N, C_in, C_out, _eqdt(eq, dt))
    wh = _w_hat(eq, plan, d, N, C_in, C_out, dt)
    y = Guarded(T * C_out * N, dt, (T, C_out, N))
    eq.eqlinear_forward(plan, to_dev(d["x"], dt), wh.t, y.t, T=T)
    dx, _ = run_backward_data(eq, N, C_in, C_out, T, dt, d)
    dw = run_backward_weight(eq, N, C_in, C_out, T, dt, d)
    torch.cuda.synchronize()
    lhs = np.sum(d["dy64"] * to_f64(y.t))
    tol = 1e-5 if dt == F32 else 2e-2
    scale = np.linalg.norm(d["dy64"]) * np.linalg.norm(to_f64(y.t))
    assert abs(np.sum(dx * d["x64"]) - lhs) <= tol * scale
    assert abs(np.sum(dw * d["w64"]) - lhs) <= tol * scale


@pytest.mark.parametrize("N,C_in,C_out,T", [(8, 96, 96, 700), (7, 40, 72, 333), (8, 24, 16, 500)])
def test_backward_weight_fp16_loss_scaled(eq, N, C_in, C_out, T):
    """A loss-scaled upstream gradient in fp16 (dy scaled by 2^13, exactly): the
    transformed dy held in fp16 would pass 65504 unscaled.  dw (fp32) must match
    the oracle on the plane paths and the narrow-layer path alike."""
    d = _inputs(N, C_in, C_out, T, F16, seed=N + C_in)
    dyd, dy64 = synthetic.quantize(d["dy64"] * 8192.0, F16)
    assert np.array_equal(dy64, d["dy64"] * 8192.0)
    dd = dict(d, dy=dyd, dy64=dy64)
    dw = run_backward_weight(eq, N, C_in, C_out, T, F16, dd)
    assert np.all(np.isfinite(dw))
    assert_close(dw, oracle.cn_backward_weight(d["x64"], dy64), F16, f"dw fp16 loss-scaled N={N}")


# --- the benchmark workloads at full size ------------------------------------------------

def _shift_route_dw(x64, dy64):
    """dw[o][i][m] = sum_{t,g} dy[t][o][g] x[t][i][(g - m) mod N], written as one
    fp64 matrix product of dy (o by (t, g)) with the cyclically shifted copies of
    x ((t, g) by (i, m)): an independent evaluation of every element."""
    T, C_in, N = x64.shape
    C_out = dy64.shape[1]
    g = np.arange(N)
    xs = np.stack([x64[:, :, (g - m) % N] for m in range(N)], axis=2)  # [t][i][m][g]
    A = dy64.transpose(1, 0, 2).reshape(C_out, T * N)
    B = xs.transpose(0, 3, 1, 2).reshape(T * N, C_in * N)
    return (A @ B).reshape(C_out, C_in, N)


@pytest.mark.parametrize("name", ["c2", "c3a", "c3b", "c3c", "c4"])
def test_backward_workload_full_size(eq, name):
    wl = synthetic.WORKLOADS[name]
    N, C_in, C_out, T, dt = wl.N, wl.C_in, wl.C_out, wl.T, wl.dtype
    d = _inputs(N, C_in, C_out, T, dt, seed=0)
    # input gradient: every token row against the oracle
    dx, _ = run_backward_data(eq, N, C_in, C_out, T, dt, d)
    ref = oracle.cn_backward_data(d["dy64"], d["w64"])
    r, m = assert_close(dx, ref, dt, f"{name} dx")
    print(f"{name} dx: rel-L2 {r:.3e} max/rms {m:.3e} over all {T} tokens")
    # weight gradient: whole output-channel rows against the oracle (the first
    # and last rows, so the last ragged output tile, and rows across the
    # middle), and every element against the shift-and-multiply route
    dw = run_backward_weight(eq, N, C_in, C_out, T, dt, d)
    assert np.all(np.isfinite(dw))
    rows = sorted({0, 1, 2, C_out // 3, C_out // 2, C_out - 3, C_out - 2, C_out - 1})
    ref = oracle.cn_backward_weight(d["x64"], np.ascontiguousarray(d["dy64"][:, rows]))
    r, m = assert_close(dw[rows], ref, dt, f"{name} dw rows {rows}")
    print(f"{name} dw: rel-L2 {r:.3e} max/rms {m:.3e} over output rows {rows} (all i, m)")
    full = _shift_route_dw(d["x64"], d["dy64"])
    # the route agrees with the oracle where both are computed (fp64 rounding only)
    assert rel_l2(full[rows], ref) < 1e-12
    r, m = assert_close(dw, full, dt, f"{name} dw (every element)")
    print(f"{name} dw: rel-L2 {r:.3e} max/rms {m:.3e} over all {C_out * C_in * N} elements")
