"""GPU parity: the HIP library, called through its C ABI, against the fp64 oracle.

Bars (whole output): rel-L2 <= 1e-5 for fp32 plans, <= 2e-2 for bf16 plans with
fp32 accumulation; in addition the largest element error relative to the
output's RMS must stay under 2e-4 (fp32) / 1e-1 (bf16), so a mistake confined
to a tail tile cannot hide in the norm.  Output buffers carry sentinels on both
sides to catch stray writes.  Inputs come from synthetic.py (seeded); expected
values come only from oracle/.
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


def run_cn(eq, N, C_in, C_out, T, dt, seed=0, tile=-1, inputs=None):
    import torch
    d = inputs or synthetic.cn_inputs(N, C_in, C_out, T, dt, seed)
    plan = eq.eqlinear_plan(N, C_in, C_out, _eqdt(eq, dt))
    x, w = to_dev(d["x"], dt), to_dev(d["w"], dt)
    wh = Guarded(N * C_out * C_in, dt)
    eq.eqlinear_weight_fft(plan, w, wh.t)
    y = Guarded(T * C_out * N, dt, (T, C_out, N))
    if tile == -1:
        eq.eqlinear_forward(plan, x, wh.t, y.t, T=T)
    else:
        eq.eqlinear_forward_tiled(plan, x, wh.t, y.t, tile, T=T)
    torch.cuda.synchronize()
    wh.check_guards()
    y.check_guards()
    return to_f64(y.t), d


# --- weight spectrum ---------------------------------------------------------------

@pytest.mark.parametrize("dt", [F32, BF16, F16])
@pytest.mark.parametrize("N", range(1, 17))
def test_weight_fft_matches_oracle(eq, N, dt):
    import torch
    C_in, C_out = 7, 5
    d = synthetic.cn_inputs(N, C_in, C_out, 1, dt, seed=N)
    plan = eq.eqlinear_plan(N, C_in, C_out, _eqdt(eq, dt))
    wh = Guarded(N * C_out * C_in, dt)
    eq.eqlinear_weight_fft(plan, to_dev(d["w"], dt), wh.t)
    torch.cuda.synchronize()
    wh.check_guards()
    got = to_f64(wh.t).reshape(N, C_out, C_in)
    ref = oracle.cn_weight_dft(d["w64"])
    # computed in fp64 with exact special twiddles and rounded once: the GPU
    # value is a correctly rounded neighbour of the exact DFT, which the oracle
    # gives up to fp64 noise (libm's cos(pi/2) is 6e-17, not 0, so exact ties
    # of sums of fp32 values may fall either way in the oracle).
    bits = {F32: 24, BF16: 8, F16: 11}[dt]
    _, e = np.frexp(ref)
    half_ulp = np.ldexp(0.5, e - bits)
    if dt == F16:  # below 2^-14 fp16 is subnormal: spacing 2^-24
        half_ulp = np.maximum(half_ulp, 2.0 ** -25)
    noise = 1e-13 * np.abs(d["w64"]).max()
    assert np.all(np.abs(got - ref) <= half_ulp * (1 + 1e-9) + noise)
    assert rel_l2(got, ref) <= {F32: 1e-6, BF16: 4e-3, F16: 5e-4}[dt]


# --- fused forward: sweeps over group order, shapes, tails and tile configurations ----

SHAPES = [(1, 1, 1), (3, 5, 17), (33, 17, 65), (40, 72, 130)]


@pytest.mark.parametrize("dt", [F32, BF16, F16])
@pytest.mark.parametrize("N", range(1, 17))
def test_forward_sweep(eq, N, dt):
    for (C_in, C_out, T) in SHAPES:
        d = synthetic.cn_inputs(N, C_in, C_out, T, dt, seed=N * 100 + C_in)
        ref = oracle.cn_dense(d["x64"], d["w64"])
        for tile in range(-1, 18):
            y, _ = run_cn(eq, N, C_in, C_out, T, dt, tile=tile, inputs=d)
            assert_close(y, ref, dt, f"N={N} {dt} C_in={C_in} C_out={C_out} T={T} tile={tile}")


@pytest.mark.parametrize("dt", [F32, BF16, F16])
@pytest.mark.parametrize("N,C_in,C_out,T", [
    (8, 96, 96, 1000), (7, 160, 160, 777), (8, 96, 384, 300), (8, 384, 96, 300),
    (4, 8, 8, 64), (8, 32, 32, 4096), (5, 64, 64, 129), (16, 48, 80, 97), (12, 20, 36, 200),
    (6, 48, 40, 150), (3, 64, 24, 90), (2, 16, 48, 70),
    # whole 8-channel input groups with token rows of y that are not whole
    # 16-byte pieces (the transform kernel's element-wise store path)
    (2, 32, 21, 150), (4, 24, 3, 77), (6, 16, 7, 50), (7, 8, 4, 60),
])
def test_forward_multi_tile_shapes(eq, N, C_in, C_out, T, dt):
    d = synthetic.cn_inputs(N, C_in, C_out, T, dt, seed=7)
    ref = oracle.cn_dense(d["x64"], d["w64"])
    for tile in range(-1, 18):
        y, _ = run_cn(eq, N, C_in, C_out, T, dt, tile=tile, inputs=d)
        assert_close(y, ref, dt, f"N={N} {dt} {C_in}->{C_out} T={T} tile={tile}")


# --- the benchmark workloads at full size --------------------------------------------

@pytest.mark.parametrize("name", ["c1", "c2", "c3a", "c3b", "c3c", "c4"])
def test_workload_full_size(eq, name):
    """Every token row of the benchmark layer, in the launch configuration the
    benchmark times, against the oracle's replicated matrix (fp64)."""
    wl = synthetic.WORKLOADS[name]
    y, d = run_cn(eq, wl.N, wl.C_in, wl.C_out, wl.T, wl.dtype)
    W = oracle.cn_expand(d["w64"])
    ref = oracle.apply_dense(W, d["x64"].reshape(wl.T, -1)).reshape(wl.T, wl.C_out, wl.N)
    r, m = assert_close(y, ref, wl.dtype, name)
    print(f"{name}: rel-L2 {r:.3e} max/rms {m:.3e} over all {wl.T} tokens")
    # every 64-token tile on its own: a mistake in one tile cannot hide in the norm
    for t0 in range(0, wl.T, 64):
        assert_close(y[t0:t0 + 64], ref[t0:t0 + 64], wl.dtype, f"{name} tokens {t0}..")


# --- invariants on the GPU --------------------------------------------------------------

@pytest.mark.parametrize("name", ["c2", "c3b", "c4"])
def test_fp16_workload_full_size(eq, name):
    """The benchmark layers with fp16 I/O at full size, every token row."""
    from dataclasses import replace
    wl = replace(synthetic.WORKLOADS[name], dtype=F16)
    d = synthetic.cn_inputs(wl.N, wl.C_in, wl.C_out, wl.T, F16, seed=0)
    y, _ = run_cn(eq, wl.N, wl.C_in, wl.C_out, wl.T, F16, inputs=d)
    ref = oracle.cn_dense(d["x64"], d["w64"])
    r, m = assert_close(y, ref, F16, f"{name} fp16")
    print(f"{name} fp16: rel-L2 {r:.3e} max/rms {m:.3e} over all {wl.T} tokens")


@pytest.mark.parametrize("N", [3, 4, 7, 8, 12])
def test_fp16_large_inputs_keep_their_range(eq, N):
    """fp16 x of magnitude up to ~4e4 (x ~ N(0, 1) scaled by 2^13, exactly): y
    stays below 65504, but an unscaled spectrum bin (a sum of N values) would
    not.  Every tile must still match the oracle and produce finite values."""
    C_in, C_out, T = 64, 48, 300
    d = synthetic.cn_inputs(N, C_in, C_out, T, F16, seed=N + 40)
    xd, x64 = synthetic.quantize(d["x64"] * 8192.0, F16)
    assert np.array_equal(x64, d["x64"] * 8192.0)  # the scaling is exact
    assert np.abs(x64).max() * 3 > 65504  # a DC bin of 3+ such values would overflow
    dd = dict(d, x=xd, x64=x64)
    ref = oracle.cn_dense(x64, d["w64"])
    assert np.abs(ref).max() < 65504
    for tile in range(-1, 18):
        y, _ = run_cn(eq, N, C_in, C_out, T, F16, tile=tile, inputs=dd)
        assert_close(y, ref, F16, f"N={N} fp16 x*2^13 tile={tile}")


@pytest.mark.parametrize("dt", [F32, BF16, F16])
@pytest.mark.parametrize("N", [3, 4, 7, 8])
def test_equivariance_on_gpu(eq, N, dt):
    C_in, C_out, T = 24, 40, 70
    d = synthetic.cn_inputs(N, C_in, C_out, T, dt, seed=5)
    y, _ = run_cn(eq, N, C_in, C_out, T, dt, inputs=d)
    for s in range(1, N):
        ds = dict(d)
        ds["x"] = np.ascontiguousarray(np.roll(d["x"], s, axis=-1))
        ds["x64"] = np.roll(d["x64"], s, axis=-1)
        ys, _ = run_cn(eq, N, C_in, C_out, T, dt, inputs=ds)
        assert_close(ys, np.roll(y, s, axis=-1), dt, f"roll {s}")


def test_n1_is_a_plain_matrix_product(eq):
    d = synthetic.cn_inputs(1, 37, 29, 50, F32, seed=2)
    y, _ = run_cn(eq, 1, 37, 29, 50, F32, inputs=d)
    assert_close(y[..., 0], d["x64"][..., 0] @ d["w64"][..., 0].T, F32)


def test_zero_tokens_is_a_no_op(eq):
    import torch
    plan = eq.eqlinear_plan(8, 16, 16, eq.EQL_F32)
    y = Guarded(16 * 8, F32)
    x = torch.zeros(16 * 8, device="cuda")
    wh = torch.zeros(8 * 16 * 16, device="cuda")
    eq.eqlinear_forward(plan, x[:0], wh, y.t[:0], T=0)
    torch.cuda.synchronize()
    y.check_guards()


def test_forward_is_deterministic(eq):
    d = synthetic.cn_inputs(7, 160, 160, 999, BF16, seed=3)
    y1, _ = run_cn(eq, 7, 160, 160, 999, BF16, inputs=d)
    y2, _ = run_cn(eq, 7, 160, 160, 999, BF16, inputs=d)
    assert np.array_equal(y1, y2)


def test_forward_on_a_side_stream(eq):
    import torch
    d = synthetic.cn_inputs(8, 32, 32, 513, F32, seed=4)
    ref = oracle.cn_dense(d["x64"], d["w64"])
    plan = eq.eqlinear_plan(8, 32, 32, eq.EQL_F32)
    x, w = to_dev(d["x"], F32), to_dev(d["w"], F32)
    wh = torch.empty(8 * 32 * 32, device="cuda")
    eq.eqlinear_weight_fft(plan, w, wh)
    s = torch.cuda.Stream()
    y = torch.empty(513, 32, 8, device="cuda")
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        eq.eqlinear_forward(plan, x, wh, y)
    s.synchronize()
    assert_close(to_f64(y), ref, F32)


# --- D8 Fourier-domain layer -----------------------------------------------------------

def run_d8(eq, C_in, C_out, T, dt, seed=0, inputs=None):
    import torch
    d = inputs or synthetic.d8_inputs(C_in, C_out, T, dt, seed)
    plan = eq.eqlinear_d8_plan(C_in, C_out, _eqdt(eq, dt))
    x, wb = to_dev(d["x"], dt), to_dev(d["w"], dt)
    y = Guarded(T * C_out, dt, (T, C_out))
    eq.eqlinear_d8_forward(plan, x, wb, y.t, T=T)
    torch.cuda.synchronize()
    y.check_guards()
    return to_f64(y.t), d


@pytest.mark.parametrize("dt", [F32, BF16, F16])
@pytest.mark.parametrize("C_in,C_out,T", [(8, 8, 1), (16, 24, 33), (64, 64, 130), (160, 96, 257),
                                          (256, 512, 100), (1280, 1280, 77), (512, 320, 97),
                                          (192, 640, 200)])
def test_d8_forward(eq, C_in, C_out, T, dt):
    y, d = run_d8(eq, C_in, C_out, T, dt, seed=C_in)
    ref = oracle.d8_dense(d["x64"], d["w64"], C_out)
    assert_close(y, ref, dt, f"D8 {C_in}->{C_out} T={T} {dt}")


@pytest.mark.parametrize("dt", [BF16, F16])
def test_d8_workload_full_size(eq, dt):
    """The c5 D8 layer at full size (bf16 as benchmarked, and fp16), every token row."""
    wl = synthetic.WORKLOADS["c5"]
    y, d = run_d8(eq, wl.C_in, wl.C_out, wl.T, dt)
    W = oracle.d8_expand(d["w64"], wl.C_in, wl.C_out)
    ref = oracle.apply_dense(W, d["x64"])
    r, m = assert_close(y, ref, dt, f"c5 {dt}")
    print(f"c5 {dt}: rel-L2 {r:.3e} max/rms {m:.3e} over all {wl.T} tokens")
    for t0 in range(0, wl.T, 128):
        assert_close(y[t0:t0 + 128], ref[t0:t0 + 128], dt, f"c5 {dt} tokens {t0}..")


# --- expanded-dense comparator ------------------------------------------------------------

@pytest.mark.parametrize("dt", [F32, BF16, F16])
@pytest.mark.parametrize("N,C_in,C_out,T", [(4, 8, 8, 64), (7, 20, 12, 33), (8, 32, 48, 300)])
def test_dense_comparator(eq, N, C_in, C_out, T, dt):
    import torch
    d = synthetic.cn_inputs(N, C_in, C_out, T, dt, seed=9)
    plan = eq.eqlinear_plan(N, C_in, C_out, _eqdt(eq, dt))
    Wd = Guarded(N * C_out * N * C_in, dt, (N * C_out, N * C_in))
    eq.eqlinear_expand_dense(plan, to_dev(d["w"], dt), Wd.t)
    y = Guarded(T * C_out * N, dt, (T, C_out * N))
    eq.eqlinear_dense_forward(plan, to_dev(d["x"], dt), Wd.t, y.t, T=T)
    torch.cuda.synchronize()
    Wd.check_guards()
    y.check_guards()
    # the expansion is a copy: bit-exact against the oracle's replicated matrix
    assert np.array_equal(to_f64(Wd.t), oracle.cn_expand(d["w64"]))
    ref = oracle.cn_dense(d["x64"], d["w64"]).reshape(T, -1)
    assert_close(to_f64(y.t), ref, dt, "dense comparator")


@pytest.mark.parametrize("dt", [F32, BF16, F16])
def test_d8_dense_comparator(eq, dt):
    import torch
    C_in, C_out, T = 64, 48, 70
    d = synthetic.d8_inputs(C_in, C_out, T, dt, seed=11)
    plan = eq.eqlinear_d8_plan(C_in, C_out, _eqdt(eq, dt))
    Wd = Guarded(C_in * C_out, dt, (C_out, C_in))
    eq.eqlinear_expand_dense(plan, to_dev(d["w"], dt), Wd.t)
    y = Guarded(T * C_out, dt, (T, C_out))
    eq.eqlinear_dense_forward(plan, to_dev(d["x"], dt), Wd.t, y.t, T=T)
    torch.cuda.synchronize()
    Wd.check_guards()
    y.check_guards()
    assert np.array_equal(to_f64(Wd.t), oracle.d8_expand(d["w64"], C_in, C_out))
    assert_close(to_f64(y.t), oracle.d8_dense(d["x64"], d["w64"], C_out), dt, "D8 dense comparator")
