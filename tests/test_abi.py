"""C ABI checks that need no GPU: the library loads, exports every function the
header declares, validates arguments before any HIP call, and reports the
plan counts the pages state.  Nothing here launches a kernel."""
import ctypes
import os
import re

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "eqlinear.h")


@pytest.fixture(scope="module")
def eq():
    import group_equivariant_linear_amd as eq
    from group_equivariant_linear_amd import _build
    if not eq.built():
        _build.build()
    eq.load_library()
    return eq


def header_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(eqlinear_\w+)\s*\(", src)))


def test_header_declares_the_binding_set(eq):
    assert header_functions() == sorted(eq.ABI_FUNCTIONS)


def test_library_exports_every_declared_symbol(eq):
    lib = ctypes.CDLL(eq.LIB_PATH)
    for name in header_functions():
        assert hasattr(lib, name), name


def test_header_compiles_as_c(tmp_path):
    src = tmp_path / "t.c"
    src.write_text('#include "eqlinear.h"\nint main(void){eqlinear_info i; (void)i; return 0;}\n')
    import subprocess
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"),
                    str(src), "-o", str(tmp_path / "t")], check=True)


def test_status_strings(eq):
    for s in range(5):
        assert eq.eqlinear_status_string(s).startswith("EQL_")
    assert "UNKNOWN" in eq.eqlinear_status_string(99)


@pytest.mark.parametrize("args", [(0, 4, 4, 0), (17, 4, 4, 0), (4, 0, 4, 0), (4, 4, 0, 0),
                                  (4, 4, 4, 3), (4, 4, 4, -1), (2, 1 << 20, 2, 0)])
def test_plan_rejects_invalid(eq, args):
    with pytest.raises(eq.EqlError) as e:
        eq.eqlinear_plan(*args)
    assert e.value.status == eq.EQL_ERR_INVALID


@pytest.mark.parametrize("args", [(12, 16, 0), (16, 12, 0), (0, 8, 0), (8, 8, 7)])
def test_d8_plan_rejects_invalid(eq, args):
    with pytest.raises(eq.EqlError):
        eq.eqlinear_d8_plan(*args)


def test_dihedral_plans(eq):
    """D_n plans: n = 4 is the D8 plan; widths must be multiples of 2n; counts."""
    lib = eq.load_library()
    d8 = eq.eqlinear_d8_plan(32, 64, eq.EQL_BF16).info
    d4 = eq.eqlinear_dihedral_plan(4, 32, 64, eq.EQL_BF16).info
    assert d8 == d4 and d8["N"] == 8 and d8["bins"] == 5
    for n in (2, 3, 5, 6, 12):
        C = 2 * n * 4
        info = eq.eqlinear_dihedral_plan(n, C, 2 * C, eq.EQL_F32).info
        n1 = 4 if n % 2 == 0 else 2
        n2 = n // 2 - 1 if n % 2 == 0 else (n - 1) // 2
        mi, mo = 4, 8
        assert info["N"] == 2 * n and info["bins"] == n1 + n2
        assert info["params"] == n1 * mi * mo + n2 * 4 * mi * mo == C * 2 * C // (2 * n)
        assert info["dense_macs_per_token"] == C * 2 * C
    h = ctypes.c_void_p()
    for bad in ((1, 8, 8), (13, 26, 26), (3, 8, 12), (3, 12, 8), (6, 12, 18)):
        assert lib.eqlinear_dihedral_plan(ctypes.byref(h), *bad, eq.EQL_F32) == eq.EQL_ERR_INVALID
    assert lib.eqlinear_dihedral_plan(ctypes.byref(h), 3, 12, 12, eq.EQL_F16) == eq.EQL_OK
    lib.eqlinear_plan_destroy(h)
    assert lib.eqlinear_dihedral_plan(None, 3, 12, 12, eq.EQL_F32) == eq.EQL_ERR_INVALID


def test_fp16_plans(eq):
    """fp16 plans exist for every group: C_N (weight spectrum, forward, both
    gradients, comparator) and D8 (layer, passes, comparator)."""
    lib = eq.load_library()
    p = eq.eqlinear_plan(8, 16, 24, eq.EQL_F16)
    assert p.info["dtype"] == eq.EQL_F16 and p.info["w_hat_elems"] == 8 * 16 * 24
    assert eq.eqlinear_d8_plan(16, 16, eq.EQL_F16).info["dtype"] == eq.EQL_F16
    A, B, W, S = 1 << 20, 1 << 30, 1 << 34, 1 << 38
    # the weight gradient's workspace holds fp16 planes: the same size as a bf16 plan's
    pb = eq.eqlinear_plan(8, 16, 24, eq.EQL_BF16)
    need = lib.eqlinear_backward_weight_workspace(p.handle, 100)
    assert need > 0 and need == lib.eqlinear_backward_weight_workspace(pb.handle, 100)
    # the forward's checks size fp16 tensors at 2 bytes: y one element into x's last row overlaps
    x_bytes = 5 * 16 * 8 * 2
    assert lib.eqlinear_forward(p.handle, A, W, A + x_bytes - 16, 5, None) == eq.EQL_ERR_INVALID


def test_null_out_and_null_plan(eq):
    lib = eq.load_library()
    assert lib.eqlinear_plan(None, 4, 4, 4, 0) == eq.EQL_ERR_INVALID
    assert lib.eqlinear_plan_destroy(None) == eq.EQL_ERR_INVALID
    assert lib.eqlinear_plan_info(None, None) == eq.EQL_ERR_INVALID
    assert lib.eqlinear_w_hat_elems(None) == 0
    assert lib.eqlinear_forward(None, 16, 16, 16, 1, None) == eq.EQL_ERR_INVALID


@pytest.mark.parametrize("N", range(1, 17))
def test_plan_info_counts(eq, N):
    C_in, C_out = 3, 5
    p = eq.eqlinear_plan(N, C_in, C_out, eq.EQL_F32)
    inf = p.info
    assert inf["bins"] == N // 2 + 1 == oracle.cn_kept_bins(N)
    assert inf["planes"] == N
    assert inf["has_nyquist"] == (1 if N % 2 == 0 and N > 1 else 0)
    assert inf["params"] == inf["w_hat_elems"] == oracle.cn_params(N, C_in, C_out)
    assert inf["real_gemms"] == oracle.cn_real_gemms(N) == (2 * N - 2 if N % 2 == 0 else 2 * N - 1)
    assert inf["macs_per_token"] == inf["real_gemms"] * C_in * C_out
    assert inf["dense_macs_per_token"] == N * N * C_in * C_out
    assert eq.eqlinear_w_hat_elems(p) == N * C_in * C_out


def test_page_counts_through_the_abi(eq):
    # six real products instead of sixteen for the p4 group
    p = eq.eqlinear_plan(4, 8, 8, eq.EQL_F32).info
    assert p["real_gemms"] == 6 and p["dense_macs_per_token"] // (8 * 8) == 16
    # the D8 layer: eight times fewer parameters, 5.33 times fewer multiplies
    d = eq.eqlinear_d8_plan(1280, 1280, eq.EQL_BF16).info
    assert d["dense_macs_per_token"] / d["params"] == 8
    assert abs(d["dense_macs_per_token"] / d["macs_per_token"] - 16 / 3) < 1e-12
    assert d["params"] == oracle.d8_params(1280, 1280)


@pytest.mark.skipif(os.path.exists("/dev/kfd"),
                    reason="uses fake device addresses; kept off machines with a GPU")
def test_forward_validation_before_any_hip_call(eq):
    lib = eq.load_library()
    p = eq.eqlinear_plan(8, 32, 32, eq.EQL_F32)
    h = p.handle
    A, B, W = 1 << 20, 1 << 30, 1 << 34  # aligned, disjoint fake addresses (never dereferenced)
    assert lib.eqlinear_forward(h, A, W, B, -1, None) == eq.EQL_ERR_INVALID  # T < 0
    assert lib.eqlinear_forward(h, None, None, None, 0, None) == eq.EQL_OK    # T == 0: no-op
    assert lib.eqlinear_forward(h, None, W, B, 5, None) == eq.EQL_ERR_INVALID
    assert lib.eqlinear_forward(h, A, None, B, 5, None) == eq.EQL_ERR_INVALID
    assert lib.eqlinear_forward(h, A, W, None, 5, None) == eq.EQL_ERR_INVALID
    assert lib.eqlinear_forward(h, A + 4, W, B, 5, None) == eq.EQL_ERR_INVALID  # misaligned
    assert lib.eqlinear_forward(h, A, W, B + 8, 5, None) == eq.EQL_ERR_INVALID
    assert lib.eqlinear_forward(h, A, W, A, 5, None) == eq.EQL_ERR_INVALID      # y aliases x
    assert lib.eqlinear_forward(h, A, W, A + 256, 5, None) == eq.EQL_ERR_INVALID  # overlap
    assert lib.eqlinear_forward(h, A, W, W, 5, None) == eq.EQL_ERR_INVALID      # y aliases w_hat
    assert lib.eqlinear_forward_tiled(h, A, W, B, 5, None, 18) == eq.EQL_ERR_INVALID
    assert lib.eqlinear_forward_tiled(h, A, W, B, 5, None, -2) == eq.EQL_ERR_INVALID
    d8 = eq.eqlinear_d8_plan(16, 16, eq.EQL_F32)
    assert lib.eqlinear_forward(d8.handle, A, W, B, 5, None) == eq.EQL_ERR_INVALID  # wrong kind
    assert lib.eqlinear_d8_forward(h, A, W, B, 5, None) == eq.EQL_ERR_INVALID       # wrong kind
    assert lib.eqlinear_weight_fft(d8.handle, A, W) == eq.EQL_ERR_INVALID
    assert lib.eqlinear_weight_fft(h, A, A) == eq.EQL_ERR_INVALID
    assert lib.eqlinear_weight_fft(h, A + 2, W) == eq.EQL_ERR_INVALID
    assert lib.eqlinear_d8_forward(d8.handle, A, W, A, 5, None) == eq.EQL_ERR_INVALID
    assert lib.eqlinear_d8_forward(d8.handle, A, W, B, -3, None) == eq.EQL_ERR_INVALID
    assert lib.eqlinear_d8_forward(d8.handle, None, None, None, 0, None) == eq.EQL_OK
    assert lib.eqlinear_expand_dense(h, A, A, None) == eq.EQL_ERR_INVALID
    assert lib.eqlinear_expand_dense(h, None, B, None) == eq.EQL_ERR_INVALID
    assert lib.eqlinear_dense_forward(h, A, W, A, 5, None) == eq.EQL_ERR_INVALID
    assert lib.eqlinear_dense_forward(h, A, W, B, -1, None) == eq.EQL_ERR_INVALID
    assert lib.eqlinear_dense_forward(h, None, None, None, 0, None) == eq.EQL_OK


@pytest.mark.skipif(os.path.exists("/dev/kfd"),
                    reason="uses fake device addresses; kept off machines with a GPU")
def test_backward_validation_before_any_hip_call(eq):
    lib = eq.load_library()
    p = eq.eqlinear_plan(8, 32, 16, eq.EQL_BF16)
    h = p.handle
    A, B, W, S = 1 << 20, 1 << 30, 1 << 34, 1 << 38  # aligned, disjoint fake addresses
    d8 = eq.eqlinear_d8_plan(16, 16, eq.EQL_F32)
    # adjoint spectrum
    assert lib.eqlinear_w_hat_adjoint(d8.handle, A, W, None) == eq.EQL_ERR_INVALID
    assert lib.eqlinear_w_hat_adjoint(h, None, W, None) == eq.EQL_ERR_INVALID
    assert lib.eqlinear_w_hat_adjoint(h, A, A + 16, None) == eq.EQL_ERR_INVALID   # overlap
    assert lib.eqlinear_w_hat_adjoint(h, A + 2, W, None) == eq.EQL_ERR_INVALID    # misaligned
    # input gradient
    assert lib.eqlinear_backward_data(h, A, W, B, -1, None) == eq.EQL_ERR_INVALID
    assert lib.eqlinear_backward_data(h, None, None, None, 0, None) == eq.EQL_OK
    assert lib.eqlinear_backward_data(h, A, W, A, 5, None) == eq.EQL_ERR_INVALID  # dx aliases dy
    assert lib.eqlinear_backward_data(h, A, W, W, 5, None) == eq.EQL_ERR_INVALID  # dx aliases w_hat_adj
    assert lib.eqlinear_backward_data(d8.handle, A, W, B, 5, None) == eq.EQL_ERR_INVALID
    # weight gradient
    need = lib.eqlinear_backward_weight_workspace(h, 100)
    assert need > 0 and need % 256 == 0
    assert lib.eqlinear_backward_weight_workspace(h, 0) == 0
    assert lib.eqlinear_backward_weight_workspace(h, -5) == 0
    assert lib.eqlinear_backward_weight_workspace(d8.handle, 100) == 0
    assert lib.eqlinear_backward_weight(h, A, B, W, -1, S, need, None) == eq.EQL_ERR_INVALID
    assert lib.eqlinear_backward_weight(h, A, B, W, 100, S, need - 1, None) == eq.EQL_ERR_INVALID  # short
    assert lib.eqlinear_backward_weight(h, A, B, W, 100, S + 16, need, None) == eq.EQL_ERR_INVALID  # 256-aligned
    assert lib.eqlinear_backward_weight(h, A, B, W, 100, None, need, None) == eq.EQL_ERR_INVALID
    assert lib.eqlinear_backward_weight(h, A, B, A, 100, S, need, None) == eq.EQL_ERR_INVALID  # dw aliases x
    assert lib.eqlinear_backward_weight(h, A, B, W, 100, A, need, None) == eq.EQL_ERR_INVALID  # ws over x
    assert lib.eqlinear_backward_weight(h, A, B, None, 100, S, need, None) == eq.EQL_ERR_INVALID
    assert lib.eqlinear_backward_weight(d8.handle, A, B, W, 100, S, need, None) == eq.EQL_ERR_INVALID
    # the workspace grows with T
    assert lib.eqlinear_backward_weight_workspace(h, 10000) > need
    # the weight gradient without allocation: the same checks, no workspace argument
    assert lib.eqlinear_backward_weight_noalloc(h, A, B, W, -1, None) == eq.EQL_ERR_INVALID
    assert lib.eqlinear_backward_weight_noalloc(h, A, B, A, 100, None) == eq.EQL_ERR_INVALID  # dw aliases x
    assert lib.eqlinear_backward_weight_noalloc(h, A, B, None, 100, None) == eq.EQL_ERR_INVALID
    assert lib.eqlinear_backward_weight_noalloc(h, A + 2, B, W, 100, None) == eq.EQL_ERR_INVALID
    assert lib.eqlinear_backward_weight_noalloc(d8.handle, A, B, W, 100, None) == eq.EQL_ERR_INVALID
    # a workspace past the library-held scratch: refused before any HIP call
    # (an fp32 plan: its transformed x and dy still go through the workspace)
    wide = eq.eqlinear_plan(8, 96, 96, eq.EQL_F32)
    assert lib.eqlinear_backward_weight_workspace(wide.handle, 12608) > eq.EQL_NOALLOC_SCRATCH_BYTES
    assert lib.eqlinear_backward_weight_noalloc(wide.handle, A, B, W, 12608, None) == eq.EQL_ERR_UNSUPPORTED
    # transformed x or dy reaching 2 GiB: unsupported, refused before any HIP call
    big = eq.eqlinear_plan(7, 160, 160, eq.EQL_BF16)
    X, Y, D, WS = 1 << 40, 1 << 42, 1 << 44, 1 << 46  # farther apart than the big tensors
    T = 1_000_000  # 7 * 160 * T * 2 bytes > 2 GiB
    nb = lib.eqlinear_backward_weight_workspace(big.handle, T)
    assert nb > 2 * (1 << 31)
    assert lib.eqlinear_backward_weight(big.handle, X, Y, D, T, WS, nb, None) == eq.EQL_ERR_UNSUPPORTED


def test_bias_act_validation_before_any_hip_call(eq):
    lib = eq.load_library()
    p = eq.eqlinear_plan(8, 32, 16, eq.EQL_BF16)  # bias: 16 bf16 = 32 bytes
    h = p.handle
    X, W, Y, Bz = 1 << 20, 1 << 30, 1 << 34, 1 << 38  # aligned, disjoint fake addresses
    f = lib.eqlinear_forward_bias_act
    G, NONE = eq.EQL_ACT_GELU, eq.EQL_ACT_NONE
    assert f(h, X, W, Bz, 2, Y, 5, None, -1) == eq.EQL_ERR_INVALID       # unknown activation
    assert f(h, X, W, Bz, -1, Y, 5, None, -1) == eq.EQL_ERR_INVALID
    assert f(h, X, W, Bz, G, Y, -1, None, -1) == eq.EQL_ERR_INVALID      # negative T
    assert f(h, None, None, None, G, None, 0, None, -1) == eq.EQL_OK     # T == 0: nothing to do
    assert f(h, X, W, Bz + 1, G, Y, 5, None, -1) == eq.EQL_ERR_INVALID   # bias misaligned for bf16
    assert f(h, X, W, Y + 30, G, Y, 5, None, -1) == eq.EQL_ERR_INVALID   # bias inside y
    assert f(h, X, W, Y - 30, G, Y, 5, None, -1) == eq.EQL_ERR_INVALID   # bias runs into y
    assert f(h, X, W, Bz, G, X, 5, None, -1) == eq.EQL_ERR_INVALID       # y aliases x
    assert f(h, X, W, Bz, G, W, 5, None, -1) == eq.EQL_ERR_INVALID       # y aliases w_hat
    assert f(h, X + 2, W, Bz, G, Y, 5, None, -1) == eq.EQL_ERR_INVALID   # x misaligned
    assert f(h, X, W, Bz, NONE, Y, 5, None, 18) == eq.EQL_ERR_INVALID    # tile out of range
    assert f(h, X, W, Bz, NONE, Y, 5, None, -2) == eq.EQL_ERR_INVALID
    assert f(h, None, W, Bz, G, Y, 5, None, -1) == eq.EQL_ERR_INVALID
    d8 = eq.eqlinear_d8_plan(16, 16, eq.EQL_F32)
    assert f(d8.handle, X, W, Bz, G, Y, 5, None, -1) == eq.EQL_ERR_INVALID
    pf = eq.eqlinear_plan(8, 32, 16, eq.EQL_F32)
    assert f(pf.handle, X, W, Bz + 2, G, Y, 5, None, -1) == eq.EQL_ERR_INVALID  # fp32 bias needs 4 bytes


def test_regular_forward_validation_before_any_hip_call(eq):
    lib = eq.load_library()
    f = lib.eqlinear_d8_regular_forward
    d8 = eq.eqlinear_d8_plan(64, 128, eq.EQL_BF16)  # 8 -> 16 regular channels
    h = d8.handle
    X, W, Bz, Y = 1 << 20, 1 << 30, 1 << 34, 1 << 38
    G, NONE = eq.EQL_ACT_GELU, eq.EQL_ACT_NONE
    assert f(h, X, W, Bz, 2, Y, 5, None) == eq.EQL_ERR_INVALID           # unknown activation
    assert f(h, X, W, Bz, G, Y, -1, None) == eq.EQL_ERR_INVALID          # negative T
    assert f(h, None, None, None, G, None, 0, None) == eq.EQL_OK         # T == 0
    assert f(h, X, W, Bz, G, X + 64, 5, None) == eq.EQL_ERR_INVALID      # y over x
    assert f(h, X, W, Bz, G, W, 5, None) == eq.EQL_ERR_INVALID           # y over the blocks
    assert f(h, X, W, Y + 2, G, Y, 5, None) == eq.EQL_ERR_INVALID        # bias inside y
    assert f(h, X + 2, W, Bz, G, Y, 5, None) == eq.EQL_ERR_INVALID       # misaligned
    assert f(h, X, W, Bz + 1, G, Y, 5, None) == eq.EQL_ERR_INVALID       # bias misaligned for bf16
    assert f(h, None, W, Bz, NONE, Y, 5, None) == eq.EQL_ERR_INVALID
    cn = eq.eqlinear_plan(8, 8, 16, eq.EQL_BF16)
    assert f(cn.handle, X, W, Bz, G, Y, 5, None) == eq.EQL_ERR_INVALID   # C_N plan
    # not on this path: fp32 plans, regular channel counts that are not multiples of 8
    f32 = eq.eqlinear_d8_plan(64, 128, eq.EQL_F32)
    assert f(f32.handle, X, W, Bz, G, Y, 5, None) == eq.EQL_ERR_UNSUPPORTED
    odd = eq.eqlinear_dihedral_plan(6, 12 * 12, 12 * 8, eq.EQL_F16)  # 12 -> 8 regular channels
    assert f(odd.handle, X, W, Bz, G, Y, 5, None) == eq.EQL_ERR_UNSUPPORTED


def test_d8_passes_validation_before_any_hip_call(eq):
    lib = eq.load_library()
    d8 = eq.eqlinear_d8_plan(32, 64, eq.EQL_BF16)  # y rows: 64 bf16 = 128 bytes; bias: 8 bf16
    h = d8.handle
    A, B, Bz = 1 << 20, 1 << 30, 1 << 38
    G, NONE = eq.EQL_ACT_GELU, eq.EQL_ACT_NONE
    f = lib.eqlinear_d8_bias_act
    assert f(h, A, Bz, 2, B, 5, None) == eq.EQL_ERR_INVALID          # unknown activation
    assert f(h, A, Bz, G, B, -1, None) == eq.EQL_ERR_INVALID         # negative T
    assert f(h, None, None, G, None, 0, None) == eq.EQL_OK           # T == 0
    assert f(h, A, Bz, G, A + 128, 5, None) == eq.EQL_ERR_INVALID    # partial overlap of in and out
    assert f(h, A + 2, Bz, G, B, 5, None) == eq.EQL_ERR_INVALID      # misaligned
    assert f(h, A, Bz + 1, G, B, 5, None) == eq.EQL_ERR_INVALID      # bias misaligned for bf16
    assert f(h, A, B + 8, G, B, 5, None) == eq.EQL_ERR_INVALID       # bias inside y_out
    assert f(h, None, Bz, NONE, B, 5, None) == eq.EQL_ERR_INVALID
    cn = eq.eqlinear_plan(8, 4, 8, eq.EQL_BF16)
    assert f(cn.handle, A, Bz, G, B, 5, None) == eq.EQL_ERR_INVALID  # C_N plan
    for g in (lib.eqlinear_d8_to_fourier, lib.eqlinear_d8_to_regular):
        assert g(h, A, B, -1, None) == eq.EQL_ERR_INVALID
        assert g(h, None, None, 0, None) == eq.EQL_OK
        assert g(h, A, A, 5, None) == eq.EQL_ERR_INVALID             # no in-place transform
        assert g(h, A, A + 64, 5, None) == eq.EQL_ERR_INVALID
        assert g(h, A + 8, B, 5, None) == eq.EQL_ERR_INVALID
        assert g(cn.handle, A, B, 5, None) == eq.EQL_ERR_INVALID


def test_binding_checks_tensors_without_gpu(eq):
    import torch
    p = eq.eqlinear_plan(4, 2, 2, eq.EQL_F32)
    x = torch.zeros(3, 2, 4)  # host tensor: rejected before the C call
    with pytest.raises(ValueError):
        eq.eqlinear_forward(p, x, x, x)


def test_plan_is_freed(eq):
    p = eq.eqlinear_plan(4, 2, 2, eq.EQL_F32)
    eq.eqlinear_plan_destroy(p)
    assert p.handle.value is None or p.handle.value == 0
    eq.eqlinear_plan_destroy(p)  # second destroy through the binding is a no-op
