"""Python binding of libeqlinear.so, the MI355X (gfx950) equivariant linear layers.

A thin ctypes layer over the C ABI in include/eqlinear.h: every function has the
C name, turns tensors into device pointers and the current torch stream into a
hipStream_t, checks shapes and dtypes, and raises EqlError on a non-OK status.
All arithmetic runs in the library's HIP kernels; there is no fallback path.
If the library has not been built, loading fails loudly.

Tensor arguments may be torch tensors on a ROCm device, or plain integers
(raw device addresses, for callers that manage memory themselves).
"""
from __future__ import annotations

import ctypes
import os
import threading

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libeqlinear.so")

EQL_OK, EQL_ERR_INVALID, EQL_ERR_UNSUPPORTED, EQL_ERR_HIP, EQL_ERR_NOMEM = range(5)
EQL_F32, EQL_BF16, EQL_F16 = 0, 1, 2
EQL_KIND_CN, EQL_KIND_D8 = 0, 1
EQL_ACT_NONE, EQL_ACT_GELU = 0, 1

# Every entry point of include/eqlinear.h.
ABI_FUNCTIONS = (
    "eqlinear_status_string", "eqlinear_plan", "eqlinear_d8_plan", "eqlinear_plan_destroy",
    "eqlinear_plan_info", "eqlinear_w_hat_elems", "eqlinear_weight_fft", "eqlinear_forward",
    "eqlinear_forward_tiled", "eqlinear_d8_forward", "eqlinear_expand_dense",
    "eqlinear_dense_forward", "eqlinear_w_hat_adjoint", "eqlinear_backward_data",
    "eqlinear_backward_weight_workspace", "eqlinear_backward_weight", "eqlinear_forward_bias_act",
    "eqlinear_d8_bias_act", "eqlinear_d8_to_fourier", "eqlinear_d8_to_regular", "eqlinear_dihedral_plan",
    "eqlinear_backward_weight_noalloc", "eqlinear_d8_regular_forward",
)

# Size of the library-held scratch array of eqlinear_backward_weight_noalloc.
EQL_NOALLOC_SCRATCH_BYTES = 32 << 20


class EqlError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {eqlinear_status_string(status)}")


class eqlinear_info(ctypes.Structure):
    _fields_ = [
        ("kind", ctypes.c_int32), ("dtype", ctypes.c_int32), ("N", ctypes.c_int32),
        ("C_in", ctypes.c_int32), ("C_out", ctypes.c_int32), ("bins", ctypes.c_int32),
        ("planes", ctypes.c_int32), ("has_nyquist", ctypes.c_int32),
        ("params", ctypes.c_int64), ("w_hat_elems", ctypes.c_int64),
        ("real_gemms", ctypes.c_int64), ("macs_per_token", ctypes.c_int64),
        ("dense_macs_per_token", ctypes.c_int64),
    ]

    def as_dict(self):
        return {k: getattr(self, k) for k, _ in self._fields_}


_lib = None
_lock = threading.Lock()


def load_library(path: str | None = None):
    """Load libeqlinear.so (raises OSError if it has not been built)."""
    global _lib
    with _lock:
        if _lib is not None and path is None:
            return _lib
        p = path or LIB_PATH
        if not os.path.exists(p):
            raise OSError(f"{p} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'`")
        lib = ctypes.CDLL(p)
        vp, i32, i64, st = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int
        plan_p = ctypes.POINTER(ctypes.c_void_p)
        sig = {
            "eqlinear_status_string": ([st], ctypes.c_char_p),
            "eqlinear_plan": ([plan_p, i32, i32, i32, i32], st),
            "eqlinear_d8_plan": ([plan_p, i32, i32, i32], st),
            "eqlinear_plan_destroy": ([vp], st),
            "eqlinear_plan_info": ([vp, ctypes.POINTER(eqlinear_info)], st),
            "eqlinear_w_hat_elems": ([vp], ctypes.c_size_t),
            "eqlinear_weight_fft": ([vp, vp, vp], st),
            "eqlinear_forward": ([vp, vp, vp, vp, i64, vp], st),
            "eqlinear_forward_tiled": ([vp, vp, vp, vp, i64, vp, i32], st),
            "eqlinear_d8_forward": ([vp, vp, vp, vp, i64, vp], st),
            "eqlinear_expand_dense": ([vp, vp, vp, vp], st),
            "eqlinear_dense_forward": ([vp, vp, vp, vp, i64, vp], st),
            "eqlinear_w_hat_adjoint": ([vp, vp, vp, vp], st),
            "eqlinear_backward_data": ([vp, vp, vp, vp, i64, vp], st),
            "eqlinear_backward_weight_workspace": ([vp, i64], ctypes.c_size_t),
            "eqlinear_backward_weight": ([vp, vp, vp, vp, i64, vp, ctypes.c_size_t, vp], st),
            "eqlinear_backward_weight_noalloc": ([vp, vp, vp, vp, i64, vp], st),
            "eqlinear_forward_bias_act": ([vp, vp, vp, vp, i32, vp, i64, vp, i32], st),
            "eqlinear_d8_bias_act": ([vp, vp, vp, i32, vp, i64, vp], st),
            "eqlinear_dihedral_plan": ([ctypes.POINTER(ctypes.c_void_p), i32, i32, i32, i32], st),
            "eqlinear_d8_to_fourier": ([vp, vp, vp, i64, vp], st),
            "eqlinear_d8_regular_forward": ([vp, vp, vp, vp, i32, vp, i64, vp], st),
            "eqlinear_d8_to_regular": ([vp, vp, vp, i64, vp], st),
        }
        for name, (args, res) in sig.items():
            f = getattr(lib, name)
            f.argtypes, f.restype = args, res
        if path is None:
            _lib = lib
        return lib


def eqlinear_status_string(status: int) -> str:
    return load_library().eqlinear_status_string(int(status)).decode()


def _check(status: int, where: str):
    if status != EQL_OK:
        raise EqlError(status, where)


class Plan:
    """Owns an eqlinear_plan_t; destroyed when garbage-collected."""

    def __init__(self, handle: int, lib):
        self.handle = ctypes.c_void_p(handle)
        self._lib = lib
        self.info = eqlinear_plan_info(self)

    def __del__(self):
        # may run during interpreter shutdown, when module globals (ctypes among
        # them) are already gone: touch only what the instance holds
        h = getattr(self, "handle", None)
        lib = getattr(self, "_lib", None)
        if h is not None and lib is not None and h.value:
            lib.eqlinear_plan_destroy(h)
            h.value = None

    @property
    def dtype(self):
        return self.info["dtype"]


def eqlinear_plan(N: int, C_in: int, C_out: int, dtype: int) -> Plan:
    lib = load_library()
    h = ctypes.c_void_p()
    _check(lib.eqlinear_plan(ctypes.byref(h), N, C_in, C_out, int(dtype)), "eqlinear_plan")
    return Plan(h.value, lib)


def eqlinear_d8_plan(C_in: int, C_out: int, dtype: int) -> Plan:
    lib = load_library()
    h = ctypes.c_void_p()
    _check(lib.eqlinear_d8_plan(ctypes.byref(h), C_in, C_out, int(dtype)), "eqlinear_d8_plan")
    return Plan(h.value, lib)


def eqlinear_dihedral_plan(n: int, C_in: int, C_out: int, dtype: int) -> Plan:
    """Plan of the D_n layer (dihedral group of the regular n-gon, order 2n; n = 4 is D8)."""
    lib = load_library()
    h = ctypes.c_void_p()
    _check(lib.eqlinear_dihedral_plan(ctypes.byref(h), n, C_in, C_out, int(dtype)), "eqlinear_dihedral_plan")
    return Plan(h.value, lib)


def eqlinear_plan_destroy(plan: Plan):
    if plan.handle.value:
        _check(plan._lib.eqlinear_plan_destroy(plan.handle), "eqlinear_plan_destroy")
        plan.handle = ctypes.c_void_p(0)


def eqlinear_plan_info(plan: Plan) -> dict:
    inf = eqlinear_info()
    _check(plan._lib.eqlinear_plan_info(plan.handle, ctypes.byref(inf)), "eqlinear_plan_info")
    return inf.as_dict()


def eqlinear_w_hat_elems(plan: Plan) -> int:
    return int(plan._lib.eqlinear_w_hat_elems(plan.handle))


# --- tensor marshalling --------------------------------------------------------

def _torch_dtype(plan: Plan):
    import torch
    return {EQL_F32: torch.float32, EQL_BF16: torch.bfloat16, EQL_F16: torch.float16}[plan.dtype]


def _ptr(t, plan: Plan, numel: int | None, name: str):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor or a device address")
    if t.device.type != "cuda":
        raise ValueError(f"{name}: tensor must live on the GPU, got {t.device}")
    if t.dtype != _torch_dtype(plan):
        raise ValueError(f"{name}: dtype {t.dtype} does not match the plan ({_torch_dtype(plan)})")
    if not t.is_contiguous():
        raise ValueError(f"{name}: tensor must be contiguous")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name}: expected {numel} elements, got {t.numel()}")
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _widths(plan: Plan):
    inf = plan.info
    if inf["kind"] == EQL_KIND_CN:
        return inf["N"] * inf["C_in"], inf["N"] * inf["C_out"]
    return inf["C_in"], inf["C_out"]


def _tokens(x, T, K):
    if T is not None:
        return int(T)
    if isinstance(x, int):
        raise ValueError("T is required when x is a raw address")
    return x.numel() // K


def eqlinear_weight_fft(plan: Plan, w, w_hat):
    n = eqlinear_w_hat_elems(plan)
    _check(plan._lib.eqlinear_weight_fft(plan.handle, _ptr(w, plan, n, "w"),
                                         _ptr(w_hat, plan, n, "w_hat")), "eqlinear_weight_fft")


def eqlinear_forward(plan: Plan, x, w_hat, y, T: int | None = None, stream=None):
    K, M = _widths(plan)
    T = _tokens(x, T, K)
    n = eqlinear_w_hat_elems(plan)
    _check(plan._lib.eqlinear_forward(plan.handle, _ptr(x, plan, T * K, "x"),
                                      _ptr(w_hat, plan, n, "w_hat"), _ptr(y, plan, T * M, "y"),
                                      T, _stream(stream)), "eqlinear_forward")


def eqlinear_forward_tiled(plan: Plan, x, w_hat, y, tile: int, T: int | None = None, stream=None):
    K, M = _widths(plan)
    T = _tokens(x, T, K)
    n = eqlinear_w_hat_elems(plan)
    _check(plan._lib.eqlinear_forward_tiled(plan.handle, _ptr(x, plan, T * K, "x"),
                                            _ptr(w_hat, plan, n, "w_hat"),
                                            _ptr(y, plan, T * M, "y"), T, _stream(stream),
                                            int(tile)), "eqlinear_forward_tiled")


def eqlinear_forward_bias_act(plan: Plan, x, w_hat, bias, act: int, y, T: int | None = None, stream=None,
                              tile: int = -1):
    """y = act(layer(x) + bias[o]); bias may be None (no bias), act EQL_ACT_NONE or EQL_ACT_GELU."""
    K, M = _widths(plan)
    T = _tokens(x, T, K)
    n = eqlinear_w_hat_elems(plan)
    _check(plan._lib.eqlinear_forward_bias_act(plan.handle, _ptr(x, plan, T * K, "x"),
                                               _ptr(w_hat, plan, n, "w_hat"),
                                               _ptr(bias, plan, plan.info["C_out"], "bias"), int(act),
                                               _ptr(y, plan, T * M, "y"), T, _stream(stream), int(tile)),
           "eqlinear_forward_bias_act")


def eqlinear_d8_forward(plan: Plan, x, wb, y, T: int | None = None, stream=None):
    K, M = _widths(plan)
    T = _tokens(x, T, K)
    n = eqlinear_w_hat_elems(plan)
    _check(plan._lib.eqlinear_d8_forward(plan.handle, _ptr(x, plan, T * K, "x"),
                                         _ptr(wb, plan, n, "wb"), _ptr(y, plan, T * M, "y"),
                                         T, _stream(stream)), "eqlinear_d8_forward")


def eqlinear_d8_bias_act(plan: Plan, y_in, bias, act: int, y_out, T: int | None = None, stream=None):
    """y_out = F act(F^T y_in + bias[j]) per regular channel (y_out may be y_in); bias None or
    [C_out / group order]."""
    _, M = _widths(plan)
    T = _tokens(y_in, T, M)
    _check(plan._lib.eqlinear_d8_bias_act(plan.handle, _ptr(y_in, plan, T * M, "y_in"),
                                          _ptr(bias, plan, plan.info["C_out"] // plan.info["N"], "bias"), int(act),
                                          _ptr(y_out, plan, T * M, "y_out"), T, _stream(stream)),
           "eqlinear_d8_bias_act")


def eqlinear_d8_regular_forward(plan: Plan, x_reg, wb, bias, act: int, y_reg, T: int | None = None,
                                stream=None):
    """y_reg = act(to_regular(layer(to_fourier(x_reg))) + bias[j]) in one launch; bias None or
    [C_out / group order]."""
    K, M = _widths(plan)
    T = _tokens(x_reg, T, K)
    _check(plan._lib.eqlinear_d8_regular_forward(plan.handle, _ptr(x_reg, plan, T * K, "x_reg"),
                                                 _ptr(wb, plan, eqlinear_w_hat_elems(plan), "wb"),
                                                 _ptr(bias, plan, plan.info["C_out"] // plan.info["N"], "bias"),
                                                 int(act), _ptr(y_reg, plan, T * M, "y_reg"), T, _stream(stream)),
           "eqlinear_d8_regular_forward")


def eqlinear_d8_to_fourier(plan: Plan, x_reg, x_four, T: int | None = None, stream=None):
    K, _ = _widths(plan)
    T = _tokens(x_reg, T, K)
    _check(plan._lib.eqlinear_d8_to_fourier(plan.handle, _ptr(x_reg, plan, T * K, "x_reg"),
                                            _ptr(x_four, plan, T * K, "x_four"), T, _stream(stream)),
           "eqlinear_d8_to_fourier")


def eqlinear_d8_to_regular(plan: Plan, y_four, y_reg, T: int | None = None, stream=None):
    _, M = _widths(plan)
    T = _tokens(y_four, T, M)
    _check(plan._lib.eqlinear_d8_to_regular(plan.handle, _ptr(y_four, plan, T * M, "y_four"),
                                            _ptr(y_reg, plan, T * M, "y_reg"), T, _stream(stream)),
           "eqlinear_d8_to_regular")


def eqlinear_expand_dense(plan: Plan, w, w_dense, stream=None):
    K, M = _widths(plan)
    n = eqlinear_w_hat_elems(plan)
    _check(plan._lib.eqlinear_expand_dense(plan.handle, _ptr(w, plan, n, "w"),
                                           _ptr(w_dense, plan, K * M, "w_dense"),
                                           _stream(stream)), "eqlinear_expand_dense")


def eqlinear_dense_forward(plan: Plan, x, w_dense, y, T: int | None = None, stream=None):
    K, M = _widths(plan)
    T = _tokens(x, T, K)
    _check(plan._lib.eqlinear_dense_forward(plan.handle, _ptr(x, plan, T * K, "x"),
                                            _ptr(w_dense, plan, K * M, "w_dense"),
                                            _ptr(y, plan, T * M, "y"), T, _stream(stream)),
           "eqlinear_dense_forward")


def eqlinear_w_hat_adjoint(plan: Plan, w_hat, w_hat_adj, stream=None):
    n = eqlinear_w_hat_elems(plan)
    _check(plan._lib.eqlinear_w_hat_adjoint(plan.handle, _ptr(w_hat, plan, n, "w_hat"),
                                            _ptr(w_hat_adj, plan, n, "w_hat_adj"), _stream(stream)),
           "eqlinear_w_hat_adjoint")


def eqlinear_backward_data(plan: Plan, dy, w_hat_adj, dx, T: int | None = None, stream=None):
    K, M = _widths(plan)
    T = _tokens(dy, T, M)
    n = eqlinear_w_hat_elems(plan)
    _check(plan._lib.eqlinear_backward_data(plan.handle, _ptr(dy, plan, T * M, "dy"),
                                            _ptr(w_hat_adj, plan, n, "w_hat_adj"),
                                            _ptr(dx, plan, T * K, "dx"), T, _stream(stream)),
           "eqlinear_backward_data")


def eqlinear_backward_weight_workspace(plan: Plan, T: int) -> int:
    return int(plan._lib.eqlinear_backward_weight_workspace(plan.handle, int(T)))


def _raw_ptr(t, name: str, dtype=None, numel: int | None = None):
    """Device address of a tensor whose dtype does not follow the plan."""
    if isinstance(t, int):
        return t
    import torch
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise ValueError(f"{name}: expected a GPU tensor")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: tensor must be contiguous")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name}: expected {numel} elements, got {t.numel()}")
    return t.data_ptr()


def eqlinear_backward_weight(plan: Plan, x, dy, dw, workspace, T: int | None = None, stream=None):
    """dw (fp32, N*C_in*C_out elements) from x and dy; workspace: a GPU byte
    tensor of at least eqlinear_backward_weight_workspace(plan, T) bytes."""
    import torch
    K, M = _widths(plan)
    T = _tokens(x, T, K)
    n = eqlinear_w_hat_elems(plan)
    if isinstance(workspace, int):
        raise ValueError("workspace: pass a GPU tensor (its size is checked)")
    wbytes = workspace.numel() * workspace.element_size()
    _check(plan._lib.eqlinear_backward_weight(plan.handle, _ptr(x, plan, T * K, "x"), _ptr(dy, plan, T * M, "dy"),
                                              _raw_ptr(dw, "dw", torch.float32, n),
                                              T, _raw_ptr(workspace, "workspace"), wbytes, _stream(stream)),
           "eqlinear_backward_weight")


def eqlinear_backward_weight_noalloc(plan: Plan, x, dy, dw, T: int | None = None, stream=None):
    """dw (fp32, N*C_in*C_out elements) from x and dy, with the workspace in the
    library's own scratch array on the current GPU (no allocation anywhere)."""
    import torch
    K, M = _widths(plan)
    T = _tokens(x, T, K)
    n = eqlinear_w_hat_elems(plan)
    st = plan._lib.eqlinear_backward_weight_noalloc(plan.handle, _ptr(x, plan, T * K, "x"),
                                                    _ptr(dy, plan, T * M, "dy"),
                                                    _raw_ptr(dw, "dw", torch.float32, n), T, _stream(stream))
    if st == EQL_ERR_UNSUPPORTED:
        need = eqlinear_backward_weight_workspace(plan, T)
        raise EqlError(st, f"eqlinear_backward_weight_noalloc (workspace {need} bytes > the "
                           f"{EQL_NOALLOC_SCRATCH_BYTES}-byte library scratch, or past the 2 GiB plane limit)")
    _check(st, "eqlinear_backward_weight_noalloc")


def built() -> bool:
    return os.path.exists(LIB_PATH)
