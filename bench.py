"""Benchmark of the EQ-Linear forward on one MI355X.

Prints ONE JSON line.  A step is one forward of the layer over one batch of
synthetic tokens already resident in device memory: for a C_N workload the
fused eqlinear_forward (group DFT, per-bin matrix-core products, inverse DFT),
for the D8 workload eqlinear_d8_forward.  The weight spectrum (eqlinear_weight_fft)
is computed once per weight, before the timed region, and timed on its own.

Beside the step the run times, on the same inputs:
  - the expanded-dense comparator: the replicated dense matrix multiplied by
    this library's own MFMA GEMM and by torch's F.linear (hipBLASLt); the
    faster of the two is the bar ("Flash EQ-Linear", Problem Statement and
    Experimental Results / Operator Level compare against F.linear);
  - the same step warm: back-to-back steps replayed from a HIP graph, with the
    inputs left in the 256 MiB Infinity Cache by the previous step (a labelled
    secondary figure: it measures the cache, not HBM);
  - the fp64 CPU oracle on the host cores (rank 0, N=1 only, bounded sample).

The headline time is cache-cold: every timed step starts with a 512 MiB read
that evicts the L2s and the Infinity Cache (a read leaves clean lines, so no
write-back of the flush's data is charged to the layer), and the step's layers
are bracketed by HIP events on the stream they are launched on.  ms_per_step,
value and roofline.frac all come from that cold time.

Default workload: c3, the ViT-B MLP trio of C_8 layers in bf16 at T = 64 x 197
tokens (768->768, 768->3072, 3072->768 wide, i.e. 96->96, 96->384 and 384->96
channels per group element), run as one step of three launches.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "EQ-Linear fwd tokens/sec + TFLOP/s and % roofline vs expanded-dense GEMM"
OP_METRIC = {
    "forward": METRIC,
    "backward_data": "EQ-Linear bwd (input gradient) tokens/sec + TFLOP/s and % roofline vs expanded-dense GEMM",
    "backward_weight": "EQ-Linear bwd (weight gradient) tokens/sec + TFLOP/s and % roofline vs expanded-dense GEMM",
    "regular": "EQ-Linear (dihedral, regular features in and out, one launch) fwd tokens/sec + TFLOP/s and "
               "% roofline vs expanded-dense GEMM",
}
HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = {"f32": 157.3, "bf16": 2500.0, "f16": 2500.0}
KERNEL_SOURCES = {
    "C": ["group_equivariant_linear_amd/csrc/cn_fused.h",
          "group_equivariant_linear_amd/csrc/cn_mf.h",
          "group_equivariant_linear_amd/csrc/cn_split.h",
          "group_equivariant_linear_amd/csrc/cn_dispatch.h",
          "group_equivariant_linear_amd/csrc/dft_coef.h",
          "group_equivariant_linear_amd/csrc/eq_device.h"],
    "BW": ["group_equivariant_linear_amd/csrc/cn_backward.hip",
           "group_equivariant_linear_amd/csrc/dft_coef.h",
           "group_equivariant_linear_amd/csrc/eq_device.h"],
    "D8": ["group_equivariant_linear_amd/csrc/d8_forward.hip",
           "group_equivariant_linear_amd/csrc/gemm_rows.hip",
           "group_equivariant_linear_amd/csrc/eq_device.h"],
    "REG": ["group_equivariant_linear_amd/csrc/dn_regular.hip",
            "group_equivariant_linear_amd/csrc/dn_group.h",
            "group_equivariant_linear_amd/csrc/eq_device.h"],
}
KERNEL_SOURCES["D"] = KERNEL_SOURCES["D8"]  # the dihedral layers of other orders: same kernels


def step_kernel_name(wl):
    """The kernel one forward of this workload launches (automatic tile choice)."""
    if wl.group != "C":
        # dihedral (D8 or D_n, N = group order): block columns in whole 16-byte pieces
        whole = (wl.C_in // wl.N) % 8 == 0 and (wl.C_out // wl.N) % 8 == 0
        return "d8_kernel" if wl.dtype in ("bf16", "f16") and whole else "gemm_rows_kernel"
    if wl.dtype in ("bf16", "f16") and 2 <= wl.N <= 8:
        return "cn_mf_kernel"
    if wl.dtype == "f32" and wl.N <= 10 and wl.C_in % 4 == 0 and _one_wave_shape(wl):
        return "cn_split_kernel"
    return "cn_fast_kernel"


def _one_wave_shape(wl):
    """True where the automatic choice falls to one-wave tiles (the layer is too
    small to give every CU a 4-wave workgroup); fp32 layers then run the
    input-channel split kernel.  Mirrors choose_shape in cn_dispatch.h."""
    nblk = (wl.C_out + 15) // 16
    cb = min(max(24 // wl.N, 2), 6)
    if cb > nblk:
        cb = max(nblk, 2)
    while cb >= 2:
        if ((wl.T + 63) // 64) * ((nblk + cb - 1) // cb) >= 256:
            return False
        cb -= 1
    return True


def kernel_source_hash(group):
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[group]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="c3",
                    help="c1, c2, c3a, c3b, c3c, c3 (the three MLP layers), c4, c5")
    ap.add_argument("--dtype", default="workload", choices=["workload", "f32", "bf16", "f16"],
                    help="element type of the workload's tensors (default: the workload's own)")
    ap.add_argument("--tile", type=int, default=-1,
                    help="fixed tile configuration of the C_N kernel (eqlinear_forward_tiled); -1 = automatic")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="target CPU time of the oracle sample (0 disables)")
    ap.add_argument("--op", default="forward", choices=["forward", "backward_data", "backward_weight", "regular"],
                    help="which pass of a C_N workload to time (the default line is the forward); "
                         "regular: a dihedral workload between regular-representation features in one "
                         "launch (eqlinear_d8_regular_forward; --epilogue sets bias/GELU)")
    ap.add_argument("--epilogue", default="none", choices=["none", "bias", "bias_gelu"],
                    help="forward with its pointwise neighbours: C_N workloads through "
                         "eqlinear_forward_bias_act (bias and GELU fused into the store), D8 through "
                         "eqlinear_d8_forward + the fused regular-domain round trip eqlinear_d8_bias_act; "
                         "the comparators add the same in torch")
    ap.add_argument("--mode", default="bench", choices=["bench", "cold", "traffic"],
                    help="cold: only the timed cache-cold steps (for rocprofv3 --kernel-trace); "
                         "traffic: a few forwards and a copy of known size, for rocprofv3 --pmc")
    ap.add_argument("--counters-from", nargs="+", metavar="PMC_DIR",
                    help="read the counter_collection.csv of one or more rocprofv3 --pmc runs (one pass "
                         "each) of --mode cold and write profiles/counters_<workload>.md")
    ap.add_argument("--trace-from", metavar="TRACE_DIR",
                    help="read the kernel_trace.csv of a rocprofv3 --kernel-trace run of --mode cold "
                         "and write profiles/kernel_trace_<workload>.md")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="read the counter CSVs of a FETCH_SIZE and a WRITE_SIZE run of "
                         "--mode traffic and write profiles/traffic_<workload>.{json,md}")
    return ap.parse_args()


class Layer:
    """One layer of a workload: device buffers, plan, and the step callables."""

    def __init__(self, eq, wl, seed=0, tile=-1, op="forward", epilogue="none"):
        import numpy as np
        import torch

        import synthetic
        self.wl = wl
        self.dt = wl.dtype
        self.tdt = {synthetic.F32: torch.float32, synthetic.BF16: torch.bfloat16,
                    synthetic.F16: torch.float16}[wl.dtype]
        eqdt = {synthetic.F32: eq.EQL_F32, synthetic.BF16: eq.EQL_BF16, synthetic.F16: eq.EQL_F16}[wl.dtype]
        d = synthetic.workload_inputs(wl, seed=seed)
        self.inputs = d

        def dev(a):
            if wl.dtype == synthetic.F32:
                return torch.from_numpy(a).cuda()
            return torch.from_numpy(a.view(np.int16)).view(self.tdt).cuda()

        self.x = dev(d["x"]).reshape(wl.T, -1)
        w = dev(d["w"])
        if wl.group == "C":
            self.plan = eq.eqlinear_plan(wl.N, wl.C_in, wl.C_out, eqdt)
            self.w_hat = torch.empty(eq.eqlinear_w_hat_elems(self.plan), dtype=self.tdt, device="cuda")
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            eq.eqlinear_weight_fft(self.plan, w, self.w_hat)
            self.weight_fft_ms = (time.perf_counter() - t0) * 1e3
            self.K, self.M = wl.N * wl.C_in, wl.N * wl.C_out
            if tile < 0:
                self.step = lambda: eq.eqlinear_forward(self.plan, self.x, self.w_hat, self.y, T=wl.T)
            else:
                self.step = lambda: eq.eqlinear_forward_tiled(self.plan, self.x, self.w_hat, self.y, tile, T=wl.T)
        else:
            self.plan = eq.eqlinear_dihedral_plan(wl.N // 2, wl.C_in, wl.C_out, eqdt)
            self.w_hat = w
            self.weight_fft_ms = None
            self.K, self.M = wl.C_in, wl.C_out
            self.step = lambda: eq.eqlinear_d8_forward(self.plan, self.x, self.w_hat, self.y, T=wl.T)
        self.y = torch.empty(wl.T, self.M, dtype=self.tdt, device="cuda")
        self.w = w
        info = self.plan.info
        self.macs_per_token = info["macs_per_token"]
        self.dense_macs_per_token = info["dense_macs_per_token"]
        es = 4 if wl.dtype == synthetic.F32 else 2
        self.bytes_per_token = (self.K + self.M) * es
        self.w_hat_bytes = info["w_hat_elems"] * es
        self.bytes_per_launch = wl.T * self.bytes_per_token + self.w_hat_bytes

        # comparator: replicated dense matrix, own MFMA GEMM and torch F.linear
        self.W_dense = torch.empty(self.M, self.K, dtype=self.tdt, device="cuda")
        t0 = time.perf_counter()
        eq.eqlinear_expand_dense(self.plan, w, self.W_dense)
        torch.cuda.synchronize()
        self.expand_ms = (time.perf_counter() - t0) * 1e3
        self.y_dense = torch.empty_like(self.y)
        self.dense_own = lambda: eq.eqlinear_dense_forward(self.plan, self.x, self.W_dense, self.y_dense, T=wl.T)
        self.y_lin = torch.empty_like(self.y)
        # F.linear(x, W) without a bias is x @ W^T: the same GEMM, written into a fixed buffer
        self.dense_torch = lambda: torch.mm(self.x, self.W_dense.t(), out=self.y_lin)
        self.op = op
        self.out = self.y
        self.post = None
        # the tensors a step reads and writes per token (rotated through copies
        # for the cache-cold timing) and those of the comparators
        self.rot = ("x", "y")
        self.rot_dense = ("x", "y_dense", "y_lin")
        if op == "regular":
            self._regular(eq, wl, d, dev, es, epilogue)
        elif op != "forward":
            self._backward(eq, wl, d, dev, eqdt, es)
        elif epilogue != "none":
            self._epilogue(eq, wl, d, dev, es, tile, epilogue)

    def _epilogue(self, eq, wl, d, dev, es, tile, epilogue):
        """Forward with the fused bias (+ GELU).  The comparators run the dense GEMM
        with torch's bias add and in-place GELU after it."""
        import torch

        import synthetic
        if wl.group != "C":
            return self._d8_epilogue(eq, wl, d, dev, es, epilogue)
        bd, d["b64"] = synthetic.channel_bias(wl.C_out, wl.dtype, 500)
        self.bias = dev(bd)
        act = eq.EQL_ACT_GELU if epilogue == "bias_gelu" else eq.EQL_ACT_NONE
        d["act"] = act
        self.step = lambda: eq.eqlinear_forward_bias_act(self.plan, self.x, self.w_hat, self.bias, act, self.y,
                                                         T=wl.T, tile=tile)
        self.bytes_per_launch += wl.C_out * es
        # y is [t][o][g]: column o*N+g carries b[o]
        bias_cols = self.bias.repeat_interleave(wl.N)
        gelu_ = torch._C._nn.gelu_

        def dense_torch():
            torch.addmm(bias_cols, self.x, self.W_dense.t(), out=self.y_lin)
            if act == eq.EQL_ACT_GELU:
                gelu_(self.y_lin)
        self.dense_torch = dense_torch

        def post(t):  # the same neighbours on the own GEMM's output, for the agreement figure
            v = t.float() + bias_cols.float()
            return torch.nn.functional.gelu(v) if act == eq.EQL_ACT_GELU else v
        self.post = post

    def _d8_epilogue(self, eq, wl, d, dev, es, epilogue):
        """Dihedral layer (D8, or D_n with N = 2n), then the fused regular-domain
        round trip in place (bias per regular channel, GELU).  The torch
        comparator: dense GEMM, then gather to the regular layout, the N x N
        transform, bias, in-place GELU, transform back and scatter."""
        import numpy as np
        import torch

        import synthetic
        G, n = wl.N, wl.N // 2
        m = wl.C_out // G
        bd, d["b64"] = synthetic.channel_bias(m, wl.dtype, 500)
        self.bias = dev(bd)
        act = eq.EQL_ACT_GELU if epilogue == "bias_gelu" else eq.EQL_ACT_NONE
        d["act"] = act

        def step():
            eq.eqlinear_d8_forward(self.plan, self.x, self.w_hat, self.y, T=wl.T)
            eq.eqlinear_d8_bias_act(self.plan, self.y, self.bias, act, self.y, T=wl.T)
        self.step = step
        self.bytes_per_launch += m * es
        Fm, n1, n2 = _dihedral_fourier_matrix(n)
        F = torch.tensor(Fm, dtype=torch.float32, device="cuda").to(self.tdt)
        j = np.arange(m)[:, None]
        cols = [b * m + j for b in range(n1)]
        for k in range(n2):  # E_k copies 2j, 2j+1 in its coordinate-0 and -1 slabs
            base = n1 * m + 4 * m * k
            cols += [base + 2 * j, base + 2 * j + 1, base + 2 * m + 2 * j, base + 2 * m + 2 * j + 1]
        idx = torch.tensor(np.concatenate(cols, axis=1).reshape(-1), device="cuda")  # [m][G] Fourier columns
        gelu_ = torch._C._nn.gelu_
        bias_j = self.bias[:, None]

        def round_trip(t):
            f = torch.matmul(t[:, idx].view(wl.T, m, G), F) + bias_j  # regular values: v F
            if act == eq.EQL_ACT_GELU:
                gelu_(f)
            t[:, idx] = torch.matmul(f, F.t().contiguous()).view(wl.T, -1)

        def dense_torch():
            torch.mm(self.x, self.W_dense.t(), out=self.y_lin)
            round_trip(self.y_lin)
        self.dense_torch = dense_torch

        def post(t):
            u = t.clone()
            round_trip(u)
            return u.float()
        self.post = post

    def _regular(self, eq, wl, d, dev, es, epilogue):
        """Dihedral layer between regular features in one launch: x_reg -> group
        Fourier transform -> blocks -> inverse -> bias (+ GELU) -> y_reg.  The
        comparators: the chain of the library's separate passes it replaces
        (to_fourier, d8_forward, the round trip, to_regular: four launches) and
        torch's dense GEMM on the equivalent regular-basis matrix with the bias in
        the GEMM and an in-place GELU after it."""
        import numpy as np
        import torch

        import synthetic
        assert wl.group != "C", "--op regular applies to the dihedral workloads"
        G, n = wl.N, wl.N // 2
        m = wl.C_out // G
        bd, d["b64"] = synthetic.channel_bias(m, wl.dtype, 500)
        self.bias = dev(bd) if epilogue != "none" else None
        act = eq.EQL_ACT_GELU if epilogue == "bias_gelu" else eq.EQL_ACT_NONE
        d["act"], d["regular"], d["bias_on"] = act, True, epilogue != "none"
        self.step = lambda: eq.eqlinear_d8_regular_forward(self.plan, self.x, self.w_hat, self.bias, act, self.y,
                                                           T=wl.T)
        self.bytes_per_launch += (m * es if epilogue != "none" else 0)
        self.xf = torch.empty_like(self.x)
        self.yf = torch.empty_like(self.y)
        self.y_chain = torch.empty_like(self.y)

        def chain():
            eq.eqlinear_d8_to_fourier(self.plan, self.x, self.xf, T=wl.T)
            eq.eqlinear_d8_forward(self.plan, self.xf, self.w_hat, self.yf, T=wl.T)
            eq.eqlinear_d8_bias_act(self.plan, self.yf, self.bias, act, self.yf, T=wl.T)
            eq.eqlinear_d8_to_regular(self.plan, self.yf, self.y_chain, T=wl.T)
        self.chain = chain
        self.rot_chain = ("x", "xf", "yf", "y_chain")
        # the regular-basis dense matrix: W_reg = R_out^T W_four R_in, with R the
        # map from regular features to the Fourier layout (per channel F, then the
        # layout's columns)
        Fm, n1, n2 = _dihedral_fourier_matrix(n)

        def to_four(width):
            mm = width // G
            j = np.arange(mm)[:, None]
            cols = [b * mm + j for b in range(n1)]
            for k in range(n2):
                base = n1 * mm + 4 * mm * k
                cols += [base + 2 * j, base + 2 * j + 1, base + 2 * mm + 2 * j, base + 2 * mm + 2 * j + 1]
            idx = np.concatenate(cols, axis=1)  # [mm][G]: Fourier column of (channel, feature p)
            R = np.zeros((width, width))
            for jj in range(mm):
                for p in range(G):
                    R[idx[jj, p], jj * G:(jj + 1) * G] = Fm[p]
            return torch.tensor(R, dtype=torch.float32, device="cuda")
        W_reg = to_four(wl.C_out).t() @ self.W_dense.float() @ to_four(wl.C_in)
        self.W_dense = W_reg.to(self.tdt).contiguous()
        bias_cols = (self.bias.repeat_interleave(G) if self.bias is not None
                     else torch.zeros(wl.C_out, dtype=self.tdt, device="cuda"))
        gelu_ = torch._C._nn.gelu_

        def dense_torch():
            torch.addmm(bias_cols, self.x, self.W_dense.t(), out=self.y_lin)
            if act == eq.EQL_ACT_GELU:
                gelu_(self.y_lin)
        self.dense_torch = dense_torch
        self.dense_own = None
        self.rot_dense = ("x", "y_lin")

    def _backward(self, eq, wl, d, dev, eqdt, es):
        """Buffers and step callables of the input- or weight-gradient pass; the
        upstream gradient dy is a second seeded standard normal tensor."""
        import numpy as np
        import torch

        import synthetic
        assert wl.group == "C", "the backward pass is defined for C_N layers"
        g = synthetic.cn_inputs(wl.N, wl.C_out, wl.C_in, wl.T, wl.dtype, 1000)
        self.inputs["dy64"] = g["x64"]
        self.dy = dev(g["x"]).reshape(wl.T, -1)
        if self.op == "backward_data":
            self.w_hat_adj = torch.empty_like(self.w_hat)
            eq.eqlinear_w_hat_adjoint(self.plan, self.w_hat, self.w_hat_adj)
            self.dx = torch.empty(wl.T, self.K, dtype=self.tdt, device="cuda")
            self.step = lambda: eq.eqlinear_backward_data(self.plan, self.dy, self.w_hat_adj, self.dx, T=wl.T)
            self.out = self.dx
            self.rot = ("dy", "dx")
            self.rot_dense = ("dy", "y_dense", "y_lin")
            # bytes: dy read, dx written, the adjoint spectrum
            self.bytes_per_launch = wl.T * self.bytes_per_token + self.w_hat_bytes
            # comparators: dx = dy W_dense, with W_dense^T materialised for the own GEMM
            plan_t = eq.eqlinear_plan(wl.N, wl.C_out, wl.C_in, eqdt)
            self._plan_t = plan_t
            self.W_dense_t = self.W_dense.t().contiguous()
            self.y_dense = torch.empty_like(self.dx)
            self.y_lin = torch.empty_like(self.dx)
            self.dense_own = lambda: eq.eqlinear_dense_forward(plan_t, self.dy, self.W_dense_t, self.y_dense, T=wl.T)
            self.dense_torch = lambda: torch.mm(self.dy, self.W_dense, out=self.y_lin)
        else:
            nb = eq.eqlinear_backward_weight_workspace(self.plan, wl.T)
            self.ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
            self.dw = torch.empty(self.w_hat.numel(), dtype=torch.float32, device="cuda")
            self.step = lambda: eq.eqlinear_backward_weight(self.plan, self.x, self.dy, self.dw, self.ws, T=wl.T)
            self.out = self.dw
            self.rot = ("x", "dy")
            self.rot_dense = ("x", "dy")
            # bytes: x and dy read once, dw written in fp32
            self.bytes_per_launch = wl.T * self.bytes_per_token + self.dw.numel() * 4
            # comparator: the dense weight gradient dy^T x (fp32 accumulation)
            self.y_dense = torch.empty(self.M, self.K, dtype=self.tdt, device="cuda")
            self.y_lin = self.y_dense
            self.dense_own = None
            self.dense_torch = lambda: torch.mm(self.dy.t().contiguous(), self.x, out=self.y_lin)


    def make_copies(self, n):
        """n copies of the rotated tensors (copy 0 is the original)."""
        keys = sorted(set(self.rot) | set(self.rot_dense) | set(getattr(self, "rot_chain", ())))
        self.copies = [{k: getattr(self, k) for k in keys}]
        for _ in range(n - 1):
            self.copies.append({k: getattr(self, k).clone() for k in keys})

    def use(self, r):
        for k, v in self.copies[r].items():
            setattr(self, k, v)


def _dihedral_fourier_matrix(n):
    """The orthonormal Fourier matrix F[p][q] of D_n (order G = 2n; n = 4: D8) for
    the torch comparator, from the irreps: rows sqrt(1/G) chi(q) for A1, A2 (and
    B1, B2 for even n), then sqrt(2/G) E_k(q)[kk][c] for each E_k; element
    q = a + n b is r^a s^b, E_k(r) the turn by 2 pi k / n, E_k(s) = diag(1,-1).
    Returns (F, number of 1-D irreps, number of 2-D irreps)."""
    import numpy as np
    G = 2 * n
    chars = [(1, 1), (1, -1)] + ([(-1, 1), (-1, -1)] if n % 2 == 0 else [])
    n2 = n // 2 - 1 if n % 2 == 0 else (n - 1) // 2
    F = np.zeros((G, G))
    for q in range(G):
        a, b = q % n, q // n
        for p, (cr, cs) in enumerate(chars):
            F[p, q] = cr ** a * cs ** b / np.sqrt(G)
        for k in range(1, n2 + 1):
            th = 2 * np.pi * k / n
            R = np.array([[np.cos(th), -np.sin(th)], [np.sin(th), np.cos(th)]])
            M = np.linalg.matrix_power(R, a) @ (np.diag([1.0, -1.0]) if b else np.eye(2))
            F[len(chars) + 4 * (k - 1):len(chars) + 4 * k, q] = np.sqrt(2.0 / G) * M.reshape(-1)
    return F, len(chars), n2


def time_loop(fns, steps, warmup):
    """Average ms per step of running every fn once per step, by events on the
    current stream (where the library launches)."""
    import torch
    for _ in range(warmup):
        for f in fns:
            f()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        for f in fns:
            f()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps


def time_graph(fns, outs, steps, warmup, per_graph=50):
    """Average ms per step with the steps captured into a HIP graph (per_graph
    steps per graph, replayed until `steps` steps ran), or None if a replay does
    not reproduce the eager outputs bit for bit (then the path stays eager).
    Launch-bound steps are measured this way because host-side launch cost is
    not part of the layer."""
    import torch
    for _ in range(max(warmup, 3)):
        for f in fns:
            f()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(per_graph):
            for f in fns:
                f()
    for _ in range(3):  # replays with eager work in between, each checked
        for o in outs:
            o.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        if not all(torch.equal(o, r) for o, r in zip(outs, ref)):
            return None
        for f in fns:
            f()
        torch.cuda.synchronize()
    reps = max(1, steps // per_graph)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / (reps * per_graph)


CACHE_BYTES = 256 * 1024 * 1024  # MI355X Infinity Cache
ROTATE_BYTES = 3 * CACHE_BYTES     # bytes a tensor copy waits before it is used again
MAX_COPIES = 64


def rotation_plan(bytes_per_step, est_us_per_step, steps):
    """(copies, steps per graph): enough copies that R x bytes >= 3x the
    Infinity Cache, and up to ~400 us of work per graph (the host's launch
    cost, ~10 us a graph, then hides behind the replay and the gap between
    graphs is spread over S steps), S a divisor of the timed step count so that
    exactly that many steps are timed; R is rounded up to a multiple of S so
    that every graph holds S distinct copies."""
    R = min(MAX_COPIES, max(2, -(-ROTATE_BYTES // max(bytes_per_step, 1))))
    S = max(1, min(R, int(400.0 // max(est_us_per_step, 1e-3))))
    while steps % S:
        S -= 1
    R = -(-R // S) * S
    return R, S


def rotation_timing(layers, fn_name, steps, warmup, bytes_per_step, est_us):
    """The timed cache-cold steps.  Each step runs fn_name of every layer on one
    of R copies of the tensors it reads and writes per token, in rotation, so
    a copy's data passes through HBM between uses (R x bytes >= 3x the
    Infinity Cache: its lines are evicted, and the previous steps' dirty y
    lines are written back while this step runs: the steady-state traffic).
    Steps are captured S to a HIP graph and replayed back to back; HIP events on
    the launch stream bracket the whole region, which synchronizes on both sides.
    Returns (ms per step, steps timed, R, S)."""
    import torch
    R, S = rotation_plan(bytes_per_step, est_us, steps)
    for L in layers:
        if not hasattr(L, "copies") or len(L.copies) < R:
            L.make_copies(R)
    graphs = []
    for g in range(R // S):
        for r in range(g * S, g * S + S):  # warm the kernels once eagerly
            for L in layers:
                L.use(r)
                getattr(L, fn_name)()
        torch.cuda.synchronize()
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            for r in range(g * S, g * S + S):
                for L in layers:
                    L.use(r)
                    getattr(L, fn_name)()
        graphs.append(gr)
    for L in layers:
        L.use(0)
    nrep = steps // S
    for k in range(-(-warmup // S)):
        graphs[k % len(graphs)].replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for k in range(nrep):
        graphs[k % len(graphs)].replay()
    b.record()
    torch.cuda.synchronize()
    del graphs
    return a.elapsed_time(b) / (nrep * S), nrep * S, R, S


def _median(v):
    v = sorted(v)
    n = len(v)
    return v[n // 2] if n % 2 else 0.5 * (v[n // 2 - 1] + v[n // 2])


def profile_tag(args):
    """The workload and the options that change the timed step, as a file-name part."""
    parts = [args.workload]
    if args.op != "forward":
        parts.append(args.op)
    if args.epilogue != "none":
        parts.append(args.epilogue)
    if args.dtype != "workload":
        parts.append(args.dtype)
    if args.tile != -1:
        parts.append(f"tile{args.tile}")
    return "_".join(parts)


def step_flags(args):
    """The command-line options that select the timed step, for the recorded commands."""
    f = f"--workload {args.workload}"
    if args.op != "forward":
        f += f" --op {args.op}"
    if args.epilogue != "none":
        f += f" --epilogue {args.epilogue}"
    if args.dtype != "workload":
        f += f" --dtype {args.dtype}"
    if args.tile != -1:
        f += f" --tile {args.tile}"
    return f


def summarize_trace(args, wls):
    """Per-dispatch durations of a rocprofv3 --kernel-trace run of --mode cold:
    the step kernel's dispatches in launch order, the eager warm-up and warmup
    steps dropped, grouped by layer; written to profiles/kernel_trace_<workload>.md."""
    import csv
    import glob
    files = glob.glob(os.path.join(args.trace_from, "**", "*kernel_trace.csv"), recursive=True)
    if len(files) != 1:
        raise SystemExit(f"expected one kernel_trace.csv under {args.trace_from}, found {files}")
    rows = list(csv.DictReader(open(files[0])))
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    step = [r for r in rows if any(k in r["Kernel_Name"] for k in STEP_KERNELS + BW_KERNELS)]
    names = sorted({r["Kernel_Name"] for r in step})
    nl = len(wls)
    nbytes = sum(algorithmic_bytes(w, args.op, args.epilogue) for w in wls)
    R, S = rotation_plan(nbytes, nbytes / 2.5e6, args.steps)
    skip = R + -(-args.warmup // S) * S  # eager warm-up of each graph's steps, then the warmup replays
    timed = -(-args.steps // S) * S
    # kernels per layer and step: 1 for a forward, 2 or 3 for the weight gradient
    kpl = len(step) // ((skip + timed) * nl)
    if kpl < 1 or len(step) != (skip + timed) * nl * kpl:
        raise SystemExit(f"{len(step)} step-kernel dispatches; expected ({skip} + {timed}) x {nl} x k")
    step = step[skip * nl * kpl:]
    per = {}  # (layer, position in the step) -> durations
    kname = {}
    gaps = []
    for i, r in enumerate(step):
        key = ((i // kpl) % nl, i % kpl)
        per.setdefault(key, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-3)
        kname[key] = r["Kernel_Name"]
        if i:
            gaps.append((int(r["Start_Timestamp"]) - int(step[i - 1]["End_Timestamp"])) * 1e-3)
    flags = step_flags(args)
    lines = [f"# Kernel trace, cache-cold steps, {profile_tag(args)}", "",
             "Commands:", "", "```",
             f"rocprofv3 --kernel-trace --stats -d {args.trace_from} -o run -f csv -- "
             f"python3 bench.py {flags} --mode cold --steps {args.steps} --warmup {args.warmup}",
             f"python3 bench.py {flags} --trace-from {args.trace_from} "
             f"--steps {args.steps} --warmup {args.warmup}", "```", "",
             f"Each step launches the layers on one of {R} copies of their per-token tensors, in rotation "
             f"({R * nbytes >> 20} MiB, over 3x the 256 MiB Infinity Cache), {S} step(s) per HIP graph; "
             f"the {skip} warm-up steps are dropped, {timed} steps remain.", "",
             "Kernels: " + ", ".join(f"`{n[:160]}`" for n in names), "",
             "| layer | kernel | grid | dispatches | mean us | median us | min us |",
             "|---|---|---|---|---|---|---|"]
    layer_mean = [0.0] * nl
    for (li, k), d in sorted(per.items()):
        grid = {r["Grid_Size_X"] for r in step[li * kpl + k::nl * kpl]}
        mean = sum(d) / max(len(d), 1)
        layer_mean[li] += mean
        short = next((n for n in STEP_KERNELS + BW_KERNELS if n in kname[(li, k)]), kname[(li, k)][:40])
        lines.append(f"| {wls[li].name} | {short} | {','.join(sorted(grid))} | {len(d)} | {mean:.2f} | "
                     f"{_median(d):.2f} | {min(d):.2f} |")
    lines += ["", "| layer | step us (sum of its kernels' means) | algorithmic bytes | GB/s | frac of 8 TB/s |",
              "|---|---|---|---|---|"]
    for li, wl in enumerate(wls):
        b = algorithmic_bytes(wl, args.op, args.epilogue)
        lines.append(f"| {wl.name} | {layer_mean[li]:.2f} | {b} | {b / layer_mean[li] / 1e3:.0f} | "
                     f"{b / layer_mean[li] / 1e3 / HBM_PEAK_GBS:.3f} |")
    tot_mean = sum(layer_mean)
    lines += ["", f"Sum of the layers' mean durations: {tot_mean:.2f} us per step ({nl * kpl} launches, mean "
                  f"{tot_mean / (nl * kpl):.2f} us); {nbytes} algorithmic bytes: {nbytes / tot_mean / 1e3:.0f} GB/s = "
                  f"{nbytes / tot_mean / 1e3 / HBM_PEAK_GBS:.3f} of 8 TB/s.",
              f"Gaps between consecutive dispatches under the profiler: median {_median(gaps):.2f} us."]
    stats = glob.glob(os.path.join(args.trace_from, "**", "*kernel_stats.csv"), recursive=True)
    if len(stats) == 1:
        # the profiler's own --stats summary of the same run (every dispatch of
        # the process: the eager warm-up and the comparators' setup included)
        srows = list(csv.DictReader(open(stats[0])))
        lines += ["", "rocprofv3 `--stats` (kernel_stats.csv of the same run, all dispatches of the process):", "",
                  "| kernel | calls | average us | min us | max us | share of GPU time |", "|---|---|---|---|---|---|"]
        for r in srows[:6]:
            lines.append(f"| `{r['Name'][:90]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                         f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.1f} % |")
    with open(os.path.join(ROOT, "profiles", f"kernel_trace_{profile_tag(args)}.md"), "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def cpu_baseline(layers, target_s, op="forward"):
    """The fp64 oracle (replicate-and-multiply) on the host cores, on a bounded
    sample: passes over the first n tokens of the batch, n sized so that a pass
    takes at most about target_s, repeated until target_s has elapsed."""
    import oracle  # CPU-baseline leg only
    per_token = 0.0
    for L in layers:
        p = min(L.wl.T, 64)
        ts = time.perf_counter()
        _run_oracle(L.wl, L.inputs, p, op)
        per_token += (time.perf_counter() - ts) / p
    n = max(1, min(layers[0].wl.T, int(target_s / max(per_token, 1e-12))))
    passes = 0
    t0 = time.perf_counter()
    while True:
        for L in layers:
            _run_oracle(L.wl, L.inputs, n, op)
        passes += 1
        el = time.perf_counter() - t0
        if el >= target_s:
            break
    names = "+".join(L.wl.name for L in layers)
    return {"value": passes * n / el, "unit": "tokens/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"{names}: {passes} pass(es) over the first {n} of {layers[0].wl.T} tokens, "
                      f"fp64 {'replicate-and-multiply' if op == 'forward' else op + ' (direct sums)'}, "
                      f"{el:.1f} s"}


def _run_oracle(wl, d, n, op="forward"):
    import oracle
    if d.get("regular"):
        nd, G = wl.N // 2, wl.N
        xr = d["x64"][:n].reshape(n, wl.C_in // G, G)
        yf = oracle.dn_dense_bias_act(nd, oracle.dn_to_fourier(nd, xr), d["w64"], wl.C_out,
                                      d["b64"] if d.get("bias_on") else None, d["act"])
        oracle.dn_to_regular(nd, yf)
    elif "b64" in d and wl.group != "C":
        oracle.dn_dense_bias_act(wl.N // 2, d["x64"][:n], d["w64"], wl.C_out, d["b64"], d["act"])
    elif "b64" in d:
        oracle.cn_dense_bias_act(d["x64"][:n], d["w64"], d["b64"], d["act"])
    elif op == "backward_data":
        oracle.cn_backward_data(d["dy64"][:n], d["w64"])
    elif op == "backward_weight":
        oracle.cn_backward_weight(d["x64"][:n], d["dy64"][:n])
    elif wl.group == "C":
        oracle.cn_dense(d["x64"][:n], d["w64"])
    else:
        oracle.dn_dense(wl.N // 2, d["x64"][:n], d["w64"], wl.C_out)


STEP_KERNELS = ("cn_fast_kernel", "cn_fused_kernel", "cn_mf_kernel", "cn_split_kernel", "cn_stream_kernel",
                "dn_regular_kernel", "d8_kernel",
                "gemm_rows_kernel")
BW_KERNELS = ("bw_planes_kernel", "bw_bin_kernel", "bw_gemm_kernel", "bw_small_kernel", "bw_xf_kernel",
              "bw_reduce_kernel")
TRAFFIC_WARM = 5   # back-to-back forwards (inputs partly cached from the previous launch)
TRAFFIC_COLD = 5   # forwards each after a 512 MiB read that evicts the L2s
TRAFFIC_COPIES = 5
TRAFFIC_COPY_BYTES = 256 * 1024 * 1024


def traffic_run(layers):
    """The launches the FETCH_SIZE / WRITE_SIZE passes count: warm forwards, cold
    forwards, and device copies of known size that calibrate the counters."""
    import torch
    for _ in range(TRAFFIC_WARM):
        for L in layers:
            L.step()
    flush = torch.ones(512 * 1024 * 1024 // 4, dtype=torch.float32, device="cuda")
    for _ in range(TRAFFIC_COLD):
        flush.sum()  # reads only: leaves clean lines, so no write-back is charged to the forward
        for L in layers:
            L.step()
    del flush
    n = TRAFFIC_COPY_BYTES // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(TRAFFIC_COPIES):
        dst.copy_(src)
    torch.cuda.synchronize()


def _counter_rows(d, counter):
    import csv
    import glob
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if len(files) != 1:
        raise SystemExit(f"expected one counter_collection.csv under {d}, found {files}")
    rows = [r for r in csv.DictReader(open(files[0])) if r["Counter_Name"] == counter]
    rows.sort(key=lambda r: int(r["Dispatch_Id"]))
    return rows


def op_kernel_name(wl, op):
    """Kernel(s) one step of the pass launches."""
    if op == "backward_data":
        from dataclasses import replace
        return step_kernel_name(replace(wl, C_in=wl.C_out, C_out=wl.C_in))
    if op == "regular":
        return "dn_regular_kernel"
    if op == "backward_weight":
        if wl.C_in <= 32 and wl.C_out <= 32:
            return "bw_small_kernel + bw_reduce_kernel"
        if wl.dtype in ("bf16", "f16") and wl.N in (2, 4, 6, 8):
            Tp = (wl.T + 31) // 32 * 32
            if max(wl.C_in, wl.C_out) * wl.N * Tp * 2 < 1 << 31:
                return "bw_xf_kernel + bw_reduce_kernel"
        return f"bw_planes_kernel + {_bw_products_kernel(wl)} + bw_reduce_kernel"
    return step_kernel_name(wl)


def _bw_products_kernel(wl):
    """Which product kernel the library picks for a wide layer's weight gradient:
    the per-bin kernel when some tile of at most 16 waves (32 x 64 outputs each)
    meets its load budget (4 loads per thread and stage above 8 waves, else 8;
    stages up to 53248 bytes) and both plane sets stay under 2 GiB; otherwise
    the 64 x 64 kernel.  A label only: the selection itself is the library's."""
    import synthetic
    S = 4 if wl.dtype == synthetic.F32 else 2
    Tp = (wl.T + 63) // 64 * 64
    if (wl.C_in + wl.C_out) * wl.N * Tp * S >= 1 << 31:
        return "bw_gemm_kernel"
    wmt, wnt = -(-wl.C_out // 32), -(-wl.C_in // 64)
    for no in range(1, wmt + 1):
        for ni in range(1, wnt + 1):
            wm, wn = -(-wmt // no), -(-wnt // ni)
            if wm * wn > 16:
                continue
            threads = 64 * wm * wn
            loads = -(-8 * (32 * wm + 64 * wn) // threads)
            if loads <= (8 if wm * wn <= 8 else 4) and loads * threads * 16 <= 53248:
                return "bw_bin_kernel"
    return "bw_gemm_kernel"


def _dense_grad_agreement(L):
    """rel-L2 between dw and the dense gradient dy^T x folded along its
    circulant diagonals: dw[o][i][m] = sum_g G[o*N+g][i*N+(g-m) mod N]."""
    import torch
    N, C_in, C_out = L.wl.N, L.wl.C_in, L.wl.C_out
    G = L.y_dense.float().reshape(C_out, N, C_in, N)
    g = torch.arange(N, device=G.device)
    # two index tensors split by a slice: the indexed axis comes first
    folded = torch.stack([G[:, g, :, (g - m) % N].sum(dim=0) for m in range(N)], dim=-1)
    dw = L.dw.reshape(C_out, C_in, N)
    return float(torch.linalg.vector_norm(dw - folded) / torch.linalg.vector_norm(folded))


def algorithmic_bytes(wl, op="forward", epilogue="none"):
    """Forward: x read once, y written once, the weight operand (w_hat, or the D8
    blocks) read once, plus the bias when one is fused.  Input gradient: dy read, dx written, the adjoint
    spectrum read.  Weight gradient: x and dy read, dw written in fp32."""
    es = 4 if wl.dtype == "f32" else 2
    if wl.group == "C":
        K, M, w = wl.N * wl.C_in, wl.N * wl.C_out, wl.N * wl.C_in * wl.C_out
    else:
        K, M = wl.C_in, wl.C_out
        nd = wl.N // 2  # dihedral D_n, N = 2n
        mi, mo = wl.C_in // wl.N, wl.C_out // wl.N
        w = (4 if nd % 2 == 0 else 2) * mi * mo + (nd // 2 - 1 if nd % 2 == 0 else (nd - 1) // 2) * 4 * mi * mo
    if op == "backward_weight":
        return es * wl.T * (K + M) + 4 * w
    bias = 0 if epilogue == "none" else (wl.C_out if wl.group == "C" else wl.C_out // wl.N)
    return es * (wl.T * (K + M) + w + bias)


def summarize_counters(args, wls):
    """Per-layer means of one or more rocprofv3 --pmc runs of --mode cold, one
    counter pass each (derived counters such as MfmaUtil, VALUBusy, LdsUtil,
    LDSBankConflict, OccupancyPercent, or raw ones), merged into one table and
    written to profiles/counters_<workload>.md."""
    import collections
    import csv
    import glob
    nl = len(wls)
    nbytes = sum(algorithmic_bytes(w, args.op, args.epilogue) for w in wls)
    R, S = rotation_plan(nbytes, nbytes / 2.5e6, args.steps)
    skip_steps = R + -(-args.warmup // S) * S
    total_steps = skip_steps + args.steps
    vals = collections.defaultdict(list)
    kname = {}
    counters = []
    flags = step_flags(args)
    cmds = []
    keys = set()
    for d in args.counters_from:
        files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        if len(files) != 1:
            raise SystemExit(f"expected one counter_collection.csv under {d}, found {files}")
        rows = [r for r in csv.DictReader(open(files[0]))
                if any(k in r["Kernel_Name"] for k in STEP_KERNELS + BW_KERNELS)]
        names = sorted({r["Counter_Name"] for r in rows})
        disp = sorted({int(r["Dispatch_Id"]) for r in rows})
        kpl = len(disp) // (total_steps * nl)  # kernels per layer and step
        if kpl < 1 or len(disp) != total_steps * nl * kpl:
            raise SystemExit(f"{d}: {len(disp)} step-kernel dispatches; expected {total_steps} x {nl} x k")
        keep = {dd: ((i // kpl) % nl, i % kpl) for i, dd in enumerate(disp) if i >= skip_steps * nl * kpl}
        for r in rows:
            dd = int(r["Dispatch_Id"])
            if dd in keep:
                vals[(keep[dd], r["Counter_Name"])].append(float(r["Counter_Value"]))
                kname[keep[dd]] = r["Kernel_Name"]
                keys.add(keep[dd])
        counters += [c for c in names if c not in counters]
        cmds.append(f"rocprofv3 --pmc {' '.join(names)} -d {d} -o run -f csv -- "
                    f"python3 bench.py {flags} --mode cold --steps {args.steps} --warmup {args.warmup}")
    tag = profile_tag(args)
    lines = [f"# Counters of the step kernel, cache-cold steps, {tag}", "", "Commands (one counter pass each):",
             "", "```", *cmds, f"python3 bench.py {flags} --counters-from {' '.join(args.counters_from)} "
             f"--steps {args.steps} --warmup {args.warmup}", "```", "",
             "Derived counters as rocprofv3 defines them: MfmaUtil = matrix-core busy cycles over all SIMDs / "
             "(GPU active cycles x SIMDs), in %; VALUBusy and LdsUtil likewise for the vector ALU and LDS; "
             "OccupancyPercent = resident waves over the CU's maximum; LDSBankConflict = conflict cycles per "
             "CU-cycle, in %.  Raw SQ_/TA_/TCP_ counters are sums over the dispatch.  Means over the timed "
             "dispatches.", "",
             "| layer | kernel | dispatches | " + " | ".join(counters) + " |",
             "|---|---|---|" + "---|" * len(counters)]
    for key in sorted(keys):
        n = len(vals[(key, counters[0])])
        cells = [f"{sum(vals[(key, c)]) / max(len(vals[(key, c)]), 1):.4g}" for c in counters]
        lines.append(f"| {wls[key[0]].name} | `{kname.get(key, '?')[:60]}` | {n} | " + " | ".join(cells) + " |")
    out = os.path.join(ROOT, "profiles", f"counters_{tag}.md")
    with open(out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def source_group(wl, op):
    """Which kernel sources the step of this workload and pass runs."""
    if op == "backward_weight":
        return "BW"
    if op == "regular":
        return "REG"
    return wl.group


def summarize_traffic(args, wls):
    """Calibrated HBM bytes per launch of the step kernel from two rocprofv3 --pmc runs
    of --mode traffic (FETCH_SIZE, then WRITE_SIZE; both count KiB per dispatch)."""
    wl = profile_tag(args)
    flags = step_flags(args)
    layers = wls
    res = {}
    for counter, d in zip(("FETCH_SIZE", "WRITE_SIZE"), args.traffic_from):
        rows = _counter_rows(d, counter)
        steps = [r for r in rows if any(k in r["Kernel_Name"] for k in STEP_KERNELS)]
        copies = [r for r in rows if "copy" in r["Kernel_Name"].lower() and int(r["Grid_Size"]) >= 65536]
        nl = len(layers)
        if len(steps) != (TRAFFIC_WARM + TRAFFIC_COLD) * nl or len(copies) < TRAFFIC_COPIES:
            raise SystemExit(f"{counter}: {len(steps)} step dispatches, {len(copies)} copies; "
                             f"expected {(TRAFFIC_WARM + TRAFFIC_COLD) * nl} and {TRAFFIC_COPIES}")
        kib = [float(r["Counter_Value"]) for r in steps]
        warm = sum(kib[:TRAFFIC_WARM * nl]) / TRAFFIC_WARM
        cold = sum(kib[TRAFFIC_WARM * nl:]) / TRAFFIC_COLD
        copy = sum(float(r["Counter_Value"]) for r in copies[-TRAFFIC_COPIES:]) / TRAFFIC_COPIES
        factor = TRAFFIC_COPY_BYTES / (copy * 1024.0)
        res[counter] = {"kib_warm": warm, "kib_cold": cold, "copy_kib": copy, "scale": factor,
                        "kernel": steps[0]["Kernel_Name"]}
    f, w = res["FETCH_SIZE"], res["WRITE_SIZE"]
    cold = f["kib_cold"] * 1024 * f["scale"] + w["kib_cold"] * 1024 * w["scale"]
    warm = f["kib_warm"] * 1024 * f["scale"] + w["kib_warm"] * 1024 * w["scale"]
    algo = sum(algorithmic_bytes(w, args.op, args.epilogue) for w in wls)
    group = source_group(wls[0], args.op)
    rec = {"workload": wl, "kernel": f["kernel"], "kernel_source_sha": kernel_source_hash(group),
           "hbm_bytes_per_launch": cold, "hbm_bytes_per_launch_warm": warm,
           "algorithmic_bytes_per_launch": algo, "traffic_over_algorithmic": cold / algo,
           "fetch": f, "write": w, "copy_bytes": TRAFFIC_COPY_BYTES,
           "command_fetch": f"rocprofv3 --pmc FETCH_SIZE -d {args.traffic_from[0]} -o run -f csv -- "
                            f"python3 bench.py {flags} --mode traffic",
           "command_write": f"rocprofv3 --pmc WRITE_SIZE -d {args.traffic_from[1]} -o run -f csv -- "
                            f"python3 bench.py {flags} --mode traffic",
           "command_summary": f"python3 bench.py {flags} --traffic-from "
                              f"{args.traffic_from[0]} {args.traffic_from[1]}"}
    with open(os.path.join(ROOT, "profiles", f"traffic_{wl}.json"), "w") as fh:
        json.dump(rec, fh, indent=1)
    md = [f"# HBM traffic of the step kernel, {wl}", "",
          f"Kernel: `{f['kernel']}`", "",
          "Commands (each counter in its own pass):", "",
          "```", rec["command_fetch"], rec["command_write"], rec["command_summary"], "```", "",
          f"`--mode traffic` launches {TRAFFIC_WARM} back-to-back steps, {TRAFFIC_COLD} steps "
          f"each after a 512 MiB read (L2s evicted, clean), then {TRAFFIC_COPIES} device copies of "
          f"{TRAFFIC_COPY_BYTES >> 20} MiB that calibrate the counters.", "",
          "| counter | KiB/launch warm | KiB/launch cold | copy KiB (expected "
          f"{TRAFFIC_COPY_BYTES >> 10}) | scale |", "|---|---|---|---|---|"]
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        r = res[c]
        md.append(f"| {c} | {r['kib_warm']:.1f} | {r['kib_cold']:.1f} | {r['copy_kib']:.1f} | {r['scale']:.4f} |")
    md += ["", f"Calibrated HBM bytes per launch: cold {cold:.0f}, warm {warm:.0f}; "
               f"algorithmic {algo} (x once, y once, w_hat once): cold/algorithmic = {cold / algo:.3f}.",
           f"Kernel source sha (the step kernel's sources): `{rec['kernel_source_sha']}`."]
    with open(os.path.join(ROOT, "profiles", f"traffic_{wl}.md"), "w") as fh:
        fh.write("\n".join(md) + "\n")
    print(json.dumps({"hbm_bytes_per_launch": cold, "algorithmic": algo, "ratio": cold / algo}))


def load_traffic(tag, group):
    p = os.path.join(ROOT, "profiles", f"traffic_{tag}.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        rec = json.load(f)
    if rec.get("kernel_source_sha") != kernel_source_hash(group):
        return None  # the kernel changed since the counters were taken
    return rec.get("hbm_bytes_per_launch")


class CopyStep:
    """A device copy of nbytes (half read, half written), with the rotation
    interface of Layer."""

    def __init__(self, nbytes):
        import torch
        self.src = torch.ones(max(nbytes // 8, 1), dtype=torch.float32, device="cuda")
        self.dst = torch.empty_like(self.src)
        self.rot, self.rot_dense = ("src", "dst"), ()

    def step(self):
        self.dst.copy_(self.src)

    make_copies = Layer.make_copies
    use = Layer.use


def precision_note(wl, kernel):
    """The arithmetic pipeline of the step kernel, stated with the line."""
    if wl.dtype == "f32":
        return {"io": "f32", "products": "fp32 x fp32 -> fp32 (matrix cores)",
                "transforms": "fp32 (VALU)"}
    io = wl.dtype
    if kernel == "cn_mf_kernel":
        return {"io": io, "products": f"{io} x {io} -> fp32 (matrix cores)",
                "forward_transform": f"on the matrix cores: {io} x, {io} DFT coefficients, fp32 out, "
                                     f"spectrum rounded to {io} for the products",
                "inverse_transform": f"on the matrix cores: the fp32 spectrum of y rounded to {io}, "
                                     f"{io} coefficients (1/N folded in), fp32 out, y rounded to {io} once"}
    if kernel == "dn_regular_kernel":
        return {"io": io, "products": f"{io} x {io} -> fp32 (matrix cores)",
                "transforms": f"group Fourier transform and its inverse in fp32 (VALU); the Fourier features of x "
                              f"rounded to {io} for the products; y rounded to {io} once"}
    if kernel in ("d8_kernel", "gemm_rows_kernel"):
        return {"io": io, "products": f"{io} x {io} -> fp32 (matrix cores)", "transforms": "none"}
    return {"io": io, "products": f"{io} x {io} -> fp32 (matrix cores)",
            "transforms": f"fp32 (VALU); spectrum of x rounded to {io} for the products, inverse in fp32"}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(tokens shard across GPUs with no exchange; see the sharding notes). "
              f"--gpus {args.gpus} is not supported.", file=sys.stderr)
        sys.exit(2)

    import synthetic
    names = ["c3a", "c3b", "c3c"] if args.workload == "c3" else [args.workload]
    wls = [synthetic.WORKLOADS[n] for n in names]
    if args.dtype != "workload":
        from dataclasses import replace
        wls = [replace(wl, dtype=args.dtype) for wl in wls]
    if args.traffic_from:
        summarize_traffic(args, wls)
        return
    if args.trace_from:
        summarize_trace(args, wls)
        return
    if args.counters_from:
        summarize_counters(args, wls)
        return

    import torch

    import group_equivariant_linear_amd as eq
    if not eq.built():
        from group_equivariant_linear_amd import _build
        _build.build()
    eq.load_library()
    torch.cuda.set_device(0)

    if args.epilogue != "none" and args.op not in ("forward", "regular"):
        print("--epilogue applies to the forward pass", file=sys.stderr)
        sys.exit(2)
    layers = [Layer(eq, wl, tile=args.tile, op=args.op, epilogue=args.epilogue) for wl in wls]
    torch.cuda.synchronize()
    for L in layers:
        assert L.bytes_per_launch == algorithmic_bytes(L.wl, args.op, args.epilogue)
    if args.mode == "traffic":
        traffic_run(layers)
        print(json.dumps({"copy_bytes": TRAFFIC_COPY_BYTES, "workload": args.workload}))
        return

    steps = [L.step for L in layers]
    bytes_launch = sum(L.bytes_per_launch for L in layers)
    tokens = wls[0].T
    est = lambda nbytes: nbytes / 2.5e6  # us at 2.5 TB/s, only to size the graphs
    # the timed region: K cache-cold steps
    ms, k_timed, R, S = rotation_timing(layers, "step", args.steps, args.warmup, bytes_launch, est(bytes_launch))
    kname = op_kernel_name(wls[0], args.op)
    group = wls[0].group
    achieved = bytes_launch / (ms * 1e-3) / 1e9
    cold = {"ms_per_step": ms, "steps_timed": k_timed, "copies": R, "steps_per_graph": S,
            "rotated_bytes": R * bytes_launch,
            "method": f"{R} copies of the per-token tensors used in rotation ({R * bytes_launch >> 20} MiB, "
                      f"over 3x the 256 MiB Infinity Cache), {S} step(s) per HIP graph, events around the region"}
    if args.mode == "cold":
        print(json.dumps({"workload": args.workload, "steps": k_timed, "warmup": args.warmup,
                          "ms_per_step": ms, "kernel": kname, "bytes_per_launch": bytes_launch,
                          "frac": achieved / HBM_PEAK_GBS, "mean_launch_us": ms * 1e3 / len(layers),
                          "cold": cold}))
        return
    if len(layers) > 1:
        cold["layers_ms"] = {L.wl.name: rotation_timing([L], "step", max(args.steps, 20), max(args.warmup, 2),
                                                        L.bytes_per_launch, est(L.bytes_per_launch))[0]
                             for L in layers}

    ms_eager = time_loop(steps, max(args.steps, 200), max(args.warmup, 20))
    ms_graph = time_graph(steps, [L.out for L in layers], max(args.steps, 200), max(args.warmup, 20))
    ms_warm = ms_graph if ms_graph is not None else ms_eager
    dsteps, dwarm = max(args.steps, 50), max(args.warmup, 5)
    has_own = all(L.dense_own is not None for L in layers)
    ms_own_eager = time_loop([L.dense_own for L in layers], dsteps, dwarm) if has_own else None
    ms_own_graph = (time_graph([L.dense_own for L in layers], [L.y_dense for L in layers], dsteps, dwarm)
                    if has_own else None)
    ms_lin_eager = time_loop([L.dense_torch for L in layers], dsteps, dwarm)
    ms_lin_graph = time_graph([L.dense_torch for L in layers], [L.y_lin for L in layers], dsteps, dwarm)
    # the dense comparators cache-cold, the same way as the step
    dense_bytes = sum(L.bytes_per_launch for L in layers)
    ms_lin_cold = rotation_timing(layers, "dense_torch", args.steps, args.warmup, dense_bytes, est(dense_bytes))[0]
    ms_own_cold = (rotation_timing(layers, "dense_own", args.steps, args.warmup, dense_bytes, est(dense_bytes))[0]
                   if has_own else None)
    ms_dense_cold = min(t for t in (ms_lin_cold, ms_own_cold) if t is not None)
    chain = None
    if all(hasattr(L, "chain") for L in layers):
        # the separate passes the one-launch path replaces, timed the same way
        ms_chain = rotation_timing(layers, "chain", args.steps, args.warmup, 3 * bytes_launch, est(3 * bytes_launch))[0]
        ms_chain_warm = time_graph([L.chain for L in layers], [L.y_chain for L in layers], dsteps, dwarm)
        chain = {"what": "eqlinear_d8_to_fourier + eqlinear_d8_forward + eqlinear_d8_bias_act + "
                         "eqlinear_d8_to_regular (four launches, the Fourier tensors through memory)",
                 "ms_cold": ms_chain, "ms_warm": ms_chain_warm, "speedup_cold": ms_chain / ms}
    # a device copy moving the same number of bytes (half read, half written): the
    # practical floor of a launch of this size, warm (graph) and cold (rotation)
    cp = CopyStep(bytes_launch)
    ms_copy = time_graph([cp.step], [cp.dst], dsteps, dwarm)
    if ms_copy is None:
        ms_copy = time_loop([cp.step], dsteps, dwarm)
    ms_copy_cold = rotation_timing([cp], "step", args.steps, args.warmup, bytes_launch, est(bytes_launch))[0]
    del cp
    for L in layers:
        L.use(0)
    own = [t for t in (ms_own_eager, ms_own_graph) if t is not None]
    ms_own = min(own) if own else None
    ms_lin = min(t for t in (ms_lin_eager, ms_lin_graph) if t is not None)
    # agreement of the fused path with the dense comparator on this very batch
    for L in layers:
        L.step()
        (L.dense_own if has_own else L.dense_torch)()
    torch.cuda.synchronize()
    if args.op == "backward_weight":
        # the dense gradient summed along its circulant diagonals is dw
        agree = max(_dense_grad_agreement(L) for L in layers)
    else:
        def ref(L):
            if not has_own:
                return L.y_lin.float()
            return L.post(L.y_dense) if L.post is not None else L.y_dense.float()
        agree = max(float(torch.linalg.vector_norm(L.out.float() - ref(L)) /
                          torch.linalg.vector_norm(ref(L))) for L in layers)

    flops = sum(2 * L.macs_per_token * L.wl.T for L in layers)
    dense_flops = sum(2 * L.dense_macs_per_token * L.wl.T for L in layers)
    dt = wls[0].dtype
    best_dense = min(t for t in (ms_own, ms_lin) if t is not None)

    same = args.tile == -1 and args.op in ("forward", "regular")
    traffic = load_traffic(profile_tag(args), source_group(wls[0], args.op)) if same else None
    out = {
        "metric": OP_METRIC[args.op],
        "value": tokens / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dt,
        "data": "synthetic",
        "config": {
            "workload": "; ".join(f"{wl.name}: {wl.note}, {'C' if wl.group == 'C' else ''}"
                                  f"{wl.N if wl.group == 'C' else 'D%d' % (wl.N // 2)} T={wl.T} "
                                  f"C_in={wl.C_in} C_out={wl.C_out} {wl.dtype}" for wl in wls),
            "tokens_per_step": tokens,
            "layers_per_step": len(layers),
            "tile": args.tile,
            "op": args.op,
            "epilogue": args.epilogue,
            "timing": "cache-cold: per-token tensors rotated through copies totalling over 3x the "
                      "Infinity Cache; HIP graphs replayed back to back, HIP events around the K steps",
        },
        "precision": precision_note(wls[0], kname.split(" ")[0]),
        "tflops_actual": flops / (ms * 1e-3) / 1e12,
        "tflops_dense_equiv": dense_flops / (ms * 1e-3) / 1e12,
        "mfma_frac": flops / (ms * 1e-3) / 1e12 / MFMA_PEAK_TFLOPS[dt],
        "cold": cold,
        "warm": {"ms_per_step": ms_warm, "ms_eager": ms_eager, "ms_graph": ms_graph,
                 "method": "graph" if ms_graph is not None else "eager",
                 "gbs": bytes_launch / (ms_warm * 1e-3) / 1e9,
                 "frac_hbm": bytes_launch / (ms_warm * 1e-3) / 1e9 / HBM_PEAK_GBS,
                 "note": "back-to-back steps: the inputs sit in the 256 MiB Infinity Cache"},
        "expanded_dense": {"ms_own_mfma": ms_own, "ms_torch_linear": ms_lin, "ms_best": best_dense,
                           "ms_own_eager": ms_own_eager, "ms_own_graph": ms_own_graph,
                           "ms_torch_eager": ms_lin_eager, "ms_torch_graph": ms_lin_graph,
                           "speedup_vs_best_warm": best_dense / ms_warm,
                           "ms_best_cold": ms_dense_cold, "speedup_vs_best_cold": ms_dense_cold / ms,
                           "expand_ms_once": sum(L.expand_ms for L in layers),
                           "agreement_rel_l2": agree},
        "chain_of_passes": chain,
        "copy_same_bytes": {"ms_warm": ms_copy, "ms_cold": ms_copy_cold,
                            "frac_hbm_cold": bytes_launch / (ms_copy_cold * 1e-3) / 1e9 / HBM_PEAK_GBS,
                            "frac_hbm_warm": bytes_launch / (ms_copy * 1e-3) / 1e9 / HBM_PEAK_GBS},
        "weight_fft_ms_once": [L.weight_fft_ms for L in layers],
        "roofline": {
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": traffic,
            "kernel": kname + (" + d8_pass_kernel" if group != "C" and args.epilogue != "none"
                               and args.op != "regular" else ""),
            "launches_per_step": len(layers),
            "mean_launch_us": ms * 1e3 / len(layers),
            "bytes_per_step": bytes_launch,
            "bytes_per_launch": [L.bytes_per_launch for L in layers],
            "timing": "cache-cold steps (rotated copies), HIP events on the launch stream around the K steps",
            "kernel_source_sha": kernel_source_hash(source_group(wls[0], args.op)),
        },
    }
    if args.cpu_seconds > 0:
        out["cpu_baseline"] = cpu_baseline(layers, args.cpu_seconds, args.op)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out))


if __name__ == "__main__":
    main()
