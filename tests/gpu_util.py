"""Helpers for the GPU tests: device transfer, guarded output buffers and error metrics."""
import numpy as np

import synthetic

GUARD = 64  # elements of sentinel on each side of an output buffer
SENTINEL_F32 = np.float32(-12345.5)
SENTINEL_BF16_BITS = np.int16(0x7F7F)  # a large finite bf16


def torch_dtype(dt):
    import torch
    return {synthetic.F32: torch.float32, synthetic.BF16: torch.bfloat16, synthetic.F16: torch.float16}[dt]


def to_dev(a, dt):
    import torch
    if dt == synthetic.F32:
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch_dtype(dt)).cuda()


def to_f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


class Guarded:
    """An output tensor with sentinel elements on both sides (detects stray writes)."""

    def __init__(self, n, dt, shape=None):
        import torch
        self.n, self.dt = n, dt
        self.buf = torch.empty(n + 2 * GUARD, dtype=torch_dtype(dt), device="cuda")
        if dt == synthetic.F32:
            self.buf.fill_(float(SENTINEL_F32))
        else:
            self.buf.view(torch.int16).fill_(int(SENTINEL_BF16_BITS))
        self.t = self.buf[GUARD:GUARD + n]
        if shape is not None:
            self.t = self.t.view(*shape)

    def check_guards(self):
        import torch
        if self.dt == synthetic.F32:
            g = torch.cat([self.buf[:GUARD], self.buf[-GUARD:]]).cpu().numpy()
            assert np.all(g == SENTINEL_F32), "write outside the output tensor"
        else:
            g = torch.cat([self.buf[:GUARD], self.buf[-GUARD:]]).view(torch.int16).cpu().numpy()
            assert np.all(g == SENTINEL_BF16_BITS), "write outside the output tensor"


def rel_l2(a, b):
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def max_err_over_rms(a, b):
    rms = np.sqrt(np.mean(b * b))
    return float(np.max(np.abs(a - b)) / max(rms, 1e-300))


# rel-L2 bars for the whole output; the max-error bar (relative to the output's
# RMS) catches a localised mistake that a whole-tensor norm would dilute.
# fp16: the bf16 bars scaled by the ratio of the unit roundoffs, 2^-11 / 2^-8
BARS = {synthetic.F32: (1e-5, 2e-4), synthetic.BF16: (2e-2, 1e-1), synthetic.F16: (2.5e-3, 1.25e-2)}


def assert_close(y, ref, dt, what=""):
    r, m = rel_l2(y, ref), max_err_over_rms(y, ref)
    bar, mbar = BARS[dt]
    assert np.all(np.isfinite(y)), f"{what}: non-finite output"
    assert r <= bar and m <= mbar, f"{what}: rel-L2 {r:.3e} (bar {bar:g}), max/rms {m:.3e} (bar {mbar:g})"
    return r, m
