"""Shared helpers of the GPU parity tests: device upload/download and the
error metric.

Error metric: for every (b, h) slice of an output, max_i |x_i - r_i| /
max_i |r_i| (normwise relative error); the worst slice is reported.  An
elementwise |x - r| / |r| is unbounded where outputs cross zero, so it is
not used as the bar.  Bars: 1e-4 for fp32 activations, 2e-2 for bf16
activations with fp32 state (input rounding excluded: the oracle consumes
the rounded inputs; output rounding included).
"""

import numpy as np

TOL = {"f32": 1e-4, "bf16": 2e-2}


def torch_mod():
    import torch
    return torch


def dev():
    return "cuda:0"


def to_dev(x, dtype):
    """float32 numpy array (already rounded to `dtype`) -> device tensor."""
    torch = torch_mod()
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(dev())
    return t.to(torch.bfloat16) if dtype == "bf16" else t


def to_host(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def slice_err(x, r, lead=2):
    """Worst normwise relative error over the leading `lead` axes."""
    x = np.asarray(x, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    assert x.shape == r.shape, (x.shape, r.shape)
    if x.size == 0:
        return 0.0
    xs = x.reshape(int(np.prod(x.shape[:lead])), -1)
    rs = r.reshape(xs.shape)
    num = np.abs(xs - rs).max(axis=1)
    den = np.abs(rs).max(axis=1)
    den = np.where(den == 0, 1.0, den)
    return float((num / den).max())


def report(name, err, tol):
    print(f"[parity] {name}: worst slice rel err {err:.3e} (bar {tol:.0e})", flush=True)
    assert err <= tol, f"{name}: {err:.3e} > {tol:.0e}"
