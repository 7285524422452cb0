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


_median = {"value": float("nan")}


def slice_err(x, r, lead=2):
    """Worst normwise relative error over the leading `lead` axes.  Also
    keeps, for the next report(), the median elementwise relative error over
    the entries whose reference is at least 1e-3 of its slice's largest (an
    elementwise ratio is unbounded where outputs cross zero, so it is logged,
    not used as the bar)."""
    x = np.asarray(x, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    assert x.shape == r.shape, (x.shape, r.shape)
    if x.size == 0:
        _median["value"] = 0.0
        return 0.0
    xs = x.reshape(int(np.prod(x.shape[:lead])), -1)
    rs = r.reshape(xs.shape)
    diff = np.abs(xs - rs)
    num = diff.max(axis=1)
    den = np.abs(rs).max(axis=1)
    big = (np.abs(rs) >= 1e-3 * den[:, None]) & (np.abs(rs) > 0)
    _median["value"] = float(np.median(diff[big] / np.abs(rs[big]))) if big.any() else 0.0
    den = np.where(den == 0, 1.0, den)
    return float((num / den).max())


def report(name, err, tol):
    print(f"[parity] {name}: worst slice rel err {err:.3e} (bar {tol:.0e}); median elementwise rel err "
          f"{_median['value']:.1e}", flush=True)
    _median["value"] = float("nan")
    assert err <= tol, f"{name}: {err:.3e} > {tol:.0e}"


def long_head_inputs(seed, h, T, d):
    """Inputs of head h of a 1 x H x T gated-delta workload, as the device
    wants them: q, k, v as bf16 bit patterns (uint16), alpha and beta float32.
    Runs in a worker process (no GPU, no torch)."""
    import synth
    q, k, v, a, b = synth.gdn_head(seed, 0, h, T, d, d, "bf16")
    bits = [np.ascontiguousarray(x).view(np.uint32) >> 16 for x in (q, k, v)]
    return h, [x.astype(np.uint16) for x in bits], a, b


def long_head_check(seed, h, T, d, C, o_gpu, S_gpu):
    """Oracle check of head h of a 1 x H x T gated-delta workload in a worker
    process: regenerate the head's inputs, run the fp64 chunked oracle over all
    T tokens, and return the normwise errors of every output position, of the
    seeded sample of positions, and of the final state."""
    from threadpoolctl import threadpool_limits

    import oracle
    import synth
    with threadpool_limits(limits=2):
        q, k, v, a, b = synth.gdn_head(seed, 0, h, T, d, d, "bf16")
        o_ref, S_ref = oracle.gdn_chunked(q, k, v, a, b, C)
    o_gpu = np.asarray(o_gpu, dtype=np.float64)
    err_all = slice_err(o_gpu[None], o_ref[None], 1)
    pos = long_sample_positions(seed, h, T, C)
    err_pos = slice_err(o_gpu[pos][None], o_ref[pos][None], 1)
    err_S = slice_err(np.asarray(S_gpu, dtype=np.float64)[None], S_ref[None], 1)
    return h, err_all, err_pos, err_S, len(pos)


def long_sample_positions(seed, h, T, C, n=4096, boundaries=32):
    """A seeded sample of output positions of one head: n uniform positions,
    the whole first and last chunk, and the first and last row of `boundaries`
    seeded chunk boundaries."""
    rng = np.random.default_rng([int(seed), 99, int(h)])
    nc = (T + C - 1) // C
    pos = set(rng.integers(0, T, size=n).tolist())
    pos.update(range(0, min(C, T)))
    pos.update(range((nc - 1) * C, T))
    for c in rng.integers(1, nc, size=boundaries).tolist():
        pos.update((c * C - 1, c * C))
    return np.array(sorted(p for p in pos if 0 <= p < T), dtype=np.int64)


def decode_step_inputs(seed, N, H, dk, dv, step):
    """Token inputs of one decode step (synth.decode_token_inputs, entry =
    step) as the device wants them: q, k, v as bf16 bit patterns (uint16),
    alpha and beta float32.  Runs in a worker process (no GPU, no torch)."""
    import synth
    q, k, v, a, b = synth.decode_token_inputs(seed, N, H, dk, dv, "bf16", step)
    bits = [(np.ascontiguousarray(x).view(np.uint32) >> 16).astype(np.uint16) for x in (q, k, v)]
    return step, bits, a, b


def bf16_bits_to_f32(bits):
    """uint16 bf16 bit patterns -> float32 values."""
    return (np.asarray(bits, dtype=np.uint32) << 16).view(np.float32)
