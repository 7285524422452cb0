"""GPU parity of the fused pre-operations of a Gated DeltaNet layer (causal
depthwise convolution with kernel 4, per-head L2 normalisation of q and k,
sigmoid gates, token-major to head-major layout) against the fp64 oracle,
through the C ABI: fp32 and bf16, every head size, ragged token counts (one
token, fewer than the three history rows, several tiles and a short last
one), with and without a carried conv state, resuming a split sequence,
zero rows, T = 0, the 2 x 16 x 8192 workload on sampled windows, and the
pre-operations feeding the gated-delta prefill.

Bar, elementwise: |gpu - ref| <= rtol |ref| + atol * max|ref row|, with
rtol = 1e-5 for fp32 outputs and 2^-8 + 1e-5 for bf16 outputs (the kernel
rounds its fp32 result once to bf16: at most half an ulp, i.e. 2^-8 of the
value), atol = 1e-5 (fp32 rounding of a 4-term sum and of the norm, relative
to the row's size); gates |gpu - ref| <= 1e-6.
"""

import numpy as np
import pytest

from oracle import preops as op
from oracle import batched as ob
import synth
from gpu_helpers import TOL, report, slice_err, to_dev, to_host

pytestmark = pytest.mark.gpu
RTOL = {"f32": 1e-5, "bf16": 2.0 ** -8 + 1e-5}
ATOL_ROW = 1e-5


@pytest.fixture(scope="module")
def gd():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_causal_amd as m
    m._load()
    return m


def check(name, x, r, rtol, atol_row=ATOL_ROW):
    x = np.asarray(x, np.float64)
    r = np.asarray(r, np.float64)
    assert x.shape == r.shape, (name, x.shape, r.shape)
    if r.size == 0:
        return
    assert np.all(np.isfinite(x)), name
    rowmax = np.abs(r).max(axis=-1, keepdims=True)
    bound = rtol * np.abs(r) + atol_row * rowmax
    excess = np.abs(x - r) - bound
    worst = float(np.max(np.abs(x - r) / np.where(np.abs(r) > 0, np.abs(r), 1.0)))
    print(f"[parity] {name}: max excess over bound {excess.max():.3e}, worst elementwise rel {worst:.3e}", flush=True)
    assert excess.max() <= 0, f"{name}: {int((excess > 0).sum())} elements beyond the bound"


def oracle_batch(x, w, a, bl, H, dk, dv, st):
    """The oracle per sequence, stacked: q, k, v, alpha, beta, new state."""
    outs = [op.gdn_preprocess(x[b], w, a[b], bl[b], H, dk, dv, None if st is None else st[b])
            for b in range(x.shape[0])]
    return [np.stack([o[i] for o in outs]) for i in range(6)]


def run(gd, x, w, a, bl, H, dk, dv, dtype, st=None, want_state=True):
    tst = None if st is None else to_dev(st, dtype)
    res = gd.gdn_preprocess(to_dev(x, dtype), to_dev(w, "f32"), to_dev(a, "f32"), to_dev(bl, "f32"), H, dk, dv,
                            conv_state=tst, want_state=want_state)
    return [None if t is None else to_host(t) for t in res]


def compare(tag, got, ref, dtype):
    names = ("q", "k", "v", "alpha", "beta", "conv_state")
    for n, g, r in zip(names, got, ref):
        if g is None:
            continue
        if n in ("alpha", "beta"):
            err = float(np.abs(g - r).max()) if r.size else 0.0
            print(f"[parity] {tag} {n}: max abs err {err:.3e} (bar 1e-06)", flush=True)
            assert err <= 1e-6, (tag, n, err)
        elif n == "conv_state":
            # a copy of input rows: bit-exact
            assert np.array_equal(g, r), f"{tag} conv_state differs"
        else:
            check(f"{tag} {n}", g, r, RTOL[dtype])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("B,T,H,dk,dv,with_state", [
    (2, 130, 3, 16, 32, True), (1, 64, 2, 128, 128, False), (2, 200, 2, 64, 16, True), (1, 5, 4, 32, 128, True),
    (3, 1, 2, 128, 64, True), (2, 2, 2, 16, 16, True), (1, 2, 3, 64, 64, False), (1, 1000, 2, 128, 128, True)])
def test_preprocess_matches_oracle(gd, dtype, B, T, H, dk, dv, with_state):
    x, w, a, bl = synth.preops_batch(61, B, T, H, dk, dv, dtype)
    st = synth.conv_state_batch(62, B, H, dk, dv, dtype) if with_state else None
    ref = oracle_batch(x, w, a, bl, H, dk, dv, st)
    got = run(gd, x, w, a, bl, H, dk, dv, dtype, st)
    compare(f"preops {dtype} B={B} T={T} H={H} dk={dk} dv={dv} state={with_state}", got, ref, dtype)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_split_sequence_resumes_bitwise(gd, dtype):
    """Two calls chained through the conv state give the same bits as one
    call over the whole sequence (cuts inside a tile, at a tile edge and
    fewer than three tokens from the start)."""
    B, T, H, dk, dv = 2, 300, 2, 128, 64
    x, w, a, bl = synth.preops_batch(63, B, T, H, dk, dv, dtype)
    whole = run(gd, x, w, a, bl, H, dk, dv, dtype)
    for cut in (2, 64, 100):
        first = run(gd, x[:, :cut], w, a[:, :cut], bl[:, :cut], H, dk, dv, dtype)
        second = run(gd, x[:, cut:], w, a[:, cut:], bl[:, cut:], H, dk, dv, dtype, st=first[5])
        for i in range(5):
            joined = np.concatenate([first[i], second[i]], axis=2)
            assert np.array_equal(joined, whole[i]), (cut, i)
        assert np.array_equal(second[5], whole[5]), cut


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_zero_rows_stay_zero(gd, dtype):
    """A q (or k) block that is zero over a token and the three before it
    convolves to zero and stays zero under the normalisation (no NaN)."""
    B, T, H, dk, dv = 1, 100, 2, 64, 64
    x, w, a, bl = synth.preops_batch(64, B, T, H, dk, dv, dtype)
    x[0, 20:30, 0:dk] = 0.0                         # head 0's q channels
    x[0, 50:60, H * dk + dk:H * dk + 2 * dk] = 0.0  # head 1's k channels
    ref = oracle_batch(x, w, a, bl, H, dk, dv, None)
    got = run(gd, x, w, a, bl, H, dk, dv, dtype)
    assert np.all(got[0][0, 0, 23:30] == 0.0) and np.all(got[1][0, 1, 53:60] == 0.0)
    assert np.all(ref[0][0, 0, 23:30] == 0.0)
    compare(f"preops zero rows {dtype}", got, ref, dtype)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_empty_sequence_copies_the_state(gd, dtype):
    import torch
    B, H, dk, dv = 2, 3, 32, 16
    C = H * (2 * dk + dv)
    st = synth.conv_state_batch(65, B, H, dk, dv, dtype)
    x = np.zeros((B, 0, C), np.float32)
    w = np.ones((C, 4), np.float32)
    a = np.zeros((B, 0, H), np.float32)
    got = run(gd, x, w, a, a, H, dk, dv, dtype, st)
    assert got[0].shape == (B, H, 0, dk)
    assert np.array_equal(got[5], st)
    got = run(gd, x, w, a, a, H, dk, dv, dtype, None)
    assert np.array_equal(got[5], np.zeros_like(st))
    torch.cuda.synchronize()


def test_workload_2x16x8192_sampled(gd):
    """The bench workload: every output on the GPU, checked against the oracle
    on token windows at the start, across tile edges and at the end of every
    sequence (the oracle gets the window and, as carried state, the three
    tokens before it)."""
    wl = synth.WORKLOADS["preops_bf16_2x16x8192"]
    B, T, H, dk, dv, dtype = wl["B"], wl["T"], wl["H"], wl["dk"], wl["dv"], wl["dtype"]
    x, w, a, bl = synth.preops_batch(wl["seed"], B, T, H, dk, dv, dtype)
    got = run(gd, x, w, a, bl, H, dk, dv, dtype)
    for s0, n in ((0, 70), (4030, 100), (T - 67, 67)):
        st = None if s0 == 0 else x[:, s0 - 3:s0]
        ref = oracle_batch(x[:, s0:s0 + n], w, a[:, s0:s0 + n], bl[:, s0:s0 + n], H, dk, dv, st)
        sub = [g[:, :, s0:s0 + n] for g in got[:5]]
        compare(f"preops workload window {s0}+{n}", sub + [None], ref, dtype)
    assert np.array_equal(got[5], x[:, T - 3:])


def test_preops_feed_the_gated_delta_prefill(gd):
    """Pre-operations then the chunked gated-delta prefill, against the
    oracle's pre-operations then its gated-delta recurrence (bf16, d = 128)."""
    B, T, H, d = 1, 300, 2, 128
    x, w, a, bl = synth.preops_batch(66, B, T, H, d, d, "bf16")
    q, k, v, al, be, _ = gd.gdn_preprocess(to_dev(x, "bf16"), to_dev(w, "f32"), to_dev(a, "f32"),
                                           to_dev(bl, "f32"), H, d, d, want_state=False)
    o, S = gd.gdn_prefill(q, k, v, al, be, form="chunked", chunk=64)
    rq, rk, rv, ra, rb, _ = oracle_batch(x, w, a, bl, H, d, d, None)
    # the oracle recurrence runs on the GPU's bf16-rounded q, k, v (the rounding is the I/O contract)
    hq, hk, hv = to_host(q), to_host(k), to_host(v)
    for name, g, r in (("q", hq, rq), ("k", hk, rk), ("v", hv, rv)):
        check(f"chained {name}", g, r, RTOL["bf16"])
    o_ref, S_ref = ob.gdn(hq, hk, hv, to_host(al), to_host(be), form="recurrent")
    report("preops -> gdn_prefill o", slice_err(to_host(o), o_ref), TOL["bf16"])
    report("  S", slice_err(to_host(S), S_ref), TOL["bf16"])


# ------------------------------------------------------------- packed batches
def run_varlen(gd, x, w, a, bl, H, dk, dv, cu, dtype, st=None):
    import torch
    tst = None if st is None else to_dev(st, dtype)
    tcu = torch.from_numpy(np.asarray(cu, np.int32)).to("cuda:0")
    res = gd.gdn_preprocess_varlen(to_dev(x, dtype), to_dev(w, "f32"), to_dev(a, "f32"), to_dev(bl, "f32"), H, dk, dv,
                                   tcu, conv_state=tst)
    return [to_host(t) for t in res]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("lens,H,dk,dv,with_state", [
    ([5, 0, 2, 130, 1, 300], 2, 128, 128, True), ([64, 64, 129], 3, 64, 32, False),
    ([1, 1, 1, 3, 200], 2, 16, 64, True), ([1000], 2, 128, 128, True)])
def test_preprocess_varlen_matches_oracle(gd, dtype, lens, H, dk, dv, with_state):
    C = H * (2 * dk + dv)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu[-1])
    x, w, a, bl = synth.preops_batch(67, 1, T, H, dk, dv, dtype)
    x, a, bl = x[0], a[0], bl[0]
    st = synth.conv_state_batch(68, len(lens), H, dk, dv, dtype) if with_state else None
    ref = op.gdn_preprocess_varlen(x, w, a, bl, H, dk, dv, cu, st)
    got = run_varlen(gd, x, w, a, bl, H, dk, dv, cu, dtype, st)
    # outputs [H, T, d] (rows per head), gates [H, T], states bit-exact
    compare(f"preops varlen {dtype} lens={lens} H={H} dk={dk} dv={dv}", [g[None] for g in got[:5]] + [got[5]],
            [r[None] for r in ref[:5]] + [ref[5]], dtype)
    assert C == x.shape[1]


def test_preprocess_varlen_feeds_the_packed_prefill(gd):
    """Packed pre-operations then the packed chunked prefill, against the
    oracle's pre-operations then its packed recurrence."""
    import torch
    from oracle import varlen as ov
    H, d = 2, 128
    lens = [300, 70, 0, 500]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu[-1])
    x, w, a, bl = synth.preops_batch(69, 1, T, H, d, d, "bf16")
    tcu = torch.from_numpy(cu).to("cuda:0")
    q, k, v, al, be, _ = gd.gdn_preprocess_varlen(to_dev(x[0], "bf16"), to_dev(w, "f32"), to_dev(a[0], "f32"),
                                                  to_dev(bl[0], "f32"), H, d, d, tcu, want_state=False)
    o, S, _ = gd.gdn_prefill_varlen(q, k, v, al, be, tcu, form="chunked")
    hq, hk, hv, ha, hb = to_host(q), to_host(k), to_host(v), to_host(al), to_host(be)
    rq, rk, rv, ra, rb, _ = op.gdn_preprocess_varlen(x[0], w, a[0], bl[0], H, d, d, cu)
    for name, g, r in (("q", hq, rq), ("k", hk, rk), ("v", hv, rv)):
        check(f"packed chain {name}", g[None], r[None], RTOL["bf16"])
    o_ref, S_ref, _ = ov.gdn_varlen(hq, hk, hv, ha, hb, cu, form="chunked")
    report("packed preops -> gdn_prefill_varlen o", slice_err(to_host(o), o_ref, lead=1), TOL["bf16"])
    report("  S", slice_err(to_host(S), S_ref), TOL["bf16"])
