"""GPU parity of packed variable-length batches with state snapshots for the
normalised, scalar-gated and KDA kinds (lin_attn_prefill_varlen, recurrent
form) against the fp64 oracle (oracle.varlen.packed_varlen), through the C
ABI: fp32 and bf16 activations, several head sizes, snapshots at several
intervals (z snapshots for the normalised kind), carried and in-place states,
empty and one-token sequences, a truncated snapshot buffer, an empty batch,
resuming a sequence from one of its snapshots with the uniform entry points
(prefix reuse), and a 16-sequence, 16-head, 16 384-token batch checked on
sampled heads; and the same cases for the block forms of every kind on the
matrix cores (form="chunked", bf16, d = 128, snapshots at whole 64-token
blocks), with sequences long enough to be cut into several segments.
"""

import numpy as np
import pytest

from oracle import varlen as ov
import synth
from gpu_helpers import TOL, report, slice_err, to_dev, to_host

pytestmark = pytest.mark.gpu

KINDS = ("normalized", "gated", "kda")
LENS = [1, 64, 130, 0, 1000, 63, 65, 300, 128]


@pytest.fixture(scope="module")
def gd():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_causal_amd as m
    m._load()
    return m


def inputs(kind, seed, lens, H, d, dtype, scale=1.0, states=True):
    q, k, v, a, b, cu = synth.varlen_kind_batch(seed, kind, lens, H, d, d, dtype, scale)
    S0 = z0 = None
    if states:
        S0 = synth.state_batch(seed + 1, len(lens), H, d, d, 0.05)
        z0 = synth.norm_batch(seed + 2, len(lens), H, d) if kind == "normalized" else None
    return q, k, v, a, b, cu, S0, z0


def run(gd, kind, q, k, v, a, b, cu, dtype, S0=None, z0=None, snap=0, inplace=False, snap_count=None):
    import torch
    tS = None if S0 is None else to_dev(S0, "f32")
    tz = None if z0 is None else to_dev(z0, "f32")
    tcu = torch.from_numpy(np.asarray(cu, np.int32)).to("cuda:0")
    opt = lambda x: None if x is None else to_dev(x, "f32")
    print(f"[case] {kind} {dtype} H={q.shape[0]} T={q.shape[1]} d={q.shape[2]} N={len(cu) - 1} snap={snap}",
          flush=True)
    o, S, z, sn, zsn = gd.lin_attn_prefill_varlen(kind, to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype), tcu,
                                                  opt(a), opt(b), tS, tz, snap_interval=snap, snap_count=snap_count,
                                                  S_out=tS if inplace else None, z_out=tz if inplace else None)
    h = lambda t: None if t is None else to_host(t)
    return h(o), h(S), h(z), h(sn), h(zsn)


def check(tag, got, ref, cu, dtype):
    o, S, z, sn, zsn = got
    o_r, S_r, z_r, sn_r, zsn_r = ref
    tol = TOL[dtype]
    worst = 0.0
    for n in range(len(cu) - 1):
        s, e = int(cu[n]), int(cu[n + 1])
        if e > s:
            worst = max(worst, slice_err(o[:, s:e], o_r[:, s:e], lead=1))
    report(f"{tag} o", worst, tol)
    report(f"{tag} S_out", slice_err(S, S_r), tol)
    if z_r is not None:
        report(f"{tag} z_out", slice_err(z, z_r), tol)
    if sn_r is not None and sn_r.shape[0] > 0:
        report(f"{tag} snapshots ({sn_r.shape[0]})", slice_err(sn, sn_r), tol)
        if zsn_r is not None:
            report(f"{tag} z snapshots", slice_err(zsn, zsn_r), tol)


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("dtype,d,snap,inplace", [("bf16", 128, 64, True), ("f32", 64, 7, False),
                                                  ("bf16", 32, 0, False), ("f32", 16, 50, True)])
def test_varlen_kind(gd, kind, dtype, d, snap, inplace):
    H = 3
    q, k, v, a, b, cu, S0, z0 = inputs(kind, 91, LENS, H, d, dtype)
    ref = ov.packed_varlen(kind, q, k, v, cu, a, b, S0, z0, snap_interval=snap)
    got = run(gd, kind, q, k, v, a, b, cu, dtype, S0, z0, snap=snap, inplace=inplace)
    check(f"varlen {kind} {dtype} d={d} snap={snap}", got, ref, cu, dtype)


@pytest.mark.parametrize("kind", KINDS)
def test_varlen_kind_truncated_snapshot_buffer(gd, kind):
    H, d = 2, 64
    q, k, v, a, b, cu, _, _ = inputs(kind, 93, LENS, H, d, "f32", states=False)
    *_, sn_r, zsn_r = ov.packed_varlen(kind, q, k, v, cu, a, b, snap_interval=64)
    *_, sn, zsn = run(gd, kind, q, k, v, a, b, cu, "f32", snap=64, snap_count=5)
    assert sn.shape[0] == 5
    report(f"varlen {kind} first 5 snapshots", slice_err(sn, sn_r[:5]), TOL["f32"])
    if zsn_r is not None:
        report(f"varlen {kind} first 5 z snapshots", slice_err(zsn, zsn_r[:5]), TOL["f32"])


@pytest.mark.parametrize("kind", KINDS)
def test_varlen_kind_empty_batch_passes_states(gd, kind):
    H, d = 2, 128
    cu = np.zeros(4, np.int32)
    q = np.zeros((H, 0, d), np.float32)
    a = None if kind == "normalized" else np.zeros((H, 0, d) if kind == "kda" else (H, 0), np.float32)
    b = np.zeros((H, 0), np.float32) if kind == "kda" else None
    S0 = synth.state_batch(95, 3, H, d, d, 0.05)
    z0 = synth.norm_batch(96, 3, H, d) if kind == "normalized" else None
    _, S, z, _, _ = run(gd, kind, q, q, q, a, b, cu, "bf16", S0, z0)
    assert np.array_equal(S, S0.astype(np.float64))
    if z0 is not None:
        assert np.array_equal(z, z0.astype(np.float64))


@pytest.mark.parametrize("kind", KINDS)
def test_varlen_kind_resume_from_snapshot(gd, kind):
    """Prefix reuse: a sequence continued from one of its snapshots with the
    kind's uniform entry point (recurrent form) gives the outputs and final
    state of the packed call."""
    import torch
    H, d, snap = 2, 128, 256
    lens = [700, 1100]
    q, k, v, a, b, cu, _, _ = inputs(kind, 97, lens, H, d, "bf16", states=False)
    o, S, z, sn, zsn = run(gd, kind, q, k, v, a, b, cu, "bf16", snap=snap)
    # sequence 1 resumed after its 4th snapshot (1024 tokens); its snapshots follow sequence 0's 2
    p, j = 1024, 2 + 3
    s0, e = int(cu[1]) + p, int(cu[2])
    up = lambda x: to_dev(np.ascontiguousarray(x[:, s0:e][None]), "bf16")
    Sj = torch.from_numpy(np.ascontiguousarray(sn[j][None], np.float32)).to("cuda:0")
    if kind == "normalized":
        zj = torch.from_numpy(np.ascontiguousarray(zsn[j][None], np.float32)).to("cuda:0")
        o_t, S_t, z_t = gd.lin_attn_prefill(up(q), up(k), up(v), Sj, zj, form="recurrent")
    elif kind == "gated":
        o_t, S_t = gd.gla_prefill(up(q), up(k), up(v), to_dev(np.ascontiguousarray(a[:, s0:e][None]), "f32"), Sj,
                                  form="recurrent")
    else:
        o_t, S_t = gd.kda_prefill(up(q), up(k), up(v), to_dev(np.ascontiguousarray(a[:, s0:e][None]), "f32"),
                                  to_dev(np.ascontiguousarray(b[:, s0:e][None]), "f32"), Sj, form="recurrent")
    report(f"resume {kind} o vs packed", slice_err(to_host(o_t)[0], o[:, s0:e], lead=1), TOL["bf16"])
    report(f"resume {kind} S vs packed", slice_err(to_host(S_t)[0], S[1]), TOL["bf16"])
    if kind == "normalized":
        report("resume normalized z vs packed", slice_err(to_host(z_t)[0][None], z[1][None]), TOL["bf16"])
    # and both agree with the oracle's sequence
    ref = ov.packed_varlen(kind, q, k, v, cu, a, b, snap_interval=snap)
    report(f"resume {kind} snapshot vs oracle", slice_err(sn[j][None], ref[3][j][None]), TOL["bf16"])
    report(f"resume {kind} o vs oracle", slice_err(to_host(o_t)[0], ref[0][:, s0:e], lead=1), TOL["bf16"])


@pytest.mark.timeout(600)
@pytest.mark.parametrize("kind", KINDS)
def test_varlen_kind_16_sequences(gd, kind):
    """16 sequences of mixed lengths, 16 heads, 16 384 tokens, d = 128, bf16,
    snapshots every 1024 tokens; heads 0, 7 and 15 checked against the oracle
    over every position, final state and snapshot."""
    H, d, snap = 16, 128, 1024
    lens = synth.varlen_lengths(98, 16, 16384)
    scale = 1 / np.sqrt(d) if kind == "normalized" else 1.0
    q, k, v, a, b, cu, S0, z0 = inputs(kind, 99, lens, H, d, "bf16", scale)
    got = run(gd, kind, q, k, v, a, b, cu, "bf16", S0, z0, snap=snap)
    hs = [0, 7, 15]
    sub = lambda x: None if x is None else x[hs]
    ref = ov.packed_varlen(kind, q[hs], k[hs], v[hs], cu, sub(a), sub(b), S0[:, hs],
                           None if z0 is None else z0[:, hs], snap_interval=snap)
    o, S, z, sn, zsn = got
    pick = (o[hs], S[:, hs], None if z is None else z[:, hs], sn[:, hs], None if zsn is None else zsn[:, hs])
    check(f"varlen {kind} 16 seq x 16 heads (heads 0, 7, 15)", pick, ref, cu, "bf16")


# ------------------------------------------------ KDA block form, packed batches
def run_chunked(gd, kind, q, k, v, a, b, cu, S0=None, z0=None, snap=0, snap_count=None, inplace=False):
    import torch
    tS = None if S0 is None else to_dev(S0, "f32")
    tz = None if z0 is None else to_dev(z0, "f32")
    tcu = torch.from_numpy(np.asarray(cu, np.int32)).to("cuda:0")
    opt = lambda x: None if x is None else to_dev(x, "f32")
    print(f"[case] {kind} chunked H={q.shape[0]} T={q.shape[1]} N={len(cu) - 1} snap={snap} inplace={inplace}",
          flush=True)
    o, S, z, sn, zsn = gd.lin_attn_prefill_varlen(kind, to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16"), tcu,
                                                  opt(a), opt(b), tS, tz, form="chunked", snap_interval=snap,
                                                  snap_count=snap_count, S_out=tS if inplace else None,
                                                  z_out=tz if inplace else None)
    h = lambda t: None if t is None else to_host(t)
    return h(o), h(S), h(z), h(sn), h(zsn)


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("snap,inplace", [(0, False), (64, True), (128, False)])
def test_varlen_chunked(gd, kind, snap, inplace):
    """The block forms on the matrix cores over a packed batch (normalised and
    scalar-gated: segment pass, combine, output pass; KDA: tile pass and
    column scan): empty, one-token and chunk-edge lengths, carried states,
    snapshots at whole 64-token blocks (z snapshots for the normalised kind)."""
    H, d = 2, 128
    q, k, v, a, b, cu, S0, z0 = inputs(kind, 101, LENS, H, d, "bf16")
    ref = ov.packed_varlen(kind, q, k, v, cu, a, b, S0, z0, snap_interval=snap)
    got = run_chunked(gd, kind, q, k, v, a, b, cu, S0, z0, snap=snap, inplace=inplace)
    check(f"varlen {kind} chunked snap={snap}", got, ref, cu, "bf16")


@pytest.mark.parametrize("kind", ("normalized", "gated"))
def test_varlen_chunked_many_segments(gd, kind):
    """Few heads and long sequences: each sequence is cut into several
    segments whose states are combined (one 8192-token sequence among short
    ones), snapshots every 512 tokens."""
    H, d = 1, 128
    lens = [8192, 5, 700, 0, 2049]
    q, k, v, a, b, cu, S0, z0 = inputs(kind, 111, lens, H, d, "bf16")
    ref = ov.packed_varlen(kind, q, k, v, cu, a, b, S0, z0, snap_interval=512)
    got = run_chunked(gd, kind, q, k, v, a, b, cu, S0, z0, snap=512, inplace=True)
    check(f"varlen {kind} chunked long sequences", got, ref, cu, "bf16")


def _resume(gd, kind, q, k, v, a, b, Sj, zj):
    """The uniform block-form entry point of the kind, one sequence."""
    if kind == "normalized":
        o, S, _ = gd.lin_attn_prefill(q, k, v, Sj, zj, form="chunked")
    elif kind == "gated":
        o, S = gd.gla_prefill(q, k, v, a, Sj, form="chunked")
    else:
        o, S = gd.kda_prefill(q, k, v, a, b, Sj, form="chunked")
    return o, S


@pytest.mark.parametrize("kind", KINDS)
def test_varlen_chunked_truncated_snapshots_and_resume(gd, kind):
    """Only the first 5 snapshots fit the buffer; a sequence resumed from one
    of its snapshots with the kind's uniform entry point (block form) gives
    the packed call's outputs and final state."""
    import torch
    H, d = 2, 128
    lens = [700, 1100]
    q, k, v, a, b, cu, _, _ = inputs(kind, 103, lens, H, d, "bf16", states=False)
    _, _, _, sn_r, zsn_r = ov.packed_varlen(kind, q, k, v, cu, a, b, snap_interval=256)
    _, _, _, sn5, zsn5 = run_chunked(gd, kind, q, k, v, a, b, cu, snap=256, snap_count=5)
    assert sn5.shape[0] == 5
    report(f"varlen {kind} chunked first 5 snapshots", slice_err(sn5, sn_r[:5]), TOL["bf16"])
    if zsn_r is not None:
        report(f"varlen {kind} chunked first 5 z snapshots", slice_err(zsn5, zsn_r[:5]), TOL["bf16"])
    o, S, _, sn, zsn = run_chunked(gd, kind, q, k, v, a, b, cu, snap=256)
    p, j = 1024, 2 + 3
    s0, e = int(cu[1]) + p, int(cu[2])
    up = lambda x, dt: None if x is None else to_dev(np.ascontiguousarray(x[:, s0:e][None]), dt)
    st = lambda x: None if x is None else torch.from_numpy(np.ascontiguousarray(x[j][None], np.float32)).to("cuda:0")
    o_t, S_t = _resume(gd, kind, up(q, "bf16"), up(k, "bf16"), up(v, "bf16"), up(a, "f32"), up(b, "f32"), st(sn),
                       st(zsn))
    report(f"resume {kind} chunked o vs packed", slice_err(to_host(o_t)[0], o[:, s0:e], lead=1), TOL["bf16"])
    report(f"resume {kind} chunked S vs packed", slice_err(to_host(S_t)[0], S[1]), TOL["bf16"])


@pytest.mark.timeout(600)
@pytest.mark.parametrize("kind,form", [("normalized", "chunked"), ("kda", "chunked"), ("gated", "recurrent")])
def test_varlen_kind_thousands_of_sequences(gd, kind, form):
    """2500 sequences, most a few chunks long, every 97th empty: the
    longest-first order of segments (block form of the normalised kind),
    of sequences (KDA's column scan, the recurrent form), against the oracle."""
    H, d = 2, 128
    lens = synth.varlen_lengths(91, 2500, 30000)
    moved = int(lens[::97].sum())
    lens[::97] = 0
    lens[-1] += moved
    q, k, v, a, b, cu, S0, z0 = inputs(kind, 93, lens, H, d, "bf16")
    ref = ov.packed_varlen(kind, q, k, v, cu, a, b, S0, z0, snap_interval=128)
    if form == "chunked":
        got = run_chunked(gd, kind, q, k, v, a, b, cu, S0, z0, snap=128)
    else:
        got = run(gd, kind, q, k, v, a, b, cu, "bf16", S0, z0, snap=128)
    check(f"varlen {kind} {form} 2500 sequences", got, ref, cu, "bf16")


@pytest.mark.timeout(600)
@pytest.mark.parametrize("kind", KINDS)
def test_varlen_chunked_16_sequences(gd, kind):
    """16 sequences of mixed lengths, 16 heads, 16 384 tokens, snapshots every
    1024 tokens; heads 0, 7 and 15 checked against the oracle."""
    H, d, snap = 16, 128, 1024
    lens = synth.varlen_lengths(98, 16, 16384)
    q, k, v, a, b, cu, S0, z0 = inputs(kind, 105, lens, H, d, "bf16")
    o, S, z, sn, zsn = run_chunked(gd, kind, q, k, v, a, b, cu, S0, z0, snap=snap)
    hs = [0, 7, 15]
    pick = lambda x: None if x is None else x[hs]
    pick2 = lambda x: None if x is None else x[:, hs]
    ref = ov.packed_varlen(kind, q[hs], k[hs], v[hs], cu, pick(a), pick(b), S0[:, hs], pick2(z0), snap_interval=snap)
    check(f"varlen {kind} chunked 16 seq x 16 heads (heads 0, 7, 15)",
          (o[hs], S[:, hs], pick2(z), pick2(sn), pick2(zsn)), ref, cu, "bf16")
