"""GPU parity of the gated delta rule over packed batches of sequences of
different lengths, with state snapshots, against the fp64 oracle
(oracle.varlen), through the C ABI: the matrix-core chunked path (bf16,
d = 128, chunk 64) and the recurrent path (fp32 and bf16, any head size,
snapshots at any interval); empty sequences, one-token sequences, lengths
around chunk edges, carried and in-place states, a truncated snapshot
buffer, many sequences (up to 2500, more than the plan kernel's threads), an
empty batch, resuming a sequence from one of its snapshots with gdn_prefill
(prefix reuse), and the 16-sequence workload on every sequence and head.
"""

import numpy as np
import pytest

from oracle import varlen as ov
import synth
from gpu_helpers import TOL, report, slice_err, to_dev, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gd():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_causal_amd as m
    m._load()
    return m


def run(gd, q, k, v, a, b, cu, dtype, S0=None, snap=0, form="chunked", inplace=False, snap_count=None):
    import torch
    tS = None if S0 is None else to_dev(S0, "f32")
    tcu = torch.from_numpy(np.asarray(cu, np.int32)).to("cuda:0")
    o, S, sn = gd.gdn_prefill_varlen(to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype), to_dev(a, "f32"),
                                     to_dev(b, "f32"), tcu, tS, form=form, snap_interval=snap,
                                     snap_count=snap_count, S_out=tS if inplace else None)
    return to_host(o), to_host(S), (None if sn is None else to_host(sn))


def check(tag, got, ref, cu, dtype):
    o, S, sn = got
    o_r, S_r, sn_r = ref
    tol = TOL[dtype]
    # outputs per (sequence, head) slice
    worst = 0.0
    for n in range(len(cu) - 1):
        s, e = int(cu[n]), int(cu[n + 1])
        if e > s:
            worst = max(worst, slice_err(o[:, s:e], o_r[:, s:e], lead=1))
    report(f"{tag} o", worst, tol)
    report(f"{tag} S_out", slice_err(S, S_r), tol)
    if sn_r is not None and sn_r.shape[0] > 0:
        report(f"{tag} snapshots ({sn_r.shape[0]})", slice_err(sn, sn_r), tol)


LENS = [1, 64, 130, 0, 1000, 63, 65, 300, 128]


@pytest.mark.parametrize("snap", [0, 64, 128])
def test_varlen_chunked(gd, snap):
    H, d = 2, 128
    q, k, v, a, b, cu = synth.varlen_batch(81, LENS, H, d, d, "bf16")
    S0 = synth.state_batch(82, len(LENS), H, d, d, 0.05)
    ref = ov.gdn_varlen(q, k, v, a, b, cu, S0, snap_interval=snap, form="chunked")
    got = run(gd, q, k, v, a, b, cu, "bf16", S0, snap=snap, inplace=True)
    check(f"varlen chunked snap={snap}", got, ref, cu, "bf16")


@pytest.mark.parametrize("dtype,d,snap", [("f32", 64, 7), ("f32", 16, 0), ("bf16", 128, 50), ("f32", 128, 64)])
def test_varlen_recurrent(gd, dtype, d, snap):
    H = 3
    q, k, v, a, b, cu = synth.varlen_batch(83, LENS, H, d, d, dtype)
    S0 = synth.state_batch(84, len(LENS), H, d, d, 0.05)
    ref = ov.gdn_varlen(q, k, v, a, b, cu, S0, snap_interval=snap, form="chunked")
    got = run(gd, q, k, v, a, b, cu, dtype, S0, snap=snap, form="recurrent")
    check(f"varlen recurrent {dtype} d={d} snap={snap}", got, ref, cu, dtype)


def test_varlen_many_sequences(gd):
    """64 sequences, several segments for the long ones, no initial state."""
    H, d = 4, 128
    lens = synth.varlen_lengths(85, 64, 20000)
    q, k, v, a, b, cu = synth.varlen_batch(86, lens, H, d, d, "bf16")
    ref = ov.gdn_varlen(q, k, v, a, b, cu, None, snap_interval=256, form="chunked")
    got = run(gd, q, k, v, a, b, cu, "bf16", None, snap=256)
    check("varlen 64 sequences", got, ref, cu, "bf16")


def _many_short_lengths(seed, N, total):
    """N lengths summing to total, every 97th sequence empty (its tokens moved
    to the last one)."""
    lens = synth.varlen_lengths(seed, N, total)
    moved = int(lens[::97].sum())
    lens[::97] = 0
    lens[-1] += moved
    return lens


@pytest.mark.timeout(600)
@pytest.mark.parametrize("form", ["chunked", "recurrent"])
def test_varlen_thousands_of_sequences(gd, form):
    """2500 sequences (more than one per plan-kernel thread), most a few
    chunks long, some empty: the device-built tables, the longest-first
    order of segments and sequences, and every sequence's output and state
    against the oracle."""
    H, d = 2, 128
    lens = _many_short_lengths(87, 2500, 60000)
    q, k, v, a, b, cu = synth.varlen_batch(88, lens, H, d, d, "bf16")
    S0 = synth.state_batch(89, len(lens), H, d, d, 0.05)
    ref = ov.gdn_varlen(q, k, v, a, b, cu, S0, snap_interval=128, form="chunked")
    got = run(gd, q, k, v, a, b, cu, "bf16", S0, snap=128, form=form)
    check(f"varlen 2500 sequences ({form})", got, ref, cu, "bf16")


def test_varlen_truncated_snapshot_buffer(gd):
    H, d = 2, 128
    q, k, v, a, b, cu = synth.varlen_batch(87, LENS, H, d, d, "bf16")
    _, _, sn_r = ov.gdn_varlen(q, k, v, a, b, cu, None, snap_interval=64, form="chunked")
    _, _, sn = run(gd, q, k, v, a, b, cu, "bf16", None, snap=64, snap_count=5)
    assert sn.shape[0] == 5
    report("varlen first 5 snapshots", slice_err(sn, sn_r[:5]), TOL["bf16"])


def test_varlen_empty_batch_passes_states(gd):
    H, d = 2, 128
    cu = np.zeros(4, np.int32)
    q = np.zeros((H, 0, d), np.float32)
    a = np.zeros((H, 0), np.float32)
    S0 = synth.state_batch(88, 3, H, d, d, 0.05)
    for form in ("chunked", "recurrent"):
        _, S, _ = run(gd, q, q, q, a, a, cu, "bf16", S0, form=form)
        assert np.array_equal(S, S0.astype(np.float64)), form


def test_resume_from_snapshot(gd):
    """Prefix reuse: a sequence continued from one of its snapshots with
    gdn_prefill gives the outputs and final state of the packed call."""
    import torch
    H, d, snap = 2, 128, 256
    lens = [700, 1100]
    q, k, v, a, b, cu = synth.varlen_batch(89, lens, H, d, d, "bf16")
    o, S, sn = run(gd, q, k, v, a, b, cu, "bf16", None, snap=snap)
    # sequence 1, resumed after its 4th snapshot (1024 tokens); its snapshots start after sequence 0's 2
    p, j = 1024, 2 + 3
    s0 = int(cu[1]) + p
    tail = lambda x: np.ascontiguousarray(x[:, s0:int(cu[2])][None])
    o_t, S_t = gd.gdn_prefill(to_dev(tail(q), "bf16"), to_dev(tail(k), "bf16"), to_dev(tail(v), "bf16"),
                              to_dev(tail(a), "f32"), to_dev(tail(b), "f32"), to_dev(sn[j][None], "f32"),
                              form="chunked", chunk=64)
    torch.cuda.synchronize()
    report("resumed tail o vs packed", slice_err(to_host(o_t)[0], o[:, s0:int(cu[2])], lead=1), TOL["bf16"])
    report("resumed final state vs packed", slice_err(to_host(S_t)[0], S[1], lead=1), TOL["bf16"])


def test_varlen_workload_16seq(gd):
    """The 16-sequence workload (16 384 tokens, 16 heads, snapshots every
    1024 tokens) in the launch the bench times: every sequence's outputs,
    final state and snapshots, on every head, against the oracle."""
    w = synth.WORKLOADS["gdn_varlen_bf16_16seq_16k"]
    H, d = w["H"], w["dk"]
    lens = synth.varlen_lengths(w["seed"], w["N"], w["T_total"])
    q, k, v, a, b, cu = synth.varlen_batch(w["seed"], lens, H, d, d, "bf16")
    got = run(gd, q, k, v, a, b, cu, "bf16", None, snap=w["snap"])
    ref = ov.gdn_varlen(q, k, v, a, b, cu, None, snap_interval=w["snap"], form="chunked")
    assert got[2].shape == ref[2].shape
    check("varlen workload, 16 sequences x 16 heads", got, ref, cu, "bf16")
