"""GPU parity of Kimi Delta Attention (the gated delta rule with a per-channel
key-side decay, S_t = S_{t-1} Diag(alpha_t)(I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
o_t = S_t q_t) against the fp64 oracle's recurrence, through the C ABI: the
recurrent prefill in fp32 and bf16 at every head size (d_k != d_v too), under
decay stress, with carried and in-place state and T = 0, the one-token decode
step chained over a sequence (bit-identical to the prefill) and against the
oracle's step at the 256 x 32 decode shape.
"""

import numpy as np
import pytest

import oracle
from oracle import batched as ob
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


def run(gd, q, k, v, a, b, dtype, S0=None, inplace=False):
    tS = None if S0 is None else to_dev(S0, "f32")
    o, S = gd.kda_prefill(to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype), to_dev(a, "f32"), to_dev(b, "f32"),
                          tS, form="recurrent", S_out=tS if inplace else None)
    return to_host(o), to_host(S)


@pytest.mark.parametrize("dtype,dk,dv", [("f32", 16, 16), ("f32", 32, 64), ("f32", 64, 32), ("f32", 128, 128),
                                         ("bf16", 64, 64), ("bf16", 128, 128), ("bf16", 128, 16)])
def test_kda_recurrent_form(gd, dtype, dk, dv):
    B, H, T = 1, 3, 200
    q, k, v, a, b = synth.kda_batch(71, B, H, T, dk, dv, dtype)
    S0 = synth.state_batch(72, B, H, dk, dv, 0.1)
    o_ref, S_ref = ob.kda(q, k, v, a, b, S0)
    o, S = run(gd, q, k, v, a, b, dtype, S0, inplace=True)
    report(f"kda recurrent {dtype} dk={dk} dv={dv} o", slice_err(o, o_ref), TOL[dtype])
    report("  S", slice_err(S, S_ref), TOL[dtype])


def test_kda_decay_stress(gd):
    """Channels that forget almost at once next to channels that barely forget."""
    B, H, T, d = 2, 2, 300, 128
    q, k, v, a, b = synth.kda_batch(73, B, H, T, d, d, "f32")
    a[..., ::2] = a[..., ::2] ** 40         # alpha down to ~1e-3 on even channels
    a[..., 1::4] = 1.0                      # no decay at all on a quarter of them
    o_ref, S_ref = ob.kda(q, k, v, a, b)
    o, S = run(gd, q, k, v, a, b, "f32")
    report("kda decay stress o", slice_err(o, o_ref), TOL["f32"])
    report("  S", slice_err(S, S_ref), TOL["f32"])


def test_kda_uniform_decay_matches_gated_delta(gd):
    """Equal decay on every channel: the oracle's Gated DeltaNet recurrence."""
    B, H, T, d = 1, 2, 150, 64
    q, k, v, a, b = synth.kda_batch(74, B, H, T, d, d, "f32")
    a[:] = a[..., :1]
    o_ref, S_ref = ob.gdn(q, k, v, a[..., 0], b, form="recurrent")
    o, S = run(gd, q, k, v, a, b, "f32")
    report("kda uniform decay vs gated delta o", slice_err(o, o_ref), TOL["f32"])
    report("  S", slice_err(S, S_ref), TOL["f32"])


def test_kda_empty_sequence_copies_state(gd):
    B, H, d = 1, 2, 32
    q, k, v, a, b = synth.kda_batch(75, B, H, 0, d, d, "f32")
    S0 = synth.state_batch(76, B, H, d, d, 0.1)
    o, S = run(gd, q, k, v, a, b, "f32", S0)
    assert o.shape == (B, H, 0, d) and np.array_equal(S, S0.astype(np.float64))


def test_kda_decode_chain_equals_prefill(gd):
    """T decode steps chained in place give the same bits as one prefill."""
    import torch
    B, H, T, d = 2, 4, 40, 128
    q, k, v, a, b = synth.kda_batch(77, B, H, T, d, d, "bf16")
    S0 = synth.state_batch(78, B, H, d, d, 0.05)
    o_pre, S_pre = run(gd, q, k, v, a, b, "bf16", S0)
    S = to_dev(S0, "f32")
    tq, tk, tv = to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16")
    ta, tb = to_dev(a, "f32"), to_dev(b, "f32")
    outs = []
    for t in range(T):
        o_t = gd.lin_attn_decode_step("kda", tq[:, :, t].contiguous(), tk[:, :, t].contiguous(),
                                      tv[:, :, t].contiguous(), S, alpha=ta[:, :, t].contiguous(),
                                      beta=tb[:, :, t].contiguous())
        outs.append(to_host(o_t))
    torch.cuda.synchronize()
    assert np.array_equal(np.stack(outs, axis=2), o_pre)
    assert np.array_equal(to_host(S), S_pre)


def test_kda_decode_workload_256x32(gd):
    """One decode step of the 256 x 32 workload, every head, against the oracle."""
    w = synth.WORKLOADS["kda_decode_256x32"]
    N, H, d = w["N"], w["H"], w["dk"]
    S0 = synth.decode_state_fast(w["seed"], N, H, d, d, w["state_std"])
    q, k, v, a, b = synth.kda_decode_token_inputs(w["seed"], N, H, d, d, "bf16", 0)
    S = to_dev(S0, "f32")
    o = gd.lin_attn_decode_step("kda", to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16"), S,
                                alpha=to_dev(a, "f32"), beta=to_dev(b, "f32"))
    n = N * H
    o_ref, S_ref = ob.kda_step_heads(q.reshape(n, d), k.reshape(n, d), v.reshape(n, d), a.reshape(n, d),
                                     b.reshape(n), S0.reshape(n, d, d))
    report("kda decode 256x32 o", slice_err(to_host(o).reshape(n, 1, d), o_ref.reshape(n, 1, d), lead=1), TOL["bf16"])
    report("  S", slice_err(to_host(S).reshape(n, d, d), S_ref, lead=1), TOL["bf16"])


# ------------------------------------------------------------ block (chunked) form
def run_chunked(gd, q, k, v, a, b, S0=None, inplace=False):
    tS = None if S0 is None else to_dev(S0, "f32")
    o, S = gd.kda_prefill(to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16"), to_dev(a, "f32"),
                          to_dev(b, "f32"), tS, form="chunked", chunk=64, S_out=tS if inplace else None)
    return to_host(o), to_host(S)


@pytest.mark.parametrize("B,H,T,with_state", [(1, 2, 300, True), (2, 1, 64, False), (1, 3, 65, True),
                                               (1, 1, 1, True), (2, 2, 777, True), (1, 2, 2000, False),
                                               (4, 16, 130, True)])
def test_kda_chunked(gd, B, H, T, with_state):
    d = 128
    q, k, v, a, b = synth.kda_batch(79, B, H, T, d, d, "bf16")
    S0 = synth.state_batch(80, B, H, d, d, 0.05) if with_state else None
    o_ref, S_ref = ob.kda(q, k, v, a, b, S0, form="chunked")
    o, S = run_chunked(gd, q, k, v, a, b, S0, inplace=with_state)
    report(f"kda chunked B={B} H={H} T={T} o", slice_err(o, o_ref), TOL["bf16"])
    report("  S", slice_err(S, S_ref), TOL["bf16"])


def test_kda_chunked_strong_decay(gd):
    """Chunks whose decay span exceeds the factored range take the exact path;
    channels without decay and with near-total decay side by side."""
    B, H, T, d = 1, 2, 400, 128
    q, k, v, a, b = synth.kda_batch(81, B, H, T, d, d, "bf16")
    a[..., ::2] = np.maximum(a[..., ::2] ** 40, np.float32(1e-30))   # decay values stay positive
    a[..., 1::4] = 1.0
    a[..., 200:, :] = np.maximum(a[..., 200:, :], 0.9)   # later chunks back on the factored path
    o_ref, S_ref = ob.kda(q, k, v, a, b, form="chunked")
    o, S = run_chunked(gd, q, k, v, a, b)
    report("kda chunked strong decay o", slice_err(o, o_ref), TOL["bf16"])
    report("  S", slice_err(S, S_ref), TOL["bf16"])


@pytest.mark.parametrize("T", [100, 37])
def test_kda_chunked_strong_decay_ragged(gd, T):
    """Every chunk on the exact path, the last one shorter than a chunk (its
    padded rows must add nothing), with an entering state."""
    B, H, d = 2, 2, 128
    q, k, v, a, b = synth.kda_batch(85, B, H, T, d, d, "bf16")
    a[..., ::2] = np.maximum(a[..., ::2] ** 60, np.float32(1e-30))
    S0 = synth.state_batch(86, B, H, d, d, 0.05)
    o_ref, S_ref = ob.kda(q, k, v, a, b, S0, form="chunked")
    o, S = run_chunked(gd, q, k, v, a, b, S0)
    report(f"kda chunked strong decay, ragged T={T} o", slice_err(o, o_ref), TOL["bf16"])
    report("  S", slice_err(S, S_ref), TOL["bf16"])


def test_kda_chunked_uniform_is_gated_delta(gd):
    B, H, T, d = 1, 2, 500, 128
    q, k, v, a, b = synth.kda_batch(82, B, H, T, d, d, "bf16")
    a[:] = a[..., :1]
    o_ref, S_ref = ob.gdn(q, k, v, a[..., 0], b, form="chunked")
    o, S = run_chunked(gd, q, k, v, a, b)
    report("kda chunked, equal decays vs gated delta o", slice_err(o, o_ref), TOL["bf16"])
    report("  S", slice_err(S, S_ref), TOL["bf16"])


def test_kda_chunked_matches_recurrent_kernel(gd):
    """The block form against the token-serial kernel on the same inputs."""
    B, H, T, d = 2, 4, 1000, 128
    q, k, v, a, b = synth.kda_batch(83, B, H, T, d, d, "bf16")
    S0 = synth.state_batch(84, B, H, d, d, 0.05)
    o_c, S_c = run_chunked(gd, q, k, v, a, b, S0)
    o_r, S_r = run(gd, q, k, v, a, b, "bf16", S0)
    report("kda chunked vs recurrent kernel o", slice_err(o_c, o_r), TOL["bf16"])
    report("  S", slice_err(S_c, S_r), TOL["bf16"])


def test_kda_chunked_workload_2x16x8192(gd):
    """The bench workload on every head; the oracle on four heads."""
    w = synth.WORKLOADS["kda_bf16_2x16x8192"]
    B, H, T, d = w["B"], w["H"], w["T"], w["dk"]
    q, k, v, a, b = synth.kda_batch(w["seed"], B, H, T, d, d, "bf16")
    o, S = run_chunked(gd, q, k, v, a, b)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(S))
    heads = [(0, 0), (0, 7), (1, 3), (1, 15)]
    o_ref, S_ref = ob.kda(q, k, v, a, b, form="chunked", heads=heads)
    for bb, hh in heads:
        report(f"kda workload head ({bb},{hh}) o", slice_err(o[bb:bb + 1, hh:hh + 1], o_ref[bb:bb + 1, hh:hh + 1]),
               TOL["bf16"])
        report("  S", slice_err(S[bb:bb + 1, hh:hh + 1], S_ref[bb:bb + 1, hh:hh + 1]), TOL["bf16"])
