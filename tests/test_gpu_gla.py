"""GPU parity of scalar-gated linear attention (S_t = alpha_t S_{t-1} + v_t k_t^T,
o_t = S_t q_t; no feature map, no normaliser) against the fp64 oracle's
recurrence, through the C ABI: the recurrent form in fp32 and bf16 at every
head size, the matrix-core chunked form (bf16, d = 128, chunk 64) at ragged
sizes, under gate stress, with carried and in-place state, at the
2 x 16 x 8192 workload, and the one-token decode step.
"""

import numpy as np
import pytest

import oracle
from oracle import batched as ob
import synth
from gpu_helpers import TOL, report, slice_err, to_dev, to_host

pytestmark = pytest.mark.gpu
D, C = 128, 64


@pytest.fixture(scope="module")
def gd():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_causal_amd as m
    m._load()
    return m


def inputs(seed, B, H, T, dk, dv, dtype, amean=3.0):
    q, k, v, a, _ = synth.gdn_batch(seed, B, H, T, dk, dv, dtype, alpha_mean=amean)
    return q, k, v, a


def run(gd, q, k, v, a, dtype, S0=None, inplace=False, form="chunked"):
    tS = None if S0 is None else to_dev(S0, "f32")
    o, S = gd.gla_prefill(to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype), to_dev(a, "f32"), tS, form=form,
                          chunk=C, S_out=tS if inplace else None)
    return to_host(o), to_host(S)


@pytest.mark.parametrize("dtype,d", [("f32", 16), ("f32", 32), ("f32", 64), ("f32", 128), ("bf16", 64),
                                     ("bf16", 128)])
def test_gla_recurrent_form(gd, dtype, d):
    B, H, T = 1, 3, 200
    q, k, v, a = inputs(51, B, H, T, d, d, dtype)
    S0 = synth.state_batch(52, B, H, d, d, 0.1)
    o_ref, S_ref = ob.gla(q, k, v, a, S0)
    o, S = run(gd, q, k, v, a, dtype, S0, inplace=True, form="recurrent")
    report(f"gla recurrent {dtype} d={d} o", slice_err(o, o_ref), TOL[dtype])
    report("  S", slice_err(S, S_ref), TOL[dtype])


# (segments of whole chunks: one chunk per segment, several with a short last
#  one (4x16x600), a single segment (16x16x130))
@pytest.mark.parametrize("B,H,T,amean,with_state", [
    (1, 2, 300, 3.0, True), (2, 1, 64, 3.0, False), (1, 3, 65, 3.0, True), (1, 1, 1, 3.0, True),
    (1, 2, 2000, 6.0, True), (2, 2, 777, 0.0, True), (4, 16, 600, 3.0, True), (16, 16, 130, 3.0, False)])
def test_gla_chunked(gd, B, H, T, amean, with_state):
    q, k, v, a = inputs(53, B, H, T, D, D, "bf16", amean)
    S0 = synth.state_batch(54, B, H, D, D, 0.05) if with_state else None
    o_ref, S_ref = ob.gla(q, k, v, a, S0)
    o, S = run(gd, q, k, v, a, "bf16", S0, inplace=with_state)
    report(f"gla chunked B={B} H={H} T={T} alpha~sig(N({amean},1)) o", slice_err(o, o_ref), TOL["bf16"])
    report("  S", slice_err(S, S_ref), TOL["bf16"])


def test_gla_chunked_no_decay(gd):
    """alpha = 1: plain unnormalised linear attention, o = tril(Q K^T) V."""
    q, k, v, a = inputs(55, 1, 2, 700, D, D, "bf16")
    a = np.ones_like(a)
    o_ref, S_ref = ob.gla(q, k, v, a)
    o, S = run(gd, q, k, v, a, "bf16")
    report("gla alpha=1 o", slice_err(o, o_ref), TOL["bf16"])
    report("  S", slice_err(S, S_ref), TOL["bf16"])


def test_gla_workload_2x16x8192(gd):
    w = synth.WORKLOADS["gla_bf16_2x16x8192"]
    q, k, v, a = inputs(w["seed"], w["B"], w["H"], w["T"], D, D, "bf16")
    o, S = run(gd, q, k, v, a, "bf16")
    o_ref, S_ref = ob.gla(q, k, v, a)
    report("gla workload 2x16x8192 o (all heads)", slice_err(o, o_ref), TOL["bf16"])
    report("  final S (all heads)", slice_err(S, S_ref), TOL["bf16"])


def test_gla_decode_steps_match_prefill_and_oracle(gd):
    """Chained one-token steps equal the recurrent prefill bit for bit, and a
    step over many heads matches the oracle's step."""
    import torch
    N, H, T = 8, 4, 12
    q, k, v, a = inputs(56, N, H, T, D, D, "bf16")
    S0 = synth.state_batch(57, N, H, D, D, 0.02)
    o_pre, S_pre = gd.gla_prefill(to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16"), to_dev(a, "f32"),
                                  to_dev(S0, "f32"), form="recurrent")
    S = to_dev(S0, "f32")
    outs = []
    for t in range(T):
        outs.append(gd.lin_attn_decode_step("gated", to_dev(q[:, :, t], "bf16"), to_dev(k[:, :, t], "bf16"),
                                            to_dev(v[:, :, t], "bf16"), S, alpha=to_dev(a[:, :, t], "f32")))
    assert torch.equal(torch.stack(outs, 2), o_pre) and torch.equal(S, S_pre)
    o_ref, S_ref = ob.gla_step_heads(q[:, :, 0].reshape(-1, D), k[:, :, 0].reshape(-1, D),
                                     v[:, :, 0].reshape(-1, D), a[:, :, 0].reshape(-1), S0.reshape(-1, D, D))
    report("gla decode step o", slice_err(to_host(outs[0]).reshape(-1, D), o_ref, 1), TOL["bf16"])
