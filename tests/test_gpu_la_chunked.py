"""GPU parity of the matrix-core chunked linear-attention kernel (bf16
activations, fp32 state and normaliser, d_k = d_v = 128, chunk 64) against
the fp64 oracle through the C ABI: the full 4 x 16 x 4096 workload, ragged
lengths, carried state, in-place update, and split-resume.
"""

import numpy as np
import pytest

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


# (the library cuts each head into up to 256 / (B*H) segments of whole chunks:
#  one chunk per segment, several per segment with a short last one
#  (4x16x600: 10 chunks -> 3,3,3,1), and a single segment (16x16x130))
@pytest.mark.parametrize("B,H,T,with_state", [(1, 2, 300, True), (2, 1, 64, False), (1, 3, 65, True),
                                              (1, 1, 1, False), (2, 2, 1000, True), (4, 16, 600, True),
                                              (16, 16, 130, True)])
def test_la_mfma_small(gd, B, H, T, with_state):
    q, k, v = synth.la_batch(41, B, H, T, D, D, "bf16", scale=1 / np.sqrt(D))
    S0 = z0 = None
    if with_state:
        S0 = synth.state_batch(42, B, H, D, D, 0.3) ** 2
        z0 = np.stack([[synth.norm_head(42, b, h, D, 5.0) for h in range(H)] for b in range(B)])
    o_ref, S_ref, z_ref = ob.lin_attn(q, k, v, form="chunked", chunk=C, S0=S0, z0=z0)
    tS = None if S0 is None else to_dev(S0, "f32")
    tz = None if z0 is None else to_dev(z0, "f32")
    o, S, z = gd.lin_attn_prefill(to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16"), tS, tz,
                                  form="chunked", chunk=C, S_out=tS, z_out=tz)
    report(f"la mfma B={B} H={H} T={T} o", slice_err(to_host(o), o_ref), TOL["bf16"])
    report("  S", slice_err(to_host(S), S_ref), TOL["bf16"])
    report("  z", slice_err(to_host(z), z_ref), TOL["bf16"])


def test_la_workload_4x16x4096(gd):
    w = synth.WORKLOADS["la_bf16_4x16x4096"]
    q, k, v = synth.la_batch(w["seed"], w["B"], w["H"], w["T"], D, D, "bf16", w["scale"])
    o, S, z = gd.lin_attn_prefill(to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16"), form="chunked",
                                  chunk=C)
    o_ref, S_ref, z_ref = ob.lin_attn(q, k, v, form="chunked", chunk=C)
    report("la workload 4x16x4096 o (all heads)", slice_err(to_host(o), o_ref), TOL["bf16"])
    report("  final S", slice_err(to_host(S), S_ref), TOL["bf16"])
    report("  final z", slice_err(to_host(z), z_ref), TOL["bf16"])


def test_la_mfma_split_resume_and_determinism(gd):
    import torch
    q, k, v = synth.la_batch(43, 1, 2, 777, D, D, "bf16", scale=1 / np.sqrt(D))
    tq, tk, tv = to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16")
    o_w, S_w, z_w = gd.lin_attn_prefill(tq, tk, tv, form="chunked", chunk=C)
    o_w2, S_w2, z_w2 = gd.lin_attn_prefill(tq, tk, tv, form="chunked", chunk=C)
    assert torch.equal(o_w, o_w2) and torch.equal(S_w, S_w2) and torch.equal(z_w, z_w2)
    T1 = 320
    o1, S1, z1 = gd.lin_attn_prefill(tq[:, :, :T1].contiguous(), tk[:, :, :T1].contiguous(),
                                     tv[:, :, :T1].contiguous(), form="chunked", chunk=C)
    o2, S2, z2 = gd.lin_attn_prefill(tq[:, :, T1:].contiguous(), tk[:, :, T1:].contiguous(),
                                     tv[:, :, T1:].contiguous(), S1, z1, form="chunked", chunk=C)
    report("la split-resume o", slice_err(to_host(torch.cat([o1, o2], 2)), to_host(o_w)), TOL["bf16"])
    report("la split-resume S", slice_err(to_host(S2), to_host(S_w)), TOL["bf16"])
    report("la split-resume z", slice_err(to_host(z2), to_host(z_w)), TOL["bf16"])
