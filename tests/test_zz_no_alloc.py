"""The allocation-free variant of the chunked gated-delta prefill
(gdn_prefill_noalloc, which uses the library's own device array instead of a
caller workspace) against gdn_prefill with a caller workspace, through the C
ABI: two calls in a row on one device, the second smaller, each bitwise equal
to gdn_prefill on the same inputs and within the bf16 bar of the fp64 oracle
on sampled heads."""

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


def _case(gd, seed, B, H, T, with_state, heads):
    import torch
    print(f"[no-alloc] case B={B} H={H} T={T} state={with_state}", flush=True)
    q, k, v, a, b = synth.gdn_batch(seed, B, H, T, D, D, "bf16")
    S0 = synth.state_batch(seed + 1, B, H, D, D, 0.05) if with_state else None
    args = [to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16"), to_dev(a, "f32"), to_dev(b, "f32")]
    tS = None if S0 is None else to_dev(S0, "f32")
    ws_need = gd.la_workspace_bytes("gdn_prefill", "bf16", B, H, T, D, D, "chunked", C)
    assert 0 < ws_need <= 72 << 20, ws_need
    o_ref_dev, S_ref_dev = gd.gdn_prefill(*args, tS, form="chunked", chunk=C)
    out = torch.empty_like(args[2])
    S_out = torch.empty((B, H, D, D), dtype=torch.float32, device=out.device)
    o, S = gd.gdn_prefill_noalloc(*args, tS, form="chunked", chunk=C, out=out, S_out=S_out)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref_dev), "o differs from gdn_prefill"
    assert torch.equal(S, S_ref_dev), "S_out differs from gdn_prefill"
    sel = [(bb, hh) for bb, hh in heads]
    o_h = np.stack([to_host(o[bb, hh]) for bb, hh in sel])
    S_h = np.stack([to_host(S[bb, hh]) for bb, hh in sel])
    o_r, S_r = [], []
    for bb, hh in sel:
        x, y = ob.gdn(q[bb:bb + 1, hh:hh + 1], k[bb:bb + 1, hh:hh + 1], v[bb:bb + 1, hh:hh + 1],
                      a[bb:bb + 1, hh:hh + 1], b[bb:bb + 1, hh:hh + 1], form="chunked", chunk=C,
                      S0=None if S0 is None else S0[bb:bb + 1, hh:hh + 1])
        o_r.append(x[0, 0])
        S_r.append(y[0, 0])
    report(f"no-alloc B={B} H={H} T={T} o (heads {sel})", slice_err(o_h, np.stack(o_r), 1), TOL["bf16"])
    report("  S", slice_err(S_h, np.stack(S_r), 1), TOL["bf16"])


def test_noalloc_two_calls_second_smaller(gd):
    # first call: the 2 x 16 x 8192 workload (288 of the array's 384
    # head-segments); second call: fewer heads, a ragged length and a carried
    # state, so it reads only the part of the array it writes itself
    _case(gd, 71, 2, 16, 8192, False, [(0, 0), (1, 15)])
    _case(gd, 73, 1, 3, 1000, True, [(0, 0), (0, 1), (0, 2)])


def test_noalloc_recurrent_form_needs_no_array(gd):
    import torch
    q, k, v, a, b = synth.gdn_batch(75, 1, 2, 130, D, D, "bf16")
    args = [to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16"), to_dev(a, "f32"), to_dev(b, "f32")]
    o1, S1 = gd.gdn_prefill(*args, form="recurrent")
    o2, S2 = gd.gdn_prefill_noalloc(*args, form="recurrent")
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S2)
