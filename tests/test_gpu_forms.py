"""GPU parity of the decode step, the recurrent and parallel forms and the
fp32-arithmetic chunked kernels against the fp64 oracle, through the C ABI.

Also: cross-form invariants (chained decode steps equal a prefill, split
prefill with carried state equals one prefill), in-place state update,
determinism, and the empty / single-token edge cases.
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


def la_inputs(seed, B, H, T, dk, dv, dtype, scale=1.0):
    return synth.la_batch(seed, B, H, T, dk, dv, dtype, scale)


def gdn_inputs(seed, B, H, T, dk, dv, dtype, alpha_mean=3.0):
    return synth.gdn_batch(seed, B, H, T, dk, dv, dtype, alpha_mean=alpha_mean)


# ----------------------------------------------------------------- workload 1
@pytest.mark.parametrize("form", ["parallel", "recurrent", "chunked"])
def test_la_fp32_small_workload(gd, form):
    """B=1, H=2, T=256, d=16, fp32; the GPU runs each of the three forms."""
    w = synth.WORKLOADS["la_fp32_small"]
    q, k, v = la_inputs(w["seed"], w["B"], w["H"], w["T"], w["dk"], w["dv"], "f32")
    o_ref, S_ref, z_ref = ob.lin_attn(q, k, v, form="recurrent")
    o, S, z = gd.lin_attn_prefill(to_dev(q, "f32"), to_dev(k, "f32"), to_dev(v, "f32"), form=form,
                                  chunk=w["chunk"])
    report(f"la f32 small {form} o", slice_err(to_host(o), o_ref), TOL["f32"])
    report(f"la f32 small {form} S", slice_err(to_host(S), S_ref), TOL["f32"])
    report(f"la f32 small {form} z", slice_err(to_host(z), z_ref), TOL["f32"])


@pytest.mark.parametrize("dtype,dk,dv,T,C", [
    ("f32", 64, 64, 1000, 64), ("f32", 32, 128, 77, 16), ("bf16", 128, 64, 300, 32),
    ("f32", 128, 128, 130, 32), ("bf16", 16, 16, 1, 16), ("f32", 32, 32, 300, 128), ("bf16", 16, 64, 257, 128)])
def test_la_chunked_generic_with_state(gd, dtype, dk, dv, T, C):
    q, k, v = la_inputs(7, 2, 3, T, dk, dv, dtype, scale=0.5)
    S0 = synth.state_batch(8, 2, 3, dk, dv, 0.3) ** 2
    z0 = np.stack([[synth.norm_head(8, b, h, dk) for h in range(3)] for b in range(2)])
    o_ref, S_ref, z_ref = ob.lin_attn(q, k, v, form="chunked", chunk=C, S0=S0, z0=z0)
    tS, tz = to_dev(S0, "f32"), to_dev(z0, "f32")
    o, S, z = gd.lin_attn_prefill(to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype), tS, tz,
                                  form="chunked", chunk=C, S_out=tS, z_out=tz)  # in place
    report(f"la chunked {dtype} {dk}x{dv} T={T} C={C} o", slice_err(to_host(o), o_ref), TOL[dtype])
    report("  S (in place)", slice_err(to_host(S), S_ref), TOL["f32"])
    report("  z (in place)", slice_err(to_host(z), z_ref), TOL["f32"])


@pytest.mark.parametrize("dtype,dk,dv,T", [("f32", 16, 16, 200), ("bf16", 128, 128, 100),
                                           ("f32", 64, 32, 33), ("bf16", 32, 64, 1)])
def test_la_recurrent_with_state(gd, dtype, dk, dv, T):
    q, k, v = la_inputs(9, 1, 4, T, dk, dv, dtype)
    S0 = synth.state_batch(10, 1, 4, dk, dv, 0.5) ** 2
    z0 = np.stack([[synth.norm_head(10, 0, h, dk) for h in range(4)]])
    o_ref, S_ref, z_ref = ob.lin_attn(q, k, v, form="recurrent", S0=S0, z0=z0)
    o, S, z = gd.lin_attn_prefill(to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype), to_dev(S0, "f32"),
                                  to_dev(z0, "f32"), form="recurrent")
    report(f"la recurrent {dtype} {dk}x{dv} T={T} o", slice_err(to_host(o), o_ref), TOL[dtype])
    report("  S", slice_err(to_host(S), S_ref), TOL["f32"])
    report("  z", slice_err(to_host(z), z_ref), TOL["f32"])


@pytest.mark.parametrize("dtype,dk,dv,T", [("f32", 16, 16, 300), ("bf16", 128, 128, 256),
                                           ("f32", 128, 32, 65)])
def test_la_parallel(gd, dtype, dk, dv, T):
    q, k, v = la_inputs(11, 2, 2, T, dk, dv, dtype, scale=0.3)
    o_ref = np.stack([[oracle.la_parallel(q[b, h], k[b, h], v[b, h]) for h in range(2)] for b in range(2)])
    o, S, z = gd.lin_attn_prefill(to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype), form="parallel")
    report(f"la parallel {dtype} {dk}x{dv} T={T}", slice_err(to_host(o), o_ref), TOL[dtype])
    _, S_ref, z_ref = ob.lin_attn(q, k, v, form="recurrent")
    report("  final S", slice_err(to_host(S), S_ref), TOL["f32"])
    report("  final z", slice_err(to_host(z), z_ref), TOL["f32"])


# ---------------------------------------------------------- gated delta rule
@pytest.mark.parametrize("dtype,dk,dv,T", [("f32", 16, 16, 300), ("bf16", 128, 128, 200),
                                           ("f32", 64, 128, 50), ("f32", 128, 16, 1)])
def test_gdn_recurrent_with_state(gd, dtype, dk, dv, T):
    q, k, v, a, b = gdn_inputs(12, 2, 2, T, dk, dv, dtype, alpha_mean=1.0)
    S0 = synth.state_batch(13, 2, 2, dk, dv, 0.2)
    o_ref, S_ref = ob.gdn(q, k, v, a, b, form="recurrent", S0=S0)
    tS = to_dev(S0, "f32")
    o, S = gd.gdn_prefill(to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype), to_dev(a, "f32"),
                          to_dev(b, "f32"), tS, form="recurrent", S_out=tS)
    report(f"gdn recurrent {dtype} {dk}x{dv} T={T} o", slice_err(to_host(o), o_ref), TOL[dtype])
    report("  S (in place)", slice_err(to_host(S), S_ref), TOL["f32"])


@pytest.mark.parametrize("dtype,dk,dv,T,C,amean", [
    ("f32", 64, 64, 1000, 64, 3.0), ("f32", 32, 32, 333, 16, 6.0), ("f32", 16, 128, 129, 64, 1.0),
    ("bf16", 64, 64, 500, 32, 3.0), ("f32", 128, 128, 200, 32, 6.0), ("f32", 32, 32, 300, 128, 3.0),
    ("bf16", 16, 16, 257, 128, 1.0)])
def test_gdn_chunked_generic(gd, dtype, dk, dv, T, C, amean):
    q, k, v, a, b = gdn_inputs(14, 1, 3, T, dk, dv, dtype, alpha_mean=amean)
    S0 = synth.state_batch(15, 1, 3, dk, dv, 0.2)
    o_ref, S_ref = ob.gdn(q, k, v, a, b, form="chunked", chunk=C, S0=S0)
    o, S = gd.gdn_prefill(to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype), to_dev(a, "f32"),
                          to_dev(b, "f32"), to_dev(S0, "f32"), form="chunked", chunk=C)
    report(f"gdn chunked generic {dtype} {dk}x{dv} T={T} C={C} o", slice_err(to_host(o), o_ref), TOL[dtype])
    report("  S", slice_err(to_host(S), S_ref), TOL["f32"])


# -------------------------------------------------------------- decode step
@pytest.mark.parametrize("dtype,dk,dv", [("bf16", 128, 128), ("f32", 64, 32), ("f32", 16, 128)])
def test_decode_gated_delta_small(gd, dtype, dk, dv):
    N, H, steps = 3, 4, 5
    S = synth.state_batch(16, N, H, dk, dv, 0.02)
    tS = to_dev(S, "f32")
    S_ref = S.astype(np.float64).reshape(N * H, dv, dk)
    for s in range(steps):
        q, k, v, a, b = synth.decode_token_inputs(17, N, H, dk, dv, dtype, s)
        o = gd.lin_attn_decode_step("gated_delta", to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype), tS,
                                    alpha=to_dev(a, "f32"), beta=to_dev(b, "f32"))
        o_ref, S_ref = ob.gdn_step_heads(q.reshape(-1, dk), k.reshape(-1, dk), v.reshape(-1, dv),
                                         a.reshape(-1), b.reshape(-1), S_ref)
        report(f"decode gdn {dtype} {dk}x{dv} step {s} o", slice_err(to_host(o).reshape(N * H, dv), o_ref, 1),
               TOL[dtype])
    report("  S after steps", slice_err(to_host(tS).reshape(N * H, dv, dk), S_ref, 1), TOL["f32"])


@pytest.mark.parametrize("dtype,dk,dv", [("bf16", 128, 128), ("f32", 32, 64)])
def test_decode_normalized_small(gd, dtype, dk, dv):
    N, H, steps = 2, 3, 4
    S = synth.state_batch(18, N, H, dk, dv, 0.5) ** 2
    z = np.stack([[synth.norm_head(18, n, h, dk) for h in range(H)] for n in range(N)])
    tS, tz = to_dev(S, "f32"), to_dev(z, "f32")
    S_ref, z_ref = S.astype(np.float64).reshape(N * H, dv, dk), z.astype(np.float64).reshape(N * H, dk)
    for s in range(steps):
        q, k, v = synth.la_decode_token_inputs(19, N, H, dk, dv, dtype, s, scale=0.5)
        o = gd.lin_attn_decode_step("normalized", to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype), tS, z=tz)
        o_ref, S_ref, z_ref = ob.la_step_heads(q.reshape(-1, dk), k.reshape(-1, dk), v.reshape(-1, dv), S_ref,
                                               z_ref)
        report(f"decode normalized {dtype} {dk}x{dv} step {s} o",
               slice_err(to_host(o).reshape(N * H, dv), o_ref, 1), TOL[dtype])
    report("  S", slice_err(to_host(tS).reshape(N * H, dv, dk), S_ref, 1), TOL["f32"])
    report("  z", slice_err(to_host(tz).reshape(N * H, dk), z_ref, 1), TOL["f32"])


@pytest.mark.timeout(600)
def test_decode_workload_full_size(gd):
    """256 sequences x 32 heads, d = 128, bf16 token inputs, fp32 state N(0, 0.02^2),
    1000 steps with fresh token inputs every step (drawn on the host by worker
    processes, in step order): every head checked after step 1; a seeded
    sample of 256 heads checked on every step (outputs) and at the end
    (state)."""
    import multiprocessing as mp
    from concurrent.futures import ProcessPoolExecutor

    import torch
    from gpu_helpers import bf16_bits_to_f32, decode_step_inputs

    w = synth.WORKLOADS["gdn_decode_256x32"]
    N, H, dk, dv, steps, seed = w["N"], w["H"], w["dk"], w["dv"], w["steps"], w["seed"]
    S0 = synth.decode_state_fast(seed, N, H, dk, dv, w["state_std"])
    tS = to_dev(S0, "f32")
    rng = np.random.default_rng(4242)
    sample = np.sort(rng.choice(N * H, size=256, replace=False))
    idx = torch.from_numpy(sample).to(tS.device)
    S_s = S0.reshape(N * H, dv, dk)[sample].astype(np.float64)
    out = torch.empty((N, H, dv), dtype=torch.bfloat16, device=tS.device)
    up_bits = lambda x: torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(tS.device)
    worst = 0.0
    ctx = mp.get_context("spawn")
    with ProcessPoolExecutor(max_workers=8, mp_context=ctx) as ex:
        draws = ex.map(decode_step_inputs, [seed] * steps, [N] * steps, [H] * steps, [dk] * steps, [dv] * steps,
                       range(steps), chunksize=4)
        for s, (step, (bq, bk, bv), ha, hb) in enumerate(draws):
            assert step == s
            gd.lin_attn_decode_step("gated_delta", up_bits(bq), up_bits(bk), up_bits(bv), tS,
                                    alpha=torch.from_numpy(ha).to(tS.device), beta=torch.from_numpy(hb).to(tS.device),
                                    out=out)
            hq, hk, hv = (bf16_bits_to_f32(x).reshape(N * H, -1) for x in (bq, bk, bv))
            ha, hb = ha.reshape(N * H), hb.reshape(N * H)
            if s == 0:
                o_all, S1 = ob.gdn_step_heads(hq, hk, hv, ha, hb, S0.reshape(N * H, dv, dk))
                report("decode full step 1: all heads o", slice_err(to_host(out).reshape(N * H, dv), o_all, 1),
                       TOL["bf16"])
                report("decode full step 1: all heads S", slice_err(to_host(tS).reshape(N * H, dv, dk), S1, 1),
                       TOL["f32"])
                del S1
            o_s, S_s = ob.gdn_step_heads(hq[sample], hk[sample], hv[sample], ha[sample], hb[sample], S_s)
            got = to_host(out.reshape(N * H, dv).index_select(0, idx))
            worst = max(worst, slice_err(got, o_s, 1))
            if s % 250 == 249:
                print(f"[parity] decode full: step {s + 1} of {steps}", flush=True)
    report(f"decode full: sampled heads o, worst over {steps} steps", worst, TOL["bf16"])
    got_S = to_host(tS.reshape(N * H, dv, dk).index_select(0, idx))
    report(f"decode full: sampled heads S after {steps} steps", slice_err(got_S, S_s, 1), TOL["f32"])


# --------------------------------------------------------- cross-form checks
def test_decode_steps_equal_recurrent_prefill(gd):
    """T chained decode steps give the same outputs and state as one prefill."""
    import torch
    B, H, T, d = 2, 2, 12, 64
    q, k, v, a, b = gdn_inputs(20, B, H, T, d, d, "bf16")
    S0 = synth.state_batch(21, B, H, d, d, 0.1)
    tq, tk, tv = to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16")
    ta, tb = to_dev(a, "f32"), to_dev(b, "f32")
    o_p, S_p = gd.gdn_prefill(tq, tk, tv, ta, tb, to_dev(S0, "f32"), form="recurrent")
    tS = to_dev(S0, "f32")
    outs = []
    for t in range(T):
        outs.append(gd.lin_attn_decode_step("gated_delta", tq[:, :, t].contiguous(), tk[:, :, t].contiguous(),
                                            tv[:, :, t].contiguous(), tS, alpha=ta[:, :, t].contiguous(),
                                            beta=tb[:, :, t].contiguous()))
    o_d = torch.stack(outs, dim=2)
    assert torch.equal(o_d, o_p), "decode chain and recurrent prefill differ"
    assert torch.equal(tS, S_p)


def test_split_prefill_equals_whole(gd):
    B, H, T, T1, d = 1, 2, 300, 131, 32
    q, k, v, a, b = gdn_inputs(22, B, H, T, d, d, "f32")
    dq, dk_, dv_, da, db = (to_dev(x, "f32") for x in (q, k, v, a, b))
    o_w, S_w = gd.gdn_prefill(dq, dk_, dv_, da, db, form="chunked", chunk=32)
    o1, S1 = gd.gdn_prefill(dq[:, :, :T1].contiguous(), dk_[:, :, :T1].contiguous(), dv_[:, :, :T1].contiguous(),
                            da[:, :, :T1].contiguous(), db[:, :, :T1].contiguous(), form="chunked", chunk=32)
    o2, S2 = gd.gdn_prefill(dq[:, :, T1:].contiguous(), dk_[:, :, T1:].contiguous(), dv_[:, :, T1:].contiguous(),
                            da[:, :, T1:].contiguous(), db[:, :, T1:].contiguous(), S1, form="chunked", chunk=32)
    import torch
    report("split-resume o", slice_err(to_host(torch.cat([o1, o2], dim=2)), to_host(o_w)), TOL["f32"])
    report("split-resume S", slice_err(to_host(S2), to_host(S_w)), TOL["f32"])


def test_determinism_and_edge_cases(gd):
    import torch
    q, k, v, a, b = gdn_inputs(23, 1, 2, 70, 64, 64, "f32")
    args = [to_dev(x, "f32") for x in (q, k, v, a, b)]
    r1 = gd.gdn_prefill(*args, form="chunked", chunk=16)
    r2 = gd.gdn_prefill(*args, form="chunked", chunk=16)
    assert torch.equal(r1[0], r2[0]) and torch.equal(r1[1], r2[1])
    # T = 0: the state passes through, the output is empty
    S0 = to_dev(synth.state_batch(24, 1, 2, 64, 64, 0.1), "f32")
    e = [x[:, :, :0].contiguous() for x in args]
    o, S = gd.gdn_prefill(*e, S0, form="chunked", chunk=16)
    assert o.numel() == 0 and torch.equal(S, S0)
    o, S, z = gd.lin_attn_prefill(*[x[:, :, :0].contiguous() for x in args[:3]], form="recurrent")
    assert o.numel() == 0 and float(S.abs().max()) == 0.0 and float(z.abs().max()) == 0.0
    # T = 1: o = S_1 q_1 with S_1 = alpha S0 (I - beta k k^T) + beta v k^T
    o, S = gd.gdn_prefill(*[x[:, :, :1].contiguous() for x in args], S0, form="chunked", chunk=64)
    o_ref, S_ref = ob.gdn(q[:, :, :1], k[:, :, :1], v[:, :, :1], a[:, :, :1], b[:, :, :1], form="recurrent",
                          S0=to_host(S0))
    report("T=1 o", slice_err(to_host(o), o_ref), TOL["f32"])
    report("T=1 S", slice_err(to_host(S), S_ref), TOL["f32"])


# ------------------------------------ matrix-core path at any chunk length
@pytest.mark.parametrize("C", [16, 32, 128])
def test_matrix_core_path_serves_every_chunk_length(gd, C):
    """bf16 with d = 128 runs on the matrix-core kernels (64-token blocks)
    whatever valid chunk is asked for; the chunk form is exact for any block
    length, so the oracle's chunk form at the requested C is the reference
    (states at the bf16 bar: the matrix-core state products take bf16
    operands)."""
    T = 200
    q, k, v = la_inputs(16, 1, 2, T, 128, 128, "bf16", scale=0.1)
    o_ref, S_ref, z_ref = ob.lin_attn(q, k, v, form="chunked", chunk=C)
    o, S, z = gd.lin_attn_prefill(to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16"), form="chunked", chunk=C)
    report(f"la matrix-core C={C} o", slice_err(to_host(o), o_ref), TOL["bf16"])
    report("  S", slice_err(to_host(S), S_ref), TOL["bf16"])
    report("  z", slice_err(to_host(z), z_ref), TOL["bf16"])
    q, k, v, a, b = gdn_inputs(17, 1, 2, T, 128, 128, "bf16", alpha_mean=3.0)
    S0 = synth.state_batch(18, 1, 2, 128, 128, 0.2)
    o_ref, S_ref = ob.gdn(q, k, v, a, b, form="chunked", chunk=C, S0=S0)
    o, S = gd.gdn_prefill(to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16"), to_dev(a, "f32"), to_dev(b, "f32"),
                          to_dev(S0, "f32"), form="chunked", chunk=C)
    report(f"gdn matrix-core C={C} o", slice_err(to_host(o), o_ref), TOL["bf16"])
    report("  S", slice_err(to_host(S), S_ref), TOL["bf16"])
