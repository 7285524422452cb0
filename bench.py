"""Benchmark of the gated-delta prefill and decode hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--legs a,b,...]

One timed step is one chunked gated-delta prefill (one gdn_prefill call: the
map pass, the combine and the output pass) over the 2 x 16 x 8192 workload (B=2, H=16, T=8192,
d_k = d_v = 128, bf16 activations, fp32 state, chunk 64), inputs resident in
HBM.  `value` is prefill tokens/s (B*T tokens per step).  In the same run,
each reported beside the headline: the decode workload (256 sequences x 32
heads, d = 128, fp32 state, 1000 steps) as state HBM GB/s; the normalised and
the scalar-gated linear-attention prefills; the 1 x 16 x 262144 long-context
prefill; the fused pre-operations of a Gated DeltaNet layer; the KDA decode
and prefill (block and recurrent forms); a packed batch of 16 sequences of
mixed lengths with state snapshots (gated delta, and the same batch for the
normalised, scalar-gated and KDA kinds); and the fp64 CPU oracle on a bounded
sample of the prefill workload.  Prints one JSON line.

Every leg's inputs are drawn and uploaded first; then the GPU runs about 0.3 s
of untimed work and the timed parts of the legs follow back to back, the
headline prefill last (the memory-bound decode legs first, the long-context
prefill right before the headline, and that leg after three untimed calls),
as in a serving process that is already busy (an idle GPU lowers its clocks,
and the first milliseconds of work after an idle gap run slower).  The
untimed decode steps settle the memory-bound legs; compute-bound work still
speeds up over its own first tens of milliseconds, so a short timed run of
the headline (20 steps after 5) stays slower than a long one (200 after 100).  `--legs` runs a subset (e.g. one leg under a profiler); the legs not
run are null in the JSON line.

Per-kernel durations come from HIP events recorded on the stream the kernels
are launched on (torch's current stream, which the binding passes to the C
ABI): around the call of every fourth timed prefill step, and around
each other leg's run of back-to-back calls (an event record costs a few
microseconds of GPU time).  Input sets rotate over three copies so the 256 MB
last-level cache cannot serve one step's inputs from the previous step.
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2516.6       # 256 CU x 2.4 GHz x 4096 flop/clk, dense
PREFILL = "gdn_bf16_2x16x8192"
DECODE = "gdn_decode_256x32"
LA_PREFILL = "la_bf16_4x16x4096"
GLA_PREFILL = "gla_bf16_2x16x8192"
PREOPS = "preops_bf16_2x16x8192"
KDA_DECODE = "kda_decode_256x32"
KDA_PREFILL = "kda_bf16_2x16x8192"
VARLEN = "gdn_varlen_bf16_16seq_16k"
LONG = "gdn_bf16_1x16x262144"
LEGS = ["decode", "kda_decode", "la", "gla", "preops", "kda_prefill", "varlen", "varlen_kinds", "long", "prefill",
        "copy"]


# Algorithmic work per head-token of the chunked gated-delta path, chunk C,
# d = d_k = d_v: bytes = q, k, v, o in bf16 + alpha, beta in fp32; flops as
# the chunk form computes them with triangular halves counted once:
# 5 C d + C^2 / 3 + 6 d^2.
def path_bytes_per_head_token(d):
    return 4 * d * 2 + 8


def path_flops_per_head_token(d, C):
    return 5 * C * d + C * C / 3 + 6 * d * d


# Counter figures measured with rocprofv3 (profile_summary.py writes them),
# stored per kernel with the hash of the source file it was built from;
# numbers taken on another version of that source are not used.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")
PMC_FILE = os.path.join(ROOT, "profiles", "pmc_counters.json")


def _current(rec):
    src = os.path.join(ROOT, rec["source"])
    return hashlib.sha256(open(src, "rb").read()).hexdigest() == rec["source_sha256"]


def measured_traffic(kernels):
    """Summed HBM bytes per launch of `kernels` (rocprofv3 FETCH_SIZE and
    WRITE_SIZE scaled by the same counters on a plain copy), or None when any
    of them has no counters for its current source."""
    try:
        rec = json.load(open(TRAFFIC_FILE))["kernels"]
        if not all(_current(rec[k]) for k in kernels):
            return None
        return sum(rec[k]["bytes_per_dispatch"] for k in kernels)
    except (OSError, KeyError, ValueError):
        return None


def measured_pmc(kernels):
    """MFMA and LDS counters of `kernels` (rocprofv3 --pmc MfmaUtil, LdsUtil,
    LdsBankConflict, MfmaFlopsBF16 per dispatch): the MFMA busy fraction over
    the kernels weighted by their durations in the same run, the summed BF16
    MFMA flops, and the per-kernel records.  None when any kernel's source has
    changed since."""
    try:
        rec = json.load(open(PMC_FILE))["kernels"]
        if not all(_current(rec[k]) for k in kernels):
            return None
        t = sum(rec[k]["avg_us"] for k in kernels)
        busy = sum(rec[k]["MfmaUtil"] / 100.0 * rec[k]["avg_us"] for k in kernels) / t
        return {"busy_frac": busy, "flops": sum(rec[k]["MfmaFlopsBF16"] for k in kernels),
                "kernels": {k: {m: rec[k][m] for m in ("MfmaUtil", "LdsUtil", "LdsBankConflict", "avg_us")}
                            for k in kernels}}
    except (OSError, KeyError, ValueError, ZeroDivisionError):
        return None


def hbm_roofline(kernel, nbytes, ms, traffic_kernels=None):
    gbps = nbytes / (ms * 1e-3) / 1e9
    return {"kernel": kernel, "bound": "hbm", "achieved": gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": gbps / HBM_PEAK_GBPS,
            "traffic": measured_traffic(traffic_kernels) if traffic_kernels else None,
            "bytes_per_launch": nbytes, "avg_launch_ms": ms}


class Ctx:
    """What every leg needs: torch, the binding, the device, the arguments."""

    def __init__(self, args):
        import torch

        import gated_delta_rule_causal_amd as gd
        assert torch.cuda.is_available(), "bench.py needs a GPU"
        self.torch, self.gd, self.args = torch, gd, args
        self.dev = torch.device("cuda:0")
        gd._load()

    def up(self, x, bf16=False):
        t = self.torch.from_numpy(x).to(self.dev)
        return t.to(self.torch.bfloat16) if bf16 else t

    def timed(self, calls, fn, warm=2):
        """Mean event time (ms) of `calls` back-to-back calls fn(i), after
        `warm` untimed ones."""
        torch = self.torch
        for i in range(warm):
            fn(i)
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record()
        for i in range(calls):
            fn(i)
        ev[1].record()
        torch.cuda.synchronize()
        return ev[0].elapsed_time(ev[1]) / calls


# ------------------------------------------------------------------ legs
def leg_la(c):
    import synth
    torch, gd, n = c.torch, c.gd, c.args.la_steps
    w = synth.WORKLOADS[LA_PREFILL]
    B, H, T, d, C = w["B"], w["H"], w["T"], w["dk"], w["chunk"]
    q, k, v = synth.la_batch(w["seed"], B, H, T, d, d, "bf16", w["scale"])
    sets = [tuple(c.up(x, True) for x in (q, k, v)) for _ in range(3)]
    del q, k, v
    out = torch.empty((B, H, T, d), dtype=torch.bfloat16, device=c.dev)
    S = torch.empty((B, H, d, d), dtype=torch.float32, device=c.dev)
    z = torch.empty((B, H, d), dtype=torch.float32, device=c.dev)
    yield   # inputs prepared; the timed part runs when every leg is prepared
    ms = c.timed(n, lambda i: gd.lin_attn_prefill(*sets[i % 3], form="chunked", chunk=C, out=out, S_out=S, z_out=z))
    ht = B * H * T
    roof = hbm_roofline("la_chunked_mfma_kernel (state pass + combine + output pass)", ht * 4 * d * 2, ms,
                        ["la_chunked_mfma_kernel_state", "la_combine_kernel", "la_chunked_mfma_kernel_out"])
    roof["achieved_TFLOPs"] = ht * (2 * C * d + 4 * d * d) / (ms * 1e-3) / 1e12
    return {"workload": "normalised linear attention prefill B=4 H=16 T=4096 d=128 chunk=64, bf16 I/O, fp32 state",
            "calls": n, "ms_per_call": ms, "tokens_per_s": B * T / (ms * 1e-3), "roofline": roof}


def leg_gla(c):
    import synth
    torch, gd, n = c.torch, c.gd, c.args.la_steps
    w = synth.WORKLOADS[GLA_PREFILL]
    B, H, T, d, C = w["B"], w["H"], w["T"], w["dk"], w["chunk"]
    q, k, v, a, _ = synth.gdn_batch(w["seed"], B, H, T, d, d, "bf16")
    sets = [tuple(c.up(x, True) for x in (q, k, v)) + (c.up(a),) for _ in range(3)]
    del q, k, v, a
    out = torch.empty((B, H, T, d), dtype=torch.bfloat16, device=c.dev)
    S = torch.empty((B, H, d, d), dtype=torch.float32, device=c.dev)
    yield
    ms = c.timed(n, lambda i: gd.gla_prefill(*sets[i % 3], form="chunked", chunk=C, out=out, S_out=S))
    nbytes = B * H * T * (4 * d * 2 + 4)   # q, k, v, o bf16 + alpha fp32
    return {"workload": "scalar-gated linear attention prefill B=2 H=16 T=8192 d=128 chunk=64, bf16 I/O, fp32 state",
            "calls": n, "ms_per_call": ms, "tokens_per_s": B * T / (ms * 1e-3),
            "roofline": hbm_roofline("la_chunked_mfma_kernel, gated (state pass + combine + output pass)", nbytes, ms,
                                     ["gla_chunked_mfma_kernel_state", "gla_combine_kernel",
                                      "gla_chunked_mfma_kernel_out"])}


def leg_preops(c):
    import synth
    torch, gd, n = c.torch, c.gd, c.args.la_steps
    w = synth.WORKLOADS[PREOPS]
    B, T, H, dk, dv = w["B"], w["T"], w["H"], w["dk"], w["dv"]
    x, cw, al, bl = synth.preops_batch(w["seed"], B, T, H, dk, dv, "bf16")
    x0 = c.up(x, True)
    sets = [(x0 if i == 0 else x0.clone(), c.up(cw), c.up(al), c.up(bl)) for i in range(3)]
    del x, cw, al, bl, x0
    outs = dict(q=torch.empty((B, H, T, dk), dtype=torch.bfloat16, device=c.dev),
                k=torch.empty((B, H, T, dk), dtype=torch.bfloat16, device=c.dev),
                v=torch.empty((B, H, T, dv), dtype=torch.bfloat16, device=c.dev),
                alpha=torch.empty((B, H, T), dtype=torch.float32, device=c.dev),
                beta=torch.empty((B, H, T), dtype=torch.float32, device=c.dev))
    yield
    ms = c.timed(n, lambda i: gd.gdn_preprocess(*sets[i % 3], H, dk, dv, want_state=False, **outs))
    # x read + gate logits read, q, k, v written + alpha, beta written
    nbytes = B * H * T * (2 * ((2 * dk + dv) * 2 + 8))
    return {"workload": "Gated DeltaNet pre-operations (conv k=4, q/k L2 norm, sigmoid gates) B=2 H=16 T=8192 d=128, "
                        "bf16 I/O", "calls": n, "ms_per_call": ms, "tokens_per_s": B * T / (ms * 1e-3),
            "roofline": hbm_roofline("gdn_preprocess_kernel", nbytes, ms, ["gdn_preprocess_kernel"])}


def _decode(c, kind, wname, traffic_key, warm=5):
    """A decode leg: `steps` consecutive steps from one evolving state, every
    step with token inputs of its own, drawn on the device with torch's seeded
    generator in the recipe's distributions (q, k unit rows, v ~ N(0, 1),
    beta = sigmoid(N(0, 1)); alpha = sigmoid(N(3, 1)), or for KDA
    sigmoid(N(0, 1) + mu_c) with mu_c spread evenly over [1, 5] across the key
    channels): a thousand steps of inputs would take minutes to draw on the
    host.  The parity tests check the same shape on host-drawn inputs."""
    import synth
    torch, gd = c.torch, c.gd
    w = synth.WORKLOADS[wname]
    N, H, d, steps = w["N"], w["H"], w["dk"], c.args.decode_steps
    S = c.up(synth.decode_state_fast(w["seed"], N, H, d, d, w["state_std"]))
    g = torch.Generator(device=c.dev)
    g.manual_seed(w["seed"])
    norm = torch.nn.functional.normalize
    mu = torch.linspace(1.0, 5.0, d, device=c.dev)
    draws = []
    for _ in range(steps + warm):
        q = norm(torch.randn(N, H, d, device=c.dev, generator=g), dim=-1).to(torch.bfloat16)
        k = norm(torch.randn(N, H, d, device=c.dev, generator=g), dim=-1).to(torch.bfloat16)
        v = torch.randn(N, H, d, device=c.dev, generator=g).to(torch.bfloat16)
        if kind == "kda":
            a = torch.sigmoid(torch.randn(N, H, d, device=c.dev, generator=g) + mu)
        else:
            a = torch.sigmoid(torch.randn(N, H, device=c.dev, generator=g) + 3.0)
        b = torch.sigmoid(torch.randn(N, H, device=c.dev, generator=g))
        draws.append((q, k, v, a, b))
    o = torch.empty((N, H, d), dtype=torch.bfloat16, device=c.dev)

    def call(i):
        tq, tk, tv, ta, tb = draws[i]
        gd.lin_attn_decode_step(kind, tq, tk, tv, S, alpha=ta, beta=tb, out=o)

    yield
    for i in range(warm):
        call(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ms = c.timed(steps, lambda i: call(warm + i), warm=0)
    wall = time.perf_counter() - t0
    state_bytes = 2 * N * H * d * d * 4
    a_bytes = d * 4 if kind == "kda" else 4
    io_bytes = N * H * (4 * d * 2 + a_bytes + 4)   # q, k, v, o bf16; alpha, beta fp32
    rec = {"steps": steps, "ms_per_step": ms, "steps_per_s": 1e3 / ms, "wall_steps_per_s": steps / wall,
           "state_GBps": state_bytes / (ms * 1e-3) / 1e9, "total_GBps": (state_bytes + io_bytes) / (ms * 1e-3) / 1e9,
           "roofline": hbm_roofline(f"recurrent_kernel ({kind} decode)", state_bytes + io_bytes, ms, [traffic_key])}
    del S, draws
    return rec


def leg_decode(c):
    r = yield from _decode(c, "gated_delta", DECODE, "recurrent_kernel_gated_delta_decode")
    return dict(workload="gated delta decode 256 seq x 32 heads, d=128, fp32 state, bf16 token I/O (fresh token "
                         "inputs every step, drawn on the device)", **r)


def leg_kda_decode(c):
    r = yield from _decode(c, "kda", KDA_DECODE, "recurrent_kernel_kda_decode")
    return dict(workload="KDA decode 256 seq x 32 heads, d=128, per-channel decay, fp32 state, bf16 token I/O "
                         "(fresh token inputs every step, drawn on the device)", **r)


def leg_long(c):
    # Inputs drawn on the device (torch's seeded generator, the distributions
    # of the synthetic recipe): 3 GiB of bf16 activations would take minutes
    # to draw on the host.  Values do not change the work; the parity tests
    # check this shape against the oracle on the host-drawn inputs.
    import synth
    torch, gd, n = c.torch, c.gd, c.args.long_calls
    w = synth.WORKLOADS[LONG]
    B, H, T, d = w["B"], w["H"], w["T"], w["dk"]
    g = torch.Generator(device=c.dev)
    g.manual_seed(w["seed"])
    norm = torch.nn.functional.normalize
    q = norm(torch.randn(B, H, T, d, device=c.dev, generator=g), dim=-1).to(torch.bfloat16)
    k = norm(torch.randn(B, H, T, d, device=c.dev, generator=g), dim=-1).to(torch.bfloat16)
    v = torch.randn(B, H, T, d, device=c.dev, generator=g).to(torch.bfloat16)
    a = torch.sigmoid(torch.randn(B, H, T, device=c.dev, generator=g) + 3.0)
    b = torch.sigmoid(torch.randn(B, H, T, device=c.dev, generator=g))
    ws = gd.gdn_workspace(q, v, 64)
    out = torch.empty_like(v)
    S = torch.empty((B, H, d, d), dtype=torch.float32, device=c.dev)
    yield
    ms = c.timed(n, lambda i: gd.gdn_prefill(q, k, v, a, b, form="chunked", chunk=64, out=out, S_out=S, workspace=ws),
                 warm=3)
    nbytes = B * H * T * path_bytes_per_head_token(d)
    # the plan with a lead segment when the workspace holds more than 256 / (B*H) segments per head
    lead = ws.numel() // (B * H * 3 * d * d * 4) * B * H > 256
    kernels = ["gdn_lead_map_kernel" if lead else "gdn_map_kernel", "gdn_combine_kernel", "gdn_out_kernel"]
    return {"workload": "gated delta prefill B=1 H=16 T=262144 d=128 chunk=64, bf16 I/O, fp32 state (inputs drawn "
                        "on the device)", "calls": n, "ms_per_call": ms, "tokens_per_s": B * T / (ms * 1e-3),
            "roofline": hbm_roofline("gdn_prefill (" + " + ".join(kernels) + ")", nbytes, ms,
                                     [x + "_long" for x in kernels])}


def leg_kda_prefill(c):
    import synth
    torch, gd, n = c.torch, c.gd, c.args.la_steps
    w = synth.WORKLOADS[KDA_PREFILL]
    B, H, T, d = w["B"], w["H"], w["T"], w["dk"]
    q, k, v, a, b = synth.kda_batch(w["seed"], B, H, T, d, d, "bf16")
    sets = [tuple(c.up(x, True) for x in (q, k, v)) + tuple(c.up(x) for x in (a, b)) for _ in range(2)]
    del q, k, v, a, b
    ws = torch.empty(gd.la_workspace_bytes("kda_prefill", "bf16", B, H, T, d, d, "chunked", 64), dtype=torch.uint8,
                     device=c.dev)
    out = torch.empty((B, H, T, d), dtype=torch.bfloat16, device=c.dev)
    S = torch.empty((B, H, d, d), dtype=torch.float32, device=c.dev)

    def call(i, form="chunked"):
        gd.kda_prefill(*sets[i % 2], form=form, out=out, S_out=S, workspace=ws)

    yield
    ms = c.timed(n, call)
    rec_ms = c.timed(1, lambda i: call(i, "recurrent"), warm=0)
    # q, k, v, o in bf16, per-channel alpha and beta in fp32
    nbytes = B * H * T * (4 * d * 2 + d * 4 + 4)
    return {"workload": "KDA prefill B=2 H=16 T=8192 d=128 chunk=64 (block form: tile pass + column-parallel scan), "
                        "bf16 I/O, fp32 state", "calls": n, "ms_per_call": ms, "tokens_per_s": B * T / (ms * 1e-3),
            "recurrent_form_ms": rec_ms,
            "roofline": hbm_roofline("kda_tile_kernel + kda_scan_kernel", nbytes, ms,
                                     ["kda_tile_kernel", "kda_scan_kernel"])}


def leg_varlen(c):
    import synth
    torch, gd, n = c.torch, c.gd, c.args.la_steps
    w = synth.WORKLOADS[VARLEN]
    H, d, snap, N, Tt = w["H"], w["dk"], w["snap"], w["N"], w["T_total"]
    lens = synth.varlen_lengths(w["seed"], N, Tt)
    q, k, v, a, b, cu = synth.varlen_batch(w["seed"], lens, H, d, d, "bf16")
    sets = [tuple(c.up(x, True) for x in (q, k, v)) + tuple(c.up(x) for x in (a, b)) for _ in range(3)]
    cu_t = c.up(cu)
    del q, k, v, a, b
    nsnap = int(sum(int(L) // snap for L in lens))
    out = torch.empty((H, Tt, d), dtype=torch.bfloat16, device=c.dev)
    S = torch.empty((N, H, d, d), dtype=torch.float32, device=c.dev)
    S_snap = torch.empty((nsnap, H, d, d), dtype=torch.float32, device=c.dev)
    ws = torch.empty(gd.la_workspace_bytes("gdn_prefill_varlen", "bf16", N, H, Tt, d, d), dtype=torch.uint8,
                     device=c.dev)
    yield
    ms = c.timed(n, lambda i: gd.gdn_prefill_varlen(*sets[i % 3], cu_t, snap_interval=snap, snap_count=nsnap, out=out,
                                                     S_out=S, S_snap=S_snap, workspace=ws))
    nbytes = H * Tt * path_bytes_per_head_token(d) + (nsnap + N) * H * d * d * 4
    return {"workload": f"gated delta prefill, packed batch of {N} sequences ({Tt} tokens, lengths "
                        f"{int(min(lens))}..{int(max(lens))}), H=16 d=128 chunk=64, snapshots every {snap} tokens "
                        f"({nsnap})", "calls": n, "ms_per_call": ms, "tokens_per_s": Tt / (ms * 1e-3),
            "roofline": hbm_roofline("gdn_prefill_varlen (plan + map + combine + out)", nbytes, ms,
                                     [x + "_varlen_16seq" for x in ("gdn_varlen_plan_kernel", "gdn_map_kernel",
                                                                    "gdn_combine_kernel", "gdn_out_kernel")])}


def leg_varlen_kinds(c):
    """The packed batch of the varlen leg (same lengths, snapshots every 1024
    tokens) for the other kinds through lin_attn_prefill_varlen: block form
    on the matrix cores, and one call of the recurrent form for reference."""
    import numpy as np

    import synth
    torch, gd, n = c.torch, c.gd, c.args.la_steps
    w = synth.WORKLOADS[VARLEN]
    H, d, snap, N, Tt = w["H"], w["dk"], w["snap"], w["N"], w["T_total"]
    lens = synth.varlen_lengths(w["seed"], N, Tt)
    nsnap = int(sum(int(L) // snap for L in lens))
    ws = torch.empty(gd.la_workspace_bytes("prefill_varlen", "bf16", N, H, Tt, d, d, "chunked", 64), dtype=torch.uint8,
                     device=c.dev)
    out = torch.empty((H, Tt, d), dtype=torch.bfloat16, device=c.dev)
    S = torch.empty((N, H, d, d), dtype=torch.float32, device=c.dev)
    z = torch.empty((N, H, d), dtype=torch.float32, device=c.dev)
    S_snap = torch.empty((nsnap, H, d, d), dtype=torch.float32, device=c.dev)
    z_snap = torch.empty((nsnap, H, d), dtype=torch.float32, device=c.dev)
    inputs = {}
    for kind in ("normalized", "gated", "kda"):
        q, k, v, a, b, cu = synth.varlen_kind_batch(w["seed"], kind, lens, H, d, d, "bf16",
                                                    1 / np.sqrt(d) if kind == "normalized" else 1.0)
        inputs[kind] = tuple(c.up(x, True) for x in (q, k, v)) + tuple(None if x is None else c.up(x) for x in (a, b))
        cu_t = c.up(cu)
    del q, k, v, a, b

    def call(kind, form):
        has_z = kind == "normalized"
        gd.lin_attn_prefill_varlen(kind, *inputs[kind][:3], cu_t, *inputs[kind][3:], form=form, snap_interval=snap,
                                   snap_count=nsnap, out=out, S_out=S, z_out=z if has_z else None, S_snap=S_snap,
                                   z_snap=z_snap if has_z else None, workspace=ws)

    yield
    res = {"workload": f"packed batch of {N} sequences ({Tt} tokens, lengths {int(min(lens))}..{int(max(lens))}), "
                       f"H=16 d=128, bf16 I/O, fp32 state, snapshots every {snap} tokens ({nsnap}); kinds through "
                       "lin_attn_prefill_varlen", "calls": n, "block_form_ms": {}, "recurrent_form_ms": {}}
    for kind in inputs:
        res["block_form_ms"][kind] = c.timed(n, lambda i: call(kind, "chunked"))
        res["recurrent_form_ms"][kind] = c.timed(1, lambda i: call(kind, "recurrent"), warm=0)
    return res


def leg_copy(c):
    # a plain copy of known size: under rocprofv3 --pmc its FETCH_SIZE and
    # WRITE_SIZE give the factor that turns those counters into bytes
    yield
    torch = c.torch
    src = torch.empty(64 << 20, dtype=torch.float32, device=c.dev).fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    return {"bytes": src.numel() * 4}


def leg_prefill(c):
    """The headline: W untimed steps, then exactly K timed steps between two
    synchronisations; events around the call of every fourth step."""
    import numpy as np

    import synth
    torch, gd, args = c.torch, c.gd, c.args
    w = synth.WORKLOADS[PREFILL]
    B, H, T, d, C = w["B"], w["H"], w["T"], w["dk"], w["chunk"]
    q, k, v, a, b = synth.gdn_batch(w["seed"], B, H, T, d, d, "bf16")
    sets = [tuple(c.up(x, True) for x in (q, k, v)) + tuple(c.up(x) for x in (a, b)) for _ in range(3)]
    del q, k, v, a, b
    ws = gd.gdn_workspace(sets[0][0], sets[0][2], C)
    out = torch.empty((B, H, T, d), dtype=torch.bfloat16, device=c.dev)
    S_out = torch.empty((B, H, d, d), dtype=torch.float32, device=c.dev)

    def step(i, ev=None):
        tq, tk, tv, ta, tb = sets[i % 3]
        if ev is not None:
            ev[0].record()
        gd.gdn_prefill(tq, tk, tv, ta, tb, None, form="chunked", chunk=C, out=out, S_out=S_out, workspace=ws)
        if ev is not None:
            ev[1].record()

    yield
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # an event record costs a few microseconds of GPU time, so only every
    # fourth timed step carries events
    sampled = set(range(min(1, args.steps - 1), args.steps, 4))
    evs = {i: [torch.cuda.Event(enable_timing=True) for _ in range(2)] for i in sampled}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, evs.get(i))
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    step_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs.values()]))
    head_tokens = B * H * T
    # segments per head, from the workspace size (3 fp32 d x d matrices per
    # head-segment); more than 256 / (B*H) means the plan with a lead segment
    # (segment 0 runs beside the maps in gdn_lead_map_kernel)
    G = max(1, ws.numel() // (B * H * 3 * d * d * 4)) if ws is not None and ws.numel() > 16 else 1
    lead = G * B * H > 256
    # Roofline of the whole step (every kernel of the call: gdn_lead_map_kernel
    # or gdn_map_kernel, gdn_combine_kernel, gdn_out_kernel): algorithmic
    # bytes = the path's minimal I/O per head-token (q, k, v, o in bf16, alpha,
    # beta in fp32) times the head-tokens of the step, over the event time of
    # the call.  The counter figures (HBM bytes, MFMA busy) come from rocprofv3
    # runs stored under profiles/ and are null once the source has changed.
    step_kernels = ["gdn_lead_map_kernel" if lead else "gdn_map_kernel", "gdn_combine_kernel", "gdn_out_kernel"]
    alg_bytes = head_tokens * path_bytes_per_head_token(d)
    alg_flops = head_tokens * path_flops_per_head_token(d, C)
    tflops = alg_flops / (step_ms * 1e-3) / 1e12
    pmc = measured_pmc(step_kernels)
    roof = hbm_roofline("gdn_prefill step (" + " + ".join(step_kernels) + ")", alg_bytes, step_ms, step_kernels)
    roof["segments_per_head"] = G
    roof["lead_segment"] = lead
    # The HBM roofline is the one that bounds this path (its intensity, 136
    # flop/B, is below the chip's ridge); what holds the step below it is the
    # serial chain of 64-token chunks inside each segment: per chunk, the
    # state carriers' matrix-core groups, operand conversions and barriers.
    roof["limiter"] = ("latency of the per-chunk chain in each segment (MFMA busy "
                       + (f"{pmc['busy_frac']:.0%}" if pmc else "n/a") + " by counters)")
    return {"elapsed": elapsed, "ms_per_step": elapsed * 1e3 / args.steps,
            "tokens_per_s": B * T * args.steps / elapsed, "roofline": roof,
            "mfma": {"algorithmic_flops_per_step": alg_flops, "achieved_TFLOPs": tflops,
                     "peak_TFLOPs": BF16_PEAK_TFLOPS, "frac": tflops / BF16_PEAK_TFLOPS,
                     "counter_busy_frac": None if pmc is None else pmc["busy_frac"],
                     "counter_flops_per_step": None if pmc is None else pmc["flops"],
                     "counter_kernels": None if pmc is None else pmc["kernels"]}}


def settle(c, ms):
    """About `ms` milliseconds of untimed GPU work (repeated decode steps of a
    small batch) before anything is measured: the GPU raises its clocks only
    after several milliseconds of sustained work, and without this the first
    leg would be timed on a cold GPU (this memory-bound load does not bring
    the compute-bound legs to their settled speed)."""
    torch, gd = c.torch, c.gd
    if ms <= 0:
        return
    N, H, d = 64, 32, 128
    S = torch.zeros((N, H, d, d), dtype=torch.float32, device=c.dev)
    x = torch.zeros((N, H, d), dtype=torch.bfloat16, device=c.dev)
    o = torch.empty_like(x)
    a = torch.ones((N, H), dtype=torch.float32, device=c.dev)
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < ms:
        for _ in range(50):
            gd.lin_attn_decode_step("gated_delta", x, x, x, S, alpha=a, beta=a, out=o)
        torch.cuda.synchronize()


# ------------------------------------------------------ CPU oracle baseline
def _oracle_worker(job):
    """One host process of the CPU baseline: the fp64 chunked oracle, BLAS held
    to one thread, over heads of the prefill workload (cycling from `first`)
    until `budget` seconds of oracle time have passed.  Input drawing is not
    timed."""
    seed, heads, first, T, d, C, budget = job
    from threadpoolctl import threadpool_limits

    import oracle
    import synth
    done, spent = 0, 0.0
    with threadpool_limits(limits=1):
        while spent < budget:
            bb, hh = heads[(first + done) % len(heads)]
            q, k, v, a, b = synth.gdn_head(seed, bb, hh, T, d, d, "bf16")
            ts = time.perf_counter()
            oracle.gdn_chunked(q, k, v, a, b, C)
            spent += time.perf_counter() - ts
            done += 1
    return done, spent


def cpu_baseline(w, seconds):
    """The fp64 oracle (chunked form) on the host's cores: one process per core
    (at most 16, the CPU share of one GPU), each with single-threaded BLAS and
    its own heads of the prefill workload, together spending about `seconds`
    of oracle time.  The rate is the sum of the processes' rates while all of
    them run."""
    import multiprocessing as mp
    from concurrent.futures import ProcessPoolExecutor

    B, H, T, d, C = w["B"], w["H"], w["T"], w["dk"], w["chunk"]
    host_cpus = len(os.sched_getaffinity(0))
    n = max(1, min(host_cpus, 16))
    heads = [(bb, hh) for bb in range(B) for hh in range(H)]
    jobs = [(w["seed"], heads, j, T, d, C, seconds / n) for j in range(n)]
    with ProcessPoolExecutor(max_workers=n, mp_context=mp.get_context("spawn")) as ex:
        res = list(ex.map(_oracle_worker, jobs))
    done = sum(r[0] for r in res)
    spent = sum(r[1] for r in res)
    head_tokens_per_s = sum(r[0] * T / r[1] for r in res)
    # one token of the workload carries H heads
    return {"value": head_tokens_per_s / H, "unit": "tokens/s", "cores": n, "kind": "oracle",
            "sample": f"{done} head passes over the {B * H} heads of the prefill workload ({done * T} head-tokens), "
                      f"fp64 chunked form, {n} processes x 1 BLAS thread, {spent:.1f} s of oracle time in all",
            "host_cpus": host_cpus, "blas_threads_per_process": 1, "seconds": spent}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--decode-steps", type=int, default=1000)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=24.0,
                    help="oracle time of the CPU baseline, summed over its processes")
    ap.add_argument("--la-steps", type=int, default=10, help="timed calls of each secondary prefill leg")
    ap.add_argument("--long-calls", type=int, default=8, help="timed calls of the 1 x 16 x 262144 prefill")
    ap.add_argument("--settle-ms", type=float, default=300.0,
                    help="untimed decode steps before the first leg, so that no leg starts on an idle GPU")
    ap.add_argument("--legs", default="all",
                    help="comma-separated legs to run (" + ",".join(LEGS) + "; 'copy' is a 256 MiB device copy "
                    "for counter scaling, off unless named); default all but copy")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); this path has no "
              "multi-GPU mode: each GPU would run its own share of heads independently.", file=sys.stderr)
        sys.exit(2)
    legs = [l for l in LEGS if l != "copy"] if args.legs == "all" else args.legs.split(",")
    bad = [l for l in legs if l not in LEGS]
    if bad:
        ap.error(f"unknown legs {bad}")
    if args.long_calls <= 0 and "long" in legs:
        legs.remove("long")

    c = Ctx(args)
    fns = {"la": leg_la, "gla": leg_gla, "preops": leg_preops, "decode": leg_decode, "long": leg_long,
           "kda_decode": leg_kda_decode, "kda_prefill": leg_kda_prefill, "varlen": leg_varlen, "varlen_kinds": leg_varlen_kinds,
           "prefill": leg_prefill, "copy": leg_copy}
    # Every leg first draws and uploads its inputs (seconds of host work, the
    # GPU idle); then the timed parts run back to back, in a fixed order with
    # the headline prefill last, so that no leg is timed right after an idle
    # gap (the GPU lowers its clocks when idle).
    order = [name for name in LEGS if name in legs]
    gens = {}
    for name in order:
        gens[name] = fns[name](c)
        next(gens[name])
    torch_sync = c.torch.cuda.synchronize
    torch_sync()
    settle(c, args.settle_ms)
    res = {}
    for name in order:
        try:
            next(gens[name])
        except StopIteration as stop:
            res[name] = stop.value

    import synth
    cpu = None if args.no_cpu else cpu_baseline(synth.WORKLOADS[PREFILL], args.cpu_seconds)
    p = res.get("prefill")
    rec = {
        "metric": "prefill tokens/s (gated delta, H=16,d=128) + decode state HBM GB/s at 1 GPU",
        "value": p["tokens_per_s"] if p else None,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": p["ms_per_step"] if p else None,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; q,k unit rows, v~N(0,1), alpha=sigmoid(N(3,1)), beta=sigmoid(N(0,1)))",
        "config": {"workload": "gated delta prefill B=2 H=16 T=8192 d_k=d_v=128 chunk=64, bf16 I/O, fp32 state",
                   "global_batch": 2, "seq_len": 8192, "heads": 16, "head_dim": 128, "chunk": 64,
                   "parallelism": "single GPU"},
        "roofline": p["roofline"] if p else None,
        "mfma": p["mfma"] if p else None,
        "decode": res.get("decode"),
        "la_prefill": res.get("la"),
        "gla_prefill": res.get("gla"),
        "preprocess": res.get("preops"),
        "long_context_prefill": res.get("long"),
        "kda_decode": res.get("kda_decode"),
        "kda_prefill": res.get("kda_prefill"),
        "varlen_prefill": res.get("varlen"),
        "varlen_prefill_other_kinds": res.get("varlen_kinds"),
        "legs_run": legs,
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
