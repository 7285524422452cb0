"""Benchmark of the gated-delta prefill and decode hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu]

One timed step is one chunked gated-delta prefill (state-independent pass +
sequential scan) over the 2 x 16 x 8192 workload (B=2, H=16, T=8192,
d_k = d_v = 128, bf16 activations, fp32 state, chunk 64), inputs resident in
HBM.  `value` is prefill tokens/s (B*T tokens per step).  In the same run,
each reported beside the headline: the decode workload (256 sequences x 32
heads, d = 128, fp32 state, 1000 steps) as state HBM GB/s; the normalised and
the scalar-gated linear-attention prefills; the 1 x 16 x 262144 long-context
prefill; the fused pre-operations of a
Gated DeltaNet layer; the KDA decode and prefill (block and recurrent forms); a packed batch of
16 sequences of mixed lengths with state snapshots; and the fp64 CPU oracle on
a bounded sample of the prefill workload.  Prints one JSON line.

Per-kernel durations come from HIP events recorded on the stream the kernels
are launched on (torch's current stream, which the binding passes to the C
ABI): around the two launches of every fourth timed prefill step, and around
each other leg's run of back-to-back calls (an event record costs a few
microseconds of GPU time).  Input sets rotate over three copies so the 256 MB
last-level cache cannot serve one step's inputs from the previous step.
"""

import argparse
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

# Algorithmic work per head-token of the chunked gated-delta path, chunk C,
# d = d_k = d_v: bytes = q, k, v, o in bf16 + alpha, beta in fp32; flops as
# the chunk form computes them with triangular halves counted once:
# 5 C d + C^2 / 3 + 6 d^2.
def path_bytes_per_head_token(d):
    return 4 * d * 2 + 8


def path_flops_per_head_token(d, C):
    return 5 * C * d + C * C / 3 + 6 * d * d


# HBM bytes per dispatch measured with rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE
# (scaled by the same counters on a plain copy of known size), stored per
# kernel with the hash of the source file it was built from; numbers taken on
# another version of that source are not used.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")


def measured_traffic(kernels):
    """Summed HBM bytes per launch of `kernels`, or None when any of them has
    no counters for its current source."""
    import hashlib
    try:
        rec = json.load(open(TRAFFIC_FILE))["kernels"]
        total = 0.0
        for k in kernels:
            src = os.path.join(ROOT, rec[k]["source"])
            if hashlib.sha256(open(src, "rb").read()).hexdigest() != rec[k]["source_sha256"]:
                return None
            total += rec[k]["bytes_per_dispatch"]
        return total
    except (OSError, KeyError, ValueError):
        return None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # the GPU's clocks take several milliseconds of work to settle: 100 untimed
    # steps (about 16 ms) come before the 200 timed ones
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--decode-steps", type=int, default=1000)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--la-steps", type=int, default=10, help="timed calls of the linear-attention prefill")
    ap.add_argument("--long-calls", type=int, default=2,
                    help="timed calls of the 1 x 16 x 262144 prefill (0 skips that leg, e.g. under a profiler)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a plain 256 MiB device copy (the reference kernel for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); this path has no "
              "multi-GPU mode: each GPU would run its own share of heads independently.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import gated_delta_rule_causal_amd as gd
    import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    gd._load()

    # ------------------------------------------------------------ prefill
    w = synth.WORKLOADS[PREFILL]
    B, H, T, d, C = w["B"], w["H"], w["T"], w["dk"], w["chunk"]
    q, k, v, a, b = synth.gdn_batch(w["seed"], B, H, T, d, d, "bf16")
    sets = []
    for _ in range(3):
        sets.append(tuple(torch.from_numpy(x).to(dev).to(torch.bfloat16) for x in (q, k, v)) +
                    tuple(torch.from_numpy(x).to(dev) for x in (a, b)))
    del q, k, v, a, b
    ws = gd.gdn_workspace(sets[0][0], sets[0][2], C)
    out = torch.empty((B, H, T, d), dtype=torch.bfloat16, device=dev)
    S_out = torch.empty((B, H, d, d), dtype=torch.float32, device=dev)

    def step(i, ev=None):
        tq, tk, tv, ta, tb = sets[i % 3]
        if ev is not None:
            ev[0].record()
        gd.gdn_prefill_prep(tq, tk, tv, ta, tb, ws, chunk=C)
        if ev is not None:
            ev[1].record()
        gd.gdn_prefill_scan(tq, tk, tv, ta, tb, ws, None, out=out, S_out=S_out, chunk=C)
        if ev is not None:
            ev[2].record()

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # Per-kernel durations come from events recorded around the two launches of
    # every fourth step of the timed run (an event record costs a few
    # microseconds of GPU time, so recording them on every step would inflate
    # the step time that `value` reports).
    sampled = set(range(min(1, args.steps - 1), args.steps, 4))
    evs = {i: [torch.cuda.Event(enable_timing=True) for _ in range(3)] for i in sampled}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, evs.get(i))
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    prep_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs.values()]))
    scan_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in evs.values()]))
    ms_per_step = elapsed * 1e3 / args.steps
    tokens_per_s = B * T * args.steps / elapsed
    head_tokens = B * H * T
    # segments per head, from the workspace size (3 fp32 d x d matrices per head-segment)
    mat = d * d * 4
    G = max(1, ws.numel() // (B * H * 3 * mat)) if ws.numel() > 16 else 1
    # compulsory bytes of each call in this design (inputs read once, outputs written once):
    #   prep  = segment maps: k, v, alpha, beta of the first G-1 segments; (M, N) per head-segment
    #   scan  = combine (maps + entering states) + outputs: q, k, v, alpha, beta, o, entering
    #           states, final state
    # roofline of the dominant launch: algorithmic bytes = the path's minimal
    # I/O per head-token (q, k, v, o in bf16, alpha, beta in fp32) times the
    # head-tokens one launch processes (all of them, for either launch)
    alg_bytes = head_tokens * path_bytes_per_head_token(d)
    kern = {"gdn_prefill_prep (gdn_map_kernel)": (prep_ms, ["gdn_map_kernel"]),
            "gdn_prefill_scan (gdn_combine_kernel + gdn_out_kernel)": (scan_ms,
                                                                       ["gdn_combine_kernel", "gdn_out_kernel"])}
    dom = max(kern, key=lambda n: kern[n][0])
    dom_ms, dom_kernels = kern[dom]
    dom_gbps = alg_bytes / (dom_ms * 1e-3) / 1e9
    dom_traffic = measured_traffic(dom_kernels)
    path_gbps = head_tokens * path_bytes_per_head_token(d) / ((prep_ms + scan_ms) * 1e-3) / 1e9
    path_tflops = head_tokens * path_flops_per_head_token(d, C) / ((prep_ms + scan_ms) * 1e-3) / 1e12

    if args.copy_probe:
        # a plain copy of known size: under rocprofv3 --pmc its FETCH_SIZE and
        # WRITE_SIZE give the factor that turns those counters into bytes
        src = torch.empty(64 << 20, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # ------------------------------------------- linear-attention prefill
    wl = synth.WORKLOADS[LA_PREFILL]
    Bl, Hl, Tl, dl, Cl = wl["B"], wl["H"], wl["T"], wl["dk"], wl["chunk"]
    lq, lk, lv = synth.la_batch(wl["seed"], Bl, Hl, Tl, dl, dl, "bf16", wl["scale"])
    la_sets = [tuple(torch.from_numpy(x).to(dev).to(torch.bfloat16) for x in (lq, lk, lv)) for _ in range(3)]
    del lq, lk, lv
    la_out = torch.empty((Bl, Hl, Tl, dl), dtype=torch.bfloat16, device=dev)
    la_S = torch.empty((Bl, Hl, dl, dl), dtype=torch.float32, device=dev)
    la_z = torch.empty((Bl, Hl, dl), dtype=torch.float32, device=dev)
    for i in range(2):
        gd.lin_attn_prefill(*la_sets[i % 3], form="chunked", chunk=Cl, out=la_out, S_out=la_S, z_out=la_z)
    torch.cuda.synchronize()
    # the calls of each leg below run back to back between two events
    la_ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    la_ev[0].record()
    for i in range(args.la_steps):
        gd.lin_attn_prefill(*la_sets[i % 3], form="chunked", chunk=Cl, out=la_out, S_out=la_S, z_out=la_z)
    la_ev[1].record()
    torch.cuda.synchronize()
    la_ms = la_ev[0].elapsed_time(la_ev[1]) / args.la_steps
    la_head_tokens = Bl * Hl * Tl
    la_bytes = la_head_tokens * 4 * dl * 2           # q, k, v, o in bf16
    la_flops = la_head_tokens * (2 * Cl * dl + 4 * dl * dl)
    la_gbps = la_bytes / (la_ms * 1e-3) / 1e9
    del la_sets

    # --------------------------------- scalar-gated linear-attention prefill
    wg = synth.WORKLOADS[GLA_PREFILL]
    gq, gk, gv, ga, _ = synth.gdn_batch(wg["seed"], wg["B"], wg["H"], wg["T"], wg["dk"], wg["dv"], "bf16")
    gla_sets = [tuple(torch.from_numpy(x).to(dev).to(torch.bfloat16) for x in (gq, gk, gv)) +
                (torch.from_numpy(ga).to(dev),) for _ in range(3)]
    del gq, gk, gv, ga
    gla_out = torch.empty((wg["B"], wg["H"], wg["T"], wg["dv"]), dtype=torch.bfloat16, device=dev)
    gla_S = torch.empty((wg["B"], wg["H"], wg["dv"], wg["dk"]), dtype=torch.float32, device=dev)
    for i in range(2):
        gd.gla_prefill(*gla_sets[i % 3], form="chunked", chunk=wg["chunk"], out=gla_out, S_out=gla_S)
    torch.cuda.synchronize()
    g_ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    g_ev[0].record()
    for i in range(args.la_steps):
        gd.gla_prefill(*gla_sets[i % 3], form="chunked", chunk=wg["chunk"], out=gla_out, S_out=gla_S)
    g_ev[1].record()
    torch.cuda.synchronize()
    gla_ms = g_ev[0].elapsed_time(g_ev[1]) / args.la_steps
    gla_bytes = wg["B"] * wg["H"] * wg["T"] * (4 * wg["dk"] * 2 + 4)   # q, k, v, o bf16 + alpha fp32
    gla_gbps = gla_bytes / (gla_ms * 1e-3) / 1e9
    del gla_sets

    # --------------------------------------- pre-operations of the layer
    wp = synth.WORKLOADS[PREOPS]
    Bp, Tp, Hp, dkp, dvp = wp["B"], wp["T"], wp["H"], wp["dk"], wp["dv"]
    px, pw, pa, pb = synth.preops_batch(wp["seed"], Bp, Tp, Hp, dkp, dvp, "bf16")
    x0 = torch.from_numpy(px).to(dev).to(torch.bfloat16)
    pre_sets = [(x0 if i == 0 else x0.clone(), torch.from_numpy(pw).to(dev), torch.from_numpy(pa).to(dev),
                 torch.from_numpy(pb).to(dev)) for i in range(3)]
    del px, pw, pa, pb, x0
    pre_out = dict(q=torch.empty((Bp, Hp, Tp, dkp), dtype=torch.bfloat16, device=dev),
                   k=torch.empty((Bp, Hp, Tp, dkp), dtype=torch.bfloat16, device=dev),
                   v=torch.empty((Bp, Hp, Tp, dvp), dtype=torch.bfloat16, device=dev),
                   alpha=torch.empty((Bp, Hp, Tp), dtype=torch.float32, device=dev),
                   beta=torch.empty((Bp, Hp, Tp), dtype=torch.float32, device=dev))
    for i in range(2):
        gd.gdn_preprocess(*pre_sets[i % 3], Hp, dkp, dvp, want_state=False, **pre_out)
    torch.cuda.synchronize()
    p_ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    p_ev[0].record()
    for i in range(args.la_steps):
        gd.gdn_preprocess(*pre_sets[i % 3], Hp, dkp, dvp, want_state=False, **pre_out)
    p_ev[1].record()
    torch.cuda.synchronize()
    pre_ms = p_ev[0].elapsed_time(p_ev[1]) / args.la_steps
    # x read + gate logits read, q, k, v written + alpha, beta written
    pre_bytes = Bp * Hp * Tp * (2 * ((2 * dkp + dvp) * 2 + 8))
    pre_gbps = pre_bytes / (pre_ms * 1e-3) / 1e9
    del pre_sets, pre_out

    # ------------------------------------------------------------- decode
    wd = synth.WORKLOADS[DECODE]
    N, Hd, dd, steps = wd["N"], wd["H"], wd["dk"], args.decode_steps
    S = torch.from_numpy(synth.decode_state_fast(wd["seed"], N, Hd, dd, dd, wd["state_std"])).to(dev)
    pool = []
    for e in range(8):
        tq, tk, tv, ta, tb = synth.decode_token_inputs(wd["seed"], N, Hd, dd, dd, "bf16", e)
        pool.append(tuple(torch.from_numpy(x).to(dev).to(torch.bfloat16) for x in (tq, tk, tv)) +
                    tuple(torch.from_numpy(x).to(dev) for x in (ta, tb)))
    o_dec = torch.empty((N, Hd, dd), dtype=torch.bfloat16, device=dev)
    for i in range(5):
        tq, tk, tv, ta, tb = pool[i % 8]
        gd.lin_attn_decode_step("gated_delta", tq, tk, tv, S, alpha=ta, beta=tb, out=o_dec)
    torch.cuda.synchronize()
    dev_ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    t0 = time.perf_counter()
    dev_ev[0].record()
    for i in range(steps):
        tq, tk, tv, ta, tb = pool[i % 8]
        gd.lin_attn_decode_step("gated_delta", tq, tk, tv, S, alpha=ta, beta=tb, out=o_dec)
    dev_ev[1].record()
    torch.cuda.synchronize()
    dec_elapsed = time.perf_counter() - t0
    dec_ms = dev_ev[0].elapsed_time(dev_ev[1]) / steps
    state_bytes = 2 * N * Hd * dd * dd * 4
    io_bytes = N * Hd * (3 * dd * 2 + dd * 2 + 8)
    dec_state_gbps = state_bytes / (dec_ms * 1e-3) / 1e9
    dec_total_gbps = (state_bytes + io_bytes) / (dec_ms * 1e-3) / 1e9

    # ------------------------------------ long-context prefill (1 x 16 x 262144)
    # Inputs drawn on the device (torch's seeded generator, the distributions
    # of the synthetic recipe): 3 GiB of bf16 activations would take minutes to
    # draw on the host.  Values do not change the work; the parity tests check
    # this shape against the oracle on the host-drawn inputs.
    long_ms = long_gbps = None
    wl5 = synth.WORKLOADS[LONG]
    B5, H5, T5, d5 = wl5["B"], wl5["H"], wl5["T"], wl5["dk"]
    if args.long_calls > 0:
        g5 = torch.Generator(device=dev)
        g5.manual_seed(wl5["seed"])
        norm = torch.nn.functional.normalize
        l_q = norm(torch.randn(B5, H5, T5, d5, device=dev, generator=g5), dim=-1).to(torch.bfloat16)
        l_k = norm(torch.randn(B5, H5, T5, d5, device=dev, generator=g5), dim=-1).to(torch.bfloat16)
        l_v = torch.randn(B5, H5, T5, d5, device=dev, generator=g5).to(torch.bfloat16)
        l_a = torch.sigmoid(torch.randn(B5, H5, T5, device=dev, generator=g5) + 3.0)
        l_b = torch.sigmoid(torch.randn(B5, H5, T5, device=dev, generator=g5))
        l_ws = gd.gdn_workspace(l_q, l_v, 64)
        l_out = torch.empty_like(l_v)
        l_S = torch.empty((B5, H5, d5, d5), dtype=torch.float32, device=dev)
        gd.gdn_prefill(l_q, l_k, l_v, l_a, l_b, form="chunked", chunk=64, out=l_out, S_out=l_S, workspace=l_ws)
        torch.cuda.synchronize()
        lev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        lev[0].record()
        for i in range(args.long_calls):
            gd.gdn_prefill(l_q, l_k, l_v, l_a, l_b, form="chunked", chunk=64, out=l_out, S_out=l_S, workspace=l_ws)
        lev[1].record()
        torch.cuda.synchronize()
        long_ms = lev[0].elapsed_time(lev[1]) / args.long_calls
        long_gbps = B5 * H5 * T5 * path_bytes_per_head_token(d5) / (long_ms * 1e-3) / 1e9
        del l_q, l_k, l_v, l_a, l_b, l_ws, l_out, l_S

    # ---------------------------------------------- KDA decode (per-channel decay)
    wk = synth.WORKLOADS[KDA_DECODE]
    Nk, Hk, dkk = wk["N"], wk["H"], wk["dk"]
    Sk = torch.from_numpy(synth.decode_state_fast(wk["seed"], Nk, Hk, dkk, dkk, wk["state_std"])).to(dev)
    kpool = []
    for e in range(8):
        tq, tk, tv, ta, tb = synth.kda_decode_token_inputs(wk["seed"], Nk, Hk, dkk, dkk, "bf16", e)
        kpool.append(tuple(torch.from_numpy(x).to(dev).to(torch.bfloat16) for x in (tq, tk, tv)) +
                     tuple(torch.from_numpy(x).to(dev) for x in (ta, tb)))
    ok_dec = torch.empty((Nk, Hk, dkk), dtype=torch.bfloat16, device=dev)
    for i in range(5):
        tq, tk, tv, ta, tb = kpool[i % 8]
        gd.lin_attn_decode_step("kda", tq, tk, tv, Sk, alpha=ta, beta=tb, out=ok_dec)
    torch.cuda.synchronize()
    kev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    kev[0].record()
    for i in range(steps):
        tq, tk, tv, ta, tb = kpool[i % 8]
        gd.lin_attn_decode_step("kda", tq, tk, tv, Sk, alpha=ta, beta=tb, out=ok_dec)
    kev[1].record()
    torch.cuda.synchronize()
    kda_dec_ms = kev[0].elapsed_time(kev[1]) / steps
    # state read + write, q k v o in bf16, alpha per channel and beta in fp32
    kda_dec_bytes = 2 * Nk * Hk * dkk * dkk * 4 + Nk * Hk * (4 * dkk * 2 + dkk * 4 + 4)
    kda_dec_gbps = kda_dec_bytes / (kda_dec_ms * 1e-3) / 1e9
    del Sk, kpool

    # ------------------------- KDA prefill: block form (and the recurrent form)
    wkp = synth.WORKLOADS[KDA_PREFILL]
    Bk, Hkp, Tk, dkp = wkp["B"], wkp["H"], wkp["T"], wkp["dk"]
    kq, kk, kv, ka, kb = synth.kda_batch(wkp["seed"], Bk, Hkp, Tk, dkp, dkp, "bf16")
    kda_sets = [tuple(torch.from_numpy(x).to(dev).to(torch.bfloat16) for x in (kq, kk, kv)) +
                tuple(torch.from_numpy(x).to(dev) for x in (ka, kb)) for _ in range(2)]
    del kq, kk, kv, ka, kb
    kda_ws = torch.empty(gd.la_workspace_bytes("kda_prefill", "bf16", Bk, Hkp, Tk, dkp, dkp, "chunked", 64),
                         dtype=torch.uint8, device=dev)
    kda_out = torch.empty((Bk, Hkp, Tk, dkp), dtype=torch.bfloat16, device=dev)
    kda_S = torch.empty((Bk, Hkp, dkp, dkp), dtype=torch.float32, device=dev)

    def kcall(i, form="chunked"):
        gd.kda_prefill(*kda_sets[i % 2], form=form, out=kda_out, S_out=kda_S, workspace=kda_ws)

    for i in range(2):
        kcall(i)
    torch.cuda.synchronize()
    kpe = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    kpe[0].record()
    for i in range(args.la_steps):
        kcall(i)
    kpe[1].record()
    torch.cuda.synchronize()
    kda_pre_ms = kpe[0].elapsed_time(kpe[1]) / args.la_steps
    # q, k, v, o in bf16, per-channel alpha and beta in fp32
    kda_pre_bytes = Bk * Hkp * Tk * (4 * dkp * 2 + dkp * 4 + 4)
    kda_pre_gbps = kda_pre_bytes / (kda_pre_ms * 1e-3) / 1e9
    kre = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    kre[0].record()
    kcall(0, "recurrent")
    kre[1].record()
    torch.cuda.synchronize()
    kda_rec_ms = kre[0].elapsed_time(kre[1])
    del kda_sets, kda_ws, kda_out, kda_S

    # ------------------------------- packed variable-length batch + snapshots
    wv = synth.WORKLOADS[VARLEN]
    Hv, dvv, snapv = wv["H"], wv["dk"], wv["snap"]
    lens = synth.varlen_lengths(wv["seed"], wv["N"], wv["T_total"])
    vq, vk, vv, va, vb, vcu = synth.varlen_batch(wv["seed"], lens, Hv, dvv, dvv, "bf16")
    vsets = [tuple(torch.from_numpy(x).to(dev).to(torch.bfloat16) for x in (vq, vk, vv)) +
             tuple(torch.from_numpy(x).to(dev) for x in (va, vb)) for _ in range(3)]
    vcu_t = torch.from_numpy(vcu).to(dev)
    del vq, vk, vv, va, vb
    nsnap = int(sum(int(L) // snapv for L in lens))
    v_out = torch.empty((Hv, wv["T_total"], dvv), dtype=torch.bfloat16, device=dev)
    v_S = torch.empty((wv["N"], Hv, dvv, dvv), dtype=torch.float32, device=dev)
    v_snap = torch.empty((nsnap, Hv, dvv, dvv), dtype=torch.float32, device=dev)
    v_ws = torch.empty(gd.la_workspace_bytes("gdn_prefill_varlen", "bf16", wv["N"], Hv, wv["T_total"], dvv, dvv),
                       dtype=torch.uint8, device=dev)

    def vcall(i):
        gd.gdn_prefill_varlen(*vsets[i % 3], vcu_t, snap_interval=snapv, snap_count=nsnap, out=v_out, S_out=v_S,
                              S_snap=v_snap, workspace=v_ws)

    for i in range(2):
        vcall(i)
    torch.cuda.synchronize()
    vev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    vev[0].record()
    for i in range(args.la_steps):
        vcall(i)
    vev[1].record()
    torch.cuda.synchronize()
    var_ms = vev[0].elapsed_time(vev[1]) / args.la_steps
    var_bytes = Hv * wv["T_total"] * path_bytes_per_head_token(dvv) + (nsnap + wv["N"]) * Hv * dvv * dvv * 4
    var_gbps = var_bytes / (var_ms * 1e-3) / 1e9
    del vsets, v_out, v_S, v_snap, v_ws

    # ----------------------------------------------------- CPU oracle baseline
    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(w, args.cpu_seconds)

    rec = {
        "metric": "prefill tokens/s (gated delta, H=16,d=128) + decode state HBM GB/s at 1 GPU",
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; q,k unit rows, v~N(0,1), alpha=sigmoid(N(3,1)), beta=sigmoid(N(0,1)))",
        "config": {"workload": "gated delta prefill B=2 H=16 T=8192 d_k=d_v=128 chunk=64, bf16 I/O, fp32 state",
                   "global_batch": B, "seq_len": T, "heads": H, "head_dim": d, "chunk": C,
                   "parallelism": "single GPU"},
        "roofline": {"kernel": dom, "bound": "hbm", "achieved": dom_gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": dom_gbps / HBM_PEAK_GBPS, "traffic": dom_traffic,
                     "bytes_per_launch": alg_bytes, "avg_launch_ms": dom_ms},
        "kernels_ms": {"gdn_prefill_prep": prep_ms, "gdn_prefill_scan": scan_ms, "segments_per_head": G},
        "path_roofline": {"bytes_per_head_token": path_bytes_per_head_token(d),
                          "flops_per_head_token": path_flops_per_head_token(d, C),
                          "achieved_GBps": path_gbps, "hbm_frac": path_gbps / HBM_PEAK_GBPS,
                          "achieved_TFLOPs": path_tflops, "mfma_frac": path_tflops / BF16_PEAK_TFLOPS},
        "decode": {"workload": "gated delta decode 256 seq x 32 heads, d=128, fp32 state, bf16 token I/O",
                   "steps": steps, "ms_per_step": dec_ms, "steps_per_s": 1e3 / dec_ms,
                   "wall_steps_per_s": steps / dec_elapsed,
                   "state_GBps": dec_state_gbps, "total_GBps": dec_total_gbps,
                   "roofline": {"kernel": "recurrent_kernel (decode)", "bound": "hbm",
                                "achieved": dec_total_gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                                "frac": dec_total_gbps / HBM_PEAK_GBPS,
                                "traffic": measured_traffic(["recurrent_kernel_gated_delta_decode"]),
                                "bytes_per_launch": state_bytes + io_bytes, "avg_launch_ms": dec_ms}},
        "la_prefill": {"workload": "normalised linear attention prefill B=4 H=16 T=4096 d=128 chunk=64, bf16 I/O, "
                                   "fp32 state", "calls": args.la_steps, "ms_per_call": la_ms,
                       "tokens_per_s": Bl * Tl / (la_ms * 1e-3),
                       "roofline": {"kernel": "la_chunked_mfma_kernel", "bound": "hbm", "achieved": la_gbps,
                                    "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": la_gbps / HBM_PEAK_GBPS,
                                    "bytes_per_launch": la_bytes, "avg_launch_ms": la_ms,
                                    "achieved_TFLOPs": la_flops / (la_ms * 1e-3) / 1e12}},
        "gla_prefill": {"workload": "scalar-gated linear attention prefill B=2 H=16 T=8192 d=128 chunk=64, bf16 "
                                    "I/O, fp32 state", "calls": args.la_steps, "ms_per_call": gla_ms,
                        "tokens_per_s": wg["B"] * wg["T"] / (gla_ms * 1e-3),
                        "roofline": {"kernel": "la_chunked_mfma_kernel (gated)", "bound": "hbm",
                                     "achieved": gla_gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                                     "frac": gla_gbps / HBM_PEAK_GBPS, "bytes_per_launch": gla_bytes,
                                     "avg_launch_ms": gla_ms}},
        "preprocess": {"workload": "Gated DeltaNet pre-operations (conv k=4, q/k L2 norm, sigmoid gates) B=2 "
                                   "H=16 T=8192 d=128, bf16 I/O", "calls": args.la_steps, "ms_per_call": pre_ms,
                       "tokens_per_s": Bp * Tp / (pre_ms * 1e-3),
                       "roofline": {"kernel": "gdn_preprocess_kernel", "bound": "hbm", "achieved": pre_gbps,
                                    "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": pre_gbps / HBM_PEAK_GBPS,
                                    "traffic": measured_traffic(["gdn_preprocess_kernel"]),
                                    "bytes_per_launch": pre_bytes, "avg_launch_ms": pre_ms}},
        "long_context_prefill": None if long_ms is None else {
            "workload": "gated delta prefill B=1 H=16 T=262144 d=128 chunk=64, bf16 I/O, fp32 state (inputs drawn "
                        "on the device)", "calls": args.long_calls, "ms_per_call": long_ms,
            "tokens_per_s": B5 * T5 / (long_ms * 1e-3),
            "roofline": {"kernel": "gdn_prefill (map + combine + out)", "bound": "hbm", "achieved": long_gbps,
                         "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": long_gbps / HBM_PEAK_GBPS,
                         "bytes_per_launch": B5 * H5 * T5 * path_bytes_per_head_token(d5), "avg_launch_ms": long_ms}},
        "kda_decode": {"workload": "KDA decode 256 seq x 32 heads, d=128, per-channel decay, fp32 state, bf16 "
                                   "token I/O", "steps": steps, "ms_per_step": kda_dec_ms,
                       "steps_per_s": 1e3 / kda_dec_ms,
                       "roofline": {"kernel": "recurrent_kernel (KDA decode)", "bound": "hbm",
                                    "achieved": kda_dec_gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                                    "frac": kda_dec_gbps / HBM_PEAK_GBPS, "bytes_per_launch": kda_dec_bytes,
                                    "avg_launch_ms": kda_dec_ms}},
        "kda_prefill": {"workload": "KDA prefill B=2 H=16 T=8192 d=128 chunk=64 (block form: tile pass + "
                                    "column-parallel scan), bf16 I/O, fp32 state", "calls": args.la_steps,
                        "ms_per_call": kda_pre_ms, "tokens_per_s": Bk * Tk / (kda_pre_ms * 1e-3),
                        "recurrent_form_ms": kda_rec_ms,
                        "roofline": {"kernel": "kda_tile_kernel + kda_scan_kernel", "bound": "hbm",
                                     "achieved": kda_pre_gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                                     "frac": kda_pre_gbps / HBM_PEAK_GBPS, "bytes_per_launch": kda_pre_bytes,
                                     "avg_launch_ms": kda_pre_ms}},
        "varlen_prefill": {"workload": f"gated delta prefill, packed batch of {wv['N']} sequences ({wv['T_total']} "
                                       f"tokens, lengths {int(min(lens))}..{int(max(lens))}), H=16 d=128 chunk=64, "
                                       f"snapshots every {snapv} tokens ({nsnap})",
                           "calls": args.la_steps, "ms_per_call": var_ms,
                           "tokens_per_s": wv["T_total"] / (var_ms * 1e-3),
                           "roofline": {"kernel": "gdn_prefill_varlen (plan + map + combine + out)", "bound": "hbm",
                                        "achieved": var_gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                                        "frac": var_gbps / HBM_PEAK_GBPS, "bytes_per_launch": var_bytes,
                                        "avg_launch_ms": var_ms}},
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


def cpu_baseline(w, seconds):
    """The fp64 oracle (chunked form), single-threaded BLAS, on the first heads
    of the prefill workload until `seconds` have passed."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle
    import synth

    B, H, T, d, C = w["B"], w["H"], w["T"], w["dk"], w["chunk"]
    done = 0
    spent = 0.0
    heads = [(bb, hh) for bb in range(B) for hh in range(H)]
    with threadpool_limits(limits=1):
        while spent < seconds:
            bb, hh = heads[done % len(heads)]
            q, k, v, a, b = synth.gdn_head(w["seed"], bb, hh, T, d, d, "bf16")
            ts = time.perf_counter()
            oracle.gdn_chunked(q, k, v, a, b, C)
            spent += time.perf_counter() - ts
            done += 1
    elapsed = spent
    # one token of the workload carries H heads
    return {"value": done * T / H / elapsed, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{done} head passes over the {B * H} heads of the prefill workload, cycling "
                      f"({done * T} head-tokens), fp64 chunked form, {elapsed:.1f} s of oracle time",
            "seconds": elapsed}


if __name__ == "__main__":
    main()
