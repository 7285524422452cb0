"""Variable-length packed batches and state snapshots for the gated delta
rule, in fp64.

TEST INFRASTRUCTURE ONLY (see the package docstring): used by tests/ and never
by the product path.

Source page: "Linear attention and hybrids" (ai.flicky.cc lesson 5.5.03),
section "Honest talk: why MiniMax went back to full attention", its point on
infrastructure: many implementations of these layers lack prefix caching
(reusing the work done for a shared beginning of different requests).  For a recurrent layer the reusable part of a prefix is
its state: the state after p tokens is everything a continuation needs.
Readings where the page is silent:
* a packed batch holds N sequences back to back along the token axis,
  per head: q, k [H, T_total, d_k], v [H, T_total, d_v], alpha, beta
  [H, T_total]; cu_seqlens[n] .. cu_seqlens[n+1] are the tokens of
  sequence n; every sequence starts from its own state S0[n] (zeros when
  absent) and returns its own final state;
* a snapshot is the state after p tokens of a sequence for every p that is a
  positive multiple of the snapshot interval and at most the sequence's
  length, numbered sequence by sequence in order of p.
Every sequence is the Gated DeltaNet recurrence of the same section
(gdn_recurrent), run on its own slice; form="chunked" evaluates each piece
with the chunk form gdn_chunked (chunk 64) instead, which is faster for large
head sizes and agrees with the recurrence up to rounding.
"""

import numpy as np

from .gated_delta import gdn_recurrent, gdn_chunked


def gdn_varlen(q, k, v, alpha, beta, cu_seqlens, S0=None, snap_interval=0, form="recurrent"):
    """Returns (o [H, T_total, d_v], S_final [N, H, d_v, d_k], snaps
    [n_snaps, H, d_v, d_k])."""
    if form == "recurrent":
        run = gdn_recurrent
    elif form == "chunked":
        def run(Q, K, V, A, B, S):
            return gdn_chunked(Q, K, V, A, B, 64, S)
    else:
        raise ValueError(form)
    q, k, v, alpha, beta = (np.asarray(a, dtype=np.float64) for a in (q, k, v, alpha, beta))
    H, Ttot, dk = q.shape
    dv = v.shape[-1]
    cu = [int(x) for x in cu_seqlens]
    N = len(cu) - 1
    o = np.zeros((H, Ttot, dv))
    S_fin = np.zeros((N, H, dv, dk))
    snaps = []
    for n in range(N):
        a, b = cu[n], cu[n + 1]
        per_head = []
        for h in range(H):
            S = None if S0 is None else np.asarray(S0[n, h], dtype=np.float64)
            states = []
            # run piecewise between snapshot positions, carrying the state
            start = a
            cuts = [a + p for p in range(snap_interval, b - a + 1, snap_interval)] if snap_interval > 0 else []
            ends = cuts + ([b] if not cuts or cuts[-1] != b else [])
            for cut in ends:
                if cut > start:
                    o[h, start:cut], S = run(q[h, start:cut], k[h, start:cut], v[h, start:cut],
                                             alpha[h, start:cut], beta[h, start:cut], S)
                elif S is None:
                    S = np.zeros((dv, dk))
                if cut in cuts:
                    states.append(S.copy())
                start = cut
            S_fin[n, h] = np.zeros((dv, dk)) if S is None else S
            per_head.append(states)
        for j in range(len(per_head[0]) if H > 0 else 0):
            snaps.append(np.stack([per_head[h][j] for h in range(H)]))
    snaps = np.stack(snaps) if snaps else np.zeros((0, H, dv, dk))
    return o, S_fin, snaps


def snapshot_count(cu_seqlens, snap_interval):
    """Number of snapshots of a packed batch."""
    if snap_interval <= 0:
        return 0
    cu = [int(x) for x in cu_seqlens]
    return sum((cu[n + 1] - cu[n]) // snap_interval for n in range(len(cu) - 1))
