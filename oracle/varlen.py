"""Variable-length packed batches and state snapshots, in fp64, for every
recurrence of the page: normalised linear attention, scalar-gated linear
attention, the gated delta rule and its per-channel-decay variant (KDA).

TEST INFRASTRUCTURE ONLY (see the package docstring): used by tests/ and never
by the product path.

Source page: "Linear attention and hybrids" (ai.flicky.cc lesson 5.5.03),
section "Honest talk: why MiniMax went back to full attention", its point on
infrastructure: many implementations of these layers lack prefix caching
(reusing the work done for a shared beginning of different requests).  For a
recurrent layer the reusable part of a prefix is its state (S, plus the
normaliser z for the normalised kind): the state after p tokens is everything
a continuation needs.
Readings where the page is silent:
* a packed batch holds N sequences back to back along the token axis,
  per head: q, k [H, T_total, d_k], v [H, T_total, d_v]; per-token gates
  alpha [H, T_total] (scalar-gated and gated-delta kinds) or
  [H, T_total, d_k] (KDA), beta [H, T_total]; cu_seqlens[n] ..
  cu_seqlens[n+1] are the tokens of sequence n; every sequence starts from
  its own state S0[n] [N, H, d_v, d_k] (and z0[n] [N, H, d_k]; zeros when
  absent) and returns its own final state;
* a snapshot is the state after p tokens of a sequence for every p that is a
  positive multiple of the snapshot interval and at most the sequence's
  length, numbered sequence by sequence in order of p.
Every sequence is the kind's own single-sequence recurrence (the separately
pinned la_recurrent, gated_recurrent, gdn_recurrent, kda_recurrent) run on its
own slice; form="chunked" evaluates each piece with the kind's chunk form
(chunk 64) instead, which agrees with the recurrence up to rounding (the
scalar-gated kind has no chunk form here).
"""

import numpy as np

from .gated_delta import gdn_recurrent, gdn_chunked
from .kda import kda_recurrent, kda_chunked
from .linear_attention import la_recurrent, la_chunked, gated_recurrent

KINDS = ("normalized", "gated_delta", "gated", "kda")


def _piece(kind, form):
    """run(Q, K, V, A, B, S, z) -> (O, S, z): one piece of one sequence of one
    head, from the carried state (None = zeros); z is None for kinds without
    a normaliser."""
    if form not in ("recurrent", "chunked"):
        raise ValueError(form)
    chunked = form == "chunked"
    if kind == "normalized":
        if chunked:
            return lambda Q, K, V, A, B, S, z: la_chunked(Q, K, V, 64, S, z)
        return lambda Q, K, V, A, B, S, z: la_recurrent(Q, K, V, S, z)
    if kind == "gated":
        if chunked:
            raise ValueError("the scalar-gated kind has no chunk form here")
        return lambda Q, K, V, A, B, S, z: gated_recurrent(Q, K, V, A, S) + (None,)
    if kind == "gated_delta":
        if chunked:
            return lambda Q, K, V, A, B, S, z: gdn_chunked(Q, K, V, A, B, 64, S) + (None,)
        return lambda Q, K, V, A, B, S, z: gdn_recurrent(Q, K, V, A, B, S) + (None,)
    if kind == "kda":
        if chunked:
            return lambda Q, K, V, A, B, S, z: kda_chunked(Q, K, V, A, B, 64, S) + (None,)
        return lambda Q, K, V, A, B, S, z: kda_recurrent(Q, K, V, A, B, S) + (None,)
    raise ValueError(kind)


def packed_varlen(kind, q, k, v, cu_seqlens, alpha=None, beta=None, S0=None, z0=None, snap_interval=0,
                  form="recurrent"):
    """Returns (o [H, T_total, d_v], S_final [N, H, d_v, d_k], z_final
    [N, H, d_k] or None, S_snaps [n_snaps, H, d_v, d_k], z_snaps
    [n_snaps, H, d_k] or None); the z outputs exist for the normalised kind
    only."""
    run = _piece(kind, form)
    has_z = kind == "normalized"
    q, k, v = (np.asarray(a, dtype=np.float64) for a in (q, k, v))
    H, Ttot, dk = q.shape
    dv = v.shape[-1]
    gate = None if alpha is None else np.asarray(alpha, dtype=np.float64)
    wgt = None if beta is None else np.asarray(beta, dtype=np.float64)
    cu = [int(x) for x in cu_seqlens]
    N = len(cu) - 1
    o = np.zeros((H, Ttot, dv))
    S_fin = np.zeros((N, H, dv, dk))
    z_fin = np.zeros((N, H, dk)) if has_z else None
    S_snaps, z_snaps = [], []
    for n in range(N):
        a, b = cu[n], cu[n + 1]
        cuts = [a + p for p in range(snap_interval, b - a + 1, snap_interval)] if snap_interval > 0 else []
        per_head = []
        for h in range(H):
            S = None if S0 is None else np.asarray(S0[n, h], dtype=np.float64)
            z = None if (not has_z or z0 is None) else np.asarray(z0[n, h], dtype=np.float64)
            states = []
            # run piecewise between snapshot positions, carrying the state
            start = a
            for cut in cuts + ([b] if not cuts or cuts[-1] != b else []):
                if cut > start:
                    A = None if gate is None else gate[h, start:cut]
                    B = None if wgt is None else wgt[h, start:cut]
                    o[h, start:cut], S, z = run(q[h, start:cut], k[h, start:cut], v[h, start:cut], A, B, S, z)
                if cut in cuts:
                    states.append((np.zeros((dv, dk)) if S is None else S.copy(),
                                   None if not has_z else (np.zeros(dk) if z is None else z.copy())))
                start = cut
            S_fin[n, h] = np.zeros((dv, dk)) if S is None else S
            if has_z:
                z_fin[n, h] = np.zeros(dk) if z is None else z
            per_head.append(states)
        for j in range(len(per_head[0]) if H > 0 else 0):
            S_snaps.append(np.stack([per_head[h][j][0] for h in range(H)]))
            if has_z:
                z_snaps.append(np.stack([per_head[h][j][1] for h in range(H)]))
    S_snaps = np.stack(S_snaps) if S_snaps else np.zeros((0, H, dv, dk))
    if has_z:
        z_snaps = np.stack(z_snaps) if z_snaps else np.zeros((0, H, dk))
    else:
        z_snaps = None
    return o, S_fin, z_fin, S_snaps, z_snaps


def gdn_varlen(q, k, v, alpha, beta, cu_seqlens, S0=None, snap_interval=0, form="recurrent"):
    """The gated delta rule over a packed batch: returns (o [H, T_total, d_v],
    S_final [N, H, d_v, d_k], snaps [n_snaps, H, d_v, d_k])."""
    o, S, _, snaps, _ = packed_varlen("gated_delta", q, k, v, cu_seqlens, alpha, beta, S0, None, snap_interval,
                                      form)
    return o, S, snaps


def snapshot_count(cu_seqlens, snap_interval):
    """Number of snapshots of a packed batch."""
    if snap_interval <= 0:
        return 0
    cu = [int(x) for x in cu_seqlens]
    return sum((cu[n + 1] - cu[n]) // snap_interval for n in range(len(cu) - 1))
