"""Loops of the single-head oracle functions over [B, H, T, d] arrays.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Heads are independent in every form on the source page, so a batch is just
a loop over (b, h); nothing is fused or reordered.  Layouts: q, k [B,H,T,d_k],
v [B,H,T,d_v], alpha/beta [B,H,T], S [B,H,d_v,d_k], z [B,H,d_k].
An optional ``heads`` list of (b, h) pairs restricts the work to a sample.
"""

import numpy as np

from .linear_attention import phi, la_parallel, la_recurrent, la_chunked, gated_recurrent
from .gated_delta import gdn_recurrent, gdn_chunked
from .kda import kda_recurrent, kda_chunked


def _heads(B, H, heads):
    return [(b, h) for b in range(B) for h in range(H)] if heads is None else list(heads)


def lin_attn(q, k, v, form="chunked", chunk=64, S0=None, z0=None, heads=None):
    """Returns (o, S, z) over the batch (only the listed heads are filled)."""
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    o = np.zeros((B, H, T, dv))
    S = np.zeros((B, H, dv, dk))
    z = np.zeros((B, H, dk))
    for b, h in _heads(B, H, heads):
        s0 = None if S0 is None else S0[b, h]
        z_0 = None if z0 is None else z0[b, h]
        if form == "parallel":
            if (s0 is not None and np.any(s0)) or (z_0 is not None and np.any(z_0)):
                raise ValueError("the parallel form has no carried state")
            o[b, h] = la_parallel(q[b, h], k[b, h], v[b, h])
            S[b, h], z[b, h] = _final_la_state(k[b, h], v[b, h])
        elif form == "recurrent":
            o[b, h], S[b, h], z[b, h] = la_recurrent(q[b, h], k[b, h], v[b, h], s0, z_0)
        elif form == "chunked":
            o[b, h], S[b, h], z[b, h] = la_chunked(q[b, h], k[b, h], v[b, h], chunk, s0, z_0)
        else:
            raise ValueError(form)
    return o, S, z


def _final_la_state(k, v):
    """S_T = sum_j v_j phi(k_j)^T and z_T = sum_j phi(k_j): the sums S_i, z_i
    of the kernel-trick equation at i = T ("The kernel trick" section)."""
    fk = phi(k)
    return v.T @ fk, fk.sum(axis=0)


def gdn(q, k, v, alpha, beta, form="chunked", chunk=64, S0=None, heads=None):
    """Returns (o, S) over the batch (only the listed heads are filled)."""
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    o = np.zeros((B, H, T, dv))
    S = np.zeros((B, H, dv, dk))
    for b, h in _heads(B, H, heads):
        s0 = None if S0 is None else S0[b, h]
        if form == "recurrent":
            o[b, h], S[b, h] = gdn_recurrent(q[b, h], k[b, h], v[b, h], alpha[b, h], beta[b, h], s0)
        elif form == "chunked":
            o[b, h], S[b, h] = gdn_chunked(q[b, h], k[b, h], v[b, h], alpha[b, h], beta[b, h], chunk, s0)
        else:
            raise ValueError(form)
    return o, S


def gdn_step_heads(q, k, v, alpha, beta, S):
    """One Gated DeltaNet step for many independent heads at once.

    q, k [n, dk]; v [n, dv]; alpha, beta [n]; S [n, dv, dk].  The equation of
    section "Delta rule and Gated DeltaNet" applied to every head; np.matmul
    broadcasts over the head axis.  Returns (o [n, dv], S_new).
    """
    q, k, v, alpha, beta, S = (np.asarray(a, dtype=np.float64) for a in (q, k, v, alpha, beta, S))
    dk = k.shape[-1]
    P = np.eye(dk)[None] - beta[:, None, None] * (k[:, :, None] * k[:, None, :])
    S_new = alpha[:, None, None] * (S @ P) + beta[:, None, None] * (v[:, :, None] * k[:, None, :])
    return (S_new @ q[:, :, None])[..., 0], S_new


def la_step_heads(q, k, v, S, z):
    """One normalised linear-attention step for many independent heads.

    q, k [n, dk]; v [n, dv]; S [n, dv, dk]; z [n, dk].  The recurrent form of
    section "Three forms of one computation" applied to every head.
    Returns (o [n, dv], S_new, z_new).
    """
    q, k, v, S, z = (np.asarray(a, dtype=np.float64) for a in (q, k, v, S, z))
    fk, fq = phi(k), phi(q)
    S_new = S + v[:, :, None] * fk[:, None, :]
    z_new = z + fk
    o = (S_new @ fq[:, :, None])[..., 0] / np.sum(z_new * fq, axis=1)[:, None]
    return o, S_new, z_new


def gla(q, k, v, alpha, S0=None, heads=None):
    """Gated (scalar-gate) unnormalised linear attention over the batch with
    the recurrent definition; returns (o, S) (only the listed heads filled)."""
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    o = np.zeros((B, H, T, dv))
    S = np.zeros((B, H, dv, dk))
    for b, h in _heads(B, H, heads):
        s0 = None if S0 is None else S0[b, h]
        o[b, h], S[b, h] = gated_recurrent(q[b, h], k[b, h], v[b, h], alpha[b, h], s0)
    return o, S


def gla_step_heads(q, k, v, alpha, S):
    """One gated linear-attention step for many independent heads at once:
    S <- alpha S + v k^T, o = S q (section "Memory must forget: decay and
    gates"), broadcast over the head axis.  Returns (o [n, dv], S_new)."""
    q, k, v, alpha, S = (np.asarray(a, dtype=np.float64) for a in (q, k, v, alpha, S))
    S_new = alpha[:, None, None] * S + v[:, :, None] * k[:, None, :]
    return (S_new @ q[:, :, None])[..., 0], S_new


def kda(q, k, v, alpha, beta, S0=None, form="recurrent", chunk=64, heads=None):
    """KDA over the batch (alpha [B,H,T,d_k] per channel); returns (o, S)
    with only the listed heads filled."""
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    o = np.zeros((B, H, T, dv))
    S = np.zeros((B, H, dv, dk))
    for b, h in _heads(B, H, heads):
        s0 = None if S0 is None else S0[b, h]
        if form == "recurrent":
            o[b, h], S[b, h] = kda_recurrent(q[b, h], k[b, h], v[b, h], alpha[b, h], beta[b, h], s0)
        elif form == "chunked":
            o[b, h], S[b, h] = kda_chunked(q[b, h], k[b, h], v[b, h], alpha[b, h], beta[b, h], chunk, s0)
        else:
            raise ValueError(form)
    return o, S


def kda_step_heads(q, k, v, alpha, beta, S):
    """One KDA step for many independent heads at once (alpha [n, d_k]):
    S <- S Diag(alpha) (I - beta k k^T) + beta v k^T, o = S q, broadcast over
    the head axis.  Returns (o [n, dv], S_new)."""
    q, k, v, alpha, beta, S = (np.asarray(a, dtype=np.float64) for a in (q, k, v, alpha, beta, S))
    Sd = S * alpha[:, None, :]
    Sk = (Sd @ k[:, :, None])[..., 0]                       # S Diag(alpha) k
    S_new = Sd - beta[:, None, None] * Sk[:, :, None] * k[:, None, :] + beta[:, None, None] * v[:, :, None] * k[:, None, :]
    return (S_new @ q[:, :, None])[..., 0], S_new
