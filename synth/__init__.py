"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module only draws and rounds numbers; it holds none of the method's
arithmetic, and it imports neither the oracle nor the HIP library, so both
sides can consume the very same values.

Recipe (one generator per head, so any sample of heads can be regenerated
without drawing the rest):

* ``np.random.default_rng([seed, stream, b, h])`` with streams
  q=0, k=1, v=2, alpha=3, beta=4, S0=5, z0=6; draws are float32 standard
  normals (``Generator.standard_normal(dtype=float32)``).
* q, k, v ~ N(0, 1), optionally scaled (1/sqrt(d) for the bf16 linear-attention
  workload) or L2-normalised per token (the gated-delta workloads), then
  rounded to the I/O dtype.  bf16 rounding is round-to-nearest-even, and the
  returned float32 arrays hold exactly the bf16 values the GPU sees.
* alpha = sigmoid(N(3, 1)), beta = sigmoid(N(0, 1)), kept in float32.
* pre-operations: the token-major projections x [B, T, H*(2dk+dv)] ~ N(0, 1)
  (one generator per sequence) rounded to the I/O dtype; depthwise conv
  weights [C, 4] ~ N(0, 0.5^2) float32; gate logits a ~ N(3, 1) and
  b ~ N(0, 1) float32 [B, T, H]; a carried conv state [B, 3, C] ~ N(0, 1)
  rounded to the I/O dtype.
* KDA: q, k, v, beta as for the gated delta rule; the per-channel decay
  alpha[t, c] = sigmoid(N(mu_c, 1)) with mu_c spread evenly over [1, 5] across
  the d_k key channels (fast- and slow-forgetting channels side by side).
* packed batches: sequence lengths from one generator (stream 11),
  lognormal(0, 1) weights scaled to the total token count (every length at
  least 1, the rounding remainder on the last sequence); the tokens of
  sequence n, head h are gdn_head(seed, n, h, ...) laid out back to back per
  head, [H, T_total, d].
* decode: the carried state S0 ~ N(0, 0.02^2) float32 per head; the per-step
  token inputs come from a pool of ``pool`` draws (step s uses pool entry
  s mod pool), generated with ``default_rng([seed, stream, 1000 + entry])``.
"""

import numpy as np

STREAM_Q, STREAM_K, STREAM_V, STREAM_ALPHA, STREAM_BETA, STREAM_S0, STREAM_Z0 = range(7)
STREAM_X, STREAM_CONV_W, STREAM_LOGITS, STREAM_CONV_STATE, STREAM_LENGTHS = range(7, 12)

# The five named workloads.  ``seed`` is the per-workload base seed.
WORKLOADS = {
    "la_fp32_small": dict(seed=1001, kind="la", B=1, H=2, T=256, dk=16, dv=16, dtype="f32",
                          chunk=32, scale=1.0),
    "la_bf16_4x16x4096": dict(seed=1002, kind="la", B=4, H=16, T=4096, dk=128, dv=128,
                              dtype="bf16", chunk=64, scale=1.0 / np.sqrt(128.0)),
    "gdn_bf16_2x16x8192": dict(seed=1003, kind="gdn", B=2, H=16, T=8192, dk=128, dv=128,
                               dtype="bf16", chunk=64),
    "gdn_decode_256x32": dict(seed=1004, kind="decode", N=256, H=32, dk=128, dv=128,
                              dtype="bf16", steps=1000, state_std=0.02),
    "gdn_bf16_1x16x262144": dict(seed=1005, kind="gdn", B=1, H=16, T=262144, dk=128, dv=128,
                                 dtype="bf16", chunk=64),
    # scalar-gated linear attention (no delta term): the gated-delta inputs
    # without beta, at the gated-delta prefill shape
    "gla_bf16_2x16x8192": dict(seed=1006, kind="gla", B=2, H=16, T=8192, dk=128, dv=128,
                               dtype="bf16", chunk=64),
    # Kimi Delta Attention (per-channel decay) at the gated-delta prefill
    # shape, and its decode at the decode shape
    "kda_bf16_2x16x8192": dict(seed=1008, kind="kda", B=2, H=16, T=8192, dk=128, dv=128, dtype="bf16"),
    "kda_decode_256x32": dict(seed=1009, kind="kda_decode", N=256, H=32, dk=128, dv=128, dtype="bf16",
                              steps=1000, state_std=0.02),
    # packed batch: 16 sequences of mixed lengths, 16384 tokens in all (the
    # head-token count of the 2 x 16 x 8192 prefill), snapshots every 1024
    "gdn_varlen_bf16_16seq_16k": dict(seed=1010, kind="gdn_varlen", N=16, H=16, T_total=16384, dk=128, dv=128,
                                      dtype="bf16", chunk=64, snap=1024),
    # pre-operations of a Gated DeltaNet layer in front of the 2 x 16 x 8192
    # prefill: x [2, 8192, 16 * (128 + 128 + 128)]
    "preops_bf16_2x16x8192": dict(seed=1007, kind="preops", B=2, H=16, T=8192, dk=128, dv=128,
                                  dtype="bf16"),
}


def round_bf16(x):
    """Round to the nearest bfloat16 (ties to even); returns float32 values."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32).astype(np.uint64)
    bits = (bits + 0x7FFF + ((bits >> 16) & 1)) & 0xFFFF0000
    return bits.astype(np.uint32).view(np.float32).reshape(x.shape)


def round_io(x, dtype):
    if dtype == "bf16":
        return round_bf16(x)
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    raise ValueError(dtype)


def _rng(seed, stream, *idx):
    return np.random.default_rng([int(seed), int(stream), *[int(i) for i in idx]])


def _normal(seed, stream, idx, shape):
    return _rng(seed, stream, *idx).standard_normal(size=shape, dtype=np.float32)


def _unit_rows(x):
    n = np.sqrt(np.sum(x.astype(np.float64) ** 2, axis=-1, keepdims=True))
    return (x / n).astype(np.float32)


def _sigmoid(x):
    return (1.0 / (1.0 + np.exp(-x.astype(np.float64)))).astype(np.float32)


def la_head(seed, b, h, T, dk, dv, dtype, scale=1.0):
    """q, k, v for one head of a linear-attention workload (float32 arrays)."""
    q = _normal(seed, STREAM_Q, (b, h), (T, dk)) * np.float32(scale)
    k = _normal(seed, STREAM_K, (b, h), (T, dk)) * np.float32(scale)
    v = _normal(seed, STREAM_V, (b, h), (T, dv)) * np.float32(scale)
    return round_io(q, dtype), round_io(k, dtype), round_io(v, dtype)


def gdn_head(seed, b, h, T, dk, dv, dtype, alpha_mean=3.0, beta_mean=0.0):
    """q, k (unit rows), v, alpha, beta for one head of a gated-delta workload."""
    q = round_io(_unit_rows(_normal(seed, STREAM_Q, (b, h), (T, dk))), dtype)
    k = round_io(_unit_rows(_normal(seed, STREAM_K, (b, h), (T, dk))), dtype)
    v = round_io(_normal(seed, STREAM_V, (b, h), (T, dv)), dtype)
    alpha = _sigmoid(_normal(seed, STREAM_ALPHA, (b, h), (T,)) + np.float32(alpha_mean))
    beta = _sigmoid(_normal(seed, STREAM_BETA, (b, h), (T,)) + np.float32(beta_mean))
    return q, k, v, alpha, beta


def state_head(seed, b, h, dk, dv, std, stream=STREAM_S0):
    """A carried fp32 state S0 for one head, N(0, std^2)."""
    return (_normal(seed, stream, (b, h), (dv, dk)) * np.float32(std)).astype(np.float32)


def norm_head(seed, b, h, dk, scale=1.0):
    """A carried normaliser z0 for one head (positive, like a sum of phi(k))."""
    return (np.abs(_normal(seed, STREAM_Z0, (b, h), (dk,))) * np.float32(scale) + 1).astype(np.float32)


def la_batch(seed, B, H, T, dk, dv, dtype, scale=1.0):
    q = np.empty((B, H, T, dk), np.float32)
    k = np.empty((B, H, T, dk), np.float32)
    v = np.empty((B, H, T, dv), np.float32)
    for b in range(B):
        for h in range(H):
            q[b, h], k[b, h], v[b, h] = la_head(seed, b, h, T, dk, dv, dtype, scale)
    return q, k, v


def gdn_batch(seed, B, H, T, dk, dv, dtype, **kw):
    q = np.empty((B, H, T, dk), np.float32)
    k = np.empty((B, H, T, dk), np.float32)
    v = np.empty((B, H, T, dv), np.float32)
    a = np.empty((B, H, T), np.float32)
    be = np.empty((B, H, T), np.float32)
    for b in range(B):
        for h in range(H):
            q[b, h], k[b, h], v[b, h], a[b, h], be[b, h] = gdn_head(seed, b, h, T, dk, dv, dtype, **kw)
    return q, k, v, a, be


def state_batch(seed, B, H, dk, dv, std, stream=STREAM_S0):
    S = np.empty((B, H, dv, dk), np.float32)
    for b in range(B):
        for h in range(H):
            S[b, h] = state_head(seed, b, h, dk, dv, std, stream)
    return S


def decode_state_fast(seed, N, H, dk, dv, std):
    """The whole decode state [N,H,dv,dk] from one generator (large sizes);
    the same values as ``decode_state_heads`` would not be produced, so the
    decode recipe uses this function on both sides."""
    rng = _rng(seed, STREAM_S0)
    return (rng.standard_normal(size=(N, H, dv, dk), dtype=np.float32) * np.float32(std))


def decode_token_inputs(seed, N, H, dk, dv, dtype, entry):
    """One pool entry of per-step decode inputs: q, k (unit), v [N,H,d], alpha, beta [N,H]."""
    q = round_io(_unit_rows(_normal(seed, STREAM_Q, (1000 + entry,), (N, H, dk))), dtype)
    k = round_io(_unit_rows(_normal(seed, STREAM_K, (1000 + entry,), (N, H, dk))), dtype)
    v = round_io(_normal(seed, STREAM_V, (1000 + entry,), (N, H, dv)), dtype)
    alpha = _sigmoid(_normal(seed, STREAM_ALPHA, (1000 + entry,), (N, H)) + np.float32(3.0))
    beta = _sigmoid(_normal(seed, STREAM_BETA, (1000 + entry,), (N, H)))
    return q, k, v, alpha, beta


def la_decode_token_inputs(seed, N, H, dk, dv, dtype, entry, scale=1.0):
    """One pool entry of per-step inputs for the normalised linear-attention decode."""
    q = round_io(_normal(seed, STREAM_Q, (2000 + entry,), (N, H, dk)) * np.float32(scale), dtype)
    k = round_io(_normal(seed, STREAM_K, (2000 + entry,), (N, H, dk)) * np.float32(scale), dtype)
    v = round_io(_normal(seed, STREAM_V, (2000 + entry,), (N, H, dv)) * np.float32(scale), dtype)
    return q, k, v


def preops_batch(seed, B, T, H, dk, dv, dtype, w_std=0.5):
    """Inputs of the pre-operations: x [B,T,C] (rounded to dtype), conv
    weights [C,4], gate logits a_logit, b_logit [B,T,H] (float32)."""
    C = H * (2 * dk + dv)
    x = np.empty((B, T, C), np.float32)
    for b in range(B):
        x[b] = round_io(_normal(seed, STREAM_X, (b,), (T, C)), dtype)
    w = (_normal(seed, STREAM_CONV_W, (), (C, 4)) * np.float32(w_std)).astype(np.float32)
    a = (_normal(seed, STREAM_LOGITS, (0,), (B, T, H)) + np.float32(3.0)).astype(np.float32)
    bl = _normal(seed, STREAM_LOGITS, (1,), (B, T, H))
    return x, w, a, bl


def conv_state_batch(seed, B, H, dk, dv, dtype):
    """A carried conv state [B, 3, H*(2dk+dv)] rounded to dtype."""
    return round_io(_normal(seed, STREAM_CONV_STATE, (), (B, 3, H * (2 * dk + dv))), dtype)


def _channel_decay(z, dk):
    """sigmoid(z + mu_c), mu_c evenly spread over [1, 5] along the last axis."""
    mu = np.linspace(1.0, 5.0, dk, dtype=np.float32)
    return _sigmoid(z + mu)


def kda_head(seed, b, h, T, dk, dv, dtype):
    """q, k (unit rows), v, per-channel alpha [T, dk], beta [T] for one head."""
    q, k, v, _, beta = gdn_head(seed, b, h, T, dk, dv, dtype)
    alpha = _channel_decay(_normal(seed, STREAM_ALPHA, (b, h, 1), (T, dk)), dk)
    return q, k, v, alpha, beta


def kda_batch(seed, B, H, T, dk, dv, dtype):
    q = np.empty((B, H, T, dk), np.float32)
    k = np.empty((B, H, T, dk), np.float32)
    v = np.empty((B, H, T, dv), np.float32)
    a = np.empty((B, H, T, dk), np.float32)
    be = np.empty((B, H, T), np.float32)
    for b in range(B):
        for h in range(H):
            q[b, h], k[b, h], v[b, h], a[b, h], be[b, h] = kda_head(seed, b, h, T, dk, dv, dtype)
    return q, k, v, a, be


def kda_decode_token_inputs(seed, N, H, dk, dv, dtype, entry):
    """One pool entry of KDA decode inputs: q, k (unit), v [N,H,d], alpha [N,H,dk], beta [N,H]."""
    q, k, v, _, beta = decode_token_inputs(seed, N, H, dk, dv, dtype, entry)
    alpha = _channel_decay(_normal(seed, STREAM_ALPHA, (3000 + entry,), (N, H, dk)), dk)
    return q, k, v, alpha, beta


def varlen_lengths(seed, N, total):
    """N sequence lengths summing to total (each >= 1 when total >= N)."""
    w = _rng(seed, STREAM_LENGTHS).lognormal(0.0, 1.0, size=N)
    lens = np.maximum(1, np.floor(w / w.sum() * total).astype(np.int64)) if total >= N else np.zeros(N, np.int64)
    lens[-1] += total - lens.sum()
    if lens[-1] < 0:
        raise ValueError("lengths do not fit")
    return lens


def varlen_batch(seed, lens, H, dk, dv, dtype):
    """q, k, v [H, T_total, d], alpha, beta [H, T_total] and cu_seqlens [N+1]
    (int32) of a packed batch with the given sequence lengths."""
    lens = [int(x) for x in lens]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu[-1])
    q = np.empty((H, T, dk), np.float32)
    k = np.empty((H, T, dk), np.float32)
    v = np.empty((H, T, dv), np.float32)
    a = np.empty((H, T), np.float32)
    b = np.empty((H, T), np.float32)
    for n, L in enumerate(lens):
        s0 = int(cu[n])
        for h in range(H):
            q[h, s0:s0 + L], k[h, s0:s0 + L], v[h, s0:s0 + L], a[h, s0:s0 + L], b[h, s0:s0 + L] = \
                gdn_head(seed, n, h, L, dk, dv, dtype)
    return q, k, v, a, b, cu


def varlen_kind_batch(seed, kind, lens, H, dk, dv, dtype, scale=1.0):
    """A packed batch for one kind of recurrence: q, k, v [H, T_total, d];
    alpha ([H, T_total] for "gated", [H, T_total, dk] for "kda", else None);
    beta ([H, T_total] for "kda", else None); cu_seqlens [N+1] int32.
    Sequence n, head h holds the inputs the uniform generators draw for batch
    index n, head h (la_head for "normalized", gdn_head for "gated",
    kda_head for "kda")."""
    lens = [int(x) for x in lens]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu[-1])
    q = np.empty((H, T, dk), np.float32)
    k = np.empty((H, T, dk), np.float32)
    v = np.empty((H, T, dv), np.float32)
    a = None if kind == "normalized" else np.empty((H, T, dk) if kind == "kda" else (H, T), np.float32)
    b = np.empty((H, T), np.float32) if kind == "kda" else None
    for n, L in enumerate(lens):
        s = slice(int(cu[n]), int(cu[n]) + L)
        for h in range(H):
            if kind == "normalized":
                q[h, s], k[h, s], v[h, s] = la_head(seed, n, h, L, dk, dv, dtype, scale)
            elif kind == "gated":
                q[h, s], k[h, s], v[h, s], a[h, s], _ = gdn_head(seed, n, h, L, dk, dv, dtype)
            elif kind == "kda":
                q[h, s], k[h, s], v[h, s], a[h, s], b[h, s] = kda_head(seed, n, h, L, dk, dv, dtype)
            else:
                raise ValueError(kind)
    return q, k, v, a, b, cu


def norm_batch(seed, B, H, dk, scale=1.0):
    """Carried normalisers z0 [B, H, dk] (norm_head per head)."""
    return np.stack([[norm_head(seed, b, h, dk, scale) for h in range(H)] for b in range(B)]).astype(np.float32)
