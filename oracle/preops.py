"""Pre-operations in front of a Gated DeltaNet layer, in fp64.

TEST INFRASTRUCTURE ONLY (see the package docstring): used by tests/ and never
by the product path.

Source page: "Linear attention and hybrids" (ai.flicky.cc lesson 5.5.03).
* Section "2025 hybrids: Qwen3-Next and Kimi Linear": before q, k and v are
  computed, a short causal depthwise convolution over time with kernel 4
  mixes each token with the three before it.
* Section "Delta rule and Gated DeltaNet" (unit keys in its example) and the
  gated-delta workloads: q and k are L2-normalised per token and head.
* Section "Memory must forget: decay and gates": the gate is a sigmoid of the
  input, alpha_t = sigma(...); beta_t lies in (0, 1) the same way.
Readings where the page is silent: the convolution has no bias and no
activation; tap w[:, 3] multiplies the current token and w[:, 3 - i] the token
i steps back; before the first token the three previous tokens come from a
carried state (zeros when there is none); a zero vector stays zero under the
L2 normalisation.  Channels of the projection are laid out q (H*dk), then k
(H*dk), then v (H*dv), each head's channels contiguous.
"""

import numpy as np


def causal_conv(x, w, state=None):
    """Depthwise causal convolution with kernel 4; returns (y, new_state).

    x [T, C]; w [C, 4]; state [3, C] = the three tokens before x.
    y_t[c] = sum_i w[c, i] x_{t-3+i}[c].  new_state = the last three tokens
    of [state; x].
    """
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    T, C = x.shape
    prev = np.zeros((3, C)) if state is None else np.asarray(state, dtype=np.float64)
    xx = np.concatenate([prev, x], axis=0)
    y = np.zeros((T, C))
    for t in range(T):
        for i in range(4):
            y[t] += w[:, i] * xx[t + i]
    return y, xx[-3:].copy()


def l2_normalize(x):
    """Each row divided by its Euclidean norm (zero rows stay zero)."""
    x = np.asarray(x, dtype=np.float64)
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    return np.where(n > 0, x / np.where(n > 0, n, 1.0), 0.0)


def sigmoid(x):
    x = np.asarray(x, dtype=np.float64)
    return 1.0 / (1.0 + np.exp(-x))


def gdn_preprocess(x, w, a_logit, b_logit, H, dk, dv, state=None):
    """One sequence: x [T, H*(2dk+dv)], w [H*(2dk+dv), 4], a_logit, b_logit
    [T, H].  Returns q [H, T, dk], k [H, T, dk] (conv, then L2-normalised),
    v [H, T, dv] (conv), alpha, beta [H, T] (sigmoids) and the new conv state."""
    y, new_state = causal_conv(x, w, state)
    T = y.shape[0]
    q = y[:, :H * dk].reshape(T, H, dk).transpose(1, 0, 2)
    k = y[:, H * dk:2 * H * dk].reshape(T, H, dk).transpose(1, 0, 2)
    v = y[:, 2 * H * dk:].reshape(T, H, dv).transpose(1, 0, 2)
    alpha = sigmoid(np.asarray(a_logit).T)
    beta = sigmoid(np.asarray(b_logit).T)
    return l2_normalize(q), l2_normalize(k), v, alpha, beta, new_state


def gdn_preprocess_varlen(x, w, a_logit, b_logit, H, dk, dv, cu_seqlens, state=None):
    """A packed batch: sequence n is rows cu[n] .. cu[n+1] of x [T_total, C]
    (a_logit, b_logit [T_total, H]); each runs gdn_preprocess on its own rows
    from its own state (state [N, 3, C], zeros when None).  Returns q, k
    [H, T_total, dk], v [H, T_total, dv], alpha, beta [H, T_total] and the
    new states [N, 3, C]."""
    x = np.asarray(x, dtype=np.float64)
    T, C = x.shape
    cu = [int(c) for c in cu_seqlens]
    N = len(cu) - 1
    q = np.zeros((H, T, dk))
    k = np.zeros((H, T, dk))
    v = np.zeros((H, T, dv))
    al = np.zeros((H, T))
    be = np.zeros((H, T))
    new = np.zeros((N, 3, C))
    for n in range(N):
        s, e = cu[n], cu[n + 1]
        st = None if state is None else state[n]
        qn, kn, vn, an, bn, new[n] = gdn_preprocess(x[s:e], w, np.asarray(a_logit)[s:e], np.asarray(b_logit)[s:e],
                                                    H, dk, dv, st)
        q[:, s:e], k[:, s:e], v[:, s:e], al[:, s:e], be[:, s:e] = qn, kn, vn, an, bn
    return q, k, v, al, be, new
