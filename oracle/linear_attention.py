"""Normalised causal linear attention, phi(x) = elu(x) + 1, in fp64.

TEST INFRASTRUCTURE ONLY (see the package docstring): used by tests/, smoke()
and bench.py's cpu_baseline, never by the product path.

Source page: "Linear attention and hybrids" (ai.flicky.cc lesson 5.5.03).
The three forms below compute the same function; they differ only in the
order of the sums, so they agree up to rounding.
"""

import numpy as np


def phi(x):
    """Feature map elu(x) + 1: x + 1 where x > 0, exp(x) elsewhere.

    [Linear attention and hybrids, section "The kernel trick: removing
    softmax", the Katharopoulos feature map and its worked example; also the
    "Practice" exercise spec of feature_map].  The result is strictly positive.
    """
    x = np.asarray(x, dtype=np.float64)
    # exp is evaluated on min(x, 0) so the unused branch never overflows.
    return np.where(x > 0, x + 1.0, np.exp(np.minimum(x, 0.0)))


def la_parallel(Q, K, V):
    """Parallel (masked) form: the definition itself.

    [Linear attention and hybrids, section "Three forms of one computation",
    form 1, and the kernel-trick equation for o_i].  A = phi(Q) phi(K)^T with
    the entries above the diagonal (future keys) set to zero; row i of the
    output is (A[i] @ V) / sum(A[i]).  Diagonal included: token i sees itself.
    """
    Q, K, V = (np.asarray(a, dtype=np.float64) for a in (Q, K, V))
    A = np.tril(phi(Q) @ phi(K).T)
    return (A @ V) / A.sum(axis=1, keepdims=True)


def la_recurrent(Q, K, V, S0=None, z0=None):
    """Recurrent form; returns (O, S, z).

    [Linear attention and hybrids, section "Three forms of one computation",
    form 2 (recurrent equation)]: S_t = S_{t-1} + v_t phi(k_t)^T,
    z_t = z_{t-1} + phi(k_t), o_t = S_t phi(q_t) / (z_t^T phi(q_t)).  The state
    is updated with token t before it is read (the exercise spec in "Practice"
    states the same order).  S has shape (d_v, d_k), z shape (d_k,).
    """
    Q, K, V = (np.asarray(a, dtype=np.float64) for a in (Q, K, V))
    T, dk = Q.shape
    dv = V.shape[1]
    S = np.zeros((dv, dk)) if S0 is None else np.array(S0, dtype=np.float64)
    z = np.zeros(dk) if z0 is None else np.array(z0, dtype=np.float64)
    O = np.zeros((T, dv))
    for t in range(T):
        fk = phi(K[t])
        fq = phi(Q[t])
        S = S + np.outer(V[t], fk)
        z = z + fk
        O[t] = (S @ fq) / (z @ fq)
    return O, S, z


def la_chunked(Q, K, V, C, S0=None, z0=None):
    """Chunked (block-parallel) form with block size C; returns (O, S, z).

    [Linear attention and hybrids, section "Three forms of one computation",
    form 3 (chunk equation and the block flowchart), and the "Practice"
    exercise spec of the chunked function].  For each block of rows [a, b)
    (the last block may be shorter than C):
        A_in = tril(phi(Q_b) phi(K_b)^T)
        numerator   = A_in V_b + phi(Q_b) S^T
        denominator = rowsum(A_in) + phi(Q_b) z
        O_b = numerator / denominator
    then the state absorbs the block: S += V_b^T phi(K_b), z += colsum phi(K_b).
    """
    Q, K, V = (np.asarray(a, dtype=np.float64) for a in (Q, K, V))
    T, dk = Q.shape
    dv = V.shape[1]
    S = np.zeros((dv, dk)) if S0 is None else np.array(S0, dtype=np.float64)
    z = np.zeros(dk) if z0 is None else np.array(z0, dtype=np.float64)
    O = np.zeros((T, dv))
    for a in range(0, T, C):
        b = min(a + C, T)
        fq = phi(Q[a:b])
        fk = phi(K[a:b])
        A_in = np.tril(fq @ fk.T)
        num = A_in @ V[a:b] + fq @ S.T
        den = A_in.sum(axis=1) + fq @ z
        O[a:b] = num / den[:, None]
        S = S + V[a:b].T @ fk
        z = z + fk.sum(axis=0)
    return O, S, z


def la_decode_step(q, k, v, S, z):
    """One generation step of the recurrent form; returns (o, S_new, z_new).

    [Linear attention and hybrids, section "Three forms of one computation",
    form 2]: the recurrent equation applied to a single token with a carried
    state (update first, then read).
    """
    O, S1, z1 = la_recurrent(np.asarray(q)[None, :], np.asarray(k)[None, :],
                             np.asarray(v)[None, :], S, z)
    return O[0], S1, z1


def decayed_recurrent(Q, K, V, gamma, S0=None):
    """Unnormalised linear attention with constant decay, phi = identity.

    [Linear attention and hybrids, section "Memory must forget: decay and
    gates", decay equation, left side]: S_t = gamma S_{t-1} + v_t k_t^T,
    o_t = S_t q_t.  From that section on the page writes k for phi(k) and
    drops the denominator; gamma = 1 gives the plain outer-product memory used
    by the "linear" column of the memory-capacity experiment.  Returns (O, S).
    """
    Q, K, V = (np.asarray(a, dtype=np.float64) for a in (Q, K, V))
    T, dk = Q.shape
    dv = V.shape[1]
    S = np.zeros((dv, dk)) if S0 is None else np.array(S0, dtype=np.float64)
    O = np.zeros((T, dv))
    for t in range(T):
        S = gamma * S + np.outer(V[t], K[t])
        O[t] = S @ Q[t]
    return O, S


def decayed_parallel(Q, K, V, gamma):
    """Masked parallel form of :func:`decayed_recurrent`; returns (O, D).

    [Linear attention and hybrids, section "Memory must forget: decay and
    gates", decay equation, right side]: O = ((Q K^T) * D) V with
    D_ij = gamma^(i-j) for j <= i and 0 above the diagonal.
    """
    Q, K, V = (np.asarray(a, dtype=np.float64) for a in (Q, K, V))
    T = Q.shape[0]
    i = np.arange(T)[:, None]
    j = np.arange(T)[None, :]
    D = np.where(j <= i, float(gamma) ** np.maximum(i - j, 0), 0.0)
    return ((Q @ K.T) * D) @ V, D



def gated_recurrent(Q, K, V, alpha, S0=None):
    """Unnormalised linear attention with a per-token scalar gate; returns (O, S).

    [Linear attention and hybrids, section "Memory must forget: decay and
    gates": the input-dependent gate alpha_t in place of the constant gamma of
    the decay equation]: S_t = alpha_t S_{t-1} + v_t k_t^T, o_t = S_t q_t
    (written first, then read, as in every recurrent form on the page).
    alpha_t = gamma for all t is the decay equation itself.
    """
    Q, K, V = (np.asarray(a, dtype=np.float64) for a in (Q, K, V))
    alpha = np.asarray(alpha, dtype=np.float64)
    T, dk = Q.shape
    dv = V.shape[1]
    S = np.zeros((dv, dk)) if S0 is None else np.array(S0, dtype=np.float64)
    O = np.zeros((T, dv))
    for t in range(T):
        S = alpha[t] * S + np.outer(V[t], K[t])
        O[t] = S @ Q[t]
    return O, S


def gated_parallel(Q, K, V, alpha, S0=None):
    """Masked parallel form of :func:`gated_recurrent`; returns (O, D).

    [Same section: with the gate, D_ij = alpha_{j+1} alpha_{j+2} ... alpha_i for
    j <= i (an empty product, 1, on the diagonal) and 0 above it]:
    O = ((Q K^T) * D) V, plus the entering state seen through all gates so
    far: row i adds (alpha_1 ... alpha_i) S0 q_i.  The products are formed
    directly, not through logarithms.
    """
    Q, K, V = (np.asarray(a, dtype=np.float64) for a in (Q, K, V))
    alpha = np.asarray(alpha, dtype=np.float64)
    T = Q.shape[0]
    D = np.zeros((T, T))
    for i in range(T):
        for j in range(i + 1):
            D[i, j] = np.prod(alpha[j + 1:i + 1])
    O = ((Q @ K.T) * D) @ V
    if S0 is not None:
        carry = np.array([np.prod(alpha[:i + 1]) for i in range(T)])
        O = O + carry[:, None] * (Q @ np.asarray(S0, dtype=np.float64).T)
    return O, D


def gated_decode_step(q, k, v, alpha, S):
    """One generation step of :func:`gated_recurrent`; returns (o, S_new)."""
    O, S1 = gated_recurrent(np.asarray(q)[None, :], np.asarray(k)[None, :], np.asarray(v)[None, :],
                            np.array([alpha]), S)
    return O[0], S1
