"""The gated delta rule (Gated DeltaNet) in fp64.

TEST INFRASTRUCTURE ONLY (see the package docstring): used by tests/, smoke()
and bench.py's cpu_baseline, never by the product path.

Source page: "Linear attention and hybrids" (ai.flicky.cc lesson 5.5.03),
section "Delta rule and Gated DeltaNet", Gated DeltaNet equation:

    S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,   o_t = S_t q_t

From the decay section on, the page writes k for phi(k) and drops the
normaliser, so this rule has no feature map and no denominator.  S has shape
(d_v, d_k); alpha_t and beta_t are per-token gate values in (0, 1); the output
reads the state after token t has been written.
"""

import numpy as np


def _as64(*arrays):
    return tuple(np.asarray(a, dtype=np.float64) for a in arrays)


def gdn_recurrent(Q, K, V, alpha, beta, S0=None):
    """Token-by-token recurrence, literally the Gated DeltaNet equation.

    [Linear attention and hybrids, section "Delta rule and Gated DeltaNet",
    Gated DeltaNet equation].  Returns (O, S_final).  alpha = 1 gives the plain
    delta rule of the same section; beta = 1 with unit keys makes a read with
    the key just written return exactly the value written.
    """
    Q, K, V, alpha, beta = _as64(Q, K, V, alpha, beta)
    T, dk = Q.shape
    dv = V.shape[1]
    S = np.zeros((dv, dk)) if S0 is None else np.array(S0, dtype=np.float64)
    I = np.eye(dk)
    O = np.zeros((T, dv))
    for t in range(T):
        k = K[t]
        S = alpha[t] * S @ (I - beta[t] * np.outer(k, k)) + beta[t] * np.outer(V[t], k)
        O[t] = S @ Q[t]
    return O, S


def gdn_chunked(Q, K, V, alpha, beta, C, S0=None):
    """Chunkwise form of the same recurrence, exact up to rounding order.

    The page says the delta rule was parallelised along the sequence (section
    "Delta rule and Gated DeltaNet") and that with the delta rule the masked
    form gets more complicated (end of section "Decay: recurrent and parallel
    forms"), but it prints no chunk formula.  This one is obtained by unrolling
    the Gated DeltaNet equation inside a chunk of c tokens with entry state S0:

      write the step as S_r = alpha_r S_{r-1} + u_r k_r^T with
      u_r = beta_r (v_r - alpha_r S_{r-1} k_r);  with g_r = sum_{s<=r} log alpha_s
      (chunk-local) and Gamma_rj = exp(g_r - g_j):
        S_r = e^{g_r} S0 + sum_{j<=r} Gamma_rj u_j k_j^T
      substituting S_{r-1} into u_r gives the unit lower-triangular system
        (I + L) U = diag(beta) V - diag(beta e^g) K S0^T,
        L_rj = beta_r Gamma_rj (k_r . k_j) for j < r, 0 otherwise,
      so with Tm = (I + L)^{-1}:  W = Tm diag(beta e^g) K,  Ut = Tm diag(beta) V,
        U   = Ut - W S0^T
        O   = diag(e^g) Q S0^T + [(Q K^T) * Gamma * tril] U      (diagonal kept)
        S_c = e^{g_c} S0 + U^T diag(e^{g_c - g}) K
    The last chunk may be shorter than C.  Returns (O, S_final).
    """
    Q, K, V, alpha, beta = _as64(Q, K, V, alpha, beta)
    T, dk = Q.shape
    dv = V.shape[1]
    S = np.zeros((dv, dk)) if S0 is None else np.array(S0, dtype=np.float64)
    O = np.zeros((T, dv))
    for a in range(0, T, C):
        b = min(a + C, T)
        c = b - a
        Qc, Kc, Vc = Q[a:b], K[a:b], V[a:b]
        bc = beta[a:b]
        g = np.cumsum(np.log(alpha[a:b]))
        Gamma = np.exp(g[:, None] - g[None, :])
        L = np.tril(bc[:, None] * Gamma * (Kc @ Kc.T), k=-1)
        Tm = np.linalg.solve(np.eye(c) + L, np.eye(c))
        W = Tm @ ((bc * np.exp(g))[:, None] * Kc)
        Ut = Tm @ (bc[:, None] * Vc)
        U = Ut - W @ S.T
        A = np.tril((Qc @ Kc.T) * Gamma)
        O[a:b] = np.exp(g)[:, None] * (Qc @ S.T) + A @ U
        S = np.exp(g[-1]) * S + U.T @ (np.exp(g[-1] - g)[:, None] * Kc)
    return O, S


def gdn_parallel(Q, K, V, alpha, beta):
    """Whole-sequence masked form: the chunked form with one chunk of length T
    and zero entry state (small T only).  Returns (O, S_final)."""
    T = np.asarray(Q).shape[0]
    return gdn_chunked(Q, K, V, alpha, beta, max(T, 1))


def gdn_decode_step(q, k, v, alpha, beta, S):
    """One generation step with a carried state; returns (o, S_new).

    [Linear attention and hybrids, section "Delta rule and Gated DeltaNet"]:
    the Gated DeltaNet equation applied to one token.
    """
    O, S1 = gdn_recurrent(np.asarray(q)[None, :], np.asarray(k)[None, :],
                          np.asarray(v)[None, :], np.atleast_1d(alpha),
                          np.atleast_1d(beta), S)
    return O[0], S1


def gdn_bruteforce_states(K, V, alpha, beta, S0, dtype=object):
    """Every state S_1..S_T from the fully unrolled recurrence (tiny T, d only).

    Unrolling the Gated DeltaNet equation gives
        S_t = S0 P(1, t) + sum_{j<=t} beta_j v_j k_j^T P(j+1, t),
        P(a, t) = A_a A_{a+1} ... A_t  (identity when a > t),
        A_s = alpha_s (I - beta_s k_s k_s^T).
    Each term is formed as an explicit matrix product, O(T^2 d^3).  Works on
    Python objects (e.g. fractions.Fraction) when ``dtype=object``, so it can
    be evaluated exactly on rational inputs.  Returns a list of T matrices as
    nested lists of that element type.
    """
    T = len(K)
    dk = len(K[0])
    dv = len(V[0])

    def zeros(r, c):
        return [[0 * K[0][0] for _ in range(c)] for _ in range(r)]

    def eye(n):
        m = zeros(n, n)
        for i in range(n):
            m[i][i] = 1 + 0 * K[0][0]
        return m

    def matmul(X, Y):
        r, n, c = len(X), len(Y), len(Y[0])
        out = zeros(r, c)
        for i in range(r):
            for j in range(c):
                acc = 0 * K[0][0]
                for p in range(n):
                    acc = acc + X[i][p] * Y[p][j]
                out[i][j] = acc
        return out

    def transition(s):
        m = zeros(dk, dk)
        for i in range(dk):
            for j in range(dk):
                m[i][j] = alpha[s] * ((1 if i == j else 0) - beta[s] * K[s][i] * K[s][j])
        return m

    A = [transition(s) for s in range(T)]

    def P(a, t):  # product A_a ... A_t over 0-based token indices a..t
        m = eye(dk)
        for s in range(a, t + 1):
            m = matmul(m, A[s])
        return m

    states = []
    for t in range(T):
        St = matmul([list(row) for row in S0], P(0, t))
        for j in range(t + 1):
            outer = [[beta[j] * V[j][i] * K[j][p] for p in range(dk)] for i in range(dv)]
            term = matmul(outer, P(j + 1, t))
            St = [[St[i][p] + term[i][p] for p in range(dk)] for i in range(dv)]
        states.append(St)
    return states
