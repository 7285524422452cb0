"""Kimi Delta Attention (KDA): the gated delta rule with a per-channel decay,
in fp64.

TEST INFRASTRUCTURE ONLY (see the package docstring): used by tests/ and never
by the product path.

Source page: "Linear attention and hybrids" (ai.flicky.cc lesson 5.5.03),
section "Delta rule and Gated DeltaNet": KDA replaces the scalar gate alpha_t
of the Gated DeltaNet equation by a diagonal matrix Diag(alpha_t), so that
every memory channel forgets at its own rate.  Reading where the page is
silent: the diagonal acts on the key side of S (shape d_v x d_k), in the place
the scalar occupies, i.e. before the delta correction:

    S_t = S_{t-1} Diag(alpha_t) (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,   o_t = S_t q_t

alpha_t has d_k entries in (0, 1]; with all entries equal it is the Gated
DeltaNet equation itself.
"""

import numpy as np


def _as64(*arrays):
    return tuple(np.asarray(a, dtype=np.float64) for a in arrays)


def kda_recurrent(Q, K, V, alpha, beta, S0=None):
    """Token-by-token recurrence, the equation above written out.

    Q, K (T, d_k); V (T, d_v); alpha (T, d_k); beta (T,).  Returns (O, S_final).
    """
    Q, K, V, alpha, beta = _as64(Q, K, V, alpha, beta)
    T, dk = Q.shape
    dv = V.shape[1]
    S = np.zeros((dv, dk)) if S0 is None else np.array(S0, dtype=np.float64)
    I = np.eye(dk)
    O = np.zeros((T, dv))
    for t in range(T):
        k = K[t]
        S = (S * alpha[t][None, :]) @ (I - beta[t] * np.outer(k, k)) + beta[t] * np.outer(V[t], k)
        O[t] = S @ Q[t]
    return O, S


def kda_chunked(Q, K, V, alpha, beta, C, S0=None):
    """Chunkwise form of the same recurrence, exact up to rounding order.

    Not on the page; obtained like the scalar-gated chunk form by unrolling
    the equation inside a chunk of c tokens with entry state S0.  Write the
    step as S_r = S_{r-1} D_r + u_r k_r^T with D_r = Diag(alpha_r) and
    u_r = beta_r (v_r - S_{r-1} D_r k_r).  With the chunk-local cumulative log
    decay per channel g_r = sum_{s<=r} log alpha_s (a d_k vector) and
    Gamma_rj = exp(g_r - g_j) (elementwise, for j <= r):
        S_r = S0 Diag(e^{g_r}) + sum_{j<=r} u_j (k_j * Gamma_rj)^T
    and substituting S_{r-1} into u_r gives the unit lower-triangular system
        (I + L) U = diag(beta) V - diag(beta) (K * e^g) S0^T,
        L_rj = beta_r sum_c k_r[c] Gamma_rj[c] k_j[c]   for j < r,
    so with Tm = (I + L)^{-1}:  W = Tm diag(beta) (K * e^g),  Ut = Tm diag(beta) V,
        U   = Ut - W S0^T
        A_rj = sum_c q_r[c] Gamma_rj[c] k_j[c]   for j <= r (0 above)
        O   = (Q * e^g) S0^T + A U
        S_c = S0 Diag(e^{g_c}) + U^T (K * e^{g_c - g})
    The decay factors are formed pairwise (exponent differences only), so no
    factor exceeds 1.  The last chunk may be shorter than C.  Returns
    (O, S_final).
    """
    Q, K, V, alpha, beta = _as64(Q, K, V, alpha, beta)
    T, dk = Q.shape
    dv = V.shape[1]
    S = np.zeros((dv, dk)) if S0 is None else np.array(S0, dtype=np.float64)
    O = np.zeros((T, dv))
    for a in range(0, T, C):
        b = min(a + C, T)
        c = b - a
        Qc, Kc, Vc, bc = Q[a:b], K[a:b], V[a:b], beta[a:b]
        g = np.cumsum(np.log(alpha[a:b]), axis=0)                      # (c, dk)
        lower = np.tril(np.ones((c, c)))
        diff = np.where(lower[:, :, None] > 0, g[:, None, :] - g[None, :, :], -np.inf)
        Gamma = np.exp(diff)                                           # (c, c, dk), 0 above the diagonal
        KK = np.einsum("rc,rjc,jc->rj", Kc, Gamma, Kc)
        L = bc[:, None] * np.tril(KK, k=-1)
        Tm = np.linalg.solve(np.eye(c) + L, np.eye(c))
        W = Tm @ (bc[:, None] * (Kc * np.exp(g)))
        Ut = Tm @ (bc[:, None] * Vc)
        U = Ut - W @ S.T
        A = np.einsum("rc,rjc,jc->rj", Qc, Gamma, Kc)
        O[a:b] = (Qc * np.exp(g)) @ S.T + A @ U
        S = S * np.exp(g[-1])[None, :] + U.T @ (Kc * np.exp(g[-1][None, :] - g))
    return O, S


def kda_decode_step(q, k, v, alpha, beta, S):
    """One generation step with a carried state; returns (o, S_new)."""
    O, S1 = kda_recurrent(np.asarray(q)[None, :], np.asarray(k)[None, :], np.asarray(v)[None, :],
                          np.asarray(alpha)[None, :], np.atleast_1d(beta), S)
    return O[0], S1


def kda_bruteforce_states(K, V, alpha, beta, S0):
    """Every state S_1..S_T from the fully unrolled recurrence (tiny sizes).

    S_t = S0 P(1, t) + sum_{j<=t} beta_j v_j k_j^T P(j+1, t), with
    P(a, t) = A_a ... A_t and A_s = Diag(alpha_s) (I - beta_s k_s k_s^T),
    each product formed explicitly.  Works on Python objects (e.g.
    fractions.Fraction), so it can be evaluated exactly on rational inputs.
    Returns a list of T matrices as nested lists.
    """
    T, dk, dv = len(K), len(K[0]), len(V[0])
    zero = 0 * K[0][0]

    def matmul(X, Y):
        return [[sum((X[i][p] * Y[p][j] for p in range(len(Y))), zero) for j in range(len(Y[0]))]
                for i in range(len(X))]

    def eye():
        return [[zero + (1 if i == j else 0) for j in range(dk)] for i in range(dk)]

    A = [[[alpha[s][i] * ((1 if i == j else 0) - beta[s] * K[s][i] * K[s][j]) for j in range(dk)]
          for i in range(dk)] for s in range(T)]

    def P(a, t):
        m = eye()
        for s in range(a, t + 1):
            m = matmul(m, A[s])
        return m

    states = []
    for t in range(T):
        St = matmul([list(r) for r in S0], P(0, t))
        for j in range(t + 1):
            outer = [[beta[j] * V[j][i] * K[j][p] for p in range(dk)] for i in range(dv)]
            term = matmul(outer, P(j + 1, t))
            St = [[St[i][p] + term[i][p] for p in range(dk)] for i in range(dv)]
        states.append(St)
    return states
