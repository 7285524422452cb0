"""Pins of the fp64 oracle against facts fixed outside the oracle itself.

Every check here runs on the CPU.  Sources of truth:

* values printed on the source page ("Linear attention and hybrids",
  ai.flicky.cc lesson 5.5.03), stored under tests/golden/ with their citation;
* closed forms and invariants of the equations (beta = 0, unit keys with
  beta = 1, orthonormal keys, identical keys, constant values);
* brute force: the gated delta rule unrolled into explicit products of
  transition matrices, evaluated exactly in rational arithmetic.

The last part plants plausible mistakes (a dropped term, a wrong sign, a
transposed operand, an off-by-one mask) into copies of the oracle source and
checks that at least one pin rejects each of them.
"""

import json
import os
import types
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import gated_delta as gd_mod
from oracle import linear_attention as la_mod

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def rand_gdn(rng, T, dk, dv, alpha_mean=3.0, unit=True):
    Q = rng.normal(size=(T, dk))
    K = rng.normal(size=(T, dk))
    if unit:
        Q /= np.linalg.norm(Q, axis=1, keepdims=True)
        K /= np.linalg.norm(K, axis=1, keepdims=True)
    V = rng.normal(size=(T, dv))
    a = 1 / (1 + np.exp(-rng.normal(alpha_mean, 1, T)))
    b = 1 / (1 + np.exp(-rng.normal(0, 1, T)))
    return Q, K, V, a, b


# --------------------------------------------------------------------------
# Pin functions.  Each takes a namespace holding the oracle functions, so the
# same checks can be run against planted mutants below.  Each raises
# AssertionError on failure.
# --------------------------------------------------------------------------

def pin_phi(ns):
    g = golden("phi_worked_example.json")
    fq, fk = ns.phi(np.array(g["q"])), ns.phi(np.array(g["k"]))
    d = g["decimals"]
    assert np.allclose(np.round(fq, d), g["phi_q"]) and np.allclose(np.round(fk, d), g["phi_k"])
    assert round(float(fq @ fk), d) == g["linear_similarity"]
    assert round(float(np.exp(np.dot(g["q"], g["k"]))), d) == g["softmax_similarity"]
    # closed form: phi(-1) = 1/e, phi(0) = 1, phi(x) = x + 1 for x > 0
    g2 = golden("phi_selfcheck.json")
    px = ns.phi(np.array(g2["x"]))
    assert np.allclose(np.round(px, g2["decimals"]), g2["phi_x"])
    assert abs(px[0] - np.exp(-1.0)) < 1e-15 and px[1] == 1.0 and px[2] == 3.0
    assert np.all(ns.phi(np.linspace(-30, 30, 101)) > 0)


def pin_three_forms(ns):
    """The page's self-check: rng(0), Q, K, V of shape (6, 4), C = 4 (last block
    of 2 tokens); all forms agree and the state is (d_v, d_k) = (4, 4)."""
    rng = np.random.default_rng(0)
    Q, K, V = rng.normal(size=(3, 6, 4))
    p = ns.la_parallel(Q, K, V)
    r, S, z = ns.la_recurrent(Q, K, V)
    c, S2, z2 = ns.la_chunked(Q, K, V, 4)
    assert np.allclose(p, r) and np.allclose(p, c)
    assert S.shape == (4, 4) and z.shape == (4,)
    assert np.abs(p - r).max() < 1e-12 and np.abs(p - c).max() < 1e-12
    assert np.abs(S - S2).max() < 1e-12 and np.abs(z - z2).max() < 1e-12


def pin_la_closed_forms(ns):
    rng = np.random.default_rng(7)
    T, d = 9, 5
    # identical keys: every weight in a row is equal, so o_t is the running mean of v
    q = rng.normal(size=(T, d))
    k = np.tile(rng.normal(size=(1, d)), (T, 1))
    v = rng.normal(size=(T, 3))
    mean = np.cumsum(v, axis=0) / np.arange(1, T + 1)[:, None]
    for o in (ns.la_parallel(q, k, v), ns.la_recurrent(q, k, v)[0], ns.la_chunked(q, k, v, 4)[0]):
        assert np.abs(o - mean).max() < 1e-12
    # a single token reads back its own value
    for o in (ns.la_parallel(q[:1], q[:1], v[:1]), ns.la_recurrent(q[:1], k[:1], v[:1])[0]):
        assert np.abs(o - v[:1]).max() < 1e-15
    # constant values: the normalised output is that constant at every step
    k2 = rng.normal(size=(T, d))
    vc = np.full((T, 2), 2.5)
    for o in (ns.la_parallel(q, k2, vc), ns.la_recurrent(q, k2, vc)[0], ns.la_chunked(q, k2, vc, 4)[0]):
        assert np.abs(o - 2.5).max() < 1e-12
    # final state is the plain sum over all tokens
    _, S, z = ns.la_recurrent(q, k2, v)
    assert np.abs(S - v.T @ ns.phi(k2)).max() < 1e-12
    assert np.abs(z - ns.phi(k2).sum(0)).max() < 1e-12


def pin_la_chunk_invariance(ns):
    rng = np.random.default_rng(11)
    T, dk, dv = 37, 6, 5
    Q, K, V = rng.normal(size=(T, dk)), rng.normal(size=(T, dk)), rng.normal(size=(T, dv))
    S0 = rng.normal(size=(dv, dk)) ** 2
    z0 = np.abs(rng.normal(size=dk)) + 1
    o_r, S_r, z_r = ns.la_recurrent(Q, K, V, S0, z0)
    for C in (1, 7, 32, 64, T):
        o_c, S_c, z_c = ns.la_chunked(Q, K, V, C, S0, z0)
        assert np.abs(o_c - o_r).max() < 1e-12
        assert np.abs(S_c - S_r).max() < 1e-12 and np.abs(z_c - z_r).max() < 1e-12
    assert np.abs(ns.la_parallel(Q, K, V) - ns.la_chunked(Q, K, V, 8)[0]).max() < 1e-12
    # split-resume: two calls with the carried state equal one call
    o1, S1, z1 = ns.la_recurrent(Q[:20], K[:20], V[:20], S0, z0)
    o2, S2, z2 = ns.la_chunked(Q[20:], K[20:], V[20:], 8, S1, z1)
    assert np.abs(np.vstack([o1, o2]) - o_r).max() < 1e-12 and np.abs(S2 - S_r).max() < 1e-12


def pin_decay(ns):
    g = golden("decay_forms.json")
    rng = np.random.default_rng(0)
    Q, K, V = rng.normal(size=(3, g["T"], g["d"]))
    o_rec, _ = ns.decayed_recurrent(Q, K, V, g["gamma"])
    o_par, D = ns.decayed_parallel(Q, K, V, g["gamma"])
    assert np.abs(o_rec - o_par).max() < 10 * g["printed_max_discrepancy"]
    assert np.array_equal(D.round(2), np.array(g["D_rounded_2dp"]))


def pin_gated_reduces_to_decay(ns):
    """A constant gate is the decay equation: same outputs as the decayed
    recurrence on the page's example inputs, and the gated mask D equals the
    page's printed gamma^(i-j) mask."""
    g = golden("decay_forms.json")
    rng = np.random.default_rng(0)
    Q, K, V = rng.normal(size=(3, g["T"], g["d"]))
    alpha = np.full(g["T"], g["gamma"])
    o_g, S_g = ns.gated_recurrent(Q, K, V, alpha)
    o_d, S_d = ns.decayed_recurrent(Q, K, V, g["gamma"])
    assert np.abs(o_g - o_d).max() < 1e-13 and np.abs(S_g - S_d).max() < 1e-13
    _, D = ns.gated_parallel(Q, K, V, alpha)
    assert np.array_equal(D.round(2), np.array(g["D_rounded_2dp"]))
    # alpha = 1: the plain outer-product memory
    o_1, _ = ns.gated_recurrent(Q, K, V, np.ones(g["T"]))
    assert np.abs(o_1 - np.tril(Q @ K.T) @ V).max() < 1e-12


def pin_gated_forms_and_exact(ns):
    """Recurrent and masked parallel forms (the gate products formed directly)
    agree with a carried state; both match the recurrence evaluated exactly in
    rational arithmetic; split-resume equals one call; the decode step is the
    recurrence for one token."""
    rng = np.random.default_rng(11)
    T, dk, dv = 23, 5, 3
    Q, K, V = rng.normal(size=(T, dk)), rng.normal(size=(T, dk)), rng.normal(size=(T, dv))
    a = 1 / (1 + np.exp(-rng.normal(1.0, 1.0, T)))
    S0 = rng.normal(size=(dv, dk))
    o_r, S_r = ns.gated_recurrent(Q, K, V, a, S0)
    o_p, _ = ns.gated_parallel(Q, K, V, a, S0)
    assert np.abs(o_r - o_p).max() < 1e-12
    F = lambda x: Fraction(float(x))
    S = [[F(S0[i, j]) for j in range(dk)] for i in range(dv)]
    for t in range(8):
        S = [[F(a[t]) * S[i][j] + F(V[t, i]) * F(K[t, j]) for j in range(dk)] for i in range(dv)]
        o_t = [sum(S[i][j] * F(Q[t, j]) for j in range(dk)) for i in range(dv)]
        assert max(abs(float(o_t[i]) - o_r[t, i]) for i in range(dv)) < 1e-12
    o1, S1 = ns.gated_recurrent(Q[:9], K[:9], V[:9], a[:9], S0)
    o2, S2 = ns.gated_recurrent(Q[9:], K[9:], V[9:], a[9:], S1)
    assert np.abs(np.vstack([o1, o2]) - o_r).max() < 1e-12 and np.abs(S2 - S_r).max() < 1e-12
    o_s, S_s = ns.gated_decode_step(Q[0], K[0], V[0], a[0], S0)
    assert np.abs(o_s - o_r[0]).max() < 1e-13


def pin_delta_example(ns):
    g = golden("delta_rule_example.json")
    k = np.array([g["key"], g["key"]])
    v = np.array(g["values_written"])
    ones = np.ones(2)
    o_delta, _ = ns.gdn_recurrent(k, k, v, ones, ones * g["beta"])
    o_delta_c, _ = ns.gdn_chunked(k, k, v, ones, ones * g["beta"], 2)
    o_lin, _ = ns.decayed_recurrent(k, k, v, 1.0)
    assert np.allclose(o_delta[-1], g["read_delta_rule"], atol=1e-15)
    assert np.allclose(o_delta_c[-1], g["read_delta_rule"], atol=1e-15)
    assert np.allclose(o_lin[-1], g["read_plain_linear"], atol=1e-15)


def pin_memory_capacity(ns):
    """The capacity table of section "Memory capacity: what a fixed state
    loses": n unit keys and random values stored in a d = 32 state, each key
    then used as the query.  Columns: softmax attention at temperature 1/20,
    plain linear attention, the delta rule (beta = 1), and the delta rule on
    the last four pairs only; each is the mean cosine between what is read
    back and the value stored.  The generator and its draw order (keys, then
    values, for each n in turn) are the page's, so the printed 3-decimal
    values must come back exactly."""
    from scipy.special import softmax

    table = golden("memory_capacity.json")
    d = 32
    draws = np.random.default_rng(0)

    def mean_cosine(read, stored):
        dots = np.einsum("nd,nd->n", read, stored)
        return float(np.mean(dots / (np.linalg.norm(read, axis=1) * np.linalg.norm(stored, axis=1))))

    for n, *printed in table["rows"]:
        keys = draws.normal(size=(n, d))
        keys /= np.linalg.norm(keys, axis=1)[:, None]
        values = draws.normal(size=(n, d))
        read_softmax = softmax(20.0 * (keys @ keys.T), axis=1) @ values
        S_plain = ns.decayed_recurrent(keys, keys, values, 1.0)[1]
        S_delta = ns.gdn_recurrent(keys, keys, values, np.ones(n), np.ones(n))[1]
        read_delta = keys @ S_delta.T
        got = [mean_cosine(read_softmax, values), mean_cosine(keys @ S_plain.T, values),
               mean_cosine(read_delta, values), mean_cosine(read_delta[-4:], values[-4:])]
        assert [round(x, table["decimals"]) for x in got] == printed, (n, got, printed)


def pin_gdn_unit_key_recall(ns):
    """beta = 1 and |k| = 1: right after the write, S_t k_t = v_t for any alpha."""
    rng = np.random.default_rng(3)
    T, d = 23, 6
    _, K, V, a, _ = rand_gdn(rng, T, d, 4)
    S0 = rng.normal(size=(4, d))
    for o in (ns.gdn_recurrent(K, K, V, a, np.ones(T), S0)[0],
              ns.gdn_chunked(K, K, V, a, np.ones(T), 8, S0)[0]):
        assert np.abs(o - V).max() < 1e-13


def pin_gdn_beta_zero(ns):
    """beta = 0: nothing is written, S_t = (prod alpha) S0 and o_t = that times q_t."""
    rng = np.random.default_rng(4)
    T, d = 17, 5
    Q, K, V, a, _ = rand_gdn(rng, T, d, 3, unit=False)
    S0 = rng.normal(size=(3, d))
    gam = np.cumprod(a)
    want = gam[:, None] * (Q @ S0.T)
    for o, S in (ns.gdn_recurrent(Q, K, V, a, np.zeros(T), S0),
                 ns.gdn_chunked(Q, K, V, a, np.zeros(T), 4, S0)):
        assert np.abs(o - want).max() < 1e-13
        assert np.abs(S - gam[-1] * S0).max() < 1e-13
    o, S = ns.gdn_recurrent(Q, K, V, np.ones(T), np.zeros(T), S0)
    assert np.abs(S - S0).max() == 0


def pin_gdn_orthonormal_recall(ns):
    """d orthonormal keys, alpha = beta = 1: every stored value is read back exactly."""
    rng = np.random.default_rng(5)
    d = 8
    Kq, _ = np.linalg.qr(rng.normal(size=(d, d)))
    K = Kq.T
    V = rng.normal(size=(d, d))
    for _, S in (ns.gdn_recurrent(K, K, V, np.ones(d), np.ones(d)),
                 ns.gdn_chunked(K, K, V, np.ones(d), np.ones(d), 3)):
        assert np.abs(K @ S.T - V).max() < 1e-12


def pin_gdn_bruteforce_exact(ns):
    """States and outputs against the unrolled product form in exact rationals."""
    rng = np.random.default_rng(6)
    T, dk, dv = 5, 3, 2

    def rat(x, den=16):
        return Fraction(int(round(x * den)), den)

    K = [[rat(x) for x in row] for row in rng.normal(size=(T, dk))]
    Qr = [[rat(x) for x in row] for row in rng.normal(size=(T, dk))]
    V = [[rat(x) for x in row] for row in rng.normal(size=(T, dv))]
    al = [Fraction(int(x), 32) for x in rng.integers(20, 32, T)]
    be = [Fraction(int(x), 32) for x in rng.integers(1, 32, T)]
    S0 = [[rat(x) for x in row] for row in rng.normal(size=(dv, dk))]
    exact = gd_mod.gdn_bruteforce_states(K, V, al, be, S0)
    f = lambda m: np.array([[float(x) for x in r] for r in m])
    Kf, Qf, Vf, S0f = f(K), f(Qr), f(V), f(S0)
    af, bf = np.array([float(x) for x in al]), np.array([float(x) for x in be])
    o_exact = np.array([[float(sum(exact[t][i][p] * Qr[t][p] for p in range(dk))) for i in range(dv)]
                        for t in range(T)])
    for C in (None, 1, 2, T):
        if C is None:
            o, S = ns.gdn_recurrent(Qf, Kf, Vf, af, bf, S0f)
        else:
            o, S = ns.gdn_chunked(Qf, Kf, Vf, af, bf, C, S0f)
        assert np.abs(o - o_exact).max() < 1e-13, C
        assert np.abs(S - f(exact[-1])).max() < 1e-13, C
    # every intermediate state of the recurrence, via its one-token steps
    S = S0f
    for t in range(T):
        o_t, S = ns.gdn_decode_step(Qf[t], Kf[t], Vf[t], af[t], bf[t], S)
        assert np.abs(S - f(exact[t])).max() < 1e-13
        assert np.abs(o_t - o_exact[t]).max() < 1e-13


def pin_gdn_chunk_invariance(ns):
    rng = np.random.default_rng(12)
    T, dk, dv = 70, 8, 6
    Q, K, V, a, b = rand_gdn(rng, T, dk, dv, alpha_mean=1.0)
    S0 = rng.normal(size=(dv, dk))
    o_r, S_r = ns.gdn_recurrent(Q, K, V, a, b, S0)
    for C in (1, 7, 32, 64, T):
        o_c, S_c = ns.gdn_chunked(Q, K, V, a, b, C, S0)
        assert np.abs(o_c - o_r).max() < 1e-12, C
        assert np.abs(S_c - S_r).max() < 1e-12, C
    o_p, S_p = ns.gdn_parallel(Q, K, V, a, b)
    o_r0, S_r0 = ns.gdn_recurrent(Q, K, V, a, b)
    assert np.abs(o_p - o_r0).max() < 1e-12 and np.abs(S_p - S_r0).max() < 1e-12
    # split-resume with the carried state
    o1, S1 = ns.gdn_chunked(Q[:29], K[:29], V[:29], a[:29], b[:29], 8, S0)
    o2, S2 = ns.gdn_chunked(Q[29:], K[29:], V[29:], a[29:], b[29:], 16, S1)
    assert np.abs(np.vstack([o1, o2]) - o_r).max() < 1e-12 and np.abs(S2 - S_r).max() < 1e-12


GDN_PINS = [pin_delta_example, pin_memory_capacity, pin_gdn_unit_key_recall, pin_gdn_beta_zero,
            pin_gdn_orthonormal_recall, pin_gdn_bruteforce_exact, pin_gdn_chunk_invariance]
LA_PINS = [pin_phi, pin_three_forms, pin_la_closed_forms, pin_la_chunk_invariance, pin_decay,
           pin_gated_reduces_to_decay, pin_gated_forms_and_exact]


@pytest.mark.parametrize("pin", LA_PINS + GDN_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(oracle)


def test_sizes_closed_forms():
    """Sizes the page states, from their closed forms; the decode bench prices
    its state traffic with the same per-head figure."""
    g = golden("sizes.json")
    d = 128
    assert d * d == g["state_numbers_per_head_d128"]
    n = 10 ** 6
    ratio = (n * n * d) / (n * d * d)
    assert abs(ratio - g["op_ratio_n1e6_d128_approx"]) / g["op_ratio_n1e6_d128_approx"] < 0.03
    kv_1m = 48 * 2 * 2 * 256 * 2 * n / 2 ** 30   # layers x (K,V) x heads x dim x bf16 x tokens
    assert round(kv_1m) == g["kv_cache_48_layers_1M_tokens_GiB_approx"]
    per_token_12 = 12 * 1024 * 2
    assert per_token_12 * 262144 / 2 ** 30 == g["kv_cache_12_layers_262K_GiB"]
    assert 4 * per_token_12 * 262144 / 2 ** 30 == g["kv_cache_48_layers_262K_GiB"]
    assert 36 * 32 * 128 * 128 * 4 / 2 ** 20 == g["gdn_states_36_layers_32_heads_MiB"]


# --------------------------------------------------------------------------
# Planted mistakes: each mutant of the oracle source must fail some pin.
# --------------------------------------------------------------------------

def _mutant(module, old, new):
    src = open(module.__file__).read()
    assert src.count(old) == 1, f"mutation anchor not unique: {old!r}"
    ns = {"__name__": module.__name__ + "_mutant"}
    exec(compile(src.replace(old, new), module.__file__ + "<mutant>", "exec"), ns)
    return ns


def _namespace(la_ns=None, gd_ns=None):
    la_src = la_ns or vars(la_mod)
    gd_src = gd_ns or vars(gd_mod)
    names = ["phi", "la_parallel", "la_recurrent", "la_chunked", "la_decode_step",
             "decayed_recurrent", "decayed_parallel", "gated_recurrent", "gated_parallel", "gated_decode_step"]
    gnames = ["gdn_recurrent", "gdn_chunked", "gdn_parallel", "gdn_decode_step"]
    return types.SimpleNamespace(**{n: la_src[n] for n in names}, **{n: gd_src[n] for n in gnames})


LA_MUTATIONS = [
    ("np.where(x > 0, x + 1.0,", "np.where(x > 0, x,"),
    ("np.exp(np.minimum(x, 0.0))", "np.exp(-np.minimum(x, 0.0))"),
    ("A = np.tril(phi(Q) @ phi(K).T)", "A = np.triu(phi(Q) @ phi(K).T)"),
    ("        z = z + fk\n", "        z = z + fq\n"),
    ("A_in = np.tril(fq @ fk.T)", "A_in = np.tril(fq @ fk.T, k=-1)"),
    ("num = A_in @ V[a:b] + fq @ S.T", "num = A_in @ V[a:b] + fq @ S"),
    ("den = A_in.sum(axis=1) + fq @ z", "den = A_in.sum(axis=0) + fq @ z"),
    ("S = S + V[a:b].T @ fk", "S = S + fk.T @ V[a:b]"),
    ("np.maximum(i - j, 0)", "np.maximum(j - i, 0)"),
    ("S = gamma * S + np.outer(V[t], K[t])", "S = gamma * S + np.outer(K[t], V[t])"),
    ("S = alpha[t] * S + np.outer(V[t], K[t])", "S = S + np.outer(V[t], K[t])"),
    ("S = alpha[t] * S + np.outer(V[t], K[t])", "S = alpha[t] * S + np.outer(V[t], Q[t])"),
    ("D[i, j] = np.prod(alpha[j + 1:i + 1])", "D[i, j] = np.prod(alpha[j:i + 1])"),
    ("carry = np.array([np.prod(alpha[:i + 1]) for i in range(T)])",
     "carry = np.array([np.prod(alpha[:i]) for i in range(T)])"),
    ("O = O + carry[:, None] * (Q @ np.asarray(S0, dtype=np.float64).T)",
     "O = O + carry[:, None] * (Q @ np.asarray(S0, dtype=np.float64))"),
]

GD_MUTATIONS = [
    ("S = alpha[t] * S @ (I - beta[t]", "S = S @ (I - beta[t]"),
    ("(I - beta[t] * np.outer(k, k))", "(I + beta[t] * np.outer(k, k))"),
    ("beta[t] * np.outer(V[t], k)", "beta[t] * np.outer(k, V[t])"),
    ("L = np.tril(bc[:, None] * Gamma * (Kc @ Kc.T), k=-1)",
     "L = np.tril(bc[:, None] * Gamma * (Kc @ Kc.T), k=0)"),
    ("L = np.tril(bc[:, None] * Gamma", "L = np.tril(Gamma"),
    ("W = Tm @ ((bc * np.exp(g))[:, None] * Kc)", "W = Tm @ (bc[:, None] * Kc)"),
    ("A = np.tril((Qc @ Kc.T) * Gamma)", "A = np.tril((Qc @ Kc.T) * Gamma, k=-1)"),
    ("U = Ut - W @ S.T", "U = Ut + W @ S.T"),
    ("S = np.exp(g[-1]) * S + U.T", "S = S + U.T"),
    ("np.exp(g[-1] - g)[:, None] * Kc)", "np.exp(g - g[-1])[:, None] * Kc)"),
    ("Gamma = np.exp(g[:, None] - g[None, :])", "Gamma = np.exp(g[None, :] - g[:, None])"),
    ("O[a:b] = np.exp(g)[:, None] * (Qc @ S.T) + A @ U", "O[a:b] = (Qc @ S.T) + A @ U"),
]


def _fails_some_pin(ns, pins):
    for pin in pins:
        try:
            with np.errstate(all="ignore"):
                pin(ns)
        except (AssertionError, ValueError, FloatingPointError, np.linalg.LinAlgError):
            return True
    return False


def test_genuine_oracle_passes_all_pins_via_namespace():
    assert not _fails_some_pin(_namespace(), LA_PINS + GDN_PINS)


@pytest.mark.parametrize("old,new", LA_MUTATIONS, ids=[m[1][:40] for m in LA_MUTATIONS])
def test_planted_la_mistake_is_caught(old, new):
    assert _fails_some_pin(_namespace(la_ns=_mutant(la_mod, old, new)), LA_PINS + GDN_PINS)


@pytest.mark.parametrize("old,new", GD_MUTATIONS, ids=[m[1][:40] for m in GD_MUTATIONS])
def test_planted_gdn_mistake_is_caught(old, new):
    assert _fails_some_pin(_namespace(gd_ns=_mutant(gd_mod, old, new)), GDN_PINS)


def test_batched_steps_equal_single_head_steps():
    """The head-batched steps used for large decode checks equal the pinned
    single-head steps, head by head."""
    from oracle import batched
    rng = np.random.default_rng(21)
    n, dk, dv = 5, 6, 4
    q, k = rng.normal(size=(n, dk)), rng.normal(size=(n, dk))
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    v = rng.normal(size=(n, dv))
    a, b = rng.uniform(0.5, 1, n), rng.uniform(0, 1, n)
    S, z = rng.normal(size=(n, dv, dk)), np.abs(rng.normal(size=(n, dk))) + 1
    o, S1 = batched.gdn_step_heads(q, k, v, a, b, S)
    o2, S2, z2 = batched.la_step_heads(q, k, v, S, z)
    o3, S3 = batched.gla_step_heads(q, k, v, a, S)
    for i in range(n):
        oi, Si = oracle.gdn_decode_step(q[i], k[i], v[i], a[i], b[i], S[i])
        assert np.abs(oi - o[i]).max() < 1e-13 and np.abs(Si - S1[i]).max() < 1e-13
        oi, Si, zi = oracle.la_decode_step(q[i], k[i], v[i], S[i], z[i])
        assert np.abs(oi - o2[i]).max() < 1e-13 and np.abs(Si - S2[i]).max() < 1e-13
        assert np.abs(zi - z2[i]).max() < 1e-13
        oi, Si = oracle.gated_decode_step(q[i], k[i], v[i], a[i], S[i])
        assert np.abs(oi - o3[i]).max() < 1e-13 and np.abs(Si - S3[i]).max() < 1e-13


# --------------------------------------------------------------------------
# Pre-operations: causal depthwise convolution, L2 normalisation, sigmoid gates
# --------------------------------------------------------------------------

from oracle import preops as pre_mod


def pin_preops(ns):
    rng = np.random.default_rng(31)
    T, C = 11, 7
    x = rng.normal(size=(T, C))
    w = rng.normal(size=(C, 4))
    st = rng.normal(size=(3, C))
    # taps: [0,0,0,1] is the identity, [1,0,0,0] a delay of three tokens
    ident = np.tile([0.0, 0.0, 0.0, 1.0], (C, 1))
    delay = np.tile([1.0, 0.0, 0.0, 0.0], (C, 1))
    assert np.array_equal(ns.causal_conv(x, ident)[0], x)
    y, _ = ns.causal_conv(x, delay, st)
    assert np.array_equal(y[3:], x[:-3]) and np.array_equal(y[:3], st)
    # against numpy's full convolution of each channel (zero history)
    y, _ = ns.causal_conv(x, w)
    for c in range(C):
        assert np.abs(y[:, c] - np.convolve(x[:, c], w[c, ::-1])[:T]).max() < 1e-12
    # a carried state equals the concatenated history; split-resume equals one call
    y_full, s_full = ns.causal_conv(np.vstack([st, x]), w)
    y_st, s_st = ns.causal_conv(x, w, st)
    assert np.abs(y_full[3:] - y_st).max() < 1e-12 and np.abs(s_full - s_st).max() == 0
    y1, s1 = ns.causal_conv(x[:4], w, st)
    y2, s2 = ns.causal_conv(x[4:], w, s1)
    assert np.abs(np.vstack([y1, y2]) - y_st).max() < 1e-12 and np.array_equal(s2, s_st)
    # L2: unit rows in the same direction; zero rows stay zero
    z = np.vstack([x, np.zeros(C)])
    n = ns.l2_normalize(z)
    assert np.abs(np.linalg.norm(n[:-1], axis=1) - 1).max() < 1e-14 and np.all(n[-1] == 0)
    assert np.abs(n[:-1] * np.linalg.norm(x, axis=1, keepdims=True) - x).max() < 1e-12
    # sigmoid: closed values and symmetry
    p = np.array([0.1, 0.5, 0.9])
    assert np.abs(ns.sigmoid(np.log(p / (1 - p))) - p).max() < 1e-15
    assert np.abs(ns.sigmoid(-x) - (1 - ns.sigmoid(x))).max() < 1e-15
    # layout of the fused call: q | k | v channel blocks, head-contiguous
    H, dk, dv = 2, 3, 2
    Ct = H * (2 * dk + dv)
    xs = rng.normal(size=(T, Ct))
    a, b = rng.normal(size=(T, H)), rng.normal(size=(T, H))
    q, k, v, al, be, _ = ns.gdn_preprocess(xs, np.tile([0.0, 0.0, 0.0, 1.0], (Ct, 1)), a, b, H, dk, dv)
    for h in range(H):
        qh = xs[:, h * dk:(h + 1) * dk]
        vh = xs[:, 2 * H * dk + h * dv:2 * H * dk + (h + 1) * dv]
        kh = xs[:, H * dk + h * dk:H * dk + (h + 1) * dk]
        assert np.abs(q[h] - qh / np.linalg.norm(qh, axis=1, keepdims=True)).max() < 1e-12
        assert np.abs(k[h] - kh / np.linalg.norm(kh, axis=1, keepdims=True)).max() < 1e-12
        assert np.array_equal(v[h], vh)
        assert np.abs(al[h] - 1 / (1 + np.exp(-a[:, h]))).max() < 1e-15
        assert np.abs(be[h] - 1 / (1 + np.exp(-b[:, h]))).max() < 1e-15


def pin_preops_varlen(ns):
    """A packed batch = each sequence alone (the pinned one-sequence
    function), with history never crossing a sequence boundary: a sequence
    run after another gives the outputs of the same sequence run alone."""
    rng = np.random.default_rng(33)
    H, dk, dv = 2, 3, 2
    C = H * (2 * dk + dv)
    lens = [5, 0, 2, 7]
    cu = np.concatenate([[0], np.cumsum(lens)])
    T = int(cu[-1])
    x = rng.normal(size=(T, C))
    w = rng.normal(size=(C, 4))
    a, b = rng.normal(size=(T, H)), rng.normal(size=(T, H))
    st = rng.normal(size=(len(lens), 3, C))
    q, k, v, al, be, new = ns.gdn_preprocess_varlen(x, w, a, b, H, dk, dv, cu, st)
    for n, L in enumerate(lens):
        s, e = cu[n], cu[n + 1]
        ref = ns.gdn_preprocess(x[s:e], w, a[s:e], b[s:e], H, dk, dv, st[n])
        for got, want in zip((q[:, s:e], k[:, s:e], v[:, s:e], al[:, s:e], be[:, s:e], new[n]), ref):
            assert np.abs(got - want).max(initial=0) < 1e-12
    # an empty sequence passes its state through; a 2-token one keeps one state row
    assert np.array_equal(new[1], st[1])
    assert np.array_equal(new[2][0], st[2][2]) and np.array_equal(new[2][1:], x[cu[2]:cu[3]])
    # the last sequence alone, from zeros, differs from the packed one only through its state
    _, _, v0, _, _, _ = ns.gdn_preprocess(x[cu[3]:], w, a[cu[3]:], b[cu[3]:], H, dk, dv)
    assert np.abs(v0[:, 3:] - v[:, cu[3] + 3:]).max() < 1e-12


def test_preops_varlen_pin():
    pin_preops_varlen(pre_mod)


PRE_MUTATIONS = [
    ("y[t] += w[:, i] * xx[t + i]", "y[t] += w[:, 3 - i] * xx[t + i]"),
    ("xx = np.concatenate([prev, x], axis=0)", "xx = np.concatenate([np.zeros_like(prev), x], axis=0)"),
    ("return y, xx[-3:].copy()", "return y, xx[:3].copy()"),
    ("n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))", "n = np.sum(x * x, axis=-1, keepdims=True)"),
    ("return 1.0 / (1.0 + np.exp(-x))", "return 1.0 / (1.0 + np.exp(x))"),
    ("k = y[:, H * dk:2 * H * dk].reshape(T, H, dk).transpose(1, 0, 2)",
     "k = y[:, H * dk:2 * H * dk].reshape(T, dk, H).transpose(2, 0, 1)"),
]


def test_preops_pins():
    pin_preops(pre_mod)


@pytest.mark.parametrize("old,new", PRE_MUTATIONS, ids=[m[1][:40] for m in PRE_MUTATIONS])
def test_planted_preops_mistake_is_caught(old, new):
    ns = types.SimpleNamespace(**_mutant(pre_mod, old, new))
    assert _fails_some_pin(ns, [pin_preops])


PRE_VARLEN_MUTATIONS = [
    ("st = None if state is None else state[n]", "st = None"),
    ("q[:, s:e], k[:, s:e], v[:, s:e], al[:, s:e], be[:, s:e] = qn, kn, vn, an, bn",
     "q[:, s:e], k[:, s:e], v[:, s:e], al[:, s:e], be[:, s:e] = qn, kn, vn, bn, an"),
]


@pytest.mark.parametrize("old,new", PRE_VARLEN_MUTATIONS, ids=[m[1][:40] for m in PRE_VARLEN_MUTATIONS])
def test_planted_preops_varlen_mistake_is_caught(old, new):
    ns = types.SimpleNamespace(**_mutant(pre_mod, old, new))
    assert _fails_some_pin(ns, [pin_preops_varlen])


# ------------------------------------------------------------------ KDA
from oracle import kda as kda_mod


def rand_kda(rng, T, dk, dv, spread=1.5):
    Q = rng.normal(size=(T, dk))
    K = rng.normal(size=(T, dk))
    K /= np.linalg.norm(K, axis=1, keepdims=True)
    V = rng.normal(size=(T, dv))
    # per-channel decay: slow and fast channels side by side
    a = 1.0 / (1.0 + np.exp(-(rng.normal(size=(T, dk)) * spread + np.linspace(-1.0, 5.0, dk))))
    b = 1.0 / (1.0 + np.exp(-rng.normal(size=T)))
    return Q, K, V, a, b


def pin_kda_uniform_is_gdn(ns):
    """Equal decay on every channel is the Gated DeltaNet equation (the
    genuine, separately pinned oracle)."""
    rng = np.random.default_rng(41)
    T, dk, dv = 40, 6, 5
    Q, K, V, a, b = rand_kda(rng, T, dk, dv)
    a1 = np.repeat(a[:, :1], dk, axis=1)
    S0 = rng.normal(size=(dv, dk))
    o_ref, S_ref = oracle.gdn_recurrent(Q, K, V, a1[:, 0], b, S0)
    for o, S in (ns.kda_recurrent(Q, K, V, a1, b, S0), ns.kda_chunked(Q, K, V, a1, b, 8, S0)):
        assert np.abs(o - o_ref).max() < 1e-12 and np.abs(S - S_ref).max() < 1e-12


def pin_kda_beta_zero(ns):
    """beta = 0: pure per-channel forgetting of the key side,
    S_t = S0 Diag(prod_{s<=t} alpha_s), o_t = S_t q_t."""
    rng = np.random.default_rng(42)
    T, d = 13, 4
    Q, K, V, a, _ = rand_kda(rng, T, d, d)
    b = np.zeros(T)
    S0 = rng.normal(size=(d, d))
    P = np.cumprod(a, axis=0)
    o_ref = np.stack([(S0 * P[t][None, :]) @ Q[t] for t in range(T)])
    S_ref = S0 * P[-1][None, :]
    for o, S in (ns.kda_recurrent(Q, K, V, a, b, S0), ns.kda_chunked(Q, K, V, a, b, 4, S0)):
        assert np.abs(o - o_ref).max() < 1e-12 and np.abs(S - S_ref).max() < 1e-12


def pin_kda_unit_key_recall(ns):
    """beta = 1 and a unit key: the decay comes before the correction, so a
    read with the key just written returns exactly the value written,
    whatever the decay."""
    rng = np.random.default_rng(43)
    T, dk, dv = 9, 5, 3
    Q, K, V, a, _ = rand_kda(rng, T, dk, dv)
    b = np.ones(T)
    S = rng.normal(size=(dv, dk))
    for t in range(T):
        _, S = ns.kda_decode_step(Q[t], K[t], V[t], a[t], b[t], S)
        assert np.abs(S @ K[t] - V[t]).max() < 1e-12
    _, Sc = ns.kda_chunked(Q, K, V, a, b, 4, rng.normal(size=(dv, dk)))
    assert np.abs(Sc @ K[-1] - V[-1]).max() < 1e-12


def pin_kda_bruteforce_exact(ns):
    """States and outputs against the unrolled product form in exact rationals."""
    rng = np.random.default_rng(44)
    T, dk, dv = 5, 3, 2

    def rat(x, den=16):
        return Fraction(int(round(x * den)), den)

    K = [[rat(x) for x in row] for row in rng.normal(size=(T, dk))]
    Qr = [[rat(x) for x in row] for row in rng.normal(size=(T, dk))]
    V = [[rat(x) for x in row] for row in rng.normal(size=(T, dv))]
    al = [[Fraction(int(x), 32) for x in row] for row in rng.integers(12, 33, (T, dk))]
    be = [Fraction(int(x), 32) for x in rng.integers(1, 32, T)]
    S0 = [[rat(x) for x in row] for row in rng.normal(size=(dv, dk))]
    exact = ns.kda_bruteforce_states(K, V, al, be, S0)
    f = lambda m: np.array([[float(x) for x in r] for r in m])
    Kf, Qf, Vf, S0f, af = f(K), f(Qr), f(V), f(S0), f(al)
    bf = np.array([float(x) for x in be])
    o_exact = np.array([[float(sum(exact[t][i][p] * Qr[t][p] for p in range(dk))) for i in range(dv)]
                        for t in range(T)])
    for C in (None, 1, 2, T):
        o, S = ns.kda_recurrent(Qf, Kf, Vf, af, bf, S0f) if C is None else \
            ns.kda_chunked(Qf, Kf, Vf, af, bf, C, S0f)
        assert np.abs(o - o_exact).max() < 1e-13, C
        assert np.abs(S - f(exact[-1])).max() < 1e-13, C
    S = S0f
    for t in range(T):
        o_t, S = ns.kda_decode_step(Qf[t], Kf[t], Vf[t], af[t], bf[t], S)
        assert np.abs(S - f(exact[t])).max() < 1e-13 and np.abs(o_t - o_exact[t]).max() < 1e-13


def pin_kda_chunk_invariance(ns):
    rng = np.random.default_rng(45)
    T, dk, dv = 70, 8, 6
    Q, K, V, a, b = rand_kda(rng, T, dk, dv, spread=3.0)
    S0 = rng.normal(size=(dv, dk))
    o_r, S_r = ns.kda_recurrent(Q, K, V, a, b, S0)
    for C in (1, 5, 16, 64, T):
        o_c, S_c = ns.kda_chunked(Q, K, V, a, b, C, S0)
        assert np.abs(o_c - o_r).max() < 1e-11 and np.abs(S_c - S_r).max() < 1e-11, C
    o1, S1 = ns.kda_chunked(Q[:29], K[:29], V[:29], a[:29], b[:29], 8, S0)
    o2, S2 = ns.kda_chunked(Q[29:], K[29:], V[29:], a[29:], b[29:], 16, S1)
    assert np.abs(np.vstack([o1, o2]) - o_r).max() < 1e-11 and np.abs(S2 - S_r).max() < 1e-11


KDA_PINS = [pin_kda_uniform_is_gdn, pin_kda_beta_zero, pin_kda_unit_key_recall, pin_kda_bruteforce_exact,
            pin_kda_chunk_invariance]


@pytest.mark.parametrize("pin", KDA_PINS, ids=lambda f: f.__name__)
def test_kda_pin(pin):
    pin(kda_mod)


def test_kda_batched_step_matches_single_head():
    rng = np.random.default_rng(46)
    n, dk, dv = 5, 6, 4
    q, k, v = rng.normal(size=(n, dk)), rng.normal(size=(n, dk)), rng.normal(size=(n, dv))
    a, b, S = rng.uniform(0.2, 1.0, (n, dk)), rng.uniform(0, 1, n), rng.normal(size=(n, dv, dk))
    o, S1 = oracle.batched.kda_step_heads(q, k, v, a, b, S)
    for i in range(n):
        o_i, S_i = oracle.kda_decode_step(q[i], k[i], v[i], a[i], b[i], S[i])
        assert np.abs(o[i] - o_i).max() < 1e-12 and np.abs(S1[i] - S_i).max() < 1e-12


KDA_MUTATIONS = [
    # decay on the value side instead of the key side
    ("S = (S * alpha[t][None, :]) @", "S = (S * alpha[t][:, None]) @"),
    # decay after the delta correction
    ("S = (S * alpha[t][None, :]) @ (I - beta[t] * np.outer(k, k)) + beta[t] * np.outer(V[t], k)",
     "S = (S @ (I - beta[t] * np.outer(k, k))) * alpha[t][None, :] + beta[t] * np.outer(V[t], k)"),
    # no decay at all
    ("S = (S * alpha[t][None, :]) @", "S = (S * 1.0) @"),
    # W without the decay factor
    ("W = Tm @ (bc[:, None] * (Kc * np.exp(g)))", "W = Tm @ (bc[:, None] * Kc)"),
    # entry state decayed by the first token's factor only
    ("S = S * np.exp(g[-1])[None, :] +", "S = S * np.exp(g[0])[None, :] +"),
    # intra-chunk products without their diagonal
    ("lower = np.tril(np.ones((c, c)))", "lower = np.tril(np.ones((c, c)), k=-1)"),
    # inter-chunk output without the decay of q
    ("O[a:b] = (Qc * np.exp(g)) @ S.T + A @ U", "O[a:b] = Qc @ S.T + A @ U"),
    # beta on the column side of L
    ("L = bc[:, None] * np.tril(KK, k=-1)", "L = bc[None, :] * np.tril(KK, k=-1)"),
    # end-state key factors decayed the wrong way
    ("U.T @ (Kc * np.exp(g[-1][None, :] - g))", "U.T @ (Kc * np.exp(g - g[-1][None, :]))"),
    # brute force with the diagonal on the other side of the transition
    ("A = [[[alpha[s][i] *", "A = [[[alpha[s][j] *"),
]


@pytest.mark.parametrize("old,new", KDA_MUTATIONS, ids=[m[1][:40] for m in KDA_MUTATIONS])
def test_planted_kda_mistake_is_caught(old, new):
    ns = types.SimpleNamespace(**_mutant(kda_mod, old, new))
    assert _fails_some_pin(ns, KDA_PINS)


# ------------------------------------------------- packed batches, snapshots
from oracle import varlen as vl_mod


def pin_varlen(ns):
    """Packed sequences are independent recurrences on their own slices (the
    separately pinned gdn_recurrent); a snapshot is the final state of the
    recurrence over that prefix, and resuming from it reproduces the rest of
    the sequence."""
    rng = np.random.default_rng(51)
    H, dk, dv, iv = 2, 4, 3, 4
    lens = [9, 0, 4, 13, 3]
    cu = np.concatenate([[0], np.cumsum(lens)])
    Tt = int(cu[-1])
    q, k = rng.normal(size=(H, Tt, dk)), rng.normal(size=(H, Tt, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.normal(size=(H, Tt, dv))
    a = 1 / (1 + np.exp(-rng.normal(2, 1, (H, Tt))))
    b = 1 / (1 + np.exp(-rng.normal(size=(H, Tt))))
    S0 = rng.normal(size=(len(lens), H, dv, dk))
    o, S, snaps = ns.gdn_varlen(q, k, v, a, b, cu, S0, snap_interval=iv)
    assert ns.snapshot_count(cu, iv) == sum(L // iv for L in lens) == snaps.shape[0]
    j = 0
    for n, L in enumerate(lens):
        s, e = cu[n], cu[n + 1]
        for h in range(H):
            o_ref, S_ref = oracle.gdn_recurrent(q[h, s:e], k[h, s:e], v[h, s:e], a[h, s:e], b[h, s:e], S0[n, h])
            assert np.abs(o[h, s:e] - o_ref).max(initial=0) < 1e-12
            assert np.abs(S[n, h] - (S0[n, h] if L == 0 else S_ref)).max() < 1e-12
        for p in range(iv, L + 1, iv):
            for h in range(H):
                _, S_p = oracle.gdn_recurrent(q[h, s:s + p], k[h, s:s + p], v[h, s:s + p], a[h, s:s + p],
                                              b[h, s:s + p], S0[n, h])
                assert np.abs(snaps[j, h] - S_p).max() < 1e-12
                # prefix caching: the tail from the snapshot gives the same outputs
                o_t, S_t = oracle.gdn_recurrent(q[h, s + p:e], k[h, s + p:e], v[h, s + p:e], a[h, s + p:e],
                                                b[h, s + p:e], snaps[j, h])
                assert np.abs(o_t - o[h, s + p:e]).max(initial=0) < 1e-12
                assert np.abs(S_t - S[n, h]).max() < 1e-12
            j += 1
    # the chunk-form evaluation agrees
    o_c, S_c, snaps_c = ns.gdn_varlen(q, k, v, a, b, cu, S0, snap_interval=iv, form="chunked")
    assert np.abs(o_c - o).max() < 1e-12 and np.abs(S_c - S).max() < 1e-12 and np.abs(snaps_c - snaps).max() < 1e-12
    # without an initial state every sequence starts from zero; without snapshots none are returned
    o0, S0z, sn0 = ns.gdn_varlen(q, k, v, a, b, cu)
    assert sn0.shape[0] == 0 and np.all(S0z[1] == 0)
    o_ref, _ = oracle.gdn_recurrent(q[0, :9], k[0, :9], v[0, :9], a[0, :9], b[0, :9])
    assert np.abs(o0[0, :9] - o_ref).max() < 1e-12


def test_varlen_pin():
    pin_varlen(vl_mod)


VARLEN_MUTATIONS = [
    ("cuts = [a + p for p in range(snap_interval, b - a + 1, snap_interval)]",
     "cuts = [a + p for p in range(snap_interval, b - a, snap_interval)]"),
    ("S = None if S0 is None else np.asarray(S0[n, h], dtype=np.float64)", "S = None"),
    ("return sum((cu[n + 1] - cu[n]) // snap_interval for n in range(len(cu) - 1))",
     "return (cu[-1] - cu[0]) // snap_interval"),
    ("else S.copy(),", "else np.zeros_like(S),"),
]


@pytest.mark.parametrize("old,new", VARLEN_MUTATIONS, ids=[m[1][:40] for m in VARLEN_MUTATIONS])
def test_planted_varlen_mistake_is_caught(old, new):
    ns = types.SimpleNamespace(**_mutant(vl_mod, old, new))
    assert _fails_some_pin(ns, [pin_varlen])


def _kind_inputs(rng, kind, H, Tt, dk, dv, N):
    q, k = rng.normal(size=(H, Tt, dk)), rng.normal(size=(H, Tt, dk))
    if kind == "kda":
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.normal(size=(H, Tt, dv))
    a = b = z0 = None
    if kind == "gated":
        a = 1 / (1 + np.exp(-rng.normal(2, 1, (H, Tt))))
    elif kind == "kda":
        a = 1 / (1 + np.exp(-rng.normal(2, 1, (H, Tt, dk))))
        b = 1 / (1 + np.exp(-rng.normal(size=(H, Tt))))
    S0 = rng.normal(size=(N, H, dv, dk))
    if kind == "normalized":
        S0 = np.abs(S0)
        z0 = rng.uniform(0.5, 2.0, size=(N, H, dk))
    return q, k, v, a, b, S0, z0


def _kind_reference(kind, q, k, v, a, b, S, z):
    """The kind's pinned single-sequence recurrence on one slice: (O, S, z)."""
    if kind == "normalized":
        return oracle.la_recurrent(q, k, v, S, z)
    if kind == "gated":
        return oracle.gated_recurrent(q, k, v, a, S) + (None,)
    return oracle.kda_recurrent(q, k, v, a, b, S) + (None,)


def pin_varlen_kinds(ns):
    """For the normalised, scalar-gated and KDA kinds: packed sequences are
    independent runs of the kind's own (separately pinned) recurrence on their
    slices from their own state (S, and z for the normalised kind); a snapshot
    is the state after that prefix, and resuming from it reproduces the rest
    of the sequence and its final state."""
    H, dk, dv, iv = 2, 4, 3, 4
    lens = [9, 0, 4, 13, 3]
    cu = np.concatenate([[0], np.cumsum(lens)])
    Tt = int(cu[-1])
    for seed, kind in enumerate(("normalized", "gated", "kda")):
        rng = np.random.default_rng(60 + seed)
        q, k, v, a, b, S0, z0 = _kind_inputs(rng, kind, H, Tt, dk, dv, len(lens))
        o, S, z, snaps, zsnaps = ns.packed_varlen(kind, q, k, v, cu, a, b, S0, z0, snap_interval=iv)
        assert snaps.shape[0] == ns.snapshot_count(cu, iv) == sum(L // iv for L in lens)
        assert (z is None) == (kind != "normalized") and (zsnaps is None) == (kind != "normalized")
        sl = lambda x, h, s, e: None if x is None else x[h, s:e]
        j = 0
        for n, L in enumerate(lens):
            s, e = cu[n], cu[n + 1]
            for h in range(H):
                zi = None if z0 is None else z0[n, h]
                o_ref, S_ref, z_ref = _kind_reference(kind, q[h, s:e], k[h, s:e], v[h, s:e], sl(a, h, s, e),
                                                      sl(b, h, s, e), S0[n, h], zi)
                assert np.abs(o[h, s:e] - o_ref).max(initial=0) < 1e-12
                assert np.abs(S[n, h] - S_ref).max() < 1e-12
                if kind == "normalized":
                    assert np.abs(z[n, h] - z_ref).max() < 1e-12
            for p in range(iv, L + 1, iv):
                for h in range(H):
                    zi = None if z0 is None else z0[n, h]
                    _, S_p, z_p = _kind_reference(kind, q[h, s:s + p], k[h, s:s + p], v[h, s:s + p],
                                                  sl(a, h, s, s + p), sl(b, h, s, s + p), S0[n, h], zi)
                    assert np.abs(snaps[j, h] - S_p).max() < 1e-12
                    zs = None
                    if kind == "normalized":
                        assert np.abs(zsnaps[j, h] - z_p).max() < 1e-12
                        zs = zsnaps[j, h]
                    # prefix caching: the tail from the snapshot gives the same outputs and end state
                    o_t, S_t, z_t = _kind_reference(kind, q[h, s + p:e], k[h, s + p:e], v[h, s + p:e],
                                                    sl(a, h, s + p, e), sl(b, h, s + p, e), snaps[j, h], zs)
                    assert np.abs(o_t - o[h, s + p:e]).max(initial=0) < 1e-12
                    assert np.abs(S_t - S[n, h]).max() < 1e-12
                    if kind == "normalized":
                        assert np.abs(z_t - z[n, h]).max() < 1e-12
                j += 1
        if kind != "gated":
            # the chunk-form evaluation agrees (the scalar-gated kind has none here)
            o_c, S_c, z_c, sn_c, zs_c = ns.packed_varlen(kind, q, k, v, cu, a, b, S0, z0, iv, form="chunked")
            assert np.abs(o_c - o).max() < 1e-9 and np.abs(S_c - S).max() < 1e-9 and np.abs(sn_c - snaps).max() < 1e-9
            if kind == "normalized":
                assert np.abs(z_c - z).max() < 1e-12 and np.abs(zs_c - zsnaps).max() < 1e-12
        # without an initial state every sequence starts from zero
        o0, S0z, z0z, sn0, _ = ns.packed_varlen(kind, q, k, v, cu, a, b)
        assert sn0.shape[0] == 0 and np.all(S0z[1] == 0)
        if kind == "normalized":
            assert np.all(z0z[1] == 0)
        o_ref, _, _ = _kind_reference(kind, q[1, 13:26], k[1, 13:26], v[1, 13:26], sl(a, 1, 13, 26),
                                      sl(b, 1, 13, 26), None, None)
        assert np.abs(o0[1, 13:26] - o_ref).max() < 1e-12


def test_varlen_kinds_pin():
    pin_varlen_kinds(vl_mod)


VARLEN_KIND_MUTATIONS = [
    ("z = None if (not has_z or z0 is None) else np.asarray(z0[n, h], dtype=np.float64)", "z = None"),
    ("else z.copy())))", "else np.zeros_like(z))))"),
    ("A = None if gate is None else gate[h, start:cut]", "A = None if gate is None else gate[h, a:a + cut - start]"),
    ("B = None if wgt is None else wgt[h, start:cut]", "B = None if wgt is None else wgt[h, a:a + cut - start]"),
    ("z_fin[n, h] = np.zeros(dk) if z is None else z", "z_fin[n, h] = np.zeros(dk)"),
    ("kda_recurrent(Q, K, V, A, B, S) + (None,)", "kda_recurrent(Q, K, V, A, B, None) + (None,)"),
    ("gated_recurrent(Q, K, V, A, S) + (None,)", "gated_recurrent(Q, K, V, A, None) + (None,)"),
    ("la_recurrent(Q, K, V, S, z)", "la_recurrent(Q, K, V, S, None)"),
    ("o[h, start:cut], S, z = run(", "o[h, a:a + cut - start], S, z = run("),
]


@pytest.mark.parametrize("old,new", VARLEN_KIND_MUTATIONS, ids=[m[1][:40] for m in VARLEN_KIND_MUTATIONS])
def test_planted_varlen_kind_mistake_is_caught(old, new):
    ns = types.SimpleNamespace(**_mutant(vl_mod, old, new))
    assert _fails_some_pin(ns, [pin_varlen_kinds])
