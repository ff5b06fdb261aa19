"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Each test names the passage it follows.  None of them retypes the oracle's
own formula: they use printed worked examples, closed forms, special cases,
an independent quadrature of the expected per-table kernel, brute force on
tiny inputs, and central finite differences.
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import race_oracle as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rand_head(rng, N, d, L, P, scale=1.0):
    Q = rng.standard_normal((N, d)) * scale
    K = rng.standard_normal((N, d)) * scale
    V = rng.standard_normal((N, d))
    W = rng.standard_normal((L, P, d))
    return Q, K, V, W


# ---------------------------------------------------------------- worked examples

def test_teaching_example_readout():
    """Slides backup frame 'bucket masses change the answer' (teaching example)."""
    g = _load("teaching_example.json")
    phi_K = np.array(g["phi_K"])[None]            # (L=1, N=2, R=2)
    V = np.array(g["V"])[:, None]                 # (N=2, dv=1)
    phi_Q = np.array(g["phi_Q"])[None, None]      # (L=1, N=1, R=2)
    content, mass = orc.bucket_stats(phi_K, V)
    np.testing.assert_allclose(mass[0], g["mass_printed"], rtol=0, atol=1e-15)
    np.testing.assert_allclose(content[0, :, 0], g["content_printed"], rtol=0, atol=1e-14)
    O, num, den = orc.readout(phi_Q, content, mass)
    assert abs(num[0, 0] - g["num_printed"]) < 1e-14
    assert abs(den[0] - g["den_printed"]) < 1e-15
    # the page rounds O to 4 decimals; the exact ratio of its printed Num/Den:
    assert round(O[0, 0], g["O_printed_decimals"]) == g["O_printed"]
    assert abs(O[0, 0] - g["num_printed"] / g["den_printed"]) < 1e-14
    # equivalent pairwise weights phi(Q).phi(K_j)
    w = phi_K[0] @ phi_Q[0, 0]
    np.testing.assert_allclose(w, g["pairwise_weights_printed"], atol=1e-15)


def test_teaching_example_is_not_per_bucket_mean_mixing():
    """The same frame: mixing per-bucket means (the Fig. 7 reading) is another operator."""
    g = _load("teaching_example.json")
    phi_K = np.array(g["phi_K"])[None]
    V = np.array(g["V"])[:, None]
    phi_Q = np.array(g["phi_Q"])[None, None]
    content, mass = orc.bucket_stats(phi_K, V)
    O, _, _ = orc.readout(phi_Q, content, mass)
    mixed = float(phi_Q[0, 0] @ (content[0, :, 0] / mass[0]))
    assert round(mixed, 4) == g["per_bucket_mean_mixing_printed"]
    assert abs(O[0, 0] - mixed) > 0.2


def test_walkthrough_example():
    """Visual walkthrough, Step 5 worked example (S, Z summaries, out_1 = 14/6)."""
    g = _load("walkthrough_example.json")
    F = np.array(g["key_features"], dtype=float)[None]     # one "table" of width 3
    vals = np.array(g["values"], dtype=float)[:, None]
    S, Z = orc.bucket_stats(F, vals)
    np.testing.assert_array_equal(S[0, :, 0], g["S_printed"])
    np.testing.assert_array_equal(Z[0], g["Z_printed"])
    q = np.array(g["query_feature"], dtype=float)[None, None]
    out, num, den = orc.readout(q, S, Z)
    assert num[0, 0] == g["num_printed"] and den[0] == g["den_printed"]
    assert round(out[0, 0], g["out_printed_decimals"]) == g["out_printed"]


# ---------------------------------------------------------------- soft assignments

def test_corner_order_and_assignment_by_hand():
    """Algorithm 1 (slides frame 'Soft corner assignments ...') evaluated by hand
    for P = 2 with the corner order bit t of r set <=> v_{r,t} = +1."""
    x = np.array([0.7, -0.2, 0.4])
    W = np.array([[[0.5, 1.0, -0.3], [-1.2, 0.1, 0.8]]])    # L=1, P=2, d=3
    beta = 1.7
    u = np.tanh(W[0] @ x)
    v = {0: (-1, -1), 1: (1, -1), 2: (-1, 1), 3: (1, 1)}
    e = np.array([math.exp(beta * (u[0] * v[r][0] + u[1] * v[r][1])) for r in range(4)])
    expect = e / e.sum()
    phi = orc.soft_assign(x[None], W, beta)[0, 0]
    np.testing.assert_allclose(phi, expect, rtol=1e-14, atol=0)


@pytest.mark.parametrize("P", [1, 2, 3, 4, 6, 8])
def test_rows_are_distributions(P):
    """Each token becomes a probability vector over the buckets (slides, frame
    'Soft corner assignments ...'): entries > 0, rows sum to 1."""
    rng = np.random.default_rng(100 + P)
    X = rng.standard_normal((50, 16)) * 2.0
    W = rng.standard_normal((3, P, 16))
    for beta in (0.3, 4.0, 8.0):
        Phi = orc.soft_assign(X, W, beta)
        assert Phi.shape == (3, 50, 1 << P)
        assert np.all(Phi > 0)
        np.testing.assert_allclose(Phi.sum(-1), 1.0, atol=1e-14)


@pytest.mark.parametrize("P", [1, 2, 3, 5, 8])
def test_softmax_equals_product_of_sigmoids(P):
    """Reading notes section 2.4: phi_r = prod_t sigma(2 beta u_t v_{r,t})."""
    rng = np.random.default_rng(7 + P)
    X = rng.standard_normal((40, 12))
    W = rng.standard_normal((2, P, 12))
    for beta in (0.5, 2.0, 8.0):
        a = orc.soft_assign(X, W, beta)
        b = orc.soft_assign_sigmoid_product(X, W, beta)
        np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-300)


def test_beta_zero_is_uniform():
    """beta -> 0 gives uniform buckets (slides, frame 'Soft corner assignments ...'),
    so every output is the plain mean of the visible values and dQ = dK = 0."""
    rng = np.random.default_rng(3)
    Q, K, V, W = _rand_head(rng, 33, 8, 2, 3)
    Phi = orc.soft_assign(Q, W, 0.0)
    np.testing.assert_allclose(Phi, 1.0 / 8, atol=1e-16)
    O = orc.forward_head(Q, K, V, W, 0.0)
    np.testing.assert_allclose(O, np.broadcast_to(V.mean(0), O.shape), atol=1e-14)
    Oc = orc.causal_forward_head(Q, K, V, W, 0.0)
    run = np.cumsum(V, axis=0) / np.arange(1, 34)[:, None]
    np.testing.assert_allclose(Oc, run, atol=1e-14)
    dO = rng.standard_normal(V.shape)
    for causal in (False, True):
        dQ, dK, dV = orc.backward_head(Q, K, V, W, 0.0, dO, causal)
        assert np.abs(dQ).max() == 0.0 and np.abs(dK).max() == 0.0


# ---------------------------------------------------------------- hashing limits

def _unit_pair(d, theta, rng):
    a = rng.standard_normal(d)
    a /= np.linalg.norm(a)
    b = rng.standard_normal(d)
    b -= a * (a @ b)
    b /= np.linalg.norm(b)
    return a, math.cos(theta) * a + math.sin(theta) * b


def _per_table_kernel(q, k, W, beta):
    Phi = orc.soft_assign(np.stack([q, k]), W, beta)      # (T, 2, R)
    return np.einsum("tr,tr->t", Phi[:, 0], Phi[:, 1])


@pytest.mark.parametrize("P", [1, 2, 3])
def test_hard_hash_limit_is_powered_angular_kernel(P):
    """At large beta the collision frequency of the soft buckets tends to
    kappa_ang^P with kappa_ang = 1 - theta/pi (slides, frames 'A hash collision
    estimates a powered angular kernel' and 'Choose a nonnegative kernel ...'):
    values 1, 1/2 and 0 at angles 0, pi/2, pi."""
    rng = np.random.default_rng(11 * P)
    d, T, beta = 6, 1 << 17, 1.0e4
    for theta in (0.0, math.pi / 3, math.pi / 2, 2 * math.pi / 3, math.pi):
        q, k = _unit_pair(d, theta, rng)
        W = rng.standard_normal((T, P, d))
        s = _per_table_kernel(q, k, W, beta)
        kappa = 1.0 - theta / math.pi
        se = s.std() / math.sqrt(T)
        assert abs(s.mean() - kappa ** P) <= 5 * se + 2e-3, (theta, s.mean(), kappa ** P)
    # closed forms at 0, pi/2, pi
    q, k = _unit_pair(d, 0.0, rng)
    assert abs(_per_table_kernel(q, q, rng.standard_normal((4096, P, d)), beta).mean() - 1.0) < 2e-3
    assert _per_table_kernel(q, -q, rng.standard_normal((4096, P, d)), beta).mean() < 2e-3


def _expected_kernel_quadrature(q, k, beta, P, n=160):
    """E_W[phi(q).phi(k)] for one table with iid N(0, I) rows, by 2-D Gauss-Hermite
    quadrature.  Rows are independent, so the expectation is E_bit^P with
    E_bit = E[s1 s2 + (1 - s1)(1 - s2)], s_i = sigma(2 beta tanh z_i) and
    (z1, z2) bivariate normal with covariance [[|q|^2, q.k], [q.k, |k|^2]]."""
    x, w = np.polynomial.hermite_e.hermegauss(n)
    cov = np.array([[q @ q, q @ k], [q @ k, k @ k]])
    Lc = np.linalg.cholesky(cov)
    X1, X2 = np.meshgrid(x, x, indexing="ij")
    z1 = Lc[0, 0] * X1
    z2 = Lc[1, 0] * X1 + Lc[1, 1] * X2
    s1 = 1.0 / (1.0 + np.exp(-2 * beta * np.tanh(z1)))
    s2 = 1.0 / (1.0 + np.exp(-2 * beta * np.tanh(z2)))
    f = s1 * s2 + (1 - s1) * (1 - s2)
    e_bit = np.einsum("i,j,ij->", w, w, f) / (2 * math.pi)
    return e_bit ** P


@pytest.mark.parametrize("beta,P,norm", [(2.0, 2, 1.0), (1.0, 3, 2.0), (0.5, 1, 0.7)])
def test_finite_beta_expectation_matches_quadrature(beta, P, norm):
    """Monte Carlo over Gaussian tables of the oracle's per-table kernel equals an
    independent quadrature of its expectation (Gaussian W: slides frame 'Soft
    corner assignments ...'; factorisation: reading notes section 2.4).  This
    pins tanh, the sign of the logits, beta and the corner enumeration."""
    rng = np.random.default_rng(int(beta * 100) + P)
    d, T = 5, 1 << 17
    q, k = _unit_pair(d, 1.1, rng)
    q, k = q * norm, k * 1.3
    W = rng.standard_normal((T, P, d))
    s = _per_table_kernel(q, k, W, beta)
    ref = _expected_kernel_quadrature(q, k, beta, P)
    se = s.std() / math.sqrt(T)
    assert abs(s.mean() - ref) <= 5 * se, (s.mean(), ref, se)
    # a plausible mistake (tanh left out) is separated by far more than 5 sigma
    x, w = np.polynomial.hermite_e.hermegauss(80)
    assert abs(ref - _no_tanh_quad(q, k, beta, P)) > 10 * se


def _no_tanh_quad(q, k, beta, P, n=80):
    x, w = np.polynomial.hermite_e.hermegauss(n)
    cov = np.array([[q @ q, q @ k], [q @ k, k @ k]])
    Lc = np.linalg.cholesky(cov)
    X1, X2 = np.meshgrid(x, x, indexing="ij")
    z1 = Lc[0, 0] * X1
    z2 = Lc[1, 0] * X1 + Lc[1, 1] * X2
    s1 = 1.0 / (1.0 + np.exp(-2 * beta * z1))
    s2 = 1.0 / (1.0 + np.exp(-2 * beta * z2))
    f = s1 * s2 + (1 - s1) * (1 - s2)
    return (np.einsum("i,j,ij->", w, w, f) / (2 * math.pi)) ** P


def test_lemma10_setting():
    """Slides backup frame 'Lemma 10 omits the soft-hash bias': all Q, K equal one
    unit vector, P = 2, beta = 0.1 -> per-table S_hat_ij = |phi|^2 < e^0.4/4,
    while normalisation still returns the mean of V."""
    rng = np.random.default_rng(5)
    d, N = 7, 20
    x = rng.standard_normal(d)
    x /= np.linalg.norm(x)
    X = np.tile(x, (N, 1))
    V = rng.standard_normal((N, 3))
    for L in (1, 4, 16):
        W = rng.standard_normal((L, 2, d))
        O, S = orc.brute_force_head(X, X, V, W, 0.1)
        assert S.max() < math.exp(0.4) / 4 < 0.373
        np.testing.assert_allclose(O, np.broadcast_to(V.mean(0), O.shape), atol=1e-14)
        np.testing.assert_allclose(orc.forward_head(X, X, V, W, 0.1), O, atol=1e-14)


# ---------------------------------------------------------------- readout structure

@pytest.mark.parametrize("causal", [False, True])
def test_associative_form_equals_brute_force(causal):
    """Phi_Q (Phi_K^T V) = (Phi_Q Phi_K^T) V (slides, frame 'Normalize after
    combining the tables'); causal keeps j <= i (Algorithm 2)."""
    rng = np.random.default_rng(21 + causal)
    for (N, d, L, P, beta) in [(17, 5, 2, 3, 1.0), (64, 8, 3, 2, 4.0), (200, 16, 4, 4, 8.0)]:
        Q, K, V, W = _rand_head(rng, N, d, L, P)
        Ob, _ = orc.brute_force_head(Q, K, V, W, beta, causal)
        if causal:
            O1 = orc.causal_forward_head(Q, K, V, W, beta, block=7)
            O2 = orc.causal_forward_head_loop(Q, K, V, W, beta)
            np.testing.assert_allclose(O2, Ob, rtol=1e-12, atol=1e-12)
        else:
            O1 = orc.forward_head(Q, K, V, W, beta)
        np.testing.assert_allclose(O1, Ob, rtol=1e-12, atol=1e-12)


def test_rank_bound():
    """The non-causal kernel S_hat has rank at most L*R (slides, frame 'Linear
    cost assumes a fixed bucket budget', reader's deduction)."""
    rng = np.random.default_rng(8)
    Q, K, V, W = _rand_head(rng, 96, 10, 2, 2)
    _, S = orc.brute_force_head(Q, K, V, W, 1.5)
    sv = np.linalg.svd(S, compute_uv=False)
    assert np.sum(sv > 1e-10 * sv[0]) <= 2 * 4


@pytest.mark.parametrize("causal", [False, True])
def test_convex_combination(causal):
    """Normalisation makes each output a convex combination of values (slides,
    frame 'Choose a nonnegative kernel ...'): inside V's per-column range, and
    constant V gives that constant."""
    rng = np.random.default_rng(9 + causal)
    Q, K, V, W = _rand_head(rng, 80, 6, 3, 3)
    f = orc.causal_forward_head if causal else orc.forward_head
    O = f(Q, K, V, W, 3.0)
    assert np.all(O <= V.max(0) + 1e-12) and np.all(O >= V.min(0) - 1e-12)
    c = np.array([1.5, -2.0, 0.0, 3.25, 7.0, -0.5])
    Oc = f(Q, K, np.tile(c, (80, 1)), W, 3.0)
    np.testing.assert_allclose(Oc, np.broadcast_to(c, Oc.shape), rtol=1e-13, atol=1e-13)


def test_causal_first_token_attends_to_itself():
    """Update before read (slides, frame 'Causality is a prefix update ...'), so
    O_1 = V_1 -- the walkthrough's Step 6 Case B (a lone token)."""
    rng = np.random.default_rng(12)
    Q, K, V, W = _rand_head(rng, 10, 4, 2, 3)
    O = orc.causal_forward_head(Q, K, V, W, 6.0)
    np.testing.assert_allclose(O[0], V[0], rtol=1e-14, atol=1e-15)
    # a one-token non-causal input returns its value as well (Case B)
    O1 = orc.forward_head(Q[:1], K[:1], V[:1], W, 6.0)
    np.testing.assert_allclose(O1[0], V[0], rtol=1e-14, atol=1e-15)


def test_causal_prefix_only_sees_past():
    """Causal output at t depends only on tokens j <= t (Algorithm 2)."""
    rng = np.random.default_rng(13)
    Q, K, V, W = _rand_head(rng, 40, 4, 2, 3)
    O = orc.causal_forward_head(Q, K, V, W, 2.0)
    K2, V2 = K.copy(), V.copy()
    K2[25:] = rng.standard_normal(K2[25:].shape)
    V2[25:] = rng.standard_normal(V2[25:].shape)
    O2 = orc.causal_forward_head(Q, K2, V2, W, 2.0)
    np.testing.assert_array_equal(O[:25], O2[:25])
    assert np.abs(O[25:] - O2[25:]).max() > 1e-3


def test_corner_relabeling_invariance():
    """Flipping the sign of one hyperplane (or reordering them) relabels the
    corners consistently, which permutes Phi but leaves O unchanged."""
    rng = np.random.default_rng(14)
    Q, K, V, W = _rand_head(rng, 30, 5, 2, 3)
    O = orc.forward_head(Q, K, V, W, 2.5)
    W2 = W.copy()
    W2[1, 2] *= -1.0
    W2[0] = W2[0][[2, 0, 1]]
    np.testing.assert_allclose(orc.forward_head(Q, K, V, W2, 2.5), O, rtol=1e-12, atol=1e-13)
    Phi, Phi2 = orc.soft_assign(Q, W, 2.5), orc.soft_assign(Q, W2, 2.5)
    r = np.arange(8)
    np.testing.assert_allclose(Phi2[1], Phi[1][:, r ^ 4], rtol=1e-13)


def test_tables_normalised_jointly_not_per_table():
    """Tables are combined before the ratio ('ratio of summed numerators and
    denominators, rather than an average of ratios')."""
    rng = np.random.default_rng(15)
    Q, K, V, W = _rand_head(rng, 25, 4, 3, 2)
    O = orc.forward_head(Q, K, V, W, 4.0)
    per = np.mean([orc.forward_head(Q, K, V, W[l:l + 1], 4.0) for l in range(3)], axis=0)
    assert np.abs(O - per).max() > 1e-3


def test_batched_wrappers():
    rng = np.random.default_rng(16)
    B, H, N, d = 2, 3, 20, 4
    Q = rng.standard_normal((B, H, N, d))
    K = rng.standard_normal((B, H, N, d))
    V = rng.standard_normal((B, H, N, d))
    W = rng.standard_normal((2, 2, d))
    for causal in (False, True):
        O = orc.forward(Q, K, V, W, 1.0, causal)
        f = orc.causal_forward_head if causal else orc.forward_head
        np.testing.assert_array_equal(O[1, 2], f(Q[1, 2], K[1, 2], V[1, 2], W, 1.0))


# ---------------------------------------------------------------- backward

def _loss(Q, K, V, W, beta, dO, causal):
    f = orc.causal_forward_head if causal else orc.forward_head
    return float(np.sum(f(Q, K, V, W, beta) * dO))


@pytest.mark.parametrize("causal", [False, True])
def test_backward_finite_differences(causal):
    """dQ, dK, dV equal central finite differences of sum(O * dO)."""
    rng = np.random.default_rng(30 + causal)
    N, d, L, P, beta = 7, 4, 2, 2, 1.5
    Q, K, V, W = _rand_head(rng, N, d, L, P)
    dO = rng.standard_normal((N, d))
    dQ, dK, dV = orc.backward_head(Q, K, V, W, beta, dO, causal)
    eps = 1e-6
    for X, G in ((Q, dQ), (K, dK), (V, dV)):
        num = np.empty_like(X)
        for idx in np.ndindex(X.shape):
            old = X[idx]
            X[idx] = old + eps
            lp = _loss(Q, K, V, W, beta, dO, causal)
            X[idx] = old - eps
            lm = _loss(Q, K, V, W, beta, dO, causal)
            X[idx] = old
            num[idx] = (lp - lm) / (2 * eps)
        assert np.abs(num - G).max() <= 1e-6 * max(1.0, np.abs(G).max()), (causal, np.abs(num - G).max())


@pytest.mark.parametrize("causal", [False, True])
def test_backward_invariants(causal):
    """Rows of the normalised kernel sum to one, so sum_j dV_j = sum_i dO_i;
    constant V gives dQ = dK = 0; V -> V + c changes no gradient."""
    rng = np.random.default_rng(40 + causal)
    N, d, L, P, beta = 300, 8, 3, 3, 4.0
    Q, K, V, W = _rand_head(rng, N, d, L, P)
    dO = rng.standard_normal((N, d))
    dQ, dK, dV = orc.backward_head(Q, K, V, W, beta, dO, causal)
    np.testing.assert_allclose(dV.sum(0), dO.sum(0), rtol=1e-11, atol=1e-11)
    c = rng.standard_normal(d)
    dQ2, dK2, dV2 = orc.backward_head(Q, K, V + c, W, beta, dO, causal)
    for a, b in ((dQ, dQ2), (dK, dK2), (dV, dV2)):
        np.testing.assert_allclose(a, b, rtol=1e-9, atol=1e-11 * np.abs(a).max())
    dQc, dKc, _ = orc.backward_head(Q, K, np.tile(c, (N, 1)), W, beta, dO, causal)
    assert np.abs(dQc).max() < 1e-11 * np.abs(dQ).max()
    assert np.abs(dKc).max() < 1e-11 * np.abs(dK).max()


def test_backward_causal_equals_masked_brute_force_gradient():
    """Causal gradients via prefix/suffix sums equal the gradients of the masked
    N x N form computed by finite differences on a second tiny case."""
    rng = np.random.default_rng(50)
    N, d, L, P, beta = 5, 3, 1, 3, 2.0
    Q, K, V, W = _rand_head(rng, N, d, L, P)
    dO = rng.standard_normal((N, d))
    dQ, dK, dV = orc.backward_head(Q, K, V, W, beta, dO, True)

    def loss(Q, K, V):
        return float(np.sum(orc.brute_force_head(Q, K, V, W, beta, True)[0] * dO))

    eps = 1e-6
    for which, G in ((0, dQ), (1, dK), (2, dV)):
        args = [Q.copy(), K.copy(), V.copy()]
        num = np.empty_like(G)
        for idx in np.ndindex(G.shape):
            a = [x.copy() for x in args]
            a[which][idx] += eps
            lp = loss(*a)
            a[which][idx] -= 2 * eps
            lm = loss(*a)
            num[idx] = (lp - lm) / (2 * eps)
        assert np.abs(num - G).max() <= 1e-6 * max(1.0, np.abs(G).max())


def test_causal_blocks_with_initial_bank_equal_whole_sequence():
    """Evaluating the tail of a causal sequence from the bank of its prefix
    gives the same outputs and gradients of the tail as the whole sequence."""
    rng = np.random.default_rng(60)
    N, d, L, P, beta, cut = 90, 5, 2, 3, 3.0, 57
    Q, K, V, W = _rand_head(rng, N, d, L, P)
    dO = rng.standard_normal((N, d))
    O = orc.causal_forward_head(Q, K, V, W, beta)
    dQ, dK, dV = orc.backward_head(Q, K, V, W, beta, dO, True)
    c0, m0 = orc.state_head(K[:cut], V[:cut], W, beta)
    Ot = orc.causal_forward_head(Q[cut:], K[cut:], V[cut:], W, beta, content0=c0, mass0=m0)
    np.testing.assert_allclose(Ot, O[cut:], rtol=1e-12, atol=1e-13)
    tq, tk, tv = orc.backward_head(Q[cut:], K[cut:], V[cut:], W, beta, dO[cut:], True, content0=c0, mass0=m0)
    for a, b in ((tq, dQ[cut:]), (tk, dK[cut:]), (tv, dV[cut:])):
        np.testing.assert_allclose(a, b, rtol=1e-10, atol=1e-12 * np.abs(b).max())


def test_causal_kernel_blocks_equal_prefix_readout():
    """The block-wise causal evaluation (statistics of the keys before a
    block plus the implicit kernel over the block's keys j <= t) gives the
    O and Den of the per-token prefix readout, the one-token loop and the
    masked brute-force kernel, for blocks that do not divide N, with and
    without a starting bank; its final statistics are those of all keys."""
    rng = np.random.default_rng(62)
    for (N, d, L, P, beta, block) in [(37, 5, 2, 3, 2.0, 8), (130, 6, 3, 2, 6.0, 32), (64, 4, 2, 4, 1.0, 64)]:
        Q, K, V, W = _rand_head(rng, N, d, L, P)
        O_ref, Den_ref = orc.causal_forward_head(Q, K, V, W, beta, return_den=True)
        O, Den, c, m = orc.causal_forward_head_kernel_blocks(Q, K, V, W, beta, block=block)
        np.testing.assert_allclose(O, O_ref, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(Den, Den_ref, rtol=1e-12)
        np.testing.assert_allclose(O, orc.causal_forward_head_loop(Q, K, V, W, beta), rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(O, orc.brute_force_head(Q, K, V, W, beta, True)[0], rtol=1e-12, atol=1e-13)
        c_all, m_all = orc.state_head(K, V, W, beta)
        np.testing.assert_allclose(c, c_all, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(m, m_all, rtol=1e-12)
        cut = N // 3
        c0, m0 = orc.state_head(K[:cut], V[:cut], W, beta)
        Ot, Dt, _, _ = orc.causal_forward_head_kernel_blocks(Q[cut:], K[cut:], V[cut:], W, beta, block=block,
                                                             content0=c0, mass0=m0)
        np.testing.assert_allclose(Ot, O_ref[cut:], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(Dt, Den_ref[cut:], rtol=1e-12)


def test_bank_level_pieces_compose_to_backward():
    """query_grads / grad_banks / key_grads evaluated in two halves and summed
    give the single-call gradients (bank sums are additive over rows)."""
    rng = np.random.default_rng(61)
    Q, K, V, W = _rand_head(rng, 70, 6, 2, 3)
    dO = rng.standard_normal((70, 6))
    dQ, dK, dV = orc.backward_head(Q, K, V, W, 2.0, dO, False)
    content, mass = orc.state_head(K, V, W, 2.0)
    parts = [orc.query_grads(Q[s], dO[s], W, 2.0, content, mass) for s in (slice(0, 30), slice(30, 70))]
    np.testing.assert_allclose(np.concatenate([p[0] for p in parts]), dQ, rtol=1e-12, atol=1e-14)
    banks = [orc.grad_banks(Q[s], W, 2.0, p[3], p[4]) for s, p in zip((slice(0, 30), slice(30, 70)), parts)]
    dc = banks[0][0] + banks[1][0]
    dm = banks[0][1] + banks[1][1]
    gk, gv = orc.key_grads(K, V, W, 2.0, dc, dm)
    np.testing.assert_allclose(gk, dK, rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(gv, dV, rtol=1e-11, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("beta", [0.7, 4.0])
def test_dbeta_finite_differences(causal, beta):
    """dL/dbeta (query-side plus key-side terms) equals the central finite
    difference of sum(O * dO) in beta (logits beta * u . v_r)."""
    rng = np.random.default_rng(60 + 2 * causal + int(beta))
    N, d, L, P = 9, 5, 2, 3
    Q, K, V, W = _rand_head(rng, N, d, L, P)
    dO = rng.standard_normal((N, d))
    tq, tk = orc.dbeta_head(Q, K, V, W, beta, dO, causal)
    eps = 1e-6
    num = (_loss(Q, K, V, W, beta + eps, dO, causal) - _loss(Q, K, V, W, beta - eps, dO, causal)) / (2 * eps)
    got = tq.sum() + tk.sum()
    assert abs(got - num) <= 1e-7 * max(1.0, np.abs(tq).sum() + np.abs(tk).sum()), (causal, beta, got, num)
    # the batched wrapper adds the same terms
    assert abs(orc.dbeta(Q[None, None], K[None, None], V[None, None], W, beta, dO[None, None], causal) - got) < 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_dbeta_invariants(causal):
    """Constant V makes O independent of beta, so dbeta = 0; V -> V + c
    shifts O by c and leaves dbeta unchanged."""
    rng = np.random.default_rng(70 + causal)
    N, d, L, P, beta = 200, 6, 3, 3, 2.5
    Q, K, V, W = _rand_head(rng, N, d, L, P)
    dO = rng.standard_normal((N, d))
    tq, tk = orc.dbeta_head(Q, K, V, W, beta, dO, causal)
    scale = np.abs(tq).sum() + np.abs(tk).sum()
    c = rng.standard_normal(d)
    tq2, tk2 = orc.dbeta_head(Q, K, V + c, W, beta, dO, causal)
    assert abs((tq2.sum() + tk2.sum()) - (tq.sum() + tk.sum())) < 1e-10 * scale
    tqc, tkc = orc.dbeta_head(Q, K, np.tile(c, (N, 1)), W, beta, dO, causal)
    assert abs(tqc.sum() + tkc.sum()) < 1e-11 * scale


@pytest.mark.parametrize("causal", [False, True])
def test_dW_finite_differences(causal):
    """dL/dW (query-side plus key-side parts) equals the central finite
    difference of sum(O * dO) in every entry of the tables (the
    pre-activations are W^(l) x; slides, frame "Soft corner assignments make
    hashing differentiable")."""
    rng = np.random.default_rng(80 + causal)
    N, d, L, P, beta = 9, 5, 2, 3, 1.5
    Q, K, V, W = _rand_head(rng, N, d, L, P)
    dO = rng.standard_normal((N, d))
    wq, wk = orc.dW_head(Q, K, V, W, beta, dO, causal)
    got = wq + wk
    eps = 1e-6
    num = np.empty_like(W)
    for idx in np.ndindex(*W.shape):
        Wp, Wm = W.copy(), W.copy()
        Wp[idx] += eps
        Wm[idx] -= eps
        num[idx] = (_loss(Q, K, V, Wp, beta, dO, causal) - _loss(Q, K, V, Wm, beta, dO, causal)) / (2 * eps)
    scale = max(1.0, np.abs(got).max())
    assert np.abs(got - num).max() <= 1e-7 * scale, (causal, np.abs(got - num).max())
    # the batched wrapper adds the same parts
    np.testing.assert_allclose(orc.dW(Q[None, None], K[None, None], V[None, None], W, beta, dO[None, None], causal),
                               got, rtol=0, atol=1e-12 * scale)


@pytest.mark.parametrize("causal", [False, True])
def test_dW_scaling_identity(causal):
    """Scaling the rows of one side by s and its projection by 1/s leaves
    every pre-activation W^(l) x unchanged, so per side
    <dW_side, W> = <dX, X> with dX the finite-difference-pinned input
    gradient (Q side: dQ, K side: dK)."""
    rng = np.random.default_rng(90 + causal)
    N, d, L, P, beta = 150, 6, 3, 3, 2.5
    Q, K, V, W = _rand_head(rng, N, d, L, P)
    dO = rng.standard_normal((N, d))
    wq, wk = orc.dW_head(Q, K, V, W, beta, dO, causal)
    dQ, dK, _ = orc.backward_head(Q, K, V, W, beta, dO, causal)
    for part, dX, X in ((wq, dQ, Q), (wk, dK, K)):
        lhs, rhs = float(np.sum(part * W)), float(np.sum(dX * X))
        assert abs(lhs - rhs) <= 1e-10 * max(1.0, float(np.sum(np.abs(dX * X)))), (causal, lhs, rhs)


def test_dW_zero_beta_and_per_head_tables():
    """beta = 0 makes every assignment uniform whatever W is, so dW = 0.
    Per-head tables that are all equal give per-head gradients whose sum over
    heads is the shared-table gradient; a finite difference in one head's
    table moves only that head's loss."""
    rng = np.random.default_rng(95)
    B, H, N, d, L, P = 2, 3, 40, 6, 2, 3
    Q = rng.standard_normal((B, H, N, d))
    K = rng.standard_normal((B, H, N, d))
    V = rng.standard_normal((B, H, N, d))
    dO = rng.standard_normal((B, H, N, d))
    W = rng.standard_normal((L, P, d))
    for causal in (False, True):
        assert np.abs(orc.dW(Q, K, V, W, 0.0, dO, causal)).max() == 0.0
        shared = orc.dW(Q, K, V, W, 1.7, dO, causal)
        per_head = orc.dW(Q, K, V, np.stack([W] * H), 1.7, dO, causal)
        np.testing.assert_allclose(per_head.sum(axis=0), shared, rtol=0, atol=1e-12 * np.abs(shared).max())
    W4 = rng.standard_normal((H, L, P, d))
    for causal in (False, True):
        g = orc.dW(Q, K, V, W4, 1.7, dO, causal)
        eps = 1e-6
        for idx in [(0, 0, 1, 2), (2, 1, 0, 5), (1, 1, 2, 0)]:
            Wp, Wm = W4.copy(), W4.copy()
            Wp[idx] += eps
            Wm[idx] -= eps
            num = (np.sum(orc.forward(Q, K, V, Wp, 1.7, causal) * dO)
                   - np.sum(orc.forward(Q, K, V, Wm, 1.7, causal) * dO)) / (2 * eps)
            assert abs(g[idx] - num) <= 1e-7 * max(1.0, np.abs(g).max()), (causal, idx, g[idx], num)
