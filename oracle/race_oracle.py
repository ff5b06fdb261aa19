"""Plain float64 CPU oracle of the RACE attention layer.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the test suite, the smoke check and the CPU
baseline leg of the benchmark use it.  It shares no code with the HIP
library and imports nothing from the product package.

Sources (the method's definition; cited by page title and section):

* "RACE Attention" slides (English deck on arXiv 2510.04008v5):
  frame "Soft corner assignments make hashing differentiable" (paper
  Algorithm 1), frame "Each bucket stores mass and a weighted value sum",
  frame "Normalize after combining the tables", frame "Causality is a prefix
  update of the same statistics" (paper Algorithm 2), backup frame "bucket
  masses change the answer" (teaching example).
* "RACE Attention" reading notes (Chinese): section 2.2 (notation),
  section 2.4 (soft bucketing, product-of-sigmoids identity),
  section 2.5 (aggregation and global-ratio readout),
  section 2.6 (causal prefix buckets).
* "Long-context architectures: Visual walkthrough": Step 4/5 (the S, Z
  summaries and their worked example), Step 6 (degenerate cases).

Conventions (readings where the pages are silent):

* Corner r of the P-cube has coordinate t equal to +1 exactly when bit t of
  r is set (bit 0 is the least significant bit).
* The 1/L factor the slides put on both Num and Den is left out: it cancels
  in Num/Den exactly.  ``brute_force`` keeps it, as the implicit kernel is
  written with it.
* No epsilon is added to the denominator; all features are positive.
* W has shape (L, P, d) and is shared by every batch row and head; the
  batched functions also take per-head tables (H, L, P, d).
* The backward pass is the exact gradient of the forward map with W and beta
  held fixed; ``dbeta_head`` adds the gradient with respect to beta, the
  inverse temperature the pages train (logits beta * u . v_r), and
  ``dW_head`` the gradient with respect to the tables, for tables that are
  trained or differ per head.

Everything is float64 numpy.  Arrays for one head are (N, d); batched
arrays are (B, H, N, d).
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "corners",
    "soft_assign",
    "soft_assign_sigmoid_product",
    "bucket_stats",
    "readout",
    "forward_head",
    "causal_forward_head",
    "causal_forward_head_loop",
    "brute_force_head",
    "backward_head",
    "forward",
    "backward",
    "state_head",
    "query_grads",
    "query_terms",
    "grad_banks",
    "key_grads",
    "beta_terms",
    "dbeta_head",
    "dbeta",
]


def corners(P: int) -> np.ndarray:
    """Hypercube corners v_r in {+1,-1}^P as an (R, P) float64 matrix, R = 2^P.

    The corner set is defined in the slides' frame "Soft corner assignments
    make hashing differentiable"; the pages leave their order open, so row r
    has +1 in column t exactly when bit t of r is 1.
    """
    R = 1 << P
    r = np.arange(R)[:, None]
    t = np.arange(P)[None, :]
    return np.where((r >> t) & 1, 1.0, -1.0)


def _projected(X: np.ndarray, W: np.ndarray) -> np.ndarray:
    """u^(l)(x) = tanh(W^(l) x) for every table: (N, d) x (L, P, d) -> (L, N, P).

    Slides, frame "Soft corner assignments make hashing differentiable".
    """
    X = np.asarray(X, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    pre = np.matmul(X[None], W.transpose(0, 2, 1))
    return np.tanh(pre)


def soft_assign(X: np.ndarray, W: np.ndarray, beta: float) -> np.ndarray:
    """Soft corner assignments Phi^(l)(X), shape (L, N, R).

    phi_r(x) = exp(beta u.v_r) / sum_r' exp(beta u.v_r'), u = tanh(W x)
    (slides, frame "Soft corner assignments make hashing differentiable";
    reading notes section 2.4).  The row maximum is subtracted before exp,
    which changes nothing in exact arithmetic.
    """
    U = _projected(X, W)                       # (L, N, P)
    C = corners(W.shape[1])                    # (R, P)
    logits = float(beta) * np.matmul(U, C.T)
    logits = logits - logits.max(axis=-1, keepdims=True)
    E = np.exp(logits)
    return E / E.sum(axis=-1, keepdims=True)


def soft_assign_sigmoid_product(X: np.ndarray, W: np.ndarray, beta: float) -> np.ndarray:
    """Same assignments through the identity phi_r = prod_t sigma(2 beta u_t v_{r,t}).

    Reading notes section 2.4 (the factorisation taken from the paper's
    Sec. 6.2).  Used only to cross-check ``soft_assign``.
    """
    U = _projected(X, W)                       # (L, N, P)
    C = corners(W.shape[1])                    # (R, P)
    z = 2.0 * float(beta) * U[:, :, None, :] * C[None, None, :, :]   # (L, N, R, P)
    sig = np.exp(np.minimum(z, 0.0)) / (1.0 + np.exp(-np.abs(z)))   # logistic, no overflow
    return np.prod(sig, axis=-1)


def bucket_stats(Phi_K: np.ndarray, V: np.ndarray):
    """Per-table bucket mass and content.

    mass^(l) = Phi_K^(l)^T 1_N (R,), content^(l) = Phi_K^(l)^T V (R, dv).
    Slides, frame "Each bucket stores mass and a weighted value sum" (there
    mass is lettered A and content B); reading notes section 2.5.
    Phi_K: (L, N, R); V: (N, dv).  Returns (content (L, R, dv), mass (L, R)).
    """
    Phi_K = np.asarray(Phi_K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    content = np.matmul(Phi_K.transpose(0, 2, 1), V)
    mass = Phi_K.sum(axis=1)
    return content, mass


def readout(Phi_Q: np.ndarray, content: np.ndarray, mass: np.ndarray):
    """Combine tables, then one global ratio.

    Num = sum_l Phi_Q^(l) content^(l), Den = sum_l Phi_Q^(l) mass^(l),
    O = diag(Den)^-1 Num (slides, frame "Normalize after combining the
    tables"; reading notes section 2.5).  Returns (O, Num, Den).
    """
    Phi_Q = np.asarray(Phi_Q, dtype=np.float64)
    L, N, R = Phi_Q.shape
    F = Phi_Q.transpose(1, 0, 2).reshape(N, L * R)        # tables side by side
    Num = F @ np.asarray(content, dtype=np.float64).reshape(L * R, -1)
    Den = F @ np.asarray(mass, dtype=np.float64).reshape(L * R)
    return Num / Den[:, None], Num, Den


def state_head(K, V, W, beta):
    """Non-causal bucket state of one head: (content (L, R, d), mass (L, R))."""
    return bucket_stats(soft_assign(K, W, beta), V)


def forward_head(Q, K, V, W, beta):
    """Non-causal RACE output of one head, (N, d) -> (N, d).

    Algorithm 1 as the slides state it: assignments, bucket statistics,
    readout, normalisation.
    """
    content, mass = bucket_stats(soft_assign(K, W, beta), V)
    O, _, _ = readout(soft_assign(Q, W, beta), content, mass)
    return O


def causal_forward_head_loop(Q, K, V, W, beta):
    """Causal RACE output of one head, one token at a time.

    Algorithm 2 as in the slides' frame "Causality is a prefix update of the
    same statistics": at step t first add phi(K_t) to the masses and
    phi(K_t) V_t^T to the contents, then read with phi(Q_t).  Small N only.
    """
    Phi_Q = soft_assign(Q, W, beta)            # (L, N, R)
    Phi_K = soft_assign(K, W, beta)
    V = np.asarray(V, dtype=np.float64)
    L, N, R = Phi_K.shape
    content = np.zeros((L, R, V.shape[1]))
    mass = np.zeros((L, R))
    O = np.empty((N, V.shape[1]))
    for t in range(N):
        mass += Phi_K[:, t, :]
        content += Phi_K[:, t, :, None] * V[t][None, None, :]
        num = np.einsum("lr,lrc->c", Phi_Q[:, t, :], content)
        den = np.einsum("lr,lr->", Phi_Q[:, t, :], mass)
        O[t] = num / den
    return O


def _prefix_states(Phi_K, V, t0, t1, content0, mass0):
    """Inclusive prefix states for tokens t0..t1-1 starting from given sums."""
    pc = np.cumsum(Phi_K[:, t0:t1, :, None] * V[None, t0:t1, None, :], axis=1)
    pm = np.cumsum(Phi_K[:, t0:t1, :], axis=1)
    return content0[:, None] + pc, mass0[:, None] + pm


def causal_forward_head(Q, K, V, W, beta, block=256, return_den=False, content0=None, mass0=None):
    """Causal RACE output of one head through inclusive prefix sums.

    Same quantities as ``causal_forward_head_loop``; the running sums
    content_t = sum_{j<=t} phi(K_j) V_j^T and mass_t = sum_{j<=t} phi(K_j)
    are formed with cumulative sums, ``block`` tokens at a time only to bound
    memory (the sums themselves are the plain prefix sums).  ``content0`` and
    ``mass0`` (default zero) are the bank of keys that precede this block of
    the sequence, so a long sequence can be evaluated piece by piece.
    """
    Phi_Q = soft_assign(Q, W, beta)
    Phi_K = soft_assign(K, W, beta)
    V = np.asarray(V, dtype=np.float64)
    L, N, R = Phi_K.shape
    dv = V.shape[1]
    O = np.empty((N, dv))
    Den = np.empty(N)
    c0 = np.zeros((L, R, dv)) if content0 is None else np.array(content0, dtype=np.float64)
    m0 = np.zeros((L, R)) if mass0 is None else np.array(mass0, dtype=np.float64)
    for t0 in range(0, N, block):
        t1 = min(N, t0 + block)
        pc, pm = _prefix_states(Phi_K, V, t0, t1, c0, m0)
        num = np.einsum("lnr,lnrc->nc", Phi_Q[:, t0:t1], pc)
        den = np.einsum("lnr,lnr->n", Phi_Q[:, t0:t1], pm)
        O[t0:t1] = num / den[:, None]
        Den[t0:t1] = den
        c0, m0 = pc[:, -1], pm[:, -1]
    return (O, Den) if return_den else O


def causal_forward_head_kernel_blocks(Q, K, V, W, beta, block=256, content0=None, mass0=None):
    """Causal RACE output of one head, evaluated a block of tokens at a time
    through the two equal forms the pages give for one readout (slides frame
    "Normalize after combining the tables": bucket statistics read out by
    phi(Q), or the implicit kernel S_tj = sum_l phi^(l)(Q_t) . phi^(l)(K_j)
    applied to the keys; reading notes section 2.5).  The causal readout of
    token t sums over the keys j <= t (slides frame "Causality is a prefix
    update of the same statistics"); here the keys before t's block enter
    through their statistics (content0 / mass0 plus earlier blocks) and the
    block's own keys j <= t through S_tj [V_j | 1].  Every key is counted
    once, so O and Den equal those of ``causal_forward_head``, without one
    bank per token (long sequences stay affordable).

    Returns (O, Den, content, mass); content / mass are the statistics of all
    keys seen, content0 / mass0 included.
    """
    Phi_Q = soft_assign(Q, W, beta)
    Phi_K = soft_assign(K, W, beta)
    V = np.asarray(V, dtype=np.float64)
    L, N, R = Phi_K.shape
    dv = V.shape[1]
    content = np.zeros((L, R, dv)) if content0 is None else np.array(content0, dtype=np.float64)
    mass = np.zeros((L, R)) if mass0 is None else np.array(mass0, dtype=np.float64)
    O = np.empty((N, dv))
    Den = np.empty(N)
    for t0 in range(0, N, block):
        t1 = min(N, t0 + block)
        pq, pk = Phi_Q[:, t0:t1], Phi_K[:, t0:t1]
        # keys before the block: their statistics, read out as in the non-causal layer
        num = np.matmul(pq, content).sum(axis=0)
        den = np.matmul(pq, mass[:, :, None])[:, :, 0].sum(axis=0)
        # keys of the block: the implicit kernel, keys j <= t only
        S = np.tril(np.matmul(pq, pk.transpose(0, 2, 1)).sum(axis=0))
        num = num + S @ V[t0:t1]
        den = den + S.sum(axis=1)
        O[t0:t1] = num / den[:, None]
        Den[t0:t1] = den
        content = content + np.matmul(pk.transpose(0, 2, 1), V[t0:t1])
        mass = mass + pk.sum(axis=1)
    return O, Den, content, mass


def brute_force_head(Q, K, V, W, beta, causal=False):
    """Explicit N x N kernel S_hat = (1/L) sum_l Phi_Q^(l) Phi_K^(l)^T, masked
    to j <= i when causal, then row-normalised: O = diag(S_hat 1)^-1 S_hat V.

    Slides, frame "Normalize after combining the tables" (the implicit
    kernel).  Tiny N only.  Returns (O, S_hat).
    """
    Phi_Q = soft_assign(Q, W, beta)
    Phi_K = soft_assign(K, W, beta)
    L = Phi_Q.shape[0]
    S = np.einsum("lir,ljr->ij", Phi_Q, Phi_K) / L
    if causal:
        S = np.tril(S)
    V = np.asarray(V, dtype=np.float64)
    return (S @ V) / S.sum(axis=1, keepdims=True), S


def _assign_backward(X, W, beta, Phi, dPhi):
    """Pull dL/dPhi back to dL/dX through softmax, beta, corners, tanh and W.

    dLambda = Phi * (dPhi - rowsum(Phi * dPhi)), dU = beta dLambda C,
    dPre = dU * (1 - U^2), dX = sum_l dPre^(l) W^(l).
    """
    U = _projected(X, W)                                   # (L, N, P)
    C = corners(W.shape[1])
    dLam = Phi * (dPhi - np.sum(Phi * dPhi, axis=-1, keepdims=True))
    dU = float(beta) * np.matmul(dLam, C)
    dPre = dU * (1.0 - U * U)
    return np.matmul(dPre, np.asarray(W, dtype=np.float64)).sum(axis=0)


def beta_terms(X, W, beta, Phi, dPhi):
    """Per-row contribution to dL/dbeta of the soft assignments Phi(X).

    The logits are Lambda_r = beta (u . v_r) (slides, frame "Soft corner
    assignments make hashing differentiable"), so with the softmax backward
    dLambda = Phi * (dPhi - rowsum(Phi * dPhi)) each row contributes
    sum_l sum_r dLambda_r (u . v_r).  Returns an (N,) array.
    """
    U = _projected(X, W)                                   # (L, N, P)
    C = corners(W.shape[1])
    dLam = Phi * (dPhi - np.sum(Phi * dPhi, axis=-1, keepdims=True))
    return np.sum(dLam * np.matmul(U, C.T), axis=(0, 2))


def _assignment_grads(Q, K, V, W, beta, dO, causal=False):
    """Soft assignments of both sides and the gradients of sum(O * dO) with
    respect to them, as backward_head forms them: returns
    (Phi_Q, dPhi_Q, Phi_K, dPhi_K), each (L, N, R)."""
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    dO = np.asarray(dO, dtype=np.float64)
    Phi_Q = soft_assign(Q, W, beta)
    Phi_K = soft_assign(K, W, beta)
    if not causal:
        content, mass = state_head(K, V, W, beta)
        _, O, Den, g, h = query_terms(Q, dO, W, beta, content, mass)
        dPhi_Q = np.matmul(g[None], content.transpose(0, 2, 1)) + h[None, :, None] * mass[:, None, :]
        dcontent, dmass = grad_banks(Q, W, beta, g, h, Phi_Q)
        dPhi_K = np.matmul(V[None], dcontent.transpose(0, 2, 1)) + dmass[:, None, :]
    else:
        O, Den = causal_forward_head(Q, K, V, W, beta, return_den=True)
        g = dO / Den[:, None]
        h = -np.sum(dO * O, axis=1) / Den
        # prefix sums read by query t, suffix sums reaching key j (inclusive)
        pc = np.cumsum(Phi_K[:, :, :, None] * V[None, :, None, :], axis=1)
        pm = np.cumsum(Phi_K, axis=1)
        dPhi_Q = np.einsum("nc,lnrc->lnr", g, pc) + h[None, :, None] * pm
        sD = np.cumsum((Phi_Q[:, :, :, None] * g[None, :, None, :])[:, ::-1], axis=1)[:, ::-1]
        sE = np.cumsum((Phi_Q * h[None, :, None])[:, ::-1], axis=1)[:, ::-1]
        dPhi_K = np.einsum("nc,lnrc->lnr", V, sD) + sE
    return Phi_Q, dPhi_Q, Phi_K, dPhi_K


def dbeta_head(Q, K, V, W, beta, dO, causal=False):
    """dL/dbeta of L = sum(O * dO) for one head, as per-row terms of the
    query side and of the key side: returns (terms_Q, terms_K), each (N,);
    dbeta is their total.  The dPhi of each side are those of backward_head."""
    Phi_Q, dPhi_Q, Phi_K, dPhi_K = _assignment_grads(Q, K, V, W, beta, dO, causal)
    return beta_terms(Q, W, beta, Phi_Q, dPhi_Q), beta_terms(K, W, beta, Phi_K, dPhi_K)


def weight_terms(X, W, beta, Phi, dPhi):
    """Contribution of the rows X to dL/dW through their soft assignments.

    The pre-activations are W^(l) x (slides, frame "Soft corner assignments
    make hashing differentiable"), so with dPre = beta dLambda C * (1 - U^2)
    (the chain _assign_backward follows) the rows contribute
    dW^(l) = dPre^(l)^T X.  Returns an (L, P, d) array.
    """
    X = np.asarray(X, dtype=np.float64)
    U = _projected(X, W)                                   # (L, N, P)
    C = corners(W.shape[1])
    dLam = Phi * (dPhi - np.sum(Phi * dPhi, axis=-1, keepdims=True))
    dPre = float(beta) * np.matmul(dLam, C) * (1.0 - U * U)
    return np.matmul(dPre.transpose(0, 2, 1), X)


def dW_head(Q, K, V, W, beta, dO, causal=False):
    """dL/dW of L = sum(O * dO) for one head whose tables are W (L, P, d):
    returns the query-side and key-side parts (dW_Q, dW_K), each (L, P, d);
    dW is their sum (W enters both projections)."""
    Phi_Q, dPhi_Q, Phi_K, dPhi_K = _assignment_grads(Q, K, V, W, beta, dO, causal)
    return weight_terms(Q, W, beta, Phi_Q, dPhi_Q), weight_terms(K, W, beta, Phi_K, dPhi_K)


def head_tables(W, hh):
    """Tables of head hh: W is (L, P, d), shared by every head, or
    (H, L, P, d), one set of tables per head."""
    W = np.asarray(W)
    return W[hh] if W.ndim == 4 else W


def dW(Q, K, V, W, beta, dO, causal=False):
    """Batched dL/dW over (B, H, N, d) arrays.  Shared tables (L, P, d) sum
    the contributions of every batch row and head; per-head tables
    (H, L, P, d) sum those of every batch row for each head."""
    W = np.asarray(W)
    out = np.zeros(W.shape, dtype=np.float64)
    for b in range(np.asarray(Q).shape[0]):
        for hh in range(np.asarray(Q).shape[1]):
            wq, wk = dW_head(Q[b, hh], K[b, hh], V[b, hh], head_tables(W, hh), beta, dO[b, hh], causal)
            if W.ndim == 4:
                out[hh] += wq + wk
            else:
                out += wq + wk
    return out


def dbeta(Q, K, V, W, beta, dO, causal=False):
    """Batched dL/dbeta over (B, H, N, d) arrays (one beta for every head;
    W shared (L, P, d) or per head (H, L, P, d))."""
    tot = 0.0
    for b in range(np.asarray(Q).shape[0]):
        for hh in range(np.asarray(Q).shape[1]):
            tq, tk = dbeta_head(Q[b, hh], K[b, hh], V[b, hh], head_tables(W, hh), beta, dO[b, hh], causal)
            tot += float(tq.sum() + tk.sum())
    return tot


def query_terms(Q, dO, W, beta, content, mass):
    """For query rows that read the bank (content, mass): Phi_Q, O, Den and the
    upstream terms g = dO / Den, h = -rowdot(dO, O) / Den."""
    Phi_Q = soft_assign(Q, W, beta)
    O, _, Den = readout(Phi_Q, content, mass)
    dO = np.asarray(dO, dtype=np.float64)
    g = dO / Den[:, None]
    h = -np.einsum("nc,nc->n", dO, O) / Den
    return Phi_Q, O, Den, g, h


def query_grads(Q, dO, W, beta, content, mass):
    """Query-side gradient of sum(O * dO) for rows that read the bank
    (content, mass): dPhi_Q = g content^T + h mass^T, then softmax / tanh /
    projection backward.  Returns (dQ, O, Den, g, h)."""
    Phi_Q, O, Den, g, h = query_terms(Q, dO, W, beta, content, mass)
    dPhi_Q = np.matmul(g[None], content.transpose(0, 2, 1)) + h[None, :, None] * mass[:, None, :]
    return _assign_backward(Q, W, beta, Phi_Q, dPhi_Q), O, Den, g, h


def grad_banks(Q, W, beta, g, h, Phi_Q=None):
    """Gradient banks dcontent = Phi_Q^T g (L, R, d) and dmass = Phi_Q^T h (L, R)
    summed over the given query rows (Phi_Q may be passed in when known)."""
    if Phi_Q is None:
        Phi_Q = soft_assign(Q, W, beta)
    return np.matmul(Phi_Q.transpose(0, 2, 1), g), np.matmul(Phi_Q.transpose(0, 2, 1), h[:, None])[:, :, 0]


def key_grads(K, V, W, beta, dcontent, dmass):
    """Key-side gradients for rows that wrote the bank: dV = sum_l Phi_K dcontent,
    dPhi_K = V dcontent^T + 1 dmass^T, then softmax / tanh / projection backward."""
    Phi_K = soft_assign(K, W, beta)
    V = np.asarray(V, dtype=np.float64)
    dV = np.matmul(Phi_K, dcontent).sum(axis=0)
    dPhi_K = np.matmul(V[None], dcontent.transpose(0, 2, 1)) + dmass[:, None, :]
    return _assign_backward(K, W, beta, Phi_K, dPhi_K), dV


def backward_head(Q, K, V, W, beta, dO, causal=False, content0=None, mass0=None):
    """Exact gradient (dQ, dK, dV) of sum(O * dO) for one head.

    With g = dO / Den and h = -rowdot(dO, O) / Den:
    non-causal: dPhi_Q = g content^T + h mass^T; dcontent = Phi_Q^T g;
    dmass = Phi_Q^T h; dV = sum_l Phi_K dcontent; dPhi_K = V dcontent^T +
    1 dmass^T.  Causal: the contents/masses read by query t are the prefix
    sums at t, and the gradients reaching key j are the suffix sums over
    t >= j.  Then softmax, tanh and projection backward on both sides.
    Causal only: content0 / mass0 are the bank of earlier keys (the rows are
    then the last block of a longer sequence; gradients of the earlier keys
    are not returned).
    """
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    dO = np.asarray(dO, dtype=np.float64)
    if not causal:
        content, mass = state_head(K, V, W, beta)
        dQ, _, _, g, h = query_grads(Q, dO, W, beta, content, mass)
        dcontent, dmass = grad_banks(Q, W, beta, g, h)
        dK, dV = key_grads(K, V, W, beta, dcontent, dmass)
        return dQ, dK, dV
    Phi_Q = soft_assign(Q, W, beta)
    Phi_K = soft_assign(K, W, beta)
    L, N, R = Phi_Q.shape
    dv = V.shape[1]
    O, Den = causal_forward_head(Q, K, V, W, beta, return_den=True, content0=content0, mass0=mass0)
    g = dO / Den[:, None]
    h = -np.sum(dO * O, axis=1) / Den
    dPhi_Q = np.empty((L, N, R))
    dPhi_K = np.empty((L, N, R))
    dV = np.empty((N, dv))
    block = 256
    # Prefix sums (read by each query).
    c0 = np.zeros((L, R, dv)) if content0 is None else np.array(content0, dtype=np.float64)
    m0 = np.zeros((L, R)) if mass0 is None else np.array(mass0, dtype=np.float64)
    for t0 in range(0, N, block):
        t1 = min(N, t0 + block)
        pc, pm = _prefix_states(Phi_K, V, t0, t1, c0, m0)
        dPhi_Q[:, t0:t1] = (np.einsum("nc,lnrc->lnr", g[t0:t1], pc)
                            + h[None, t0:t1, None] * pm)
        c0, m0 = pc[:, -1], pm[:, -1]
    # Suffix sums D_j = sum_{t>=j} phi(Q_t) g_t^T, E_j = sum_{t>=j} phi(Q_t) h_t.
    Dn = np.zeros((L, R, dv))
    En = np.zeros((L, R))
    for t1 in range(N, 0, -block):
        t0 = max(0, t1 - block)
        outer = Phi_Q[:, t0:t1, :, None] * g[None, t0:t1, None, :]
        sD = np.cumsum(outer[:, ::-1], axis=1)[:, ::-1] + Dn[:, None]
        sE = np.cumsum(Phi_Q[:, t0:t1][:, ::-1] * h[None, t0:t1][:, ::-1, None],
                       axis=1)[:, ::-1] + En[:, None]
        dV[t0:t1] = np.einsum("lnr,lnrc->nc", Phi_K[:, t0:t1], sD)
        dPhi_K[:, t0:t1] = np.einsum("nc,lnrc->lnr", V[t0:t1], sD) + sE
        Dn, En = sD[:, 0], sE[:, 0]
    dQ = _assign_backward(Q, W, beta, Phi_Q, dPhi_Q)
    dK = _assign_backward(K, W, beta, Phi_K, dPhi_K)
    return dQ, dK, dV


def forward(Q, K, V, W, beta, causal=False):
    """Batched forward over (B, H, N, d) arrays; returns float64 O.  W is
    (L, P, d), shared by every head, or (H, L, P, d), per head."""
    Q = np.asarray(Q)
    out = np.empty(Q.shape, dtype=np.float64)
    for b in range(Q.shape[0]):
        for hh in range(Q.shape[1]):
            Wh = head_tables(W, hh)
            if causal:
                out[b, hh] = causal_forward_head(Q[b, hh], K[b, hh], V[b, hh], Wh, beta)
            else:
                out[b, hh] = forward_head(Q[b, hh], K[b, hh], V[b, hh], Wh, beta)
    return out


def backward(Q, K, V, W, beta, dO, causal=False):
    """Batched backward over (B, H, N, d) arrays; returns float64 (dQ, dK, dV).
    W as in forward."""
    Q = np.asarray(Q)
    dQ = np.empty(Q.shape, dtype=np.float64)
    dK = np.empty(Q.shape, dtype=np.float64)
    dV = np.empty(np.asarray(V).shape, dtype=np.float64)
    for b in range(Q.shape[0]):
        for hh in range(Q.shape[1]):
            dQ[b, hh], dK[b, hh], dV[b, hh] = backward_head(
                Q[b, hh], K[b, hh], V[b, hh], head_tables(W, hh), beta, dO[b, hh], causal)
    return dQ, dK, dV
