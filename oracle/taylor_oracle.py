"""fp64 CPU oracle for causal attention under a truncated Taylor kernel.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, tables or
constants with the HIP library; the two meet only at seeded inputs.

Sources (page titles as published):

* [ExpAttn] "Expanding Attention: A Taylor-Series Route to Linear-Time
  Transformers with a Fixed Number of Recurrent States" -- the arXiv
  2610.20637v1 abstract reproduced on that page.  Primary authority.
* [arXivNews] "arXiv Introduces New Linear-Time Transformer Method via Taylor
  Series Expansion and Fixed-State Recurrence" -- sections "Technical
  Mechanism Analysis" and "Engineering Trade-offs and Performance".
* [HN-thread] the comment thread on the paper (remix-clone-hacker-news item
  46888355): the replies explaining the (Q'K)V = Q'(KV) construction and
  the extra "+1" column of the state.

Notation: d = key/query width, e = value width, n = number of Taylor terms
(orders m = 0 .. n-1), W = sum_m C(d+m-1, m) feature rows.

Readings where the pages leave a step open:

* no temperature inside the exponential: the kernel is K_n(q.k) on inputs
  the caller has already L2-normalised; the optional normalised path
  (``normalized_inputs``) makes the unit rows itself in fp64, folds a
  temperature tau into the queries, and rounds each unit coordinate once to
  the nearest value of the input dtype;
* "n terms" means the orders 0 .. n-1;
* the state stores *raw* symmetric monomials mu_t(k) = prod_l k_{t_l}; the
  multinomial weight 1/alpha(t)! lives on the query side,
  phi_t(q) = mu_t(q) / alpha(t)!, so phi(q).mu(k) = K_n(q.k);
* feature rows: blocks m = 0 .. n-1 in ascending order, inside a block the
  order of ``itertools.combinations_with_replacement(range(d), m)``;
* causal mask inclusive (token i attends to j <= i); a decode step updates
  the state first and then reads out;
* the "+1" (normaliser) column is the last logical column, index e.

Every function here is a plain definition; there is no blocking, fusion or
reordering beyond what the pages' algorithm states.  Pins that fix each
function against something other than itself are in
``tests/test_oracle_pins.py``.
"""

from __future__ import annotations

import itertools
import math
from typing import List, Sequence, Tuple

import numpy as np

__all__ = [
    "multi_indices", "block_widths", "state_rows", "state_floats",
    "multinomial_weights", "feature_map", "taylor_kernel",
    "quadratic_attention", "quadratic_rows", "states_definition",
    "recurrent_attention", "chunked_attention", "decode_step",
    "prefill_from_numden", "prefill_from_states", "prefill_from_rows",
    "merge_states", "softmax_attention", "states_to_planes",
    "planes_to_states", "block_row_ranges",
    "normalize_rows", "round_to_dtype", "normalized_inputs",
    "softmax_rows",
]


# ---------------------------------------------------------------------------
# Symmetric tensor-power packing  [ExpAttn abstract: the m-th state is
# C(d+m-1, m) wide; arXivNews "Engineering Trade-offs": same width, 9945
# elements per head at the optimum]
# ---------------------------------------------------------------------------

def multi_indices(d: int, m: int) -> List[Tuple[int, ...]]:
    """Non-decreasing index tuples of length m over range(d), lexicographic.

    These are the distinct coordinates of the symmetric tensor x^{(x)m}; there
    are C(d+m-1, m) of them [ExpAttn abstract].
    """
    return list(itertools.combinations_with_replacement(range(d), m))


def block_widths(d: int, n: int) -> List[int]:
    """Width of each of the n states: C(d+m-1, m) for m = 0 .. n-1 [ExpAttn abstract]."""
    return [math.comb(d + m - 1, m) for m in range(n)]


def state_rows(d: int, n: int) -> int:
    """Total number of feature rows W over the n states."""
    return sum(block_widths(d, n))


def state_floats(d: int, e: int, n: int) -> int:
    """Elements of one head's state: W rows times (e + 1) columns.

    The extra column carries the softmax normaliser [HN-thread, reply on the
    "+1"]; with d=16, e=64, n=3 this is 153*65 = 9945 [ExpAttn abstract].
    """
    return state_rows(d, n) * (e + 1)


def block_row_ranges(d: int, n: int) -> List[Tuple[int, int]]:
    """[start, stop) row range of each m-block inside the W rows."""
    out, r = [], 0
    for w in block_widths(d, n):
        out.append((r, r + w))
        r += w
    return out


def multinomial_weights(d: int, n: int) -> np.ndarray:
    """c_t = 1/alpha(t)! for every feature row t, in row order.

    alpha(t) is the multiplicity vector of tuple t.  The multinomial theorem
    gives (q.k)^m / m! = sum_{|t| = m} mu_t(q) mu_t(k) / alpha(t)!, which is
    how the tensor-power inner product of each Taylor term is folded into a
    packed symmetric state [ExpAttn abstract].
    """
    w = []
    for m in range(n):
        for t in multi_indices(d, m):
            denom = 1
            for i in set(t):
                denom *= math.factorial(t.count(i))
            w.append(1.0 / denom)
    return np.array(w, dtype=np.float64)


def feature_map(X: np.ndarray, n: int, weighted: bool) -> np.ndarray:
    """Packed symmetric tensor powers of every row of X.

    Returns [..., W] with mu_t(x) = prod_l x[t_l] (weighted=False, key side)
    or phi_t(x) = c_t mu_t(x) (weighted=True, query side).  The m = 0 row is
    the constant 1.  [ExpAttn abstract: each Taylor term factorised into a
    tensor-power inner product.]
    """
    X = np.asarray(X, dtype=np.float64)
    d = X.shape[-1]
    blocks = []
    for m in range(n):
        T = np.array(multi_indices(d, m), dtype=np.intp).reshape(len(multi_indices(d, m)), m)
        v = np.ones(X.shape[:-1] + (T.shape[0],), dtype=np.float64)
        for l in range(m):  # coordinates multiplied left to right along each tuple
            v = v * X[..., T[:, l]]
        blocks.append(v)
    F = np.concatenate(blocks, axis=-1)
    if weighted:
        F = F * multinomial_weights(d, n)
    return F


def taylor_kernel(x, n: int):
    """K_n(x) = sum_{m=0}^{n-1} x^m / m!  -- the first n terms of exp(x) [ExpAttn abstract]."""
    x = np.asarray(x, dtype=np.float64)
    out = np.zeros_like(x)
    for m in range(n):
        out = out + x ** m / math.factorial(m)
    return out


# ---------------------------------------------------------------------------
# The definition: quadratic-form causal attention with the truncated kernel
# ---------------------------------------------------------------------------

def _heads(A: np.ndarray) -> Tuple[np.ndarray, Tuple[int, ...]]:
    A = np.asarray(A, dtype=np.float64)
    lead = A.shape[:-2]
    return A.reshape((-1,) + A.shape[-2:]), lead


def quadratic_attention(Q, K, V, n: int) -> np.ndarray:
    """o_i = sum_{j<=i} K_n(q_i.k_j) v_j / sum_{j<=i} K_n(q_i.k_j).

    Q, K: [..., N, d]; V: [..., N, e].  This is softmax attention with exp
    replaced by its n-term Taylor truncation [ExpAttn abstract], causal and
    inclusive of the diagonal, normalised by the same kernel sum (the "+1"
    column of the recurrent form) [HN-thread, reply on the "+1"].
    """
    Qh, lead = _heads(Q)
    Kh, _ = _heads(K)
    Vh, _ = _heads(V)
    N = Qh.shape[1]
    out = np.empty(Vh.shape, dtype=np.float64)
    for h in range(Qh.shape[0]):
        P = taylor_kernel(Qh[h] @ Kh[h].T, n)
        for i in range(N):  # row i sums over keys 0 .. i only
            p = P[i, : i + 1]
            out[h, i] = (p @ Vh[h, : i + 1]) / p.sum()
    return out.reshape(lead + Vh.shape[1:])


def quadratic_rows(q_rows, K, V, rows: Sequence[int], n: int) -> np.ndarray:
    """The definition evaluated for selected query rows of one head.

    q_rows: [len(rows), d] (the queries at those positions); K: [N, d]; V:
    [N, e].  Row i uses keys 0 .. i.  Used to check long sequences on sampled
    outputs without forming the N x N matrix.
    """
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    q_rows = np.asarray(q_rows, dtype=np.float64)
    out = np.empty((len(rows), V.shape[1]), dtype=np.float64)
    for r, i in enumerate(rows):
        p = taylor_kernel(K[: i + 1] @ q_rows[r], n)
        out[r] = (p @ V[: i + 1]) / p.sum()
    return out


def states_definition(K, V, n: int, block: int = 4096) -> np.ndarray:
    """S[t, :e] = sum_j mu_t(k_j) v_j and S[t, e] = sum_j mu_t(k_j).

    K: [..., N, d]; V: [..., N, e]; returns [..., W, e+1].  The n states of
    the abstract stacked row-wise; the last column carries the normaliser
    [ExpAttn abstract; HN-thread reply on the "+1"].  Summed over token blocks
    of ``block`` rows only to bound memory (the sum is the same sum).
    """
    Kh, lead = _heads(K)
    Vh, _ = _heads(V)
    H, N, d = Kh.shape
    e = Vh.shape[2]
    W = state_rows(d, n)
    S = np.zeros((H, W, e + 1), dtype=np.float64)
    for h in range(H):
        for s in range(0, N, block):
            mu = feature_map(Kh[h, s:s + block], n, weighted=False)
            Vp = np.concatenate([Vh[h, s:s + block], np.ones((mu.shape[0], 1))], axis=1)
            S[h] += mu.T @ Vp
    return S.reshape(lead + (W, e + 1))


# ---------------------------------------------------------------------------
# Recurrent, chunked and decode forms  [ExpAttn abstract; arXivNews
# "Technical Mechanism Analysis" items 1, 2 and 4]
# ---------------------------------------------------------------------------

def _readout(phi: np.ndarray, S: np.ndarray) -> np.ndarray:
    """o = phi(q).S[:, :e] / phi(q).S[:, e] for rows of phi [HN-thread "+1" reply]."""
    num = phi @ S[..., :-1]
    den = phi @ S[..., -1]
    return num / den[..., None]


def recurrent_attention(Q, K, V, n: int) -> Tuple[np.ndarray, np.ndarray]:
    """Token-by-token recurrence: S += mu(k_j) (x) [v_j, 1], then read out.

    One rank-one outer-product update of the state per token, independent of
    the context length [ExpAttn abstract].  Returns (O, final states).
    """
    Qh, lead = _heads(Q)
    Kh, _ = _heads(K)
    Vh, _ = _heads(V)
    H, N, d = Qh.shape
    e = Vh.shape[2]
    W = state_rows(d, n)
    O = np.empty((H, N, e))
    S_all = np.empty((H, W, e + 1))
    for h in range(H):
        phi = feature_map(Qh[h], n, weighted=True)
        mu = feature_map(Kh[h], n, weighted=False)
        S = np.zeros((W, e + 1))
        for j in range(N):
            S += np.outer(mu[j], np.append(Vh[h, j], 1.0))
            O[h, j] = _readout(phi[j], S)
        S_all[h] = S
    return O.reshape(lead + (N, e)), S_all.reshape(lead + (W, e + 1))


def chunked_attention(Q, K, V, n: int, chunk: int) -> Tuple[np.ndarray, np.ndarray]:
    """Chunk-parallel form: inter-chunk readout from the running state plus
    the intra-chunk block of the quadratic form, then the state update.

    For chunk c with rows i: num_i = phi(q_i).S_prev[:, :e] +
    sum_{j in c, j <= i} K_n(q_i.k_j) v_j (likewise den with the "+1"
    column), then S_prev += mu(K_c)^T [V_c, 1].  Valid because the states are
    sums over tokens, so they add across chunks [ExpAttn abstract: additive
    states, prefill admits a parallel scan] and (Q'K)V = Q'(KV)
    [HN-thread, reply on the associativity].
    """
    Qh, lead = _heads(Q)
    Kh, _ = _heads(K)
    Vh, _ = _heads(V)
    H, N, d = Qh.shape
    e = Vh.shape[2]
    W = state_rows(d, n)
    O = np.empty((H, N, e))
    S_all = np.empty((H, W, e + 1))
    for h in range(H):
        S = np.zeros((W, e + 1))
        for s in range(0, N, chunk):
            q, k, v = Qh[h, s:s + chunk], Kh[h, s:s + chunk], Vh[h, s:s + chunk]
            L = q.shape[0]
            phi = feature_map(q, n, weighted=True)
            mu = feature_map(k, n, weighted=False)
            vp = np.concatenate([v, np.ones((L, 1))], axis=1)
            P = np.where(np.tril(np.ones((L, L), dtype=bool)), taylor_kernel(q @ k.T, n), 0.0)
            acc = phi @ S + P @ vp
            O[h, s:s + L] = acc[:, :e] / acc[:, e:]
            S = S + mu.T @ vp
        S_all[h] = S
    return O.reshape(lead + (N, e)), S_all.reshape(lead + (W, e + 1))


def decode_step(q, k, v, S, n: int) -> Tuple[np.ndarray, np.ndarray]:
    """One generated token: rank-one update of the state, then readout.

    q, k: [..., d]; v: [..., e]; S: [..., W, e+1].  Returns (o, S_new) with
    S_new = S + mu(k) (x) [v, 1] and o = phi(q).S_new[:, :e] / phi(q).S_new[:, e]
    (inclusive: the token attends to itself).  Constant work per token
    whatever the context length [ExpAttn abstract; arXivNews "Technical
    Mechanism Analysis" item 4].
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    S = np.asarray(S, dtype=np.float64)
    mu = feature_map(k, n, weighted=False)
    phi = feature_map(q, n, weighted=True)
    vp = np.concatenate([v, np.ones(v.shape[:-1] + (1,))], axis=-1)
    S_new = S + mu[..., :, None] * vp[..., None, :]
    num = np.einsum("...t,...tc->...c", phi, S_new[..., :-1])
    den = np.einsum("...t,...t->...", phi, S_new[..., -1])
    return num / den[..., None], S_new


def prefill_from_numden(Q, K, V, S0, n: int) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Numerator and normaliser of a prefill that continues from states S0.

    Q, K: [..., N, d]; V: [..., N, e]; S0: [..., W, e+1], or None for zero
    states.  For row i,
        num_i = phi(q_i).S0[:, :e] + sum_{j<=i} K_n(q_i.k_j) v_j,
        den_i = phi(q_i).S0[:, e]  + sum_{j<=i} K_n(q_i.k_j),
    before any division.  Both are sums over keys, so results computed over
    separate key segments add, which is how segments are combined; the
    returned states are S0 plus the states of the new tokens [ExpAttn
    abstract: additive states, constant-size recurrent state; HN-thread,
    reply on the "+1" column for the den part].  Returns (num [..., N, e],
    den [..., N], states [..., W, e+1]).
    """
    Qh, lead = _heads(Q)
    Kh, _ = _heads(K)
    Vh, _ = _heads(V)
    H, N, d = Qh.shape
    e = Vh.shape[2]
    W = state_rows(d, n)
    S0h = np.zeros((H, W, e + 1)) if S0 is None else np.asarray(S0, dtype=np.float64).reshape(H, W, e + 1)
    num = np.empty((H, N, e))
    den = np.empty((H, N))
    S_all = np.empty((H, W, e + 1))
    for h in range(H):
        phi = feature_map(Qh[h], n, weighted=True)
        vp = np.concatenate([Vh[h], np.ones((N, 1))], axis=1)
        P = taylor_kernel(Qh[h] @ Kh[h].T, n)
        acc = phi @ S0h[h]
        for i in range(N):  # row i sums over the new keys 0 .. i only
            acc[i] = acc[i] + P[i, : i + 1] @ vp[: i + 1]
        num[h] = acc[:, :e]
        den[h] = acc[:, e]
        S_all[h] = S0h[h] + states_definition(Kh[h], Vh[h], n)
    return num.reshape(lead + (N, e)), den.reshape(lead + (N,)), S_all.reshape(lead + (W, e + 1))


def prefill_from_states(Q, K, V, S0, n: int) -> Tuple[np.ndarray, np.ndarray]:
    """Prefill of new tokens that continues from the states S0 of earlier ones.

    o_i = num_i / den_i with num and den from ``prefill_from_numden``; the
    returned states are S0 plus the states of the new tokens.  The earlier
    tokens enter only through their summed state, which is what lets a
    prefill resume after decoding or start from another segment's total
    [ExpAttn abstract: additive states, constant-size recurrent state].
    """
    num, den, S_all = prefill_from_numden(Q, K, V, S0, n)
    return num / den[..., None], S_all


def prefill_from_rows(q_rows, K, V, S0, rows: Sequence[int], n: int) -> np.ndarray:
    """``prefill_from_states`` evaluated for selected query rows of one head.

    q_rows: [len(rows), d]; K: [N, d]; V: [N, e]; S0: [W, e+1].  Row i reads
    out the carried-in states and adds the kernel sum over the new keys
    0 .. i.  Used to check long sequences on sampled outputs.
    """
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    S0 = np.asarray(S0, dtype=np.float64)
    q_rows = np.asarray(q_rows, dtype=np.float64)
    e = V.shape[1]
    base = feature_map(q_rows, n, weighted=True) @ S0
    out = np.empty((len(rows), e), dtype=np.float64)
    for r, i in enumerate(rows):
        p = taylor_kernel(K[: i + 1] @ q_rows[r], n)
        num = base[r, :e] + p @ V[: i + 1]
        den = base[r, e] + p.sum()
        out[r] = num / den
    return out


def merge_states(a, b) -> np.ndarray:
    """States of two token sets add: S(A u B) = S(A) + S(B) [ExpAttn abstract]."""
    return np.asarray(a, dtype=np.float64) + np.asarray(b, dtype=np.float64)


def softmax_attention(Q, K, V) -> np.ndarray:
    """Exact causal softmax attention (exp kernel, no scale), the quantity the
    truncated kernel approximates [ExpAttn abstract].  The row max is
    subtracted before exp, which leaves the ratio unchanged."""
    Qh, lead = _heads(Q)
    Kh, _ = _heads(K)
    Vh, _ = _heads(V)
    N = Qh.shape[1]
    mask = np.tril(np.ones((N, N), dtype=bool))
    out = np.empty(Vh.shape)
    for h in range(Qh.shape[0]):
        X = np.where(mask, Qh[h] @ Kh[h].T, -np.inf)
        X = X - X.max(axis=1, keepdims=True)
        P = np.exp(X)
        out[h] = (P @ Vh[h]) / P.sum(axis=1, keepdims=True)
    return out.reshape(lead + Vh.shape[1:])


# ---------------------------------------------------------------------------
# Input side: L2 normalisation of q and k, optional temperature  [ExpAttn
# abstract: normalisation is the prerequisite that keeps q.k inside the
# series' convergence radius; arXivNews "Engineering Trade-offs and
# Performance": without it, more terms stop helping]
# ---------------------------------------------------------------------------

def normalize_rows(X, scale: float = 1.0) -> np.ndarray:
    """scale * x / ||x||_2 for every row x of X (last axis), in fp64.

    With unit q and k, |q.k| <= 1, the region where the truncated series
    converges fast [ExpAttn abstract].  A temperature tau is folded into the
    queries as scale = tau, which turns the kernel into K_n(tau q.k) on the
    unit vectors.  A zero row has no direction and gives NaN.
    """
    X = np.asarray(X, dtype=np.float64)
    with np.errstate(invalid="ignore", divide="ignore"):
        return X * (float(scale) / np.sqrt(np.sum(X * X, axis=-1, keepdims=True)))


def round_to_dtype(X, dtype: str) -> np.ndarray:
    """fp64 values rounded once to the nearest value of the working dtype,
    ties to even, returned as fp64.

    "f32": numpy's fp64 -> fp32 cast.  "bf16": 8 significant bits (the
    fp32 exponent range): with |x| = m 2^p, m in [0.5, 1), the spacing of
    bf16 values around x is u = 2^(p-8) (at least 2^-133, the subnormal
    spacing), and x is rounded to rint(x / u) u, where rint rounds half to
    even; x / u is exact (a power-of-two scaling).  Values beyond the largest
    bf16 round to infinity.  This is the correctly rounded unit row of the
    normalised path; rounding to fp32 first would round twice.
    """
    X = np.asarray(X, dtype=np.float64)
    if dtype == "f32":
        with np.errstate(over="ignore"):
            return X.astype(np.float32).astype(np.float64)
    if dtype == "bf16":
        out = X.copy()
        fin = np.isfinite(X) & (X != 0.0)
        x = X[fin]
        _, p = np.frexp(np.abs(x))
        u = np.ldexp(1.0, np.maximum(p - 8, -133))
        r = np.rint(x / u) * u
        big = (2.0 - 2.0 ** -7) * 2.0 ** 127
        r = np.where(np.abs(r) > big, np.copysign(np.inf, r), r)
        out[fin] = r
        return out
    raise ValueError(f"unknown dtype {dtype!r}")


def normalized_inputs(Q, K, temperature: float, dtype: str) -> Tuple[np.ndarray, np.ndarray]:
    """(q_hat, k_hat): q_hat = round(tau q/||q||), k_hat = round(k/||k||),
    the fp64 unit rows of ``normalize_rows`` rounded once to the nearest
    value of the working dtype (``round_to_dtype``).

    The attention of the normalised path is then the definition above on
    these rows, e.g. quadratic_attention(q_hat, k_hat, V, n), whose kernel is
    K_n(tau q.k / (||q|| ||k||)) up to the rounding of the unit rows.
    """
    return (round_to_dtype(normalize_rows(Q, temperature), dtype),
            round_to_dtype(normalize_rows(K, 1.0), dtype))


def softmax_rows(q_rows, K, V, rows: Sequence[int]) -> np.ndarray:
    """``softmax_attention`` evaluated for selected query rows of one head:
    row i is the exp-weighted average of v_0 .. v_i with weights
    exp(q_i.k_j) (no scale), the baseline the truncated kernel is compared
    against [ExpAttn abstract; arXivNews "Engineering Trade-offs and
    Performance"].  The largest score is subtracted before exp.  A decode
    step of softmax attention at position i is row i of this.

    q_rows: [len(rows), d]; K: [N, d]; V: [N, e].
    """
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    q_rows = np.asarray(q_rows, dtype=np.float64)
    out = np.empty((len(rows), V.shape[1]), dtype=np.float64)
    for r, i in enumerate(rows):
        x = K[: i + 1] @ q_rows[r]
        p = np.exp(x - x.max())
        out[r] = (p @ V[: i + 1]) / p.sum()
    return out


# ---------------------------------------------------------------------------
# Boundary layout converters (logical [.., W, e+1] <-> the library's planes)
# ---------------------------------------------------------------------------

def states_to_planes(S) -> np.ndarray:
    """Logical states [B, H, W, e+1] -> flat buffer: the value plane
    [B, H, W, e] followed by the normaliser plane [B, H, W]."""
    S = np.asarray(S)
    num = S[..., :-1]
    den = S[..., -1]
    return np.concatenate([num.reshape(-1), den.reshape(-1)])


def planes_to_states(flat, B: int, H: int, W: int, e: int) -> np.ndarray:
    """Inverse of states_to_planes."""
    flat = np.asarray(flat)
    nnum = B * H * W * e
    num = flat[:nnum].reshape(B, H, W, e)
    den = flat[nnum:nnum + B * H * W].reshape(B, H, W, 1)
    return np.concatenate([num, den], axis=-1)
