"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Each ``pin_*`` function raises AssertionError when the oracle disagrees with
an independent fact: a hand-derived example, exact rational arithmetic, the
full (unpacked) tensor powers, a textbook special case, a library routine,
or a bound from Taylor's theorem.  ``tests/test_oracle_pins.py`` runs them
on the oracle; ``tests/test_oracle_mutants.py`` plants plausible mistakes in
the oracle and checks that some pin catches each one.

Pages: [ExpAttn] = "Expanding Attention: A Taylor-Series Route to
Linear-Time Transformers with a Fixed Number of Recurrent States" (the
arXiv 2610.20637v1 abstract); [arXivNews] = "arXiv Introduces New
Linear-Time Transformer Method via Taylor Series Expansion and Fixed-State
Recurrence"; [HN-thread] = the comment thread on the paper (item 46888355).
"""

from __future__ import annotations

import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np

import oracle.taylor_oracle as orc
from taylor_recurrent_states_amd import workloads as wl

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _frac(p):
    return Fraction(p[0], p[1])


def _unit(d, rng):
    return wl.l2_normalise(rng.standard_normal(d))


def rel_err(x, ref):
    x, ref = np.asarray(x, np.float64), np.asarray(ref, np.float64)
    return float(np.max(np.abs(x - ref)) / np.max(np.abs(ref)))


# ---------------------------------------------------------------------------
# Hand-derived example and page numbers
# ---------------------------------------------------------------------------

def pin_hand_example():
    """The d=2 example worked by hand in tests/golden/hand_example_d2.json."""
    g = json.load(open(os.path.join(GOLDEN, "hand_example_d2.json")))
    to_f = lambda a: np.array([[float(_frac(x)) for x in row] for row in a])
    q, k, v = to_f(g["q"]), to_f(g["k"]), to_f(g["v"])
    o_ref, S_ref = to_f(g["o"]), to_f(g["S"])
    n = g["n"]
    assert np.allclose(orc.quadratic_attention(q, k, v, n), o_ref, rtol=0, atol=1e-15)
    o_r, S_r = orc.recurrent_attention(q, k, v, n)
    assert np.allclose(o_r, o_ref, rtol=0, atol=1e-15)
    assert np.allclose(S_r, S_ref, rtol=0, atol=1e-15)
    assert np.allclose(orc.states_definition(k, v, n), S_ref, rtol=0, atol=1e-15)
    o_c, S_c = orc.chunked_attention(q, k, v, n, 1)
    assert np.allclose(o_c, o_ref, rtol=0, atol=1e-15)
    assert np.allclose(S_c, S_ref, rtol=0, atol=1e-15)
    w = np.array([float(_frac(x)) for x in g["weights"]])
    assert np.array_equal(orc.multinomial_weights(2, n), w)


def pin_page_widths():
    """Widths C(d+m-1, m) and 9,945 elements per head at d=16, e=64, n=3
    [ExpAttn abstract; arXivNews 'Engineering Trade-offs']."""
    g = json.load(open(os.path.join(GOLDEN, "page_numbers.json")))
    c = g["elements_per_head_n3"]
    assert orc.state_floats(c["d"], c["e"], c["n"]) == c["value"]
    # block sizes against brute-force enumeration of multisets
    for d in (1, 2, 3, 5, 16):
        for m in range(5):
            brute = {tuple(sorted(t)) for t in itertools.product(range(d), repeat=m)}
            assert orc.block_widths(d, m + 1)[m] == len(brute)
            assert sorted(brute) == orc.multi_indices(d, m)


# ---------------------------------------------------------------------------
# P1: exact rational brute force
# ---------------------------------------------------------------------------

_RATIONAL_UNITS = {
    2: [(Fraction(3, 5), Fraction(4, 5)), (Fraction(5, 13), Fraction(12, 13)),
        (Fraction(-4, 5), Fraction(3, 5)), (Fraction(8, 17), Fraction(-15, 17)),
        (Fraction(-7, 25), Fraction(-24, 25)), (Fraction(1), Fraction(0))],
    3: [(Fraction(1, 3), Fraction(2, 3), Fraction(2, 3)), (Fraction(2, 7), Fraction(3, 7), Fraction(6, 7)),
        (Fraction(-2, 3), Fraction(1, 3), Fraction(2, 3)), (Fraction(6, 7), Fraction(-2, 7), Fraction(3, 7)),
        (Fraction(2, 3), Fraction(-2, 3), Fraction(-1, 3)), (Fraction(0), Fraction(-1), Fraction(0))],
}


def _exact_quadratic(q, k, v, n):
    N, e = len(q), len(v[0])
    out = []
    for i in range(N):
        num, den = [Fraction(0)] * e, Fraction(0)
        for j in range(i + 1):
            x = sum(a * b for a, b in zip(q[i], k[j]))
            w = sum(x ** m / math.factorial(m) for m in range(n))
            den += w
            num = [a + w * b for a, b in zip(num, v[j])]
        out.append([a / den for a in num])
    return out


def _exact_recurrent_kron(q, k, v, n):
    """Recurrence on the FULL tensor powers x^{(x)m} (d^m entries, no packing)."""
    d, e = len(q[0]), len(v[0])
    S = {m: {} for m in range(n)}
    out = []
    for i in range(len(q)):
        for m in range(n):
            for t in itertools.product(range(d), repeat=m):
                mu = Fraction(1)
                for a in t:
                    mu *= k[i][a]
                row = S[m].setdefault(t, [Fraction(0)] * (e + 1))
                for c in range(e):
                    row[c] += mu * v[i][c]
                row[e] += mu
        num, den = [Fraction(0)] * e, Fraction(0)
        for m in range(n):
            for t, row in S[m].items():
                qm = Fraction(1)
                for a in t:
                    qm *= q[i][a]
                w = qm / math.factorial(m)
                num = [a + w * row[c] for c, a in enumerate(num)]
                den += w * row[e]
        out.append([a / den for a in num])
    return out, S


def pin_exact_rational():
    """Exact recurrence over unpacked tensor powers equals the exact quadratic
    form, and the fp64 oracle matches both within 1e-15 (relative)
    [ExpAttn abstract: lossless with respect to the truncated kernel]."""
    rng = np.random.Generator(np.random.PCG64(11))
    for d in (2, 3):
        units = _RATIONAL_UNITS[d]
        for n in (1, 2, 3, 4):
            N = 5
            qi = rng.integers(0, len(units), N)
            ki = rng.integers(0, len(units), N)
            q = [units[i] for i in qi]
            k = [units[i] for i in ki]
            v = [[Fraction(int(a), 4) for a in rng.integers(-8, 9, 2)] for _ in range(N)]
            exact_q = _exact_quadratic(q, k, v, n)
            exact_r, S = _exact_recurrent_kron(q, k, v, n)
            assert exact_q == exact_r
            qf = np.array([[float(a) for a in r] for r in q])
            kf = np.array([[float(a) for a in r] for r in k])
            vf = np.array([[float(a) for a in r] for r in v])
            ref = np.array([[float(a) for a in r] for r in exact_q])
            for o in (orc.quadratic_attention(qf, kf, vf, n),
                      orc.recurrent_attention(qf, kf, vf, n)[0],
                      orc.chunked_attention(qf, kf, vf, n, 2)[0]):
                assert np.max(np.abs(o - ref)) <= 1e-15 * max(1.0, np.max(np.abs(ref))) * 4
            # packed oracle states equal the unpacked exact states at every
            # tuple (every permutation of a multiset holds the same value)
            Sp = orc.states_definition(kf, vf, n)
            r = 0
            for m in range(n):
                for t in orc.multi_indices(d, m):
                    for perm in set(itertools.permutations(t)):
                        exact_row = [float(x) for x in S[m][perm]]
                        assert np.allclose(Sp[r], exact_row, rtol=0, atol=1e-14)
                    r += 1


# ---------------------------------------------------------------------------
# P2: packed features against full Kronecker powers
# ---------------------------------------------------------------------------

def pin_kron_features():
    """phi(q).mu(k) restricted to block m equals <q^{(x)m}, k^{(x)m}>/m!
    computed with np.kron (no packing) [ExpAttn abstract]."""
    rng = np.random.Generator(np.random.PCG64(5))
    for d in (1, 2, 3, 4):
        for n in (1, 2, 3, 4):
            q, k = rng.standard_normal(d), rng.standard_normal(d)
            phi = orc.feature_map(q, n, weighted=True)
            mu = orc.feature_map(k, n, weighted=False)
            r = 0
            kq, kk = np.ones(1), np.ones(1)
            for m, w in enumerate(orc.block_widths(d, n)):
                packed = float(phi[r:r + w] @ mu[r:r + w])
                full = float(kq @ kk) / math.factorial(m)
                assert abs(packed - full) <= 1e-13 * max(1.0, abs(full))
                # each packed mu entry is the product of its tuple's coordinates
                for t_idx, t in enumerate(orc.multi_indices(d, m)):
                    assert abs(mu[r + t_idx] - np.prod([k[a] for a in t])) <= 1e-15 * (1 + abs(mu[r + t_idx]))
                r += w
                kq, kk = np.kron(kq, q), np.kron(kk, k)


# ---------------------------------------------------------------------------
# O1-O3: identities and the pages' fp64 figures
# ---------------------------------------------------------------------------

def pin_unit_identity():
    """phi(x).mu(x) = sum_{m<n} 1/m! for unit x, and phi(q).mu(k) tends to
    exp(q.k) within the Taylor remainder e|x|^n/n!."""
    rng = np.random.Generator(np.random.PCG64(7))
    for d in (3, 16):
        for n in (1, 2, 3, 5):
            x = _unit(d, rng)
            val = float(orc.feature_map(x, n, True) @ orc.feature_map(x, n, False))
            assert abs(val - sum(1.0 / math.factorial(m) for m in range(n))) < 1e-13
            q, k = _unit(d, rng), _unit(d, rng)
            s = float(q @ k)
            val = float(orc.feature_map(q, n, True) @ orc.feature_map(k, n, False))
            assert abs(val - math.exp(s)) <= math.e * abs(s) ** n / math.factorial(n) + 1e-14
            assert abs(float(orc.taylor_kernel(s, n)) - val) < 1e-13


def pin_recurrent_vs_quadratic(N=256, d=16, e=64, n=3, seed=0):
    """fp64 recurrence vs quadratic form: <= 1e-14 relative (the pages report
    2.2e-16 [ExpAttn abstract]).  Returns the measured value."""
    q, k, v = wl.draw_qkv(seed, 1, 1, N, d, e, "f32")
    o_q = orc.quadratic_attention(q.exact, k.exact, v.exact, n)
    o_r, S_r = orc.recurrent_attention(q.exact, k.exact, v.exact, n)
    err = rel_err(o_r, o_q)
    assert err <= 1e-14, err
    S_d = orc.states_definition(k.exact, v.exact, n)
    assert rel_err(S_r, S_d) <= 1e-13
    return err


def pin_chunk_additivity(N=256, d=16, e=64, n=3, seed=0):
    """States of random splits merge to the single-pass states: <= 1e-13
    (the pages report 5.7e-14 [ExpAttn abstract]); the chunked form's output
    does not depend on the chunk length."""
    q, k, v = wl.draw_qkv(seed, 1, 1, N, d, e, "f32")
    kx, vx = k.exact[0, 0], v.exact[0, 0]
    cuts = [0] + wl.draw_split_points(N, 7, seed=(9, 9)) + [N]
    merged = None
    for a, b in zip(cuts[:-1], cuts[1:]):
        s = orc.chunked_attention(q.exact[0, 0, a:b], kx[a:b], vx[a:b], n, 16)[1]
        merged = s if merged is None else orc.merge_states(merged, s)
    single = orc.states_definition(kx, vx, n)
    err = rel_err(merged, single)
    assert err <= 1e-13, err
    o_ref = orc.quadratic_attention(q.exact, k.exact, v.exact, n)
    for L in (1, 7, 64, 100, 256, 300):
        o_c, S_c = orc.chunked_attention(q.exact, k.exact, v.exact, n, L)
        assert rel_err(o_c, o_ref) <= 1e-13
        assert rel_err(S_c[0, 0], single) <= 1e-13
    return err


def pin_decode_equals_recurrence(N=40, d=5, e=3, n=3, seed=3):
    """N decode steps from zero states reproduce the quadratic form and the
    single-pass states; merge of two halves matches."""
    q, k, v = wl.draw_qkv(seed, 1, 2, N, d, e, "f32")
    o_q = orc.quadratic_attention(q.exact, k.exact, v.exact, n)
    W = orc.state_rows(d, n)
    S = np.zeros((1, 2, W, e + 1))
    outs = []
    for t in range(N):
        o, S = orc.decode_step(q.exact[:, :, t], k.exact[:, :, t], v.exact[:, :, t], S, n)
        outs.append(o)
    o_d = np.stack(outs, axis=2)
    assert rel_err(o_d, o_q) <= 1e-13
    assert rel_err(S, orc.states_definition(k.exact, v.exact, n)) <= 1e-13


# ---------------------------------------------------------------------------
# O4, O8: convergence to softmax and the normalisation prerequisite
# ---------------------------------------------------------------------------

def pin_softmax_library():
    """The oracle's softmax attention equals torch's scaled_dot_product_attention
    (causal, scale 1) in fp64 on the CPU."""
    import torch
    q, k, v = wl.draw_qkv(21, 1, 2, 48, 8, 4, "f32")
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q.exact), torch.from_numpy(k.exact), torch.from_numpy(v.exact),
        is_causal=True, scale=1.0).numpy()
    assert rel_err(orc.softmax_attention(q.exact, k.exact, v.exact), ref) <= 1e-13


def pin_softmax_rows():
    """Row-sampled softmax equals torch's causal scaled_dot_product_attention
    (scale 1, fp64 CPU) on those rows, also where the scores are large
    (raw, unnormalised inputs scaled by 8: the subtracted maximum matters)."""
    import torch
    for scale, norm in ((1.0, True), (8.0, False)):
        q, k, v = wl.draw_qkv(22, 1, 1, 90, 6, 3, "f32", normalise=norm)
        Q, K, V = q.exact * scale, k.exact * scale, v.exact
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(Q), torch.from_numpy(K), torch.from_numpy(V), is_causal=True, scale=1.0).numpy()[0, 0]
        rows = [0, 1, 2, 45, 88, 89]
        got = orc.softmax_rows(Q[0, 0, rows], K[0, 0], V[0, 0], rows)
        assert rel_err(got, ref[rows]) <= 1e-13
        assert np.all(np.isfinite(got))


def pin_softmax_convergence(N=128, d=16, e=8, seed=2):
    """With unit q, k: |o_n - o_softmax| <= eps/(1-eps) max_j |v_j - o_softmax|
    per coordinate with eps = e/n! (Taylor remainder on |x| <= 1), and the error
    falls by > 100x from n=3 to n=8 [ExpAttn abstract: accuracy improves
    exponentially in n].  Returns {n: err}."""
    q, k, v = wl.draw_qkv(seed, 1, 1, N, d, e, "f32")
    o_s = orc.softmax_attention(q.exact, k.exact, v.exact)[0, 0]
    V = v.exact[0, 0]
    errs = {}
    for n in range(1, 9):
        o_n = orc.quadratic_attention(q.exact, k.exact, v.exact, n)[0, 0]
        errs[n] = float(np.max(np.abs(o_n - o_s)))
        eps = math.e / math.factorial(n)
        if eps < 1:
            for i in range(N):
                spread = np.max(np.abs(V[: i + 1] - o_s[i]), axis=0)
                assert np.all(np.abs(o_n[i] - o_s[i]) <= eps / (1 - eps) * spread + 1e-14)
    assert errs[8] < errs[3] / 100
    for a, b in zip(range(3, 8), range(4, 9)):
        assert errs[b] < errs[a]
    return errs


def pin_normalisation_required(N=128, d=16, e=8, seed=2):
    """Raw Gaussian q, k (no L2 normalisation): the error against softmax stays
    above 1e-1 for n = 3..8 [ExpAttn abstract; arXivNews 'Normalization
    Requirement']."""
    q, k, v = wl.draw_qkv(seed, 1, 1, N, d, e, "f32", normalise=False)
    o_s = orc.softmax_attention(q.exact, k.exact, v.exact)
    for n in range(3, 9):
        err = float(np.max(np.abs(orc.quadratic_attention(q.exact, k.exact, v.exact, n) - o_s)))
        assert err > 1e-1, (n, err)


# ---------------------------------------------------------------------------
# O6: SVD rank of the stacked tensor powers
# ---------------------------------------------------------------------------

def pin_svd_rank(cases=((16, 1), (16, 2), (16, 3), (6, 4))):
    """The span of x^{(x)m} over many unit x has dimension C(d+m-1, m) [ExpAttn
    abstract: the width bound is confirmed by SVD]."""
    rng = np.random.Generator(np.random.PCG64(13))
    for d, m in cases:
        C = orc.block_widths(d, m + 1)[m]
        X = wl.l2_normalise(rng.standard_normal((2 * C, d)))
        rows = []
        for x in X:
            t = np.ones(1)
            for _ in range(m):
                t = np.kron(t, x)
            rows.append(t)
        s = np.linalg.svd(np.array(rows), compute_uv=False)
        rank = int(np.sum(s > s[0] * 1e-10))
        assert rank == C, (d, m, rank, C)


# ---------------------------------------------------------------------------
# O7, O9: textbook special cases and the convex hull
# ---------------------------------------------------------------------------

def pin_special_cases():
    rng = np.random.Generator(np.random.PCG64(17))
    N, d, e = 50, 6, 4
    q, k, v = wl.draw_qkv(23, 1, 1, N, d, e, "f32")
    Q, K, V = q.exact[0, 0], k.exact[0, 0], v.exact[0, 0]
    cnt = np.arange(1, N + 1)[:, None]
    # n = 1: causal running mean of v
    mean = np.cumsum(V, axis=0) / cnt
    for o in (orc.quadratic_attention(Q, K, V, 1), orc.recurrent_attention(Q, K, V, 1)[0],
              orc.chunked_attention(Q, K, V, 1, 8)[0]):
        assert rel_err(o, mean) <= 1e-13
    # n = 2: linear attention with feature map [1, x]
    ckv = np.cumsum(K[:, :, None] * V[:, None, :], axis=0)
    ck = np.cumsum(K, axis=0)
    cv = np.cumsum(V, axis=0)
    num = cv + np.einsum("id,ide->ie", Q, ckv)
    den = cnt[:, 0] + np.einsum("id,id->i", Q, ck)
    lin = num / den[:, None]
    for o in (orc.quadratic_attention(Q, K, V, 2), orc.recurrent_attention(Q, K, V, 2)[0],
              orc.chunked_attention(Q, K, V, 2, 16)[0]):
        assert rel_err(o, lin) <= 1e-12
    # d = 1: x = q k = +-1; closed form with K_n(+-1) as exact rationals
    for n in (1, 2, 3, 4, 5):
        q1 = rng.choice([-1.0, 1.0], size=(N, 1))
        k1 = rng.choice([-1.0, 1.0], size=(N, 1))
        kp = float(sum(Fraction(1, math.factorial(m)) for m in range(n)))
        km = float(sum(Fraction((-1) ** m, math.factorial(m)) for m in range(n)))
        w = np.where(q1 @ k1.T > 0, kp, km) * np.tril(np.ones((N, N)))
        with np.errstate(invalid="ignore", divide="ignore"):
            ref = (w @ V) / w.sum(axis=1, keepdims=True)
            got = orc.quadratic_attention(q1, k1, V, n)
        # n = 2 gives K_2(-1) = 0: rows whose keys all oppose the query have a
        # zero normaliser and must come out NaN on both sides, not masked
        assert np.array_equal(np.isnan(got), np.isnan(ref))
        fin = ~np.isnan(ref)
        assert np.max(np.abs(got[fin] - ref[fin])) <= 1e-12 * np.max(np.abs(ref[fin])) + 1e-12
        if n == 2:
            assert np.isnan(ref).any()
    # state rows with closed forms
    for n in (1, 2, 3):
        S = orc.states_definition(K, V, n)
        assert S[0, -1] == N
        assert np.allclose(S[0, :-1], V.sum(axis=0), rtol=1e-14, atol=1e-13)
        if n >= 2:
            assert np.allclose(S[1:1 + d, -1], K.sum(axis=0), rtol=1e-14, atol=1e-13)
            assert np.allclose(S[1:1 + d, :-1], K.T @ V, rtol=1e-14, atol=1e-13)


def pin_convex_hull(N=96, d=16, e=8, seed=4):
    """Odd n: the truncated kernel is > 0, so each output coordinate lies
    between the min and max of the values seen so far."""
    q, k, v = wl.draw_qkv(seed, 1, 1, N, d, e, "f32")
    V = v.exact[0, 0]
    lo = np.minimum.accumulate(V, axis=0)
    hi = np.maximum.accumulate(V, axis=0)
    for n in (1, 3, 5):
        o = orc.quadratic_attention(q.exact, k.exact, v.exact, n)[0, 0]
        assert np.all(o >= lo - 1e-12) and np.all(o <= hi + 1e-12)
        x = np.linspace(-1, 1, 2001)
        assert np.all(orc.taylor_kernel(x, n) > 0)


def pin_planes_layout():
    """Plane converters: value plane [B,H,W,e] first, then the normaliser plane."""
    B, H, W, e = 2, 3, 5, 4
    S = np.arange(B * H * W * (e + 1), dtype=np.float64).reshape(B, H, W, e + 1)
    flat = orc.states_to_planes(S)
    assert flat[((1 * H + 2) * W + 3) * e + 1] == S[1, 2, 3, 1]
    assert flat[B * H * W * e + (1 * H + 2) * W + 3] == S[1, 2, 3, e]
    assert np.array_equal(orc.planes_to_states(flat, B, H, W, e), S)


def pin_quadratic_rows():
    """Row-sampled definition equals the full quadratic form."""
    q, k, v = wl.draw_qkv(31, 1, 1, 70, 6, 3, "f32")
    full = orc.quadratic_attention(q.exact, k.exact, v.exact, 3)[0, 0]
    rows = [0, 1, 17, 69]
    part = orc.quadratic_rows(q.exact[0, 0, rows], k.exact[0, 0], v.exact[0, 0], rows, 3)
    assert rel_err(part, full[rows]) <= 1e-14


def pin_prefill_from_states():
    """Prefill resumed from the states of a prefix equals the quadratic form
    over the whole sequence on the resumed rows, and its states equal the
    single-pass states [ExpAttn abstract: additive states].  Checked against
    exact rational arithmetic (d = 2, 3) and in fp64 at d = 5; zero states
    reduce it to the plain prefill."""
    rng = np.random.Generator(np.random.PCG64(12))
    for d in (2, 3):
        units = _RATIONAL_UNITS[d]
        for n in (1, 2, 3, 4):
            N = 6
            q = [units[i] for i in rng.integers(0, len(units), N)]
            k = [units[i] for i in rng.integers(0, len(units), N)]
            v = [[Fraction(int(a), 4) for a in rng.integers(-8, 9, 2)] for _ in range(N)]
            exact = _exact_quadratic(q, k, v, n)
            qf = np.array([[float(a) for a in r] for r in q])
            kf = np.array([[float(a) for a in r] for r in k])
            vf = np.array([[float(a) for a in r] for r in v])
            for p in (1, 3, 5):
                S0 = orc.states_definition(kf[:p], vf[:p], n)
                o, _ = orc.prefill_from_states(qf[p:], kf[p:], vf[p:], S0, n)
                ref = np.array([[float(a) for a in r] for r in exact[p:]])
                assert np.max(np.abs(o - ref)) <= 4e-15 * max(1.0, np.max(np.abs(ref)))
    q, k, v = wl.draw_qkv(13, 1, 2, 40, 5, 3, "f32")
    for n in (1, 2, 3):
        o_full = orc.quadratic_attention(q.exact, k.exact, v.exact, n)
        S_full = orc.states_definition(k.exact, v.exact, n)
        for p in (1, 13, 39):
            S0 = orc.states_definition(k.exact[:, :, :p], v.exact[:, :, :p], n)
            o, S = orc.prefill_from_states(q.exact[:, :, p:], k.exact[:, :, p:], v.exact[:, :, p:], S0, n)
            assert rel_err(o, o_full[:, :, p:]) <= 1e-13
            assert rel_err(S, S_full) <= 1e-13
        Z = np.zeros_like(S_full)
        o0, S0r = orc.prefill_from_states(q.exact, k.exact, v.exact, Z, n)
        assert rel_err(o0, o_full) <= 1e-13 and rel_err(S0r, S_full) <= 1e-13
    # sampled-row form against the quadratic form over the whole sequence
    q, k, v = wl.draw_qkv(14, 1, 1, 90, 4, 3, "f32")
    Qx, Kx, Vx = q.exact[0, 0], k.exact[0, 0], v.exact[0, 0]
    p, n = 30, 3
    S0 = orc.states_definition(Kx[:p], Vx[:p], n)
    rows = [0, 1, 7, 31, 59]
    got = orc.prefill_from_rows(Qx[p:][rows], Kx[p:], Vx[p:], S0, rows, n)
    ref = orc.quadratic_rows(Qx[[p + r for r in rows]], Kx, Vx, [p + r for r in rows], n)
    assert rel_err(got, ref) <= 1e-13


# ---------------------------------------------------------------------------
# Input side: L2 normalisation and temperature [ExpAttn abstract: unit q and
# k keep q.k inside the convergence radius; arXivNews "Engineering
# Trade-offs and Performance"]
# ---------------------------------------------------------------------------

def pin_prefill_from_numden(N=7, p=4, d=3, e=2, seed=21):
    """Numerator and normaliser of a resumed prefill against brute force over
    the whole sequence: num_i = sum over every key j of the prefix and of the
    new tokens up to i of K_n(q_i.k_j) v_j, den_i the same sum of weights,
    with K_n written out as its power series; the division gives
    prefill_from_states, and zero states give the plain prefill's sums
    [ExpAttn abstract: additive states]."""
    rng = np.random.Generator(np.random.PCG64(seed))
    q = rng.standard_normal((p + N, d)); q /= np.linalg.norm(q, axis=1, keepdims=True)
    k = rng.standard_normal((p + N, d)); k /= np.linalg.norm(k, axis=1, keepdims=True)
    v = rng.standard_normal((p + N, e))
    for n in (1, 2, 3, 4):
        kn = lambda x: sum(x ** m / math.factorial(m) for m in range(n))
        S0 = orc.states_definition(k[:p], v[:p], n)
        num, den, S = orc.prefill_from_numden(q[p:], k[p:], v[p:], S0, n)
        for i in range(N):
            t = p + i
            w = [kn(float(q[t] @ k[j])) for j in range(t + 1)]
            ref_num = sum(wj * v[j] for j, wj in enumerate(w))
            assert np.max(np.abs(num[i] - ref_num)) <= 1e-13 * max(1.0, np.max(np.abs(ref_num)))
            assert abs(den[i] - sum(w)) <= 1e-13 * max(1.0, abs(sum(w)))
        o, S2 = orc.prefill_from_states(q[p:], k[p:], v[p:], S0, n)
        assert np.array_equal(o, num / den[:, None]) and np.array_equal(S, S2)
        num0, den0, _ = orc.prefill_from_numden(q, k, v, None, n)
        w0 = [sum(kn(float(q[t] @ k[j])) for j in range(t + 1)) for t in range(p + N)]
        assert np.max(np.abs(den0 - np.array(w0))) <= 1e-13 * max(w0)


def pin_normalize_rows():
    """Hand values, unit norms, invariance to positive scale (exact for
    powers of two), the NaN of a zero row, and a temperature worked by hand
    in tests/golden/normalized_d1_temperature.json."""
    got = orc.normalize_rows(np.array([[3.0, 4.0], [1.0, 2.0]]), 2.0)
    assert np.allclose(got[0], [1.2, 1.6], rtol=0, atol=1e-15)
    assert np.allclose(got[1], [2 / math.sqrt(5), 4 / math.sqrt(5)], rtol=0, atol=1e-15)
    assert np.allclose(orc.normalize_rows([[1.0, 2.0, 2.0]]), [[1 / 3, 2 / 3, 2 / 3]], rtol=0, atol=1e-16)
    X = np.random.Generator(np.random.PCG64(40)).standard_normal((50, 16)) * 7.0
    for tau in (1.0, 0.5, 3.0):
        U = orc.normalize_rows(X, tau)
        assert np.max(np.abs(np.linalg.norm(U, axis=1) - tau)) <= 1e-14 * tau
        assert np.array_equal(orc.normalize_rows(X * 8.0, tau), U)
        assert np.array_equal(orc.normalize_rows(-X, tau), -U)
        # same direction: x . u = tau |x|
        assert np.allclose(np.sum(X * U, axis=1), tau * np.linalg.norm(X, axis=1), rtol=1e-14, atol=0)
    assert np.isnan(orc.normalize_rows([[0.0, 0.0]])).all()
    g = json.load(open(os.path.join(GOLDEN, "normalized_d1_temperature.json")))
    tau = float(_frac(g["tau"]))
    q = np.array([[float(_frac(x))] for x in g["q"]])
    k = np.array([[float(_frac(x))] for x in g["k"]])
    v = np.array([[float(_frac(x))] for x in g["v"]])
    for n_str, o in g["o"].items():
        qh, kh = orc.normalized_inputs(q, k, tau, "f32")
        ref = np.array([[float(_frac(x))] for x in o])
        assert np.allclose(orc.quadratic_attention(qh, kh, v, int(n_str)), ref, rtol=0, atol=1e-15)


def pin_normalized_inputs():
    """The normalised inputs are the fp64 unit rows rounded once to the
    nearest value of the dtype, worked by hand: (21, 28) has norm 35, so the
    unit row is (3/5, 4/5); 3/5 = 1.0011001100...b x 2^-1 rounds up to
    1.0011010b x 2^-1 = 0.6015625 in bf16, and 4/5 = 1.1001100110...b x 2^-1
    rounds up to 1.1001101b x 2^-1 = 0.80078125.  With temperature 2 the
    query row is (6/5, 8/5), giving 1.203125 and 1.6015625.  fp32 rows are
    the fp32 roundings of 3/5 and 4/5."""
    q = np.array([[21.0, 28.0], [-3.0, 4.0]])
    qh, kh = orc.normalized_inputs(q, q, 2.0, "bf16")
    assert np.array_equal(kh, [[0.6015625, 0.80078125], [-0.6015625, 0.80078125]])
    assert np.array_equal(qh, [[1.203125, 1.6015625], [-1.203125, 1.6015625]])
    qf, kf = orc.normalized_inputs(q, q, 1.0, "f32")
    assert np.array_equal(kf[0], np.array([0.6, 0.8], dtype=np.float32).astype(np.float64))
    assert np.array_equal(qf, kf)
    # every coordinate lies within half a bf16 spacing of the fp64 unit row
    X = np.random.Generator(np.random.PCG64(43)).standard_normal((300, 16))
    _, kb = orc.normalized_inputs(X, X, 1.0, "bf16")
    u = orc.normalize_rows(X)
    half = 2.0 ** (np.floor(np.log2(np.abs(u))) - 8)
    assert np.all(np.abs(kb - u) <= half * (1 + 2.0 ** -20))


def _bf16_nearest_brute(x: float) -> float:
    """Nearest bf16 value to a finite nonzero fp64 x (normal range) by
    enumeration: the bf16 values are the fp32 values whose low 16 bits are
    zero; take the two around x and compare exact distances (ties: the one
    with an even last mantissa bit)."""
    f = np.float32(x)
    b = int(np.array(f).view(np.uint32)) & 0xFFFF0000
    cands = set()
    for d in (-0x10000, 0, 0x10000, 0x20000):
        c = float(np.array(np.uint32((b + d) & 0xFFFFFFFF)).view(np.float32))
        if np.isfinite(c):
            cands.add(c)
    best = min(cands, key=lambda c: (abs(c - x), (int(np.array(np.float32(c)).view(np.uint32)) >> 16) & 1))
    return best


def pin_round_to_dtype():
    """bf16 rounding is a single round to nearest even from fp64: hand ties
    around 1 (spacing 2^-7), a value that rounding to fp32 first would round
    the other way (1 + 2^-8 + 2^-30: fp32 would make it the exact tie 1 +
    2^-8 and then round down to 1), agreement with a brute-force nearest
    search on random values, and with the fp32 bit rule on values that are
    already fp32; f32 rounding is numpy's cast."""
    ulp = 2.0 ** -7
    x = np.array([1 + ulp / 2, 1 + 1.5 * ulp, 1 + ulp / 2 + 2.0 ** -20, -(1 + 1.5 * ulp), 3.0, 1 + 2.0 ** -8 + 2.0 ** -30])
    assert np.array_equal(orc.round_to_dtype(x, "bf16"), [1.0, 1 + 2 * ulp, 1 + ulp, -(1 + 2 * ulp), 3.0, 1 + ulp])
    r = np.random.Generator(np.random.PCG64(41)).standard_normal(2000) * 3.0
    got = orc.round_to_dtype(r, "bf16")
    assert all(got[i] == _bf16_nearest_brute(float(r[i])) for i in range(len(r)))
    r32 = r.astype(np.float32)
    bits = wl.f32_to_bf16_bits(r32)
    assert np.array_equal(orc.round_to_dtype(r32.astype(np.float64), "bf16"),
                          wl.bf16_bits_to_f32(bits).astype(np.float64))
    assert np.array_equal(orc.round_to_dtype(r, "f32"), r.astype(np.float32).astype(np.float64))
    assert np.isnan(orc.round_to_dtype(np.array([np.nan]), "bf16")).all()
    assert np.array_equal(orc.round_to_dtype(np.array([0.0, np.inf, -np.inf]), "bf16"), [0.0, np.inf, -np.inf])


ALL_PINS = [
    pin_hand_example, pin_page_widths, pin_exact_rational, pin_kron_features,
    pin_unit_identity, pin_recurrent_vs_quadratic, pin_chunk_additivity,
    pin_decode_equals_recurrence, pin_softmax_library, pin_softmax_convergence,
    pin_normalisation_required, pin_svd_rank, pin_special_cases, pin_convex_hull,
    pin_planes_layout, pin_quadratic_rows, pin_prefill_from_states, pin_prefill_from_numden,
    pin_normalize_rows, pin_normalized_inputs, pin_round_to_dtype, pin_softmax_rows,
]
