"""Pins for the fp64 oracle: checks against values the pages print, closed
forms, invariants, special cases and finite differences -- never against a
retyped copy of the oracle's own formula.

Each pin takes an ``oracle.Oracle`` instance and raises AssertionError when it
does not hold.  ``test_oracle.py`` runs them against the real oracle;
``test_oracle_mutants.py`` runs them against deliberately broken builds and
requires every mutant to fail at least one pin.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rng(seed):
    return np.random.default_rng(seed)


def _qkv(seed, B, H, Nq, Nk, d, with_dO=True):
    r = _rng(seed)
    out = [r.standard_normal((B, H, Nq, d)), r.standard_normal((B, H, Nk, d)),
           r.standard_normal((B, H, Nk, d))]
    if with_dO:
        out.append(r.standard_normal((B, H, Nq, d)))
    return out


# ---------------------------------------------------------------- the pages' examples

def pin_worked_row_state(o):
    """research-attention section 03: state after the first tile and the final row."""
    g = _golden("online_row_example.json")
    tol = g["tolerance"]
    m, l, u = o.online_row(g["scores"], g["values"], g["tile"], ntiles=1)
    first = g["after_first_tile"]
    assert abs(m - first["m"]) <= tol, m
    assert abs(l - first["l"]) <= tol, l
    assert np.max(np.abs(u - np.array(first["u"]))) <= tol, u
    m, l, u = o.online_row(g["scores"], g["values"], g["tile"])
    assert np.max(np.abs(u / l - np.array(g["result"]))) <= tol, u / l


def pin_worked_row_untiled(o):
    """The same row through the untiled forward: Q = e1, K_j = s_j e1, scale 1."""
    g = _golden("online_row_example.json")
    s = np.array(g["scores"])
    v = np.array(g["values"])
    Q = np.array([[[[1.0, 0.0]]]])
    K = np.zeros((1, 1, 4, 2))
    K[0, 0, :, 0] = s
    O, LSE = o.fwd(Q, K, v[None, None], scale=1.0)
    assert np.max(np.abs(O[0, 0, 0] - np.array(g["result"]))) <= g["tolerance"], O
    # LSE of the row is ln(sum_j e^{s_j}), a closed form for four numbers
    assert abs(LSE[0, 0, 0] - math.log(sum(math.exp(x) for x in s))) <= 1e-12
    # tile sizes that do and do not divide the row all reach the untiled result
    for tile in (1, 2, 3, 4, 8):
        m, l, u = o.online_row(s, v, tile)
        assert np.max(np.abs(u / l - O[0, 0, 0])) <= g["tiled_vs_untiled_bound"]


def pin_four_token_example(o):
    """Flash Attention notes, 4-token example: printed outputs and intermediates."""
    g = _golden("four_token_example.json")
    X = np.array(g["X"])[None, None]
    scale = 1.0 / math.sqrt(X.shape[-1])
    O, LSE, P = o.fwd(X, X, X, scale, want_probs=True)
    to, ti = g["tol_outputs"], g["tol_intermediates"]
    assert np.max(np.abs(O[0, 0, 0] - g["token0"])) <= to, O[0, 0, 0]
    assert np.max(np.abs(O[0, 0, 1] - g["token1"])) <= to, O[0, 0, 1]
    assert np.max(np.abs(P[0, 0, 0] - g["row0_softmax"])) <= ti, P[0, 0, 0]
    denom = math.exp(LSE[0, 0, 0])  # sum_j exp(s_0j), the page's denominator
    assert abs(denom - g["row0_denominator"]) <= ti, denom
    assert np.max(np.abs(O[0, 0, 0] * denom - g["token0_numerators"])) <= ti
    assert np.max(np.abs(O[0, 0, 1] * math.exp(LSE[0, 0, 1]) - g["token1_numerators"])) <= ti


def pin_four_token_symmetry(o):
    """Swapping the two coordinates swaps tokens 0 and 1 and fixes tokens 2, 3,
    so O_1 is O_0 reversed and O_2, O_3 have equal coordinates."""
    X = np.array(_golden("four_token_example.json")["X"])[None, None]
    O, _ = o.fwd(X, X, X, 1.0 / math.sqrt(2.0))
    O = O[0, 0]
    assert np.max(np.abs(O[1] - O[0][::-1])) <= 1e-15
    assert abs(O[2, 0] - O[2, 1]) <= 1e-15 and abs(O[3, 0] - O[3, 1]) <= 1e-15
    # tokens 2 and 3 are not printed; the symmetry fixes their form, and each
    # is a convex combination of the rows of X, so both coordinates lie in [0, 1]
    assert 0.0 < O[2, 0] < 1.0 and 0.0 < O[3, 0] < 1.0


# ---------------------------------------------------------------- tiling and softmax

def pin_tiled_vs_untiled(o):
    """Tiled and untiled forward agree within 1e-12 (research-attention section 03's bound)."""
    for causal in (False, True):
        for (Nq, Nk) in ((37, 37), (21, 53)) if not causal else ((37, 37), (29, 29)):
            Q, K, V = _qkv(11 + Nq + Nk + causal, 2, 2, Nq, Nk, 8, with_dO=False)
            O, L = o.fwd(Q, K, V, 0.35, causal)
            for tile in (1, 2, 3, 16, 64):
                Ot, Lt = o.tiled_fwd(Q, K, V, 0.35, causal, tile)
                assert np.max(np.abs(Ot - O)) <= 1e-12, (tile, causal)
                assert np.max(np.abs(Lt - L)) <= 1e-12, (tile, causal)


def pin_rows_sum_to_one(o):
    for causal in (False, True):
        Q, K, V = _qkv(5, 1, 2, 24, 24, 4, with_dO=False)
        _, _, P = o.fwd(Q * 3, K, V, 0.5, causal, want_probs=True)
        assert np.max(np.abs(P.sum(-1) - 1.0)) <= 1e-13
        assert np.all(P >= 0.0)
        if causal:
            i, j = np.indices(P.shape[-2:])
            assert np.all(P[..., j > i] == 0.0)


def pin_lse_direct(o):
    """LSE equals ln(sum_j exp(S_ij)) evaluated directly (no max shift) for moderate S."""
    Q, K, V = _qkv(6, 1, 1, 9, 13, 5, with_dO=False)
    scale = 0.4
    _, L = o.fwd(Q, K, V, scale)
    for i in range(9):
        direct = math.log(sum(math.exp(scale * float(np.dot(Q[0, 0, i], K[0, 0, j]))) for j in range(13)))
        assert abs(L[0, 0, i] - direct) <= 1e-12


def pin_large_logits(o):
    """Scores far beyond exp's range still give finite, correct results: with
    one key dominating by >1000 the output is that key's value row exactly."""
    Q = np.zeros((1, 1, 1, 2)); Q[..., 0] = 1.0
    K = np.zeros((1, 1, 3, 2)); K[0, 0, :, 0] = [2000.0, 1000.0, -500.0]
    V = np.arange(6, dtype=np.float64).reshape(1, 1, 3, 2)
    O, L = o.fwd(Q, K, V, 1.0)
    assert np.all(O[0, 0, 0] == V[0, 0, 0]) and L[0, 0, 0] == 2000.0


# ---------------------------------------------------------------- gradients

def _loss(o, Q, K, V, dO, scale, causal):
    O, _ = o.fwd(Q, K, V, scale, causal)
    return float(np.sum(dO * O))


def pin_finite_differences(o):
    """Central differences of L = sum(dO * O) agree with the analytic gradients
    to 1e-6 (relative, per tensor) for small shapes, Nq != Nk, with and
    without the causal mask."""
    h = 1e-6
    for causal, (Nq, Nk, d) in ((False, (5, 7, 3)), (False, (9, 4, 4)), (True, (6, 6, 3)), (True, (11, 16, 2))):
        Q, K, V, dO = _qkv(100 + Nq * Nk + causal, 1, 2, Nq, Nk, d)
        scale = 0.7
        dQ, dK, dV, O, L = o.bwd(Q, K, V, dO, scale, causal)
        for name, X, G in (("Q", Q, dQ), ("K", K, dK), ("V", V, dV)):
            num = np.zeros_like(X)
            for idx in np.ndindex(X.shape):
                old = X[idx]
                X[idx] = old + h
                lp = _loss(o, Q, K, V, dO, scale, causal)
                X[idx] = old - h
                lm = _loss(o, Q, K, V, dO, scale, causal)
                X[idx] = old
                num[idx] = (lp - lm) / (2 * h)
            err = np.linalg.norm(num - G) / max(np.linalg.norm(num), 1e-30)
            assert err <= 1e-6, (name, causal, Nq, Nk, err)


def pin_gradient_closed_forms(o):
    """Nk = 1: O = V_0 for every row, so dV_0 = sum_i dO_i and dQ = dK = 0.
    Q = 0 (non-causal): P is uniform 1/Nk, so dV_j = sum_i dO_i / Nk and dK = 0."""
    Q, K, V, dO = _qkv(7, 1, 1, 6, 1, 4)
    dQ, dK, dV, O, L = o.bwd(Q, K, V, dO, 0.5)
    assert np.max(np.abs(dV[0, 0, 0] - dO[0, 0].sum(0))) <= 1e-13
    assert np.max(np.abs(dQ)) <= 1e-13 and np.max(np.abs(dK)) <= 1e-13
    Q, K, V, dO = _qkv(8, 1, 1, 5, 7, 3)
    Q[:] = 0.0
    dQ, dK, dV, O, L = o.bwd(Q, K, V, dO, 0.5)
    for j in range(7):
        assert np.max(np.abs(dV[0, 0, j] - dO[0, 0].sum(0) / 7)) <= 1e-13
    assert np.max(np.abs(dK)) <= 1e-13


def pin_bwd_forward_consistent(o):
    Q, K, V, dO = _qkv(9, 2, 1, 10, 12, 4)
    for causal in (False, True):
        if causal:
            K, V = K[:, :, :10], V[:, :, :10]
        _, _, _, O, L = o.bwd(Q, K, V, dO, 0.3, causal)
        O2, L2 = o.fwd(Q, K, V, 0.3, causal)
        assert np.max(np.abs(O - O2)) <= 1e-14 and np.max(np.abs(L - L2)) <= 1e-14


# ---------------------------------------------------------------- invariants I1-I8

def pin_I1_dV_column_sum(o):
    """sum_j dV_j = sum_i dO_i (each row of P sums to 1), with or without the mask."""
    for causal in (False, True):
        Q, K, V, dO = _qkv(21 + causal, 1, 2, 12, 12, 4)
        _, _, dV, _, _ = o.bwd(Q, K, V, dO, 0.6, causal)
        assert np.max(np.abs(dV.sum(2) - dO.sum(2))) <= 1e-12


def pin_I2_dK_sums_to_zero(o):
    """sum_j dK_j = 0 (each row of dS sums to zero)."""
    for causal in (False, True):
        Q, K, V, dO = _qkv(23 + causal, 1, 2, 12, 12, 4)
        _, dK, _, _, _ = o.bwd(Q, K, V, dO, 0.6, causal)
        assert np.max(np.abs(dK.sum(2))) <= 1e-12


def pin_I3_key_shift(o):
    """Adding c to every key row leaves O unchanged and moves LSE_i by scale*q_i.c."""
    for causal in (False, True):
        Q, K, V = _qkv(25 + causal, 1, 1, 8, 8, 4, with_dO=False)
        c = np.array([0.3, -1.1, 0.7, 2.0])
        O, L = o.fwd(Q, K, V, 0.5, causal)
        O2, L2 = o.fwd(Q, K + c, V, 0.5, causal)
        assert np.max(np.abs(O2 - O)) <= 1e-12
        assert np.max(np.abs(L2 - (L + 0.5 * Q @ c))) <= 1e-12


def pin_I4_value_shift(o):
    """Adding c to every value row moves every output row by c."""
    Q, K, V = _qkv(27, 1, 1, 8, 9, 4, with_dO=False)
    c = np.array([1.5, -0.25, 3.0, 0.0])
    for causal in (False, True):
        k, v = (K[:, :, :8], V[:, :, :8]) if causal else (K, V)
        O, _ = o.fwd(Q, k, v, 0.5, causal)
        O2, _ = o.fwd(Q, k, v + c, 0.5, causal)
        assert np.max(np.abs(O2 - (O + c))) <= 1e-12


def pin_I5_single_key(o):
    """Nk = 1: O = V_0, LSE = S_00.  Causal row 0 sees only key 0: O_0 = V_0."""
    Q, K, V = _qkv(29, 1, 1, 3, 1, 4, with_dO=False)
    O, L = o.fwd(Q, K, V, 0.5)
    assert np.all(O[0, 0] == V[0, 0, 0])
    assert np.max(np.abs(L[0, 0] - 0.5 * Q[0, 0] @ K[0, 0, 0])) <= 1e-14
    Q, K, V = _qkv(30, 1, 1, 6, 6, 4, with_dO=False)
    O, L = o.fwd(Q, K, V, 0.5, causal=True)
    assert np.all(O[0, 0, 0] == V[0, 0, 0])


def pin_I6_D_identity(o):
    """rowsum(dO * O) = rowsum(P * dP) with dP = dO V^T."""
    for causal in (False, True):
        Q, K, V, dO = _qkv(31 + causal, 1, 1, 7, 7, 4)
        O, _, P = o.fwd(Q, K, V, 0.5, causal, want_probs=True)
        dP = dO[0, 0] @ V[0, 0].T
        assert np.max(np.abs((dO * O).sum(-1)[0, 0] - (P[0, 0] * dP).sum(-1))) <= 1e-12


def pin_I7_zero_query(o):
    """Q = 0: O is the mean of the allowed value rows and LSE = ln(#allowed)."""
    _, K, V = _qkv(33, 1, 1, 6, 6, 4, with_dO=False)
    Q = np.zeros((1, 1, 6, 4))
    O, L = o.fwd(Q, K, V, 0.5)
    assert np.max(np.abs(O[0, 0] - V[0, 0].mean(0))) <= 1e-14
    assert np.max(np.abs(L - math.log(6))) <= 1e-14
    O, L = o.fwd(Q, K, V, 0.5, causal=True)
    for i in range(6):
        assert np.max(np.abs(O[0, 0, i] - V[0, 0, :i + 1].mean(0))) <= 1e-14
        assert abs(L[0, 0, i] - math.log(i + 1)) <= 1e-14


def pin_I8_key_permutation(o):
    """Permuting key and value rows together leaves the (non-causal) output unchanged."""
    Q, K, V = _qkv(35, 1, 2, 6, 10, 4, with_dO=False)
    perm = _rng(36).permutation(10)
    O, L = o.fwd(Q, K, V, 0.5)
    O2, L2 = o.fwd(Q, K[:, :, perm], V[:, :, perm], 0.5)
    assert np.max(np.abs(O2 - O)) <= 1e-13 and np.max(np.abs(L2 - L)) <= 1e-13


def pin_causal_is_prefix_attention(o):
    """Row i under the causal mask equals unmasked attention over keys 0..i."""
    Q, K, V = _qkv(37, 1, 1, 7, 7, 3, with_dO=False)
    O, L = o.fwd(Q, K, V, 0.8, causal=True)
    for i in range(7):
        Oi, Li = o.fwd(Q[:, :, i:i + 1], K[:, :, :i + 1], V[:, :, :i + 1], 0.8)
        assert np.max(np.abs(Oi[0, 0, 0] - O[0, 0, i])) <= 1e-14
        assert abs(Li[0, 0, 0] - L[0, 0, i]) <= 1e-14


def pin_rows_match_full(o):
    """The sampled-row forward returns exactly the full forward's rows."""
    for causal in (False, True):
        Q, K, V = _qkv(39 + causal, 2, 3, 20, 20, 4, with_dO=False)
        O, L = o.fwd(Q, K, V, 0.5, causal)
        rows = np.stack([_rng(40 + t).choice(20, 5, replace=False) for t in range(6)])
        Or, Lr = o.fwd_rows(Q, K, V, rows, 0.5, causal)
        Of, Lf = O.reshape(6, 20, 4), L.reshape(6, 20)
        for t in range(6):
            assert np.max(np.abs(Or[t] - Of[t, rows[t]])) <= 1e-14
            assert np.max(np.abs(Lr[t] - Lf[t, rows[t]])) <= 1e-14


# ---------------------------------------------------------------- dropout (research-attention sections 01, 06)

def pin_philox_known_answers(o):
    """Philox4x32-10 reproduces the generator's published known-answer vectors."""
    g = _golden("philox4x32_10_kat.json")
    for v in g["vectors"]:
        ctr = [int(x, 16) for x in v["ctr"]]
        key = [int(x, 16) for x in v["key"]]
        out = [int(x, 16) for x in v["out"]]
        assert [int(x) for x in o.philox4x32_10(ctr, key)] == out, v


def pin_dropout_rate(o):
    """Threshold t drops a fraction t/256 of the elements (within 5 binomial
    standard deviations over 2^18 elements); t = 0 drops nothing."""
    n = 2 * 2 * 256 * 256
    for t in (0, 26, 128, 255):
        keep = o.dropout_keep(2, 2, 256, 256, t, 0x1234_5678_9abc)
        frac = 1.0 - keep.mean()
        if t == 0:
            assert frac == 0.0
        else:
            p = t / 256.0
            assert abs(frac - p) <= 5 * math.sqrt(p * (1 - p) / n), (t, frac)


def pin_dropout_streams_distinct(o):
    """Different heads, query rows, key columns and seeds draw different masks
    (the counter separates every element; a mask shared between any two of
    them would be a repeated stream)."""
    keep = o.dropout_keep(1, 3, 16, 64, 128, 99).astype(np.int64)
    for a, b in ((0, 1), (0, 2), (1, 2)):
        assert np.mean(keep[0, a] == keep[0, b]) < 0.75
    for i in range(15):  # neighbouring rows: within and across 4-row blocks
        assert np.mean(keep[0, 0, i] == keep[0, 0, i + 1]) < 0.8, i
    for j in range(63):
        assert np.mean(keep[0, 0, :, j] == keep[0, 0, :, j + 1]) < 0.85, j
    other = o.dropout_keep(1, 3, 16, 64, 128, 100).astype(np.int64)
    assert np.mean(keep == other) < 0.6
    # one head of a larger problem is that problem's head bh0
    one = o.dropout_keep(1, 1, 16, 64, 128, 99, bh0=2).astype(np.int64)
    assert np.array_equal(one[0, 0], keep[0, 2])


def pin_dropout_keep_all_is_plain(o):
    """A mask that keeps everything with scale 1 gives exactly the plain forward and backward."""
    for causal in (False, True):
        Q, K, V, dO = _qkv(51 + causal, 1, 2, 9, 9, 4)
        keep = np.ones((1, 2, 9, 9), dtype=np.uint8)
        O1, L1 = o.fwd(Q, K, V, 0.6, causal)
        O2, L2 = o.fwd_dropout(Q, K, V, keep, 1.0, 0.6, causal)
        assert np.array_equal(O1, O2) and np.array_equal(L1, L2)
        g1 = o.bwd(Q, K, V, dO, 0.6, causal)
        g2 = o.bwd_dropout(Q, K, V, dO, keep, 1.0, 0.6, causal)
        for a, b in zip(g1, g2):
            assert np.array_equal(a, b)


def pin_dropout_finite_differences(o):
    """Under a fixed keep mask the dropped forward is differentiable: central
    differences of L = sum(dO * O) agree with the dropout backward to 1e-6."""
    h = 1e-6
    for causal, (Nq, Nk, d), t in ((False, (5, 7, 3), 77), (True, (8, 8, 2), 128)):
        Q, K, V, dO = _qkv(300 + Nq * Nk + causal, 1, 2, Nq, Nk, d)
        keep = o.dropout_keep(1, 2, Nq, Nk, t, 4242)
        ks = 256.0 / (256 - t)
        scale = 0.8
        dQ, dK, dV, O, L = o.bwd_dropout(Q, K, V, dO, keep, ks, scale, causal)
        O2, _ = o.fwd_dropout(Q, K, V, keep, ks, scale, causal)
        assert np.max(np.abs(O - O2)) <= 1e-14

        def loss():
            Ox, _ = o.fwd_dropout(Q, K, V, keep, ks, scale, causal)
            return float(np.sum(dO * Ox))

        for name, X, G in (("Q", Q, dQ), ("K", K, dK), ("V", V, dV)):
            num = np.zeros_like(X)
            for idx in np.ndindex(X.shape):
                old = X[idx]
                X[idx] = old + h
                lp = loss()
                X[idx] = old - h
                lm = loss()
                X[idx] = old
                num[idx] = (lp - lm) / (2 * h)
            err = np.linalg.norm(num - G) / max(np.linalg.norm(num), 1e-30)
            assert err <= 1e-6, (name, causal, err)


def pin_dropout_unbiased(o):
    """Inverted dropout keeps the expectation: averaged over many seeds, the
    dropped output approaches the plain one (the sample mean's error stays
    within a few of its own standard errors)."""
    Q, K, V = _qkv(61, 1, 1, 4, 32, 8, with_dO=False)
    O, _ = o.fwd(Q, K, V, 0.5)
    t, n = 128, 400
    samples = np.stack([o.fwd_dropout(Q, K, V, o.dropout_keep(1, 1, 4, 32, t, s), 2.0, 0.5)[0] for s in range(n)])
    mean, se = samples.mean(0), samples.std(0) / math.sqrt(n)
    z = (mean - O) / se
    assert np.sqrt(np.mean(z ** 2)) < 1.6, np.sqrt(np.mean(z ** 2))


def pin_dropout_dK_sums_to_zero(o):
    """Under dropout each row of dS still sums to zero (r is taken with the
    undropped P), so sum_j dK_j = 0."""
    for causal in (False, True):
        Q, K, V, dO = _qkv(71 + causal, 1, 2, 12, 12, 4)
        keep = o.dropout_keep(1, 2, 12, 12, 90, 7)
        _, dK, _, _, _ = o.bwd_dropout(Q, K, V, dO, keep, 256.0 / 166, 0.6, causal)
        assert np.max(np.abs(dK.sum(2))) <= 1e-12


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
