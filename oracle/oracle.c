/*
 * oracle.c -- plain fp64 CPU reference for exact scaled-dot-product attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link,
 * load or call this file: only the test suite, the smoke check and the
 * benchmark's cpu_baseline leg use it.  It shares no code, header, table or
 * constant with the HIP kernels.
 *
 * What it computes (written from the pages, not from any listing):
 *
 *   S   = scale * Q K^T                      [Online-softmax note "research-attention",
 *   P   = row-wise softmax of S                 section 01, the three-line definition;
 *   O   = P V                                   "Flash Attention" notes page, the
 *                                               Attention(Q,K,V) formula]
 *   LSE = m + ln(l), m the row max of S, l = sum_j exp(S_j - m)
 *                                             [research-attention, section 04: saving
 *                                               L = m + log(l) is enough to rebuild P]
 *
 *   Backward (page 1 "Flash Attention 原理与实现", section "Backward 的 Tiling
 *   策略", lists dV = P^T dO, dP = dO V^T, dQ = dS K, dK = dS^T Q and leaves
 *   the softmax gradient to the paper).  The softmax vector-Jacobian product
 *   used here is the textbook one: for one row p = softmax(s) and upstream
 *   gradient g = dP_row, ds_j = p_j (g_j - sum_k p_k g_k).  The scale lands on
 *   dQ and dK by the chain rule, not on dV.
 *
 *   Causal mask: key j is allowed for query i exactly when j <= i (top-left
 *   alignment, for any Nq and Nk).  Masked keys take no part in max, sum or
 *   products; their probability is exactly 0.  Key 0 is always allowed, so
 *   every row is non-empty.
 *
 * The oracle materialises S and P for a whole head in fp64 and uses libm
 * exp/log.  Summation order is the plain ascending order of the index being
 * summed; nothing is blocked, fused or reordered.
 *
 * oracle_online_row / oracle_tiled_fwd build the result from running states
 * (research-attention section 02): each tile of keys gets its own state
 * (m_t, l_t, u_t), the tiles are folded into the row's state one after the
 * other with that section's rule for combining two states, and o = u / l with
 * one division at the end.  They serve the tiled/untiled agreement check and
 * the worked row's intermediate state.
 *
 * All arrays are contiguous row-major: Q [B,H,Nq,d], K/V [B,H,Nk,d],
 * O/dO/dQ [B,H,Nq,d], dK/dV [B,H,Nk,d], LSE [B,H,Nq].  Returns 0 on success,
 * -1 on a bad argument, -2 if a scratch allocation fails.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

static int allowed(int64_t i, int64_t j, int causal) { return !causal || j <= i; }

static double dot(const double *a, const double *b, int64_t n) {
    double acc = 0.0;
    for (int64_t c = 0; c < n; ++c) acc += a[c] * b[c];
    return acc;
}

static int bad_shape(int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d) {
    return B <= 0 || H <= 0 || Nq <= 0 || Nk <= 0 || d <= 0;
}

/* One head: S (scaled scores) then P in place, plus m, l, LSE per row. */
static void head_probs(const double *Q, const double *K, int64_t Nq, int64_t Nk, int64_t d,
                       double scale, int causal, double *P, double *LSE) {
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < Nq; ++i) {
        double *row = P + i * Nk;
        double m = -INFINITY;
        for (int64_t j = 0; j < Nk; ++j) {
            if (allowed(i, j, causal)) {
                row[j] = scale * dot(Q + i * d, K + j * d, d);
                if (row[j] > m) m = row[j];
            }
        }
        double l = 0.0;
        for (int64_t j = 0; j < Nk; ++j)
            if (allowed(i, j, causal)) l += exp(row[j] - m);
        for (int64_t j = 0; j < Nk; ++j)
            row[j] = allowed(i, j, causal) ? exp(row[j] - m) / l : 0.0;
        LSE[i] = m + log(l);
    }
}

/* O_i = sum_j P[i][j] V_j */
static void head_pv(const double *P, const double *V, int64_t Nq, int64_t Nk, int64_t d, double *O) {
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < Nq; ++i) {
        double *o = O + i * d;
        for (int64_t c = 0; c < d; ++c) o[c] = 0.0;
        for (int64_t j = 0; j < Nk; ++j) {
            const double p = P[i * Nk + j];
            for (int64_t c = 0; c < d; ++c) o[c] += p * V[j * d + c];
        }
    }
}

/*
 * Forward over all heads.  P_out may be NULL; when given it receives the
 * probabilities [B,H,Nq,Nk] (only sensible for small shapes).
 */
int oracle_fwd(const double *Q, const double *K, const double *V, int64_t B, int64_t H,
               int64_t Nq, int64_t Nk, int64_t d, double scale, int causal,
               double *O, double *LSE, double *P_out) {
    if (!Q || !K || !V || !O || !LSE || bad_shape(B, H, Nq, Nk, d)) return -1;
    double *P = (double *)malloc(sizeof(double) * (size_t)(Nq * Nk));
    if (!P) return -2;
    for (int64_t bh = 0; bh < B * H; ++bh) {
        const double *q = Q + bh * Nq * d, *k = K + bh * Nk * d, *v = V + bh * Nk * d;
        head_probs(q, k, Nq, Nk, d, scale, causal, P, LSE + bh * Nq);
        head_pv(P, v, Nq, Nk, d, O + bh * Nq * d);
        if (P_out) memcpy(P_out + bh * Nq * Nk, P, sizeof(double) * (size_t)(Nq * Nk));
    }
    free(P);
    return 0;
}

/*
 * Forward for selected query rows only: rows[bh*nrows + r] is the r-th query
 * row of head bh.  Each row's softmax runs over every allowed key, exactly as
 * in oracle_fwd; O_rows is [B*H, nrows, d], LSE_rows is [B*H, nrows].
 */
int oracle_fwd_rows(const double *Q, const double *K, const double *V, int64_t B, int64_t H,
                    int64_t Nq, int64_t Nk, int64_t d, double scale, int causal,
                    const int64_t *rows, int64_t nrows, double *O_rows, double *LSE_rows) {
    if (!Q || !K || !V || !rows || !O_rows || !LSE_rows || nrows < 0 || bad_shape(B, H, Nq, Nk, d))
        return -1;
    for (int64_t t = 0; t < B * H * nrows; ++t)
        if (rows[t] < 0 || rows[t] >= Nq) return -1;
    int err = 0;
    #pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)Nk);
        if (!s) {
            #pragma omp atomic write
            err = -2;
        }
        #pragma omp for schedule(dynamic, 1)
        for (int64_t t = 0; t < B * H * nrows; ++t) {
            if (!s) continue;
            const int64_t bh = t / nrows, i = rows[t];
            const double *q = Q + (bh * Nq + i) * d, *k = K + bh * Nk * d, *v = V + bh * Nk * d;
            double m = -INFINITY;
            for (int64_t j = 0; j < Nk; ++j) {
                if (allowed(i, j, causal)) {
                    s[j] = scale * dot(q, k + j * d, d);
                    if (s[j] > m) m = s[j];
                }
            }
            double l = 0.0;
            for (int64_t j = 0; j < Nk; ++j)
                if (allowed(i, j, causal)) l += exp(s[j] - m);
            double *o = O_rows + t * d;
            for (int64_t c = 0; c < d; ++c) o[c] = 0.0;
            for (int64_t j = 0; j < Nk; ++j) {
                if (!allowed(i, j, causal)) continue;
                const double p = exp(s[j] - m) / l;
                for (int64_t c = 0; c < d; ++c) o[c] += p * v[j * d + c];
            }
            LSE_rows[t] = m + log(l);
        }
        free(s);
    }
    return err;
}

/*
 * Gradients of one head.  P: the softmax probabilities; Pv: the matrix that
 * multiplied V in the forward (P itself, or P~ = Z P keep_scale under
 * dropout); z: the dropout keep mask, or NULL for none.
 *   dP = dO V^T (times Z keep_scale under dropout), r_i = sum_j P_ij dP_ij,
 *   dS = P (dP - r), dQ = scale dS K, dK = scale dS^T Q, dV = Pv^T dO.
 * dS is scratch [Nq][Nk].
 */
static void head_grads(const double *q, const double *k, const double *v, const double *go, int64_t Nq,
                       int64_t Nk, int64_t d, double scale, const double *P, const double *Pv, const uint8_t *z,
                       double keep_scale, double *dS, double *gq, double *gk, double *gv) {
    /* dP = dO V^T, then dS = P (dP - r) row by row */
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < Nq; ++i) {
        double *row = dS + i * Nk;
        for (int64_t j = 0; j < Nk; ++j) {
            const double g = dot(go + i * d, v + j * d, d);
            row[j] = !z ? g : (z[i * Nk + j] ? g * keep_scale : 0.0);
        }
        double r = 0.0;
        for (int64_t j = 0; j < Nk; ++j) r += P[i * Nk + j] * row[j];
        for (int64_t j = 0; j < Nk; ++j) row[j] = P[i * Nk + j] * (row[j] - r);
    }
    /* dQ_i = scale sum_j dS_ij K_j */
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < Nq; ++i) {
        double *g = gq + i * d;
        for (int64_t c = 0; c < d; ++c) g[c] = 0.0;
        for (int64_t j = 0; j < Nk; ++j) {
            const double w = dS[i * Nk + j];
            for (int64_t c = 0; c < d; ++c) g[c] += w * k[j * d + c];
        }
        for (int64_t c = 0; c < d; ++c) g[c] *= scale;
    }
    /* dK_j = scale sum_i dS_ij Q_i ; dV_j = sum_i Pv_ij dO_i */
    #pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < Nk; ++j) {
        double *a = gk + j * d, *b = gv + j * d;
        for (int64_t c = 0; c < d; ++c) { a[c] = 0.0; b[c] = 0.0; }
        for (int64_t i = 0; i < Nq; ++i) {
            const double ws = dS[i * Nk + j], wp = Pv[i * Nk + j];
            for (int64_t c = 0; c < d; ++c) {
                a[c] += ws * q[i * d + c];
                b[c] += wp * go[i * d + c];
            }
        }
        for (int64_t c = 0; c < d; ++c) a[c] *= scale;
    }
}

/*
 * Backward over all heads.  Given Q, K, V and the upstream gradient dO,
 * returns dQ, dK, dV (and, when non-NULL, O and LSE of the same forward).
 * Per head: P as in the forward, dP = dO V^T, r_i = sum_j P_ij dP_ij,
 * dS = P (dP - r), dQ = scale dS K, dK = scale dS^T Q, dV = P^T dO.
 */
int oracle_bwd(const double *Q, const double *K, const double *V, const double *dO,
               int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, double scale, int causal,
               double *dQ, double *dK, double *dV, double *O, double *LSE) {
    if (!Q || !K || !V || !dO || !dQ || !dK || !dV || bad_shape(B, H, Nq, Nk, d)) return -1;
    double *P = (double *)malloc(sizeof(double) * (size_t)(Nq * Nk));
    double *dS = (double *)malloc(sizeof(double) * (size_t)(Nq * Nk));
    double *lse = (double *)malloc(sizeof(double) * (size_t)Nq);
    if (!P || !dS || !lse) {
        free(P); free(dS); free(lse);
        return -2;
    }
    for (int64_t bh = 0; bh < B * H; ++bh) {
        const double *q = Q + bh * Nq * d, *k = K + bh * Nk * d, *v = V + bh * Nk * d;
        head_probs(q, k, Nq, Nk, d, scale, causal, P, lse);
        if (O) head_pv(P, v, Nq, Nk, d, O + bh * Nq * d);
        if (LSE) memcpy(LSE + bh * Nq, lse, sizeof(double) * (size_t)Nq);
        head_grads(q, k, v, dO + bh * Nq * d, Nq, Nk, d, scale, P, P, NULL, 1.0, dS, dQ + bh * Nq * d,
                   dK + bh * Nk * d, dV + bh * Nk * d);
    }
    free(P); free(dS); free(lse);
    return 0;
}

/* The state of one tile of keys [a, b) on its own (research-attention, section
 * 02: the three quantities a block contributes): its maximum m_t, its sum
 * l_t = sum_j exp(s_j - m_t) and its unnormalised output u_t = sum_j
 * exp(s_j - m_t) v_j. */
static void tile_state(const double *s, const double *v, int64_t a, int64_t b, int64_t dv, double *m_t,
                       double *l_t, double *u_t) {
    double mx = -INFINITY;
    for (int64_t j = a; j < b; ++j) mx = s[j] > mx ? s[j] : mx;
    double sum = 0.0;
    for (int64_t c = 0; c < dv; ++c) u_t[c] = 0.0;
    for (int64_t j = a; j < b; ++j) {
        const double w = exp(s[j] - mx);
        sum += w;
        for (int64_t c = 0; c < dv; ++c) u_t[c] += w * v[j * dv + c];
    }
    *m_t = mx;
    *l_t = sum;
}

/* Section 02's rule for combining two states into the first: with
 * m = max(m1, m2), each side's l and u are weighted by exp(m_k - m) and added.
 * The empty state (nothing seen yet: l = 0) takes the other state as it is. */
static void merge_state(double *m1, double *l1, double *u1, double m2, double l2, const double *u2, int64_t dv) {
    if (*l1 == 0.0) {
        *m1 = m2;
        *l1 = l2;
        for (int64_t c = 0; c < dv; ++c) u1[c] = u2[c];
        return;
    }
    const double m = *m1 > m2 ? *m1 : m2;
    const double w_old = exp(*m1 - m), w_new = exp(m2 - m);
    *l1 = w_old * *l1 + w_new * l2;
    for (int64_t c = 0; c < dv; ++c) u1[c] = w_old * u1[c] + w_new * u2[c];
    *m1 = m;
}

/*
 * Running state of one row (research-attention, section 02): scores s[0..n),
 * value rows v[n][dv].  Folds the states of the first `ntiles` tiles of `tile`
 * consecutive scores (all of them when ntiles < 0) into the empty state, in
 * order, and returns the result (m, l, u) unnormalised.
 */
int oracle_online_row(const double *s, const double *v, int64_t n, int64_t dv, int64_t tile,
                      int64_t ntiles, double *m_out, double *l_out, double *u_out) {
    if (!s || !v || !m_out || !l_out || !u_out || n <= 0 || dv <= 0 || tile <= 0) return -1;
    double *u_t = (double *)malloc(sizeof(double) * (size_t)dv);
    if (!u_t) return -2;
    double m = -INFINITY, l = 0.0;  /* the empty state */
    for (int64_t c = 0; c < dv; ++c) u_out[c] = 0.0;
    const int64_t tiles = (n + tile - 1) / tile;
    for (int64_t t = 0; t < tiles && (ntiles < 0 || t < ntiles); ++t) {
        const int64_t a = t * tile, b = a + tile < n ? a + tile : n;
        double m_t, l_t;
        tile_state(s, v, a, b, dv, &m_t, &l_t, u_t);
        merge_state(&m, &l, u_out, m_t, l_t, u_t, dv);
    }
    free(u_t);
    *m_out = m;
    *l_out = l;
    return 0;
}

/*
 * Tiled forward: every query row runs the running-state recurrence over its
 * allowed keys in tiles of `tile` keys, then o = u / l and LSE = m + ln l.
 */
int oracle_tiled_fwd(const double *Q, const double *K, const double *V, int64_t B, int64_t H,
                     int64_t Nq, int64_t Nk, int64_t d, double scale, int causal, int64_t tile,
                     double *O, double *LSE) {
    if (!Q || !K || !V || !O || !LSE || tile <= 0 || bad_shape(B, H, Nq, Nk, d)) return -1;
    int err = 0;
    #pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)Nk);
        double *vv = (double *)malloc(sizeof(double) * (size_t)(Nk * d));
        if (!s || !vv) {
            #pragma omp atomic write
            err = -2;
        }
        #pragma omp for schedule(static)
        for (int64_t t = 0; t < B * H * Nq; ++t) {
            if (!s || !vv) continue;
            const int64_t bh = t / Nq, i = t % Nq;
            const double *q = Q + t * d, *k = K + bh * Nk * d, *v = V + bh * Nk * d;
            int64_t n = 0; /* gather the allowed keys, in order */
            for (int64_t j = 0; j < Nk; ++j) {
                if (!allowed(i, j, causal)) continue;
                s[n] = scale * dot(q, k + j * d, d);
                memcpy(vv + n * d, v + j * d, sizeof(double) * (size_t)d);
                ++n;
            }
            double m, l;
            oracle_online_row(s, vv, n, d, tile, -1, &m, &l, O + t * d);
            for (int64_t c = 0; c < d; ++c) O[t * d + c] /= l;
            LSE[t] = m + log(l);
        }
        free(s);
        free(vv);
    }
    return err;
}

/*
 * ---- Dropout on the attention probabilities.
 *
 * The pages leave dropout out of the derivation (research-attention, section
 * 01) and ask that training comparisons use the same dropout probability over
 * the same forward and backward range (section 06); they define nothing more.
 * Reading used here: inverted dropout on P.  With keep mask Z (0/1) and
 * keep_scale = 1 / (1 - rate):
 *   P~ = Z * P * keep_scale,  O = P~ V,  LSE unchanged (the softmax itself is
 *   not touched);
 *   dV = P~^T dO,  dP = Z * (dO V^T) * keep_scale,  r_i = sum_j P_ij dP_ij,
 *   dS = P (dP - r),  dQ = scale dS K,  dK = scale dS^T Q.
 *
 * The mask is drawn from a counter-based generator so that the backward can
 * draw it again instead of storing N x N bits: Philox4x32 with 10 rounds,
 * from Salmon, Moraes, Dror and Shaw, "Parallel Random Numbers: As Easy as
 * 1, 2, 3" (SC 2011): a 4 x 32-bit counter, a 2 x 32-bit key; each round
 * multiplies counter words 0 and 2 by fixed constants, keeps both halves of
 * the 64-bit products, and mixes the high halves with the other two words
 * and the key; the key is advanced by fixed Weyl increments between rounds.
 *
 * Element (bh, i, j) (bh = b*H + h, query i, key j) is decided by byte j mod 4
 * (least significant first) of output word i mod 4 of
 * Philox4x32-10(counter = (j div 4, i div 4, bh, 0), key = (seed low 32 bits,
 * seed high 32 bits)); it is dropped when that byte is below t, the rate in
 * 1/256 units (rate realised = t / 256).
 */
static const uint32_t kPhiloxMul0 = 0xD2511F53u, kPhiloxMul1 = 0xCD9E8D57u;
static const uint32_t kPhiloxWeyl0 = 0x9E3779B9u, kPhiloxWeyl1 = 0xBB67AE85u;

void oracle_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
    uint32_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3];
    uint32_t k0 = key[0], k1 = key[1];
    for (int round = 0; round < 10; ++round) {
        if (round > 0) {
            k0 += kPhiloxWeyl0;
            k1 += kPhiloxWeyl1;
        }
        const uint64_t p0 = (uint64_t)kPhiloxMul0 * c0;
        const uint64_t p1 = (uint64_t)kPhiloxMul1 * c2;
        const uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
        const uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
        c0 = hi1 ^ c1 ^ k0;
        c1 = lo1;
        c2 = hi0 ^ c3 ^ k1;
        c3 = lo0;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/*
 * keep[h][i][j] = 1 unless element (bh0 + h, i, j) is dropped at threshold t
 * (0..255), for the B*H heads starting at head index bh0 (bh0 = 0: all heads
 * of a [B,H] problem; bh0 > 0 with B = H = 1: one head of a larger problem).
 */
int oracle_dropout_keep(int64_t B, int64_t H, int64_t Nq, int64_t Nk, int t, uint64_t seed, int64_t bh0,
                        uint8_t *keep) {
    if (!keep || B <= 0 || H <= 0 || Nq <= 0 || Nk <= 0 || t < 0 || t > 255 || bh0 < 0) return -1;
    const uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    #pragma omp parallel for schedule(static)
    for (int64_t h = 0; h < B * H; ++h)
        for (int64_t i = 0; i < Nq; ++i)
            for (int64_t j = 0; j < Nk; ++j) {
                const uint32_t ctr[4] = {(uint32_t)(j / 4), (uint32_t)(i / 4), (uint32_t)(bh0 + h), 0u};
                uint32_t w[4];
                oracle_philox4x32_10(ctr, key, w);
                const uint32_t byte = (w[i % 4] >> (8 * (j % 4))) & 0xffu;
                keep[(h * Nq + i) * Nk + j] = byte >= (uint32_t)t;
            }
    return 0;
}

/* Forward with dropout (see above): O = (Z * P * keep_scale) V, LSE of the undropped softmax. */
int oracle_fwd_dropout(const double *Q, const double *K, const double *V, int64_t B, int64_t H,
                       int64_t Nq, int64_t Nk, int64_t d, double scale, int causal,
                       const uint8_t *keep, double keep_scale, double *O, double *LSE) {
    if (!Q || !K || !V || !keep || !O || !LSE || bad_shape(B, H, Nq, Nk, d)) return -1;
    double *P = (double *)malloc(sizeof(double) * (size_t)(Nq * Nk));
    if (!P) return -2;
    for (int64_t bh = 0; bh < B * H; ++bh) {
        const double *q = Q + bh * Nq * d, *k = K + bh * Nk * d, *v = V + bh * Nk * d;
        const uint8_t *z = keep + bh * Nq * Nk;
        head_probs(q, k, Nq, Nk, d, scale, causal, P, LSE + bh * Nq);
        for (int64_t e = 0; e < Nq * Nk; ++e) P[e] = z[e] ? P[e] * keep_scale : 0.0;
        head_pv(P, v, Nq, Nk, d, O + bh * Nq * d);
    }
    free(P);
    return 0;
}

/* Backward with dropout (see above); O and LSE (of the same dropped forward) when non-NULL. */
int oracle_bwd_dropout(const double *Q, const double *K, const double *V, const double *dO,
                       int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, double scale, int causal,
                       const uint8_t *keep, double keep_scale,
                       double *dQ, double *dK, double *dV, double *O, double *LSE) {
    if (!Q || !K || !V || !dO || !keep || !dQ || !dK || !dV || bad_shape(B, H, Nq, Nk, d)) return -1;
    double *P = (double *)malloc(sizeof(double) * (size_t)(Nq * Nk));
    double *Pd = (double *)malloc(sizeof(double) * (size_t)(Nq * Nk));
    double *dS = (double *)malloc(sizeof(double) * (size_t)(Nq * Nk));
    double *lse = (double *)malloc(sizeof(double) * (size_t)Nq);
    if (!P || !Pd || !dS || !lse) {
        free(P); free(Pd); free(dS); free(lse);
        return -2;
    }
    for (int64_t bh = 0; bh < B * H; ++bh) {
        const double *q = Q + bh * Nq * d, *k = K + bh * Nk * d, *v = V + bh * Nk * d;
        const uint8_t *z = keep + bh * Nq * Nk;
        head_probs(q, k, Nq, Nk, d, scale, causal, P, lse);
        for (int64_t e = 0; e < Nq * Nk; ++e) Pd[e] = z[e] ? P[e] * keep_scale : 0.0;
        if (O) head_pv(Pd, v, Nq, Nk, d, O + bh * Nq * d);
        if (LSE) memcpy(LSE + bh * Nq, lse, sizeof(double) * (size_t)Nq);
        head_grads(q, k, v, dO + bh * Nq * d, Nq, Nk, d, scale, P, Pd, z, keep_scale, dS, dQ + bh * Nq * d,
                   dK + bh * Nk * d, dV + bh * Nk * d);
    }
    free(P); free(Pd); free(dS); free(lse);
    return 0;
}

int oracle_num_threads(void) {
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}
