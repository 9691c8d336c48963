"""Float64 CPU model of the chunkwise form of the OSDN recurrence.

TEST INFRASTRUCTURE ONLY (see the package docstring).  It exists so that the chunk algebra
the GPU kernels implement is checked against the token recurrence in float64, apart from
any kernel: the tests require it to equal ``oracle.chunk_fwd`` to ~1e-12 at every chunk
size, including chunk = 1 and chunk = T.

The pages state that OSDN keeps DeltaNet's chunkwise WY pipeline with the scaled key K~ in
place of the stored key in the chunk Gram matrix and the intra-chunk scores (OSDN: Improving
Delta Rule with Provable Online Preconditioning in Linear Attention, technical summary,
sections 1, 2.1, 2.2); they give no chunk algebra.  The algebra below is derived here from
the token step  M_t = a_t (I - b_t k~_t k_t^T) M_{t-1} + b_t k~_t v_t^T  (M = S^T).

For one chunk of C rows starting from state M0, let g_r = sum_{s<=r} ln a_s, gam_r = e^{g_r},
and the pseudo-values u_r = b_r (v_r - a_r M_{r-1}^T k_r).  Unrolling the step gives
    M_r = gam_r M0 + sum_{s<=r} (gam_r / gam_s) k~_s u_s^T,
and substituting M_{r-1} into u_r gives the unit lower-triangular system
    (I + A) U = diag(b) (V - diag(gam) K M0),
    A[r,s] = b_r e^{g_r - g_s} <k_r, k~_s>   for s < r, 0 otherwise.
Then, with L the lower triangle including the diagonal,
    O   = diag(gam) Q M0 + (L o (Q K~^T) o G) U,       G[r,s] = e^{g_r - g_s}
    M_C = gam_C M0 + (diag(e^{g_C - g}) K~)^T U .
"""
from __future__ import annotations

from typing import Optional, Tuple

import numpy as np
from scipy.linalg import solve_triangular


def chunk_fwd(q, k, v, beta, d, alpha=None, S0=None, chunk: int = 64
              ) -> Tuple[np.ndarray, np.ndarray]:
    """Same contract as ``oracle.chunk_fwd``; evaluates the chunk algebra above."""
    q, k, v, beta, d = (np.asarray(x, dtype=np.float64) for x in (q, k, v, beta, d))
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    o = np.zeros((B, H, T, dv))
    S_T = np.zeros((B, H, dk, dv))
    for b in range(B):
        for h in range(H):
            M = np.zeros((dk, dv)) if S0 is None else np.array(S0[b, h], dtype=np.float64)
            for c0 in range(0, T, chunk):
                c1 = min(c0 + chunk, T)
                Q, K, V = q[b, h, c0:c1], k[b, h, c0:c1], v[b, h, c0:c1]
                bet = beta[b, h, c0:c1]
                Kt = d[b, h, c0:c1] * K
                if alpha is None:
                    g = np.zeros(c1 - c0)
                else:
                    g = np.cumsum(np.log(np.asarray(alpha[b, h, c0:c1], dtype=np.float64)))
                gam = np.exp(g)
                G = np.exp(g[:, None] - g[None, :])
                n = c1 - c0
                A = np.tril(bet[:, None] * G * (K @ Kt.T), -1)
                rhs = bet[:, None] * (V - gam[:, None] * (K @ M))
                U = solve_triangular(np.eye(n) + A, rhs, lower=True, unit_diagonal=True)
                P = np.tril((Q @ Kt.T) * G)
                o[b, h, c0:c1] = gam[:, None] * (Q @ M) + P @ U
                M = gam[-1] * M + (np.exp(g[-1] - g)[:, None] * Kt).T @ U
            S_T[b, h] = M
    return o, S_T


def precond_scan(k, beta, eta: float, r=None, d1=None, chunk: int = 64
                 ) -> Tuple[np.ndarray, np.ndarray]:
    """Same contract as ``oracle.precond.precond_scan``; evaluates the chunk form of the
    Phase-1 preconditioner recurrence (OSDN summary, sections 2.2 and 2.3), derived here.

    The token step  d_{t+1} = r_t d_t + c_t e_t x_t,  x_t = k_t^2,  c_t = eta b_t / ||k_t||^2
    (0 for a zero key),  e_t = 1 - b_t <d_t, x_t>,  is affine in d.  Over one chunk of rows
    j = 0..C-1 starting from d0, with rho_j = prod_{i<j} r_i and R[j,i] = rho_j / rho_{i+1}:
        d_j = rho_j d0 + sum_{i<j} R[j,i] c_i e_i x_i,
    and substituting d_j into e_j gives the unit lower-triangular system
        (I + L) e = 1 - b . rho . (X d0),   L[j,i] = b_j R[j,i] c_i <x_j, x_i>   (i < j),
    after which  D = rho d0^T + W X  with  W[j,i] = R[j,i] c_i e_i  (i < j), and the state
    carried to the next chunk is  rho_C d0 + sum_i R[C,i] c_i e_i x_i .
    """
    k = np.asarray(k, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)
    B, H, T, dk = k.shape
    out = np.zeros((B, H, T, dk))
    d_next = np.zeros((B, H, dk))
    for b in range(B):
        for h in range(H):
            d0 = np.ones(dk) if d1 is None else np.array(d1[b, h], dtype=np.float64)
            for c0 in range(0, T, chunk):
                c1 = min(c0 + chunk, T)
                n = c1 - c0
                X = k[b, h, c0:c1] ** 2
                nrm = X.sum(axis=1)
                bet = beta[b, h, c0:c1]
                c = np.divide(eta * bet, nrm, out=np.zeros(n), where=nrm > 0)
                rr = np.ones(n) if r is None else np.asarray(r[b, h, c0:c1], dtype=np.float64)
                # R[j, i] = prod_{i < m < j} r_m for rows j = 0..n (row n is the chunk end)
                R = np.zeros((n + 1, n))
                for j in range(n + 1):
                    for i in range(min(j, n)):
                        R[j, i] = np.prod(rr[i + 1:j])
                rho = np.array([np.prod(rr[:j]) for j in range(n + 1)])
                L = np.tril(bet[:, None] * R[:n] * c[None, :] * (X @ X.T), -1)
                rhs = 1.0 - bet * rho[:n] * (X @ d0)
                e = solve_triangular(np.eye(n) + L, rhs, lower=True, unit_diagonal=True)
                W = R * (c * e)[None, :]
                W[:n] = np.tril(W[:n], -1)
                Dall = rho[:, None] * d0[None, :] + W @ X
                out[b, h, c0:c1] = Dall[:n]
                d0 = Dall[n]
            d_next[b, h] = d0
    return out, d_next


def _segment_products(a):
    """Per-feature products of the gates a [n, dk] (n a multiple of 16) inside aligned row
    segments of 1, 2, 4, 8 and 16 rows, built level by level from the sibling segment's total:
    pre[h][r] = prod of a over r's h-segment up to r (inclusive),
    suf[h][r] = prod of a over r's h-segment after r (exclusive),
    tot[h][r] = prod of a over r's whole h-segment."""
    n = a.shape[0]
    pre, suf, tot = {1: a.copy()}, {1: np.ones_like(a)}, {1: a.copy()}
    h = 1
    while h < 16:
        sib = tot[h][np.arange(n) ^ h]  # the sibling h-segment's total
        lower = ((np.arange(n) & h) == 0)[:, None]
        pre[2 * h] = np.where(lower, pre[h], sib * pre[h])
        suf[2 * h] = np.where(lower, suf[h] * sib, suf[h])
        tot[2 * h] = tot[h] * sib
        h *= 2
    return pre, suf, tot


def _anchored_scores(X, Y, a):
    """E[r, s] = sum_f X[r, f] Y[s, f] prod_{s < t <= r} a[t, f] for s <= r (0 above the
    diagonal), as sums of plain matrix products whose operand factors are all products of
    gates, hence at most 1 (no reciprocal of a running product):

    * r and s in different 16-row blocks i > j: anchor at the last row e of block j,
      x_r = prod_{e < t <= r} a_t (the blocks between, then r's block up to r),
      y_s = prod_{s < t <= e} a_t;
    * r and s in one block: at the level h where they first fall into different h-row
      halves of one 2h-row segment, x_r = product over r's half up to r, y_s = product over
      s's half after s; one product per level, its entries outside such pairs dropped;
    * r = s: factor 1."""
    n, dk = X.shape
    pre, suf, tot = _segment_products(a)
    r = np.arange(n)[:, None]
    s = np.arange(n)[None, :]
    E = np.where(r == s, X @ Y.T, 0.0)
    h = 8
    while h >= 1:  # inside 16-row blocks
        up = ((np.arange(n) & h) != 0)[:, None]
        Xh = np.where(up, X * pre[h], 0.0)
        Yh = np.where(~up, Y * suf[h], 0.0)
        keep = ((r ^ s) >> (2 * h).bit_length() - 1 == 0) & ((r & h) != 0) & ((s & h) == 0)
        E += np.where(keep, Xh @ Yh.T, 0.0)
        h //= 2
    nb = n // 16
    blk_tot = tot[16][::16]  # [nb, dk]
    for j in range(nb):  # blocks after j, anchored at the end of block j
        cols = slice(16 * j, 16 * j + 16)
        Yj = Y[cols] * suf[16][cols]
        for i in range(j + 1, nb):
            rows = slice(16 * i, 16 * i + 16)
            cross = np.prod(blk_tot[j + 1:i], axis=0) if i > j + 1 else np.ones(dk)
            E[rows, cols] = (X[rows] * pre[16][rows] * cross) @ Yj.T
    return E


def chunk_fwd_channel(q, k, v, beta, d, alpha_ch, S0=None, chunk: int = 64
                      ) -> Tuple[np.ndarray, np.ndarray]:
    """Chunk form of the recurrence with a channel-wise gate a_t in R^dk (Erase-then-Delta
    Attention, section 2.2, eq. 5) and the OSDN write key k~ = d (.) k; derived here.

    Inside a chunk, unrolling M_r = Diag(a_r) M_{r-1} + k~_r u_r^T gives
        M_r = Diag(G_r) M0 + sum_{s<=r} Diag(rho(s->r)) k~_s u_s^T,
    G_r = prod_{t<=r} a_t (from the chunk start), rho(s->r) = prod_{s<t<=r} a_t, so
        (I + A) U = diag(b) (V - (K o G) M0),   A[r,s] = b_r sum_f k_rf k~_sf rho_f(s->r) (s<r),
        O   = (Q o G) M0 + P U,                 P[r,s] = sum_f q_rf k~_sf rho_f(s->r)   (s<=r),
        M_C = Diag(G_C) M0 + (K~ o rho(.->C))^T U.
    Every factor here is a product of gates, so at most 1.  A and P are formed by
    ``_anchored_scores`` (plain products of gate-scaled operands, no reciprocals), which is
    how the matrix-core path forms them; the chunk is padded to a multiple of 16 rows with
    gates 1 and zero rows, which changes nothing."""
    q, k, v, beta, d, alpha_ch = (np.asarray(x, dtype=np.float64)
                                  for x in (q, k, v, beta, d, alpha_ch))
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    o = np.zeros((B, H, T, dv))
    S_T = np.zeros((B, H, dk, dv))
    for b in range(B):
        for h in range(H):
            M = np.zeros((dk, dv)) if S0 is None else np.array(S0[b, h], dtype=np.float64)
            for c0 in range(0, T, chunk):
                c1 = min(c0 + chunk, T)
                n = c1 - c0
                npad = -(-n // 16) * 16
                pad = lambda x, fill=0.0: np.concatenate(
                    [x, np.full((npad - n,) + x.shape[1:], fill)]) if npad > n else x
                a = pad(alpha_ch[b, h, c0:c1], 1.0)
                Q, K = pad(q[b, h, c0:c1]), pad(k[b, h, c0:c1])
                Kt = pad(d[b, h, c0:c1] * k[b, h, c0:c1])
                V = pad(v[b, h, c0:c1])
                bet = pad(beta[b, h, c0:c1])
                G = np.cumprod(a, axis=0)
                rest = np.concatenate([np.cumprod(a[::-1], axis=0)[::-1][1:], np.ones((1, dk))])
                A = np.tril(bet[:, None] * _anchored_scores(K, Kt, a), -1)
                P = _anchored_scores(Q, Kt, a)
                rhs = bet[:, None] * (V - (K * G) @ M)
                U = solve_triangular(np.eye(npad) + A, rhs, lower=True, unit_diagonal=True)
                o[b, h, c0:c1] = ((Q * G) @ M + P @ U)[:n]
                M = G[-1][:, None] * M + (Kt * rest).T @ U
            S_T[b, h] = M
    return o, S_T


def chunk_bwd(q, k, v, beta, d, alpha=None, S0=None, do=None, dS_T=None, chunk: int = 64):
    """Chunk form of the reverse pass of ``oracle.backward.chunk_bwd`` (same contract and
    outputs), derived here by differentiating the chunk algebra above.  Per chunk, with M0 the
    state at its start, dMC the gradient with respect to the state at its end, w_s =
    e^{g_C - g_s}, L the last row of the chunk, P = lower-inclusive((Q K~^T) o G) and A as above:

        dU  = P^T dO + diag(w) K~ dMC          dR = (I + A)^{-T} dU
        dM0 = gam_L dMC + Q^T diag(gam) dO - K^T diag(gam b) dR
        dP  = lower-inclusive(dO U^T)          dA = -strictly-lower(dR U^T)
        dQ  = diag(gam) dO M0^T + (dP o G) K~
        Gb  = dA o G scaled by b_r (row r)
        dK  = -diag(gam b) dR M0^T + Gb K~
        dK~ = diag(w) U dMC^T + (dP o G)^T Q + Gb^T K
        dV  = diag(b) dR
        db_r = <dR_r, v_r - gam_r (K M0)_r> + sum_{s<r} dA[r,s] (K K~^T)[r,s] G[r,s]
        dg_r = gam_r <dO_r, (Q M0)_r> - b_r gam_r <dR_r, (K M0)_r>
               + sum_s (dP o P)[r,s] - sum_s (dP o P)[s,r]
               + sum_s (dA o A)[r,s] - sum_s (dA o A)[s,r]  - w_r <k~_r, dMC u_r>
               + [r = L] (gam_L <dMC, M0> + sum_s w_s <k~_s, dMC u_s>)
        d ln a_t = sum_{t <= r <= L} dg_r ;  da = d ln a / a
        dd  = dK~ o K ;  dK += dK~ o D
    """
    q, k, v, beta, d = (np.asarray(x, dtype=np.float64) for x in (q, k, v, beta, d))
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    out = dict(dq=np.zeros_like(q), dk=np.zeros_like(k), dv=np.zeros_like(v),
               dbeta=np.zeros_like(beta), dd=np.zeros_like(d),
               dalpha=None if alpha is None else np.zeros((B, H, T)),
               dS0=np.zeros((B, H, dk, dv)))
    for b in range(B):
        for h in range(H):
            M = np.zeros((dk, dv)) if S0 is None else np.array(S0[b, h], dtype=np.float64)
            starts, parts = [], []
            for c0 in range(0, T, chunk):  # forward: the state at every chunk start
                c1 = min(c0 + chunk, T)
                Q, K, V, bt = q[b, h, c0:c1], k[b, h, c0:c1], v[b, h, c0:c1], beta[b, h, c0:c1]
                Kt = d[b, h, c0:c1] * K
                la = np.zeros(c1 - c0) if alpha is None else np.log(np.asarray(alpha[b, h, c0:c1], np.float64))
                g = np.cumsum(la)
                gam = np.exp(g)
                G = np.exp(g[:, None] - g[None, :])
                A = np.tril(bt[:, None] * (K @ Kt.T) * G, -1)
                R = bt[:, None] * (V - gam[:, None] * (K @ M))
                U = solve_triangular(np.eye(c1 - c0) + A, R, lower=True, unit_diagonal=True)
                P = np.tril((Q @ Kt.T) * G)
                w = np.exp(g[-1] - g)
                starts.append(M)
                parts.append((c0, c1, Q, K, V, bt, Kt, g, gam, G, A, U, P, w))
                M = gam[-1] * M + (w[:, None] * Kt).T @ U
            dM = np.zeros((dk, dv)) if dS_T is None else np.array(dS_T[b, h], dtype=np.float64)
            for (c0, c1, Q, K, V, bt, Kt, g, gam, G, A, U, P, w), M0 in zip(parts[::-1], starts[::-1]):
                n = c1 - c0
                dO = np.zeros((n, dv)) if do is None else np.asarray(do[b, h, c0:c1], np.float64)
                KdM = Kt @ dM
                dU = P.T @ dO + w[:, None] * KdM
                dR = solve_triangular(np.eye(n) + A, dU, lower=True, unit_diagonal=True, trans=1)
                dP = np.tril(dO @ U.T)
                dA = -np.tril(dR @ U.T, -1)
                KM0, QM0 = K @ M0, Q @ M0
                dPG = dP * G
                Gb = dA * G * bt[:, None]
                dQ = gam[:, None] * (dO @ M0.T) + dPG @ Kt
                dK = -(gam * bt)[:, None] * (dR @ M0.T) + Gb @ Kt
                dKt = w[:, None] * (U @ dM.T) + dPG.T @ Q + Gb.T @ K
                out["dv"][b, h, c0:c1] = bt[:, None] * dR
                out["dbeta"][b, h, c0:c1] = (np.sum(dR * (V - gam[:, None] * KM0), axis=1)
                                             + np.sum(np.tril(dA * (K @ Kt.T) * G, -1), axis=1))
                EP, EA = dP * P, dA * A
                ew = w * np.sum(KdM * U, axis=1)
                dg = (gam * np.sum(dO * QM0, axis=1) - bt * gam * np.sum(dR * KM0, axis=1)
                      + EP.sum(1) - EP.sum(0) + EA.sum(1) - EA.sum(0) - ew)
                dg[-1] += gam[-1] * np.sum(dM * M0) + ew.sum()
                if alpha is not None:
                    dla = np.cumsum(dg[::-1])[::-1]
                    out["dalpha"][b, h, c0:c1] = dla / np.asarray(alpha[b, h, c0:c1], np.float64)
                out["dq"][b, h, c0:c1] = dQ
                out["dd"][b, h, c0:c1] = dKt * K
                out["dk"][b, h, c0:c1] = dK + dKt * d[b, h, c0:c1]
                dM = gam[-1] * dM + Q.T @ (gam[:, None] * dO) - K.T @ ((gam * bt)[:, None] * dR)
            out["dS0"][b, h] = dM
    return out


def _pair_decays(a):
    """rho[r, s, f] = prod_{s < t <= r} a[t, f] for s <= r (1 on the diagonal, 0 above), by
    running products down each column: exact for gates of any size, zero included."""
    n, dk = a.shape
    rho = np.zeros((n, n, dk))
    for s in range(n):
        run = np.ones(dk)
        rho[s, s] = run
        for r in range(s + 1, n):
            run = run * a[r]
            rho[r, s] = run
    return rho


def chunk_bwd_channel(q, k, v, beta, d, alpha_ch, S0=None, do=None, dS_T=None,
                      chunk: int = 32):
    """Chunk form of the reverse pass with the channel-wise gate (same contract and outputs as
    ``oracle.backward.chunk_bwd`` with ``alpha_ch`` and no scalar decay), derived here by
    differentiating the chunk algebra of ``chunk_fwd_channel``.  Per chunk, with M0 the state at
    its start, dMC the gradient with respect to the state at its end, L its last row,
    G_r = prod_{t<=r} a_t, rho(s->r) = prod_{s<t<=r} a_t, W_s = rho(s->L) (all per feature f),
    K^ = K o G, Q^ = Q o G, K~w = K~ o W, and A, P as in ``chunk_fwd_channel``:

        dU  = P^T dO + K~w dMC                 dR = (I + A)^{-T} dU
        dM0 = Diag(G_L) dMC + Q^T dO - K^T diag(b) dR      (with Q^, K^)
        dP  = lower-inclusive(dO U^T)          dA = -strictly-lower(dR U^T)
        dQ[r,f]  = G_rf (dO M0^T)[r,f] + sum_s dP[r,s] k~_sf rho_f(s->r)
        dK'[r,f] = -b_r G_rf (dR M0^T)[r,f] + b_r sum_s dA[r,s] k~_sf rho_f(s->r)
        dK~[s,f] = W_sf (U dMC^T)[s,f] + sum_r (dP[r,s] q_rf + b_r dA[r,s] k_rf) rho_f(s->r)
        dV  = diag(b) dR
        db_r = <dR_r, v_r - (K^ M0)_r> + sum_s dA[r,s] (A[r,s] / b_r)
        dLg[r,f] = q_rf dQ[r,f] + k_rf dK'[r,f] - k~_rf dK~[r,f]
                   + [r = L] (G_Lf <dMC[f,:], M0[f,:]> + sum_s k~_sf W_sf (U dMC^T)[s,f])
        d ln a_t = sum_{t <= r <= L} dLg[r] ;  da = d ln a / a
        dd  = dK~ o K ;  dK = dK' + dK~ o D

    dLg is the gradient with respect to the running log-gate sums Lg_r = ln G_r, each row's
    taken as its own variable: it collects every place Lg_r enters (the G factors of Q^ and K^,
    both ends of rho, W, and G_L on the carried state).  The gate gradient divides by a, so it is
    defined for gates in (0, 1]."""
    q, k, v, beta, d, alpha_ch = (np.asarray(x, dtype=np.float64)
                                  for x in (q, k, v, beta, d, alpha_ch))
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    out = dict(dq=np.zeros_like(q), dk=np.zeros_like(k), dv=np.zeros_like(v),
               dbeta=np.zeros_like(beta), dd=np.zeros_like(d), dalpha=None,
               dalpha_ch=np.zeros_like(alpha_ch), dS0=np.zeros((B, H, dk, dv)))
    for b in range(B):
        for h in range(H):
            M = np.zeros((dk, dv)) if S0 is None else np.array(S0[b, h], dtype=np.float64)
            starts, parts = [], []
            for c0 in range(0, T, chunk):  # forward: the state at every chunk start
                c1 = min(c0 + chunk, T)
                Q, K, V, bt = q[b, h, c0:c1], k[b, h, c0:c1], v[b, h, c0:c1], beta[b, h, c0:c1]
                a = alpha_ch[b, h, c0:c1]
                Kt = d[b, h, c0:c1] * K
                rho = _pair_decays(a)
                G = np.cumprod(a, axis=0)
                W = rho[-1]  # W[s] = rho(s -> L)
                AS = np.tril(np.einsum("rf,sf,rsf->rs", K, Kt, rho), -1)
                A = bt[:, None] * AS
                P = np.tril(np.einsum("rf,sf,rsf->rs", Q, Kt, rho))
                R = bt[:, None] * (V - (K * G) @ M)
                U = solve_triangular(np.eye(c1 - c0) + A, R, lower=True, unit_diagonal=True)
                starts.append(M)
                parts.append((c0, c1, Q, K, V, bt, a, Kt, rho, G, W, AS, A, U, P))
                M = G[-1][:, None] * M + (Kt * W).T @ U
            dM = np.zeros((dk, dv)) if dS_T is None else np.array(dS_T[b, h], dtype=np.float64)
            for (c0, c1, Q, K, V, bt, a, Kt, rho, G, W, AS, A, U, P), M0 in zip(parts[::-1],
                                                                                 starts[::-1]):
                n = c1 - c0
                dO = np.zeros((n, dv)) if do is None else np.asarray(do[b, h, c0:c1], np.float64)
                UdM = U @ dM.T  # [n, dk]
                dU = P.T @ dO + (Kt * W) @ dM
                dR = solve_triangular(np.eye(n) + A, dU, lower=True, unit_diagonal=True, trans=1)
                dP = np.tril(dO @ U.T)
                dA = -np.tril(dR @ U.T, -1)
                dQ = G * (dO @ M0.T) + np.einsum("rs,sf,rsf->rf", dP, Kt, rho)
                dKp = bt[:, None] * (-G * (dR @ M0.T) + np.einsum("rs,sf,rsf->rf", dA, Kt, rho))
                dKt = (W * UdM + np.einsum("rs,rf,rsf->sf", dP, Q, rho)
                       + np.einsum("rs,rf,rsf->sf", bt[:, None] * dA, K, rho))
                out["dv"][b, h, c0:c1] = bt[:, None] * dR
                out["dbeta"][b, h, c0:c1] = (np.sum(dR * (V - (K * G) @ M0), axis=1)
                                             + np.sum(dA * AS, axis=1))
                dLg = Q * dQ + K * dKp - Kt * dKt
                dLg[-1] += G[-1] * np.sum(dM * M0, axis=1) + np.sum(Kt * W * UdM, axis=0)
                dla = np.cumsum(dLg[::-1], axis=0)[::-1]
                out["dalpha_ch"][b, h, c0:c1] = dla / a
                out["dq"][b, h, c0:c1] = dQ
                out["dd"][b, h, c0:c1] = dKt * K
                out["dk"][b, h, c0:c1] = dKp + dKt * d[b, h, c0:c1]
                dM = G[-1][:, None] * dM + (Q * G).T @ dO - (K * G).T @ (bt[:, None] * dR)
            out["dS0"][b, h] = dM
    return out
