"""fp64 chunk-parallel evaluation of the Gated DeltaNet-2 recurrence (test helper).

This is an independent route to the same result as the stepwise oracle: it
groups C tokens into a chunk and solves for the chunk's key reads all at
once. The tests use it in both directions: it pins the oracle (brute-force
agreement on small inputs), and it checks the chunk algebra the HIP kernels
are built on before any kernel runs.

Per chunk with entering state S (d_k x d_v), tokens t = 1..L, channel-wise
G_t = sum_{r<=t} log a_r, gamma_t = exp(G_t), ratio_i(t, s) = exp(G_t,i - G_s,i):

  beta_s = b_s * k_s,  u_s = w_s * v_s
  Akk[t,s] = sum_i k_t,i ratio_i(t,s) k_s,i      (s < t)
  Akb[t,s] = sum_i k_t,i ratio_i(t,s) beta_s,i   (s < t)
  Mqk[t,s] = sum_i q_t,i ratio_i(t,s) k_s,i      (s <= t)
  Mqb[t,s] = sum_i q_t,i ratio_i(t,s) beta_s,i   (s <= t)
  (I + Akb) R = (gamma * K) S + Akk U            row t of R is the key read r_t
  O  = (gamma * Q) S + Mqk U - Mqb R
  S' = diag(gamma_L) S + (rho * K)^T U - (rho * beta)^T R,  rho_s = exp(G_L - G_s)

The unrolled step S_t = diag(a_t) S_{t-1} - beta_t r_t^T + k_t u_t^T gives
these directly (substitute and collect the terms of S, U and R).
"""
from __future__ import annotations

import numpy as np


def bf16_round(x):
    """Round to the nearest bfloat16 (ties to even), returned as float64."""
    f = np.asarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    u = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def chunked_head(q, k, v, a, b, w, S0, C: int, anchored=False, operand_round=None):
    """One head: q, k, a, b [T, d_k]; v, w [T, d_v]; S0 [d_k, d_v] or None.

    anchored=False uses the exact per-channel ratio for every (t, s) pair.
    anchored=True (or "start") factors the ratio against the chunk start,
    (k_t gamma_t) . (k_s / gamma_s). anchored="mid" factors it against the
    middle of the chunk, m = C/2 - 1: left operands x_t gamma_t / gamma_m,
    right operands y_s gamma_m / gamma_s, the state term as
    (lam K)(diag(gamma_m) S), and the carry's operands rho_s = gamma_C /
    gamma_s -- the factorisation the HIP prefill uses for d_k = 128.
    operand_round, if given, is applied to every matrix-product operand
    (e.g. bf16_round, as the MFMA operands are rounded).
    """
    rnd = operand_round or (lambda x: x)
    q, k, v, a, b, w = (np.asarray(x, dtype=np.float64) for x in (q, k, v, a, b, w))
    T, dk = k.shape
    dv = v.shape[1]
    S = np.zeros((dk, dv)) if S0 is None else np.array(S0, dtype=np.float64)
    o = np.zeros((T, dv))
    for c0 in range(0, T, C):
        sl = slice(c0, min(c0 + C, T))
        K, Q, A, Bg, V, W = k[sl], q[sl], a[sl], b[sl], v[sl], w[sl]
        L = K.shape[0]
        beta = Bg * K
        U = W * V
        G = np.cumsum(np.log(A), axis=0)
        gam = np.exp(G)
        strict = np.tril(np.ones((L, L)), -1)
        incl = np.tril(np.ones((L, L)), 0)
        if anchored == "mid":
            m = min(C // 2, L) - 1
            lam, mu = np.exp(G - G[m]), np.exp(G[m] - G)
            Kl, Ql, Km, Bm = rnd(lam * K), rnd(lam * Q), rnd(mu * K), rnd(mu * beta)
            Akk = (Kl @ Km.T) * strict
            Akb = (Kl @ Bm.T) * strict
            Mqk = (Ql @ Km.T) * incl
            Mqb = (Ql @ Bm.T) * incl
            Sg = rnd(gam[m][:, None] * S)
            Ur = rnd(U)
            R = np.linalg.solve(np.eye(L) + Akb, Kl @ Sg + Akk @ Ur)
            o[sl] = Ql @ Sg + Mqk @ Ur - Mqb @ rnd(R)
            rho = np.exp(G[-1][None, :] - G)
            S = gam[-1][:, None] * S + rnd(rho * K).T @ Ur - rnd(rho * beta).T @ rnd(R)
            continue
        if anchored:
            inv = np.exp(-G)
            Akk = ((gam * K) @ (inv * K).T) * strict
            Akb = ((gam * K) @ (inv * beta).T) * strict
            Mqk = ((gam * Q) @ (inv * K).T) * incl
            Mqb = ((gam * Q) @ (inv * beta).T) * incl
        else:
            ratio = np.exp(np.minimum(G[:, None, :] - G[None, :, :], 0.0))  # [t, s, i]
            Akk = np.einsum("ti,tsi,si->ts", K, ratio, K) * strict
            Akb = np.einsum("ti,tsi,si->ts", K, ratio, beta) * strict
            Mqk = np.einsum("ti,tsi,si->ts", Q, ratio, K) * incl
            Mqb = np.einsum("ti,tsi,si->ts", Q, ratio, beta) * incl
        R = np.linalg.solve(np.eye(L) + Akb, (gam * K) @ S + Akk @ U)
        o[sl] = (gam * Q) @ S + Mqk @ U - Mqb @ R
        rho = np.exp(G[-1][None, :] - G)
        S = gam[-1][:, None] * S + (rho * K).T @ U - (rho * beta).T @ R
    return o, S


def chunked_forward(q, k, v, a, b, w, S0, C: int, anchored=False, operand_round=None):
    """Full layout: q, k [B,T,H_qk,d_k]; v, w [B,T,H_v,d_v]; a, b [B,T,H_v,d_k]."""
    q, k, v, a, b, w = (np.asarray(x, dtype=np.float64) for x in (q, k, v, a, b, w))
    B, T, Hqk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    G = Hv // Hqk
    o = np.zeros((B, T, Hv, dv))
    ST = np.zeros((B, Hv, dk, dv))
    for n in range(B):
        for h in range(Hv):
            g = h // G
            s0 = None if S0 is None else S0[n, h]
            o[n, :, h], ST[n, h] = chunked_head(q[n, :, g], k[n, :, g], v[n, :, h], a[n, :, h],
                                                b[n, :, h], w[n, :, h], s0, C, anchored, operand_round)
    return o, ST
