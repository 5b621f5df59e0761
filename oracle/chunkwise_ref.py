"""fp64 chunkwise (WY) form of the gated delta rule / DeltaProduct forward.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).  The tests use this
module to pin the token recurrences of the oracle by brute force: a different
algorithm that must reach the same numbers to rounding.  It is also the plain
statement of the chunkwise algorithm of the msj19 "gated_deltaproduct" test.py
page, step by step:

1. chunk-local inclusive cumsum of the log-decay (``chunk_local_cumsum`` as
   used by every kernel of that page);
2. the intra-chunk matrix A_g of ``gated_chunk_scaled_dot_kkt_fwd_kernel``:
   strictly lower over tokens, beta on the row, the step mask M[a, b] on the
   sub-key product, and the decay exp(G_t - G_s);
3. T = (I + A_g)^-1 from 16-row diagonal blocks (``solve_tril_16x16_kernel``:
   forward substitution) and block merges (``merge_16x16_to_32x32_inverse``,
   ``merge_16x16_to_64x64_inverse``).  The merges are written as the exact
   block inverse: T_ij = -T_ii * sum_{j<=m<i} A_im T_mj.  (The 64x64 merge as
   printed on the page uses T_11 where T_22 and T_33 belong; that is not a
   block inverse, and this module does not reproduce it.)
4. ``gated_fwd_recompute_w_u_kernel`` and ``preprocess_qkw``: the page forms
   W from the undecayed (I + A)^-1 applied to diag(beta) E_hat and then scales
   row t by exp(G_t).  Since diag(e^G) (I + A)^-1 = (I + A_g)^-1 diag(e^G),
   that is W = T diag(beta e^G) E_hat, the form used here; U = T diag(beta) V
   with V repeated per step;
5. ``gated_chunk_delta_rule_fwd_kernel_h``: V_new = U - W S, then
   S <- exp(G_last) S + sum_b E_b (K_b * exp(G_last - G))^T V_new[:, b],
   once per chunk;
6. ``gated_chunk_linear_attn_fwd_kernel_o``: per sub-key,
   o = scale*(exp(G) Q_b S_b + tril(Q_b K_b^T * exp(G_t - G_s)) V_new[:, b]),
   summed over the sub-keys.

Virtual rows j = t*r + a (token-major) index the r steps of each token.
"""
from __future__ import annotations

import math

import numpy as np


def unit_lower_inverse_blocked(M: np.ndarray, block: int = 16) -> np.ndarray:
    """Inverse of a unit lower-triangular matrix M, by diagonal blocks of
    ``block`` rows (forward substitution) and then block-row merges."""
    n = M.shape[0]
    nb = math.ceil(n / block)
    Tm = np.zeros_like(M)
    sl = [slice(i * block, min((i + 1) * block, n)) for i in range(nb)]
    for ib in range(nb):
        Dm = M[sl[ib], sl[ib]]
        m = Dm.shape[0]
        Ti = np.eye(m)
        for i in range(m):
            for c in range(i):
                Ti[i, c] = -sum(Dm[i, j] * Ti[j, c] for j in range(c, i))
        Tm[sl[ib], sl[ib]] = Ti
    for i in range(1, nb):
        for j in range(i):
            acc = np.zeros((Tm[sl[i], sl[j]]).shape)
            for m in range(j, i):
                acc += M[sl[i], sl[m]] @ Tm[sl[m], sl[j]]
            Tm[sl[i], sl[j]] = -Tm[sl[i], sl[i]] @ acc
    return Tm


def chunkwise_forward(q, k, v, beta, g, mask, chunk, scale=1.0, h0=None, block=16):
    """Chunkwise forward.  q,k (B,T,H,r*dk); v (B,T,H,Dv); beta (B,T,H,r);
    g (B,T,H); mask (r,r).  Returns (o (B,T,H,Dv), hT (B,H,r*dk,Dv)) fp64."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    beta = np.asarray(beta, np.float64)
    g = np.asarray(g, np.float64)
    mask = np.asarray(mask, np.float64)
    B, T, H, K = q.shape
    r = mask.shape[0]
    dk = K // r
    Dv = v.shape[-1]
    o = np.zeros((B, T, H, Dv))
    hT = np.zeros((B, H, K, Dv))
    for b in range(B):
        for h in range(H):
            S = np.zeros((K, Dv)) if h0 is None else np.array(h0[b, h], np.float64)
            for c0 in range(0, T, chunk):
                L = min(chunk, T - c0)
                toks = np.arange(L)
                G = np.cumsum(g[b, c0:c0 + L, h])
                NR = L * r
                E = np.zeros((NR, K))      # erase keys, sum_b M[a,b] E_b k_b
                Wk = np.zeros((NR, K))     # write keys, E_a k_a
                bet = np.zeros(NR)
                tok = np.zeros(NR, dtype=np.int64)
                for t in toks:
                    for a in range(r):
                        j = t * r + a
                        for bb in range(r):
                            E[j, bb * dk:(bb + 1) * dk] = mask[a, bb] * k[b, c0 + t, h, bb * dk:(bb + 1) * dk]
                        Wk[j, a * dk:(a + 1) * dk] = k[b, c0 + t, h, a * dk:(a + 1) * dk]
                        bet[j] = beta[b, c0 + t, h, a]
                        tok[j] = t
                Gv = G[tok]
                lower = tok[:, None] > tok[None, :]
                A = np.where(lower, bet[:, None] * (E @ Wk.T) * np.exp(Gv[:, None] - Gv[None, :]), 0.0)
                Tm = unit_lower_inverse_blocked(np.eye(NR) + A, block)
                W = Tm @ ((bet * np.exp(Gv))[:, None] * E)
                U = Tm @ (bet[:, None] * v[b, c0 + tok, h])
                Vnew = U - W @ S
                Qc = q[b, c0:c0 + L, h]
                QK = Qc @ Wk.T                                # (L, NR): q_t . w_j
                incl = toks[:, None] >= tok[None, :]
                P = np.where(incl, QK * np.exp(G[:, None] - Gv[None, :]), 0.0)
                o[b, c0:c0 + L, h] = scale * (np.exp(G)[:, None] * (Qc @ S) + P @ Vnew)
                S = math.exp(G[-1]) * S + Wk.T @ (np.exp(G[-1] - Gv)[:, None] * Vnew)
            hT[b, h] = S
    return o, hT
