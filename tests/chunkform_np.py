"""fp64 numpy mirror of the chunkwise-parallel form (a debugging aid, not the oracle).

The GPU prefill computes the recurrence chunk by chunk.  This mirror states the
same chunk algebra in plain numpy so that (1) the derivation can be checked
against the sequential oracle on the CPU and (2) GPU intermediates can be
compared stage by stage when a kernel misbehaves.

Chunk algebra (one head, a chunk of c tokens entering with state S, G the
running sum of the log-gates inside the chunk, Gamma_r = exp(G_r)):
  unrolling S_r = Diag(Gamma_r) S + sum_{j<=r} Diag(Gamma_r / Gamma_j) k_j u_j^T
  inside u_r = beta_r (v_r - Sbar_r^T k_r) gives the unit lower-triangular system
     (I + A_kk) U = Diag(beta) (V - (K*Gamma) S),
     A_kk[r, j] = beta_r sum_c k_r[c] k_j[c] exp(G_r[c] - G_j[c])   (j < r),
  so with T = (I + A_kk)^-1:  W = T Diag(beta) (K*Gamma),  Ut = T Diag(beta) V,
     U = Ut - W S,
     O = (Q*Gamma) S + A_qk U,   A_qk[r, j] = sum_c q_r[c] k_j[c] exp(G_r[c] - G_j[c]) (j <= r),
     S' = Diag(Gamma_c) S + (K * exp(G_c - G))^T U.
This is the triangular-solve packaging of engineermaxxing "From GPT-2 to Kimi
K3", ch. 04e, with the running per-channel decay products folded through it as
heqinghuang "From GPT2 to Kimi3, Explained", section 11 describes for the gated
rule.
"""
import numpy as np


def chunk_forward_head(q, k, v, g, beta, C, S0=None, return_stages=False):
    """q, k, g: [L, dk]; v: [L, dv]; beta: [L]; returns (O [L, dv], S [dk, dv])."""
    q, k, v, g, beta = (np.asarray(a, dtype=np.float64) for a in (q, k, v, g, beta))
    L, dk = q.shape
    dv = v.shape[1]
    S = np.zeros((dk, dv)) if S0 is None else np.array(S0, dtype=np.float64)
    O = np.zeros((L, dv))
    stages = []
    for s in range(0, L, C):
        e = min(s + C, L)
        Q, K, V, b = q[s:e], k[s:e], v[s:e], beta[s:e]
        G = np.cumsum(g[s:e], axis=0)
        c = e - s
        lower = np.tril(np.ones((c, c), dtype=bool))
        diff = np.where(lower[:, :, None], G[:, None, :] - G[None, :, :], -np.inf)
        D = np.exp(diff)                                   # [r, j, dk], zero above diagonal
        gram_k = np.einsum("rc,jc,rjc->rj", K, K, D)
        A_kk = b[:, None] * np.tril(gram_k, -1)
        A_qk = np.einsum("rc,jc,rjc->rj", Q, K, D)
        T = np.linalg.inv(np.eye(c) + A_kk)
        Gam = np.exp(G)
        W = T @ (b[:, None] * K * Gam)
        Ut = T @ (b[:, None] * V)
        U = Ut - W @ S
        O[s:e] = (Q * Gam) @ S + A_qk @ U
        if return_stages:
            stages.append(dict(G=G, A_kk=A_kk, A_qk=A_qk, T=T, W=W, Ut=Ut, U=U, S_in=S.copy()))
        S = Gam[-1][:, None] * S + (K * np.exp(G[-1] - G)).T @ U
    if return_stages:
        return O, S, stages
    return O, S


def chunk_forward(q, k, v, g, beta, C, cu_seqlens=None, s0=None):
    """Packed layout ([T, H, d]) wrapper; returns (o [T, H, dv], s [N, H, dk, dv])."""
    T, H, dk = q.shape
    dv = v.shape[2]
    cu = np.array([0, T]) if cu_seqlens is None else np.asarray(cu_seqlens)
    N = len(cu) - 1
    o = np.zeros((T, H, dv))
    s = np.zeros((N, H, dk, dv))
    for n in range(N):
        sl = slice(cu[n], cu[n + 1])
        for h in range(H):
            S0 = None if s0 is None else s0[n, h]
            o[sl, h], s[n, h] = chunk_forward_head(q[sl, h], k[sl, h], v[sl, h], g[sl, h],
                                                   beta[sl, h], C, S0)
    return o, s
