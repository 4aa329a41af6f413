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


def chunk_backward_head(q, k, v, g, beta, C, d_o, S0=None, dS_final=None):
    """Gradients through the chunk algebra above, chunk by chunk (fp64 mirror of
    the GPU backward).  Per chunk, with S the incoming state, S' the outgoing one
    and dS' its cotangent (from the later chunks):

      reverse state pass   dU  = A_qk^T dO + Kd dS'
                           dS  = (Q*Gam)^T dO + Diag(Gam_c) dS' - W^T dU
      solve                U = (I + A_kk)^-1 R with R = Diag(beta)(V - (K*Gam) S), so
                           dR = T^T dU,  dA_kk = -dR U^T (strictly lower)
      R                    dV = Diag(beta) dR,  Z = dR S^T,  d(K*Gam) = -Diag(beta) Z,
                           dbeta += rowsum(dR * V) - rowsum((K*Gam) * Z)
      A_kk = Diag(beta) M  dbeta += rowsum(dA_kk * M),  dM = Diag(beta) dA_kk
      A_qk, M (decayed)    dA_qk = tril(dO U^T); each decayed product
                           X[r, j] = sum_c a_r[c] b_j[c] exp(G_r[c] - G_j[c]) sends
                           dX[r, j] b_j exp(G_r - G_j) to a_r, dX[r, j] a_r exp(..) to b_j,
                           and +a_r * (that) to dG_r, -b_j * (..) to dG_j
      O, S' (state side)   d(Q*Gam) = dO S^T, dKd = U dS'^T, dGam_c = rowsum(dS' * S)
      gates                G = cumsum(g), so dg = reverse cumsum of dG
    Returns dq, dk, dv, dg [L, d], dbeta [L], dS0 [dk, dv].
    """
    q, k, v, g, beta, d_o = (np.asarray(a, dtype=np.float64) for a in (q, k, v, g, beta, d_o))
    L, dk = q.shape
    dv = v.shape[1]
    S = np.zeros((dk, dv)) if S0 is None else np.array(S0, dtype=np.float64)
    starts = list(range(0, L, C))
    S_in = []
    for s in starts:   # forward state pass: the state entering every chunk
        S_in.append(S.copy())
        e = min(s + C, L)
        _, S = chunk_forward_head(q[s:e], k[s:e], v[s:e], g[s:e], beta[s:e], C, S)
    dq, dk_, dv_, dg = (np.zeros_like(a) for a in (q, k, v, g))
    db = np.zeros(L)
    dS = np.zeros((dk, dv)) if dS_final is None else np.array(dS_final, dtype=np.float64)
    for ci in reversed(range(len(starts))):
        s = starts[ci]
        e = min(s + C, L)
        Q, K, V, b, dO, Sc = q[s:e], k[s:e], v[s:e], beta[s:e], d_o[s:e], S_in[ci]
        G = np.cumsum(g[s:e], axis=0)
        c = e - s
        lower = np.tril(np.ones((c, c), dtype=bool))
        strict = np.tril(np.ones((c, c), dtype=bool), -1)
        E = np.exp(np.where(lower[:, :, None], G[:, None, :] - G[None, :, :], -np.inf))
        M = np.where(strict, np.einsum("rc,jc,rjc->rj", K, K, E), 0.0)
        A_qk = np.where(lower, np.einsum("rc,jc,rjc->rj", Q, K, E), 0.0)
        T = np.linalg.inv(np.eye(c) + b[:, None] * M)
        Gam = np.exp(G)
        Kg = K * Gam
        U = T @ (b[:, None] * (V - Kg @ Sc))
        Kd = K * np.exp(G[-1] - G)
        # reverse state pass
        dU = A_qk.T @ dO + Kd @ dS
        dS_in = (Q * Gam).T @ dO + Gam[-1][:, None] * dS - (T @ (b[:, None] * Kg)).T @ dU
        # gradients inside the chunk
        dR = T.T @ dU
        dA_kk = np.where(strict, -dR @ U.T, 0.0)
        Z = dR @ Sc.T
        dv_[s:e] = b[:, None] * dR
        db[s:e] = (dR * V).sum(1) - (Kg * Z).sum(1) + (dA_kk * M).sum(1)
        dM = b[:, None] * dA_kk
        dA_qk = np.where(lower, dO @ U.T, 0.0)
        dQg = dO @ Sc.T
        dKg = -b[:, None] * Z
        dKd = U @ dS.T
        dGc = (dS * Sc).sum(1) * Gam[-1]
        dQ = dQg * Gam
        dK = dKg * Gam + dKd * np.exp(G[-1] - G)
        dG = dQg * Q * Gam + dKg * K * Gam - dKd * Kd
        dG[-1] += (dKd * Kd).sum(0) + dGc
        # decayed products: A_qk (a = q, b = k) and M (a = k, b = k)
        for dX, A_side in ((dA_qk, Q), (dM, K)):
            row = np.einsum("rj,jc,rjc->rc", dX, K, E)     # to a_r
            col = np.einsum("rj,rc,rjc->jc", dX, A_side, E)  # to b_j = k_j
            if A_side is Q:
                dQ += row
            else:
                dK += row
            dK += col
            dG += A_side * row - K * col
        dq[s:e], dk_[s:e] = dQ, dK
        dg[s:e] = np.cumsum(dG[::-1], axis=0)[::-1]
        dS = dS_in
    return dq, dk_, dv_, dg, db, dS
