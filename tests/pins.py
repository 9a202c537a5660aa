"""Independent formulations used to pin the oracle.

Each function here computes something the pages (or plain mathematics) fix,
in a form other than the oracle's per-token recurrence: a quadratic
(attention-like) closed form, separated per-expert trajectories, a chunked
solve, a dense brute force with explicit powers, the stability bound. None
of them calls the oracle.
"""
from __future__ import annotations

import numpy as np


def dense_streams(u, w_experts, H, P, G, N):
    """All experts evaluated on every token with explicit loops over experts.

    u [M, D] -> X [M, E, H, P], B [M, E, G, N], C [M, E, G, N]."""
    u = np.asarray(u, dtype=np.float64)
    E = w_experts.shape[0]
    HP, GN = H * P, G * N
    out = np.stack([u @ np.asarray(w_experts[e], dtype=np.float64).T for e in range(E)], axis=1)
    return (out[..., :HP].reshape(-1, E, H, P), out[..., HP:HP + GN].reshape(-1, E, G, N),
            out[..., HP + GN:].reshape(-1, E, G, N))


def topk_mask_bruteforce(logits, k):
    """0/1 selection matrix and rank list from a full Python sort of each row
    (key: larger logit first, then smaller index)."""
    M, E = logits.shape
    mask = np.zeros((M, E))
    ranks = np.zeros((M, k), dtype=np.int64)
    for m in range(M):
        order = sorted(range(E), key=lambda e: (-logits[m, e], e))
        ranks[m] = order[:k]
        mask[m, order[:k]] = 1.0
    return mask, ranks


def softmax_rows(g):
    g = np.asarray(g, dtype=np.float64)
    out = np.empty_like(g)
    for m in range(g.shape[0]):
        ex = [np.exp(v - max(g[m])) for v in g[m]]
        s = sum(ex)
        out[m] = [v / s for v in ex]
    return out


def brute_force(u, w_router, w_experts, a, h_init, H, P, G, N, k):
    """Whole layer on a short sequence: dense experts, masked mix, and the
    unrolled solution y_t = C~_t^T (a^{t+1} h_init + sum_{s<=t} a^{t-s} U~_s)
    with every injection U~_s formed explicitly. u [Bt, T, D]."""
    Bt, T, D = u.shape
    uf = u.reshape(Bt * T, D).astype(np.float64)
    g = uf @ np.asarray(w_router, dtype=np.float64).T
    pi = softmax_rows(g)
    mask, _ = topk_mask_bruteforce(g, k)
    X, B, C = dense_streams(uf, w_experts, H, P, G, N)
    E = w_router.shape[0]
    y = np.zeros((Bt, T, H, P))
    hT = np.zeros((Bt, H, N, P))
    for b in range(Bt):
        for h in range(H):
            gi = h // (H // G)
            U = []
            Cm = []
            for t in range(T):
                m = b * T + t
                Us = np.zeros((N, P))
                cs = np.zeros(N)
                for e in range(E):
                    wt = pi[m, e] * mask[m, e]
                    Us += wt * np.outer(B[m, e, gi], X[m, e, h])
                    cs += wt * C[m, e, gi]
                U.append(Us)
                Cm.append(cs)
            h0 = np.zeros((N, P)) if h_init is None else np.asarray(h_init, dtype=np.float64)[b, h]
            ah = float(a[h])
            for t in range(T):
                st = ah ** (t + 1) * h0
                for s in range(t + 1):
                    st = st + ah ** (t - s) * U[s]
                y[b, t, h] = Cm[t] @ st
                if t == T - 1:
                    hT[b, h] = st
    return y, hT


def quadratic_form_ssm(Bm, Cm, X, a, h0):
    """Textbook closed form of a scalar-decay SSM for one head:
    y = (L_a o (C B^T)) X + diag(a^{t+1}) C h0 with L_a[t,s] = a^{t-s} [s <= t].
    Bm, Cm [T, N]; X [T, P]; h0 [N, P] or None."""
    T = Bm.shape[0]
    t = np.arange(T)
    L = np.where(t[:, None] >= t[None, :], float(a) ** (t[:, None] - t[None, :]).clip(min=0), 0.0)
    y = (L * (Cm @ Bm.T)) @ X
    if h0 is not None:
        y = y + (float(a) ** (t + 1))[:, None] * (Cm @ h0)
    return y


def chunked_solve(B_hat, X, C_mix, a, h_init, Bt, T, L):
    """SSD-style chunked solve in fp64: intra-chunk quadratic form, chunk end
    states, a sequential pass over chunk states, and the inter-chunk readout.
    B_hat [M,k,G,N]; X [M,k,H,P]; C_mix [M,G,N]."""
    M, k, G, N = B_hat.shape
    H, P = X.shape[2], X.shape[3]
    Bh = B_hat.reshape(Bt, T, k, G, N)
    Xh = X.reshape(Bt, T, k, H, P)
    Ch = C_mix.reshape(Bt, T, G, N)
    y = np.zeros((Bt, T, H, P))
    hT = np.zeros((Bt, H, N, P))
    for b in range(Bt):
        for h in range(H):
            gi = h // (H // G)
            ah = float(a[h])
            Hprev = np.zeros((N, P)) if h_init is None else np.asarray(h_init, np.float64)[b, h].copy()
            for c0 in range(0, T, L):
                c1 = min(c0 + L, T)
                Lc = c1 - c0
                # k-concatenated keys: rows (s, j)
                Bk = Bh[b, c0:c1, :, gi].reshape(Lc * k, N)
                Xk = Xh[b, c0:c1, :, h].reshape(Lc * k, P)
                s_of = np.repeat(np.arange(Lc), k)
                tt = np.arange(Lc)
                Cc = Ch[b, c0:c1, gi]
                dec = np.where(tt[:, None] >= s_of[None, :],
                               ah ** (tt[:, None] - s_of[None, :]).clip(min=0), 0.0)
                y_intra = (dec * (Cc @ Bk.T)) @ Xk
                y_inter = (ah ** (tt + 1))[:, None] * (Cc @ Hprev)
                y[b, c0:c1, h] = y_intra + y_inter
                S = (Bk * (ah ** (Lc - 1 - s_of))[:, None]).T @ Xk
                Hprev = ah ** Lc * Hprev + S
            hT[b, h] = Hprev
    return y, hT


def separated_trajectories(u, w_router, w_experts, a, h_init, H, P, G, N, k, weighted=True):
    """One state per expert, all run every step (MoE of separated SSMs).

    weighted=True: h^(e)_t = a h^(e)_{t-1} + [e in K_t] pi_{t,e} B^(e) X^(e)^T,
      with h_init put in trajectory 0 (the sum over e then starts at h_init).
    weighted=False: the classic separated SSM, h^(e)_t = a h^(e)_{t-1} +
      B^(e) X^(e)^T, every trajectory started from h_init.
    Returns per-expert states over time [Bt, T, E, H, N, P], the routing
    weights pi [M, E], the mask [M, E] and the per-expert C [M, E, G, N]."""
    Bt, T, D = u.shape
    uf = u.reshape(Bt * T, D).astype(np.float64)
    g = uf @ np.asarray(w_router, dtype=np.float64).T
    pi = softmax_rows(g)
    mask, _ = topk_mask_bruteforce(g, k)
    X, B, C = dense_streams(uf, w_experts, H, P, G, N)
    E = w_router.shape[0]
    grp = np.arange(H) // (H // G)
    hs = np.zeros((Bt, T, E, H, N, P))
    for b in range(Bt):
        cur = np.zeros((E, H, N, P))
        if h_init is not None:
            if weighted:
                cur[0] = h_init[b]
            else:
                cur[:] = h_init[b][None]
        for t in range(T):
            m = b * T + t
            for e in range(E):
                wt = pi[m, e] * mask[m, e] if weighted else 1.0
                inj = np.einsum("hn,hp->hnp", B[m, e][grp], X[m, e])
                cur[e] = np.asarray(a, np.float64)[:, None, None] * cur[e] + wt * inj
            hs[b, t] = cur
    return hs, pi, mask, C
