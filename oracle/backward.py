"""Backward pass of the Swimba mixer in fp64 (oracle).

TEST INFRASTRUCTURE: only tests, the smoke check and the benchmark's CPU
baseline use this module. It imports numpy and the base oracle, nothing from
the HIP path.

The pages fine-tune Swimba (papernotes.org notes, Experiments: SFT of the
converted model), which needs the gradients of a loss through the mixer.
Readings (argued in the design notes of the repository): the loss is any
scalar l(y, h_T); given dy = dl/dy and dh_T = dl/dh_T this module returns
the gradients with respect to u, W_r, W_exp, a and h_init. The top-k set K_t
is piecewise constant in the logits, so it has no gradient; the weights
w_{t,j} = pi_{t,K_t[j]} do, through the softmax over all experts.

Every function is the chain rule written out for one forward step of the
base oracle (oracle/swimba.py), in reverse order:
  recurrence:  h_t = a h_{t-1} + sum_j B_hat_j X_j^T,  y_t = C~_t^T h_t
     dh_t accumulates C~_t dy_t^T and a dh_{t+1};
     dX_j = dh_t^T B_hat_j,  dB_hat_j = dh_t X_j (summed over a group's heads),
     dC~_t = h_t dy_t (summed over a group's heads),  da = sum_t <dh_t, h_{t-1}>.
  mix:         B_hat_j = w_j B_j,  C~ = sum_j w_j C_j
  projection:  z_j = W^(e_j) u  (rows X | B | C)
  router:      w_j = softmax(W_r u)[e_j]
"""
from __future__ import annotations

import numpy as np

from oracle import swimba as osw


def recurrence_backward(B_hat, X, C_mix, a, h_init, dy, dh_final, batch, seqlen):
    """Gradients of the single-trajectory recurrence, one token at a time in
    reverse ([notes] Method, key design 1, state and readout equations).

    B_hat [M,k,G,N], X [M,k,H,P], C_mix [M,G,N], a [H], h_init [Bt,H,N,P] or
    None, dy [M,H,P] (or [Bt,T,H,P]), dh_final [Bt,H,N,P] or None.
    Returns dB_hat, dX, dC_mix, da [H], dh_init [Bt,H,N,P].
    """
    M, k, G, N = B_hat.shape
    H = a.shape[0]
    P = X.shape[-1]
    grp = np.arange(H) // (H // G)
    Bh = np.asarray(B_hat, np.float64).reshape(batch, seqlen, k, G, N)
    Xh = np.asarray(X, np.float64).reshape(batch, seqlen, k, H, P)
    Ch = np.asarray(C_mix, np.float64).reshape(batch, seqlen, G, N)
    dyh = np.asarray(dy, np.float64).reshape(batch, seqlen, H, P)
    av = np.asarray(a, np.float64)
    # forward states h_t (t = -1 .. T-1)
    hs = np.zeros((seqlen + 1, batch, H, N, P))
    if h_init is not None:
        hs[0] = np.asarray(h_init, np.float64)
    for t in range(seqlen):
        U = np.einsum("bjhn,bjhp->bhnp", Bh[:, t][:, :, grp, :], Xh[:, t])
        hs[t + 1] = av[None, :, None, None] * hs[t] + U
    dB = np.zeros((batch, seqlen, k, G, N))
    dX = np.zeros((batch, seqlen, k, H, P))
    dC = np.zeros((batch, seqlen, G, N))
    da = np.zeros(H)
    dh = np.zeros((batch, H, N, P)) if dh_final is None else np.array(dh_final, np.float64)
    for t in range(seqlen - 1, -1, -1):
        c = Ch[:, t][:, grp, :]                                      # [Bt,H,N]
        dh = dh + np.einsum("bhn,bhp->bhnp", c, dyh[:, t])            # y_t = C~_t^T h_t
        ht = hs[t + 1]
        dCh = np.einsum("bhnp,bhp->bhn", ht, dyh[:, t])              # per head
        for g in range(G):
            dC[:, t, g] += dCh[:, grp == g].sum(axis=1)
        # h_t = a h_{t-1} + sum_j B_hat_j X_j^T
        dX[:, t] = np.einsum("bhnp,bjhn->bjhp", dh, Bh[:, t][:, :, grp, :])
        dBh = np.einsum("bhnp,bjhp->bjhn", dh, Xh[:, t])              # [Bt,k,H,N]
        for g in range(G):
            dB[:, t, :, g] += dBh[:, :, grp == g].sum(axis=2)
        da += np.einsum("bhnp,bhnp->h", dh, hs[t])
        dh = av[None, :, None, None] * dh
    return (dB.reshape(M, k, G, N), dX.reshape(M, k, H, P), dC.reshape(M, G, N), da, dh)


def mix_backward(streams: osw.Streams, w, dB_hat, dC_mix):
    """Gradients of the parameter-space mix ([notes] Method, key design 1,
    mixing equation: B_hat_j = w_j B_j, C~ = sum_j w_j C_j).
    Returns dB [M,k,G,N], dC [M,k,G,N] (of the per-slot expert streams) and
    dw [M,k]."""
    w = np.asarray(w, np.float64)
    dB = w[:, :, None, None] * dB_hat
    dC = w[:, :, None, None] * np.asarray(dC_mix, np.float64)[:, None]
    dw = (np.einsum("mkgn,mkgn->mk", streams.B, dB_hat)
          + np.einsum("mkgn,mgn->mk", streams.C, dC_mix))
    return dB, dC, dw


def project_backward(u, w_experts, idx, dX, dB, dC):
    """Gradients of the expert projections z_j = W^(e_j) u ([notes] Method,
    key design 1: expert-specific linear projections; rows X | B | C).
    dX [M,k,H,P], dB/dC [M,k,G,N]. Returns du [M,D] and dW [E,W,D]."""
    u = np.asarray(u, np.float64)
    M, k = idx.shape
    dz = np.concatenate([dX.reshape(M, k, -1), dB.reshape(M, k, -1), dC.reshape(M, k, -1)],
                        axis=2)                                      # [M,k,W]
    E = w_experts.shape[0]
    dW = np.zeros(w_experts.shape)
    du = np.zeros_like(u)
    for e in range(E):
        rows, slots = np.nonzero(idx == e)
        if rows.size:
            g = dz[rows, slots]                                      # [n, W]
            dW[e] = g.T @ u[rows]
            du_e = g @ np.asarray(w_experts[e], np.float64)
            np.add.at(du, rows, du_e)
    return du, dW


def route_backward(u, w_router, routing: osw.Routing, dw):
    """Gradients through w_j = pi[e_j], pi = softmax(g), g = W_r u ([notes]
    Method, key design 1; the top-k set itself is piecewise constant).
    Returns du [M,D], dW_r [E,D] and dg [M,E]."""
    u = np.asarray(u, np.float64)
    pi = routing.pi
    dpi = np.zeros_like(pi)
    np.add.at(dpi, (np.arange(pi.shape[0])[:, None], routing.idx), dw)
    dg = pi * (dpi - np.sum(pi * dpi, axis=1, keepdims=True))
    return dg @ np.asarray(w_router, np.float64), dg.T @ u, dg


def forward_backward(u, w_router, w_experts, a, h_init, dy, dh_final, *, nheads, headdim,
                     ngroups, dstate, top_k, routing=None):
    """The whole backward pass: gradients of l(y, h_T) with respect to u,
    W_r, W_exp, a and h_init, given dy [Bt,T,H,P] and dh_T [Bt,H,N,P]."""
    Bt, T, D = u.shape
    uf = u.reshape(Bt * T, D)
    r = routing if routing is not None else osw.route(uf, w_router, top_k)
    s = osw.expert_streams(uf, w_experts, r.idx, nheads, headdim, ngroups, dstate)
    B_hat, X, C_mix = osw.mix_streams(s, r.w)
    dB_hat, dX, dC_mix, da, dh0 = recurrence_backward(B_hat, X, C_mix, a, h_init, dy, dh_final,
                                                      Bt, T)
    dB, dC, dw = mix_backward(s, r.w, dB_hat, dC_mix)
    du_p, dW = project_backward(uf, w_experts, r.idx, dX, dB, dC)
    du_r, dWr, dg = route_backward(uf, w_router, r, dw)
    return {"du": (du_p + du_r).reshape(Bt, T, D), "dW_router": dWr, "dW_experts": dW,
            "da": da, "dh_init": dh0, "dB_hat": dB_hat, "dX": dX, "dC_mix": dC_mix, "dw": dw,
            "dg": dg, "routing": r}
