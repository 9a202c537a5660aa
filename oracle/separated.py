"""MoE over separated SSMs, the design Swimba is compared against, in fp64.

TEST INFRASTRUCTURE: only tests, the smoke check and the benchmark's CPU
baseline use this module. It imports numpy and the oracle's own router and
projections, nothing from the HIP path.

[notes] Research background and motivation: the "MoE over separated SSMs"
keeps one state trajectory per expert and advances every expert's recursion
at every step, so state memory and the recurrence's work grow with the
number of experts; [gist-en] Technical Summary 2, "MoE of Separated SSMs"
(independent state trajectories per expert); [notes] Method, key design 2,
Theorem 3.4: the separated output is the routing-weighted sum of the
experts' readouts of their own states, equal to the mixed output under
static routing with one shared readout, and within C * sum_e pi_e
||h^(e) - h|| of it otherwise.

Reading adopted (the pages give no equations for it beyond Theorem 3.4):
  * Every expert e has its own state h^(e) [H, N, P] with the shared
    transition a_h, advanced at every step:
        h^(e)_t = a_h h^(e)_{t-1} + [e in K_t] B^(e)_t X^(e)_t^T
    (an expert outside the token's top-k set injects nothing; its state
    still decays).
  * y_t = sum_{e in K_t} pi_{t,e} C^(e)_t^T h^(e)_t, pi the softmax over all
    E experts (as in the Swimba router), not renormalised.
  * h^(e)_{-1} = h_init[:, e] (zero when absent).
With k = E and static routing these make Theorem 3.4's equality hold; with
k = E = 1 the layer is a single SSM, as Swimba's is.

Pins (tests/test_oracle_separated.py): Theorem 3.4 equality against the
Swimba oracle under static routing with a shared readout; Theorem 3.4's bound
under dynamic routing; k = E = 1 against the textbook quadratic form; dense
k = E against the independent per-expert formulation in tests/pins.py;
brute force with explicit powers on T <= 8 for k < E; an expert never
selected keeps a^t h_init.
"""
from __future__ import annotations

import numpy as np

from . import swimba as osw


def separated_recurrence(B, X, C, mask, pi, a, h_init, batch, seqlen, heads=None):
    """E separated trajectories, one token at a time.

    B [M, E, G, N], X [M, E, Hs, P], C [M, E, G, N]: every expert's streams
    (zeros where the expert is not selected; only selected ones are read);
    mask [M, E] 0/1 selection; pi [M, E] routing probabilities; a [H] over
    all heads; h_init [Bt, E, H, N, P] or None. Returns y [Bt, T, Hs, P] and
    the final states [Bt, E, Hs, N, P].
    """
    M, E, G, N = B.shape
    H = a.shape[0]
    heads = np.arange(H) if heads is None else np.asarray(heads)
    P = X.shape[-1]
    grp = heads // (H // G)
    Bh = B.reshape(batch, seqlen, E, G, N)
    Xh = X.reshape(batch, seqlen, E, heads.size, P)
    Ch = C.reshape(batch, seqlen, E, G, N)
    mk = mask.reshape(batch, seqlen, E)
    wt = (pi * mask).reshape(batch, seqlen, E)
    av = np.asarray(a, np.float64)[heads][None, None, :, None, None]
    if h_init is None:
        h = np.zeros((batch, E, heads.size, N, P))
    else:
        h = np.array(np.asarray(h_init, np.float64)[:, :, heads], copy=True)
    y = np.zeros((batch, seqlen, heads.size, P))
    for t in range(seqlen):
        # injection of every selected expert: B^(e) X^(e)^T per head
        Bt_ = Bh[:, t][:, :, grp, :]                                  # [Bt,E,Hs,N]
        U = Bt_[..., :, None] * Xh[:, t][..., None, :]                 # [Bt,E,Hs,N,P]
        h = av * h + mk[:, t][:, :, None, None, None] * U
        # readout: sum over selected experts of pi C^(e)^T h^(e)
        c = Ch[:, t][:, :, grp, :]                                    # [Bt,E,Hs,N]
        ye = np.einsum("behn,behnp->behp", c, h)
        y[:, t] = np.einsum("be,behp->bhp", wt[:, t], ye)
    return y, h


def separated_forward(u, w_router, w_experts, a, h_init, *, nheads, headdim, ngroups, dstate,
                      top_k, heads=None, routing=None) -> dict:
    """The whole separated-SSM MoE layer: route, project the selected
    experts, run E trajectories, read out. u [Bt, T, D]; h_init [Bt, E, H,
    N, P] or None. ``routing`` as for the Swimba oracle's ``forward``."""
    Bt, T, D = u.shape
    E = w_router.shape[0]
    uf = u.reshape(Bt * T, D)
    r = routing if routing is not None else osw.route(uf, w_router, top_k)
    s = osw.expert_streams(uf, w_experts, r.idx, nheads, headdim, ngroups, dstate, heads=heads)
    M = Bt * T
    hs = s.X.shape[2]
    B = np.zeros((M, E, ngroups, dstate))
    X = np.zeros((M, E, hs, headdim))
    C = np.zeros((M, E, ngroups, dstate))
    mask = np.zeros((M, E))
    rows = np.arange(M)
    for j in range(r.idx.shape[1]):
        e = r.idx[:, j]
        B[rows, e] = s.B[:, j]
        X[rows, e] = s.X[:, j]
        C[rows, e] = s.C[:, j]
        mask[rows, e] = 1.0
    y, hT = separated_recurrence(B, X, C, mask, r.pi, a, h_init, Bt, T, heads=heads)
    return {"y": y, "h_final": hT, "routing": r, "mask": mask}
