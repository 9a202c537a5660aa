"""Expert-mixed diagonal transition: the decay mixed per token, in fp64 (oracle).

TEST INFRASTRUCTURE: only tests, the smoke check and the benchmark's CPU
baseline use this module. It imports numpy and the base oracle, nothing from
the HIP path.

The base mixer shares one transition a_h per head across experts and steps.
The pages name, as the authors' next step, extending the parameter-space mix
to the diagonal of the transition while keeping the stability guarantee
(papernotes.org notes on "Swimba: Switch Mamba Model Scales State Space
Models", Limitations and outlook, the future-improvement item). Readings
adopted (argued in the design notes of the repository):
  * Each expert e has its own per-head scalar decay a_h^(e) in [0, 1).
  * A token's decay is the convex mix over its selected experts, with the
    same routing weights as the streams renormalised over the k selected
    experts: a_{t,h} = sum_j w_{t,j} a_h^(e_j) / sum_j w_{t,j}. Equal expert
    decays then give back the shared-decay mixer exactly, and a_{t,h} never
    exceeds max_e a_h^(e) <= rho < 1, the contraction the stability theorem
    needs (Method, key design 2; Theorem 3.3 in the gist.science summary).
  * The recurrence is unchanged otherwise: h_t = a_t h_{t-1} + U~_t,
    y_t = C~_t^T h_t, with a_t the decay of token t itself.

Pins (tests/test_oracle_mixed_decay.py): equal expert decays against the
pinned shared-decay oracle; k = 1 against the selected expert's decay;
explicit products of decays on short sequences (the time-varying quadratic
form); the contraction bounds on the mixed decay and on the state; chunked
cumulative products against running products.
"""
from __future__ import annotations

import numpy as np

from oracle import swimba as osw


def mix_decay(idx: np.ndarray, w: np.ndarray, a_experts: np.ndarray) -> np.ndarray:
    """Per-token, per-head decay mixed over the selected experts.

    [notes] Limitations and outlook: the parameter-space mix extended to the
    transition's diagonal; [notes] Method, key design 1: the mix weights are
    the routing weights of the selected experts. idx, w: [M, k]; a_experts:
    [E, H]. Returns a_t [M, H] = sum_j w_j a^(idx_j) / sum_j w_j.
    """
    w = np.asarray(w, np.float64)
    ae = np.asarray(a_experts, np.float64)
    num = np.einsum("mk,mkh->mh", w, ae[np.asarray(idx)])
    return num / w.sum(axis=1)[:, None]


def recurrence_tv(B_hat: np.ndarray, X: np.ndarray, C_mix: np.ndarray, a_t: np.ndarray,
                  h_init: np.ndarray | None, batch: int, seqlen: int, heads=None):
    """The single-trajectory recurrence with a per-token decay.

    Same as the shared-decay recurrence ([notes] Method, key design 1: h_t =
    A h_{t-1} + U~_t, Y_t = C~_t^T h_t) with A = a_{t,h} for token t. a_t:
    [M, H] over all heads; the other arguments as in the base oracle.
    """
    M, k, G, N = B_hat.shape
    H = a_t.shape[1]
    heads = np.arange(H) if heads is None else np.asarray(heads)
    P = X.shape[-1]
    grp = heads // (H // G)
    Bh = B_hat.reshape(batch, seqlen, k, G, N)
    Xh = X.reshape(batch, seqlen, k, heads.size, P)
    Ch = C_mix.reshape(batch, seqlen, G, N)
    av = np.asarray(a_t, np.float64).reshape(batch, seqlen, H)[:, :, heads]
    if h_init is None:
        h = np.zeros((batch, heads.size, N, P))
    else:
        h = np.array(np.asarray(h_init, dtype=np.float64)[:, heads], copy=True)
    y = np.zeros((batch, seqlen, heads.size, P))
    for t in range(seqlen):
        Bt_ = Bh[:, t][:, :, grp, :]
        U = np.matmul(Bt_.transpose(0, 2, 3, 1), Xh[:, t].transpose(0, 2, 1, 3))
        h = av[:, t][:, :, None, None] * h + U
        c = Ch[:, t][:, grp, :]
        y[:, t] = np.matmul(c[:, :, None, :], h)[:, :, 0, :]
    return y, h


def forward_tv(u: np.ndarray, w_router: np.ndarray, w_experts: np.ndarray,
               a_experts: np.ndarray, h_init, *, nheads: int, headdim: int, ngroups: int,
               dstate: int, top_k: int, heads=None, routing=None) -> dict:
    """The whole mixer with the expert-mixed decay: route, project, mix the
    streams and the decay, recur, read out. u: [Bt, T, D]; a_experts: [E, H]."""
    Bt, T, D = u.shape
    uf = u.reshape(Bt * T, D)
    r = routing if routing is not None else osw.route(uf, w_router, top_k)
    s = osw.expert_streams(uf, w_experts, r.idx, nheads, headdim, ngroups, dstate, heads=heads)
    B_hat, X, C_mix = osw.mix_streams(s, r.w)
    a_t = mix_decay(r.idx, r.w, a_experts)
    y, hT = recurrence_tv(B_hat, X, C_mix, a_t, h_init, Bt, T, heads=heads)
    return {"y": y, "h_final": hT, "routing": r, "B_hat": B_hat, "X": X, "C_mix": C_mix,
            "a_t": a_t}


def decode_step_tv(u_t: np.ndarray, w_router: np.ndarray, w_experts: np.ndarray,
                   a_experts: np.ndarray, h: np.ndarray, *, nheads: int, headdim: int,
                   ngroups: int, dstate: int, top_k: int, heads=None, routing=None) -> dict:
    """One recurrent decode step with the expert-mixed decay ([notes] Method,
    key design 1, recurrent form). u_t: [Bt, D]; h: [Bt, H, N, P] over all
    heads; ``heads`` and ``routing`` as for ``forward_tv`` (y and the new
    state are then over those heads)."""
    out = forward_tv(u_t[:, None, :], w_router, w_experts, a_experts, h, nheads=nheads,
                     headdim=headdim, ngroups=ngroups, dstate=dstate, top_k=top_k,
                     heads=heads, routing=routing)
    return {"y": out["y"][:, 0], "h": out["h_final"], "routing": out["routing"],
            "a_t": out["a_t"]}


def chunk_decay_products(a_t: np.ndarray, batch: int, seqlen: int, chunk: int) -> np.ndarray:
    """Running product of the decay within each chunk of ``chunk`` tokens:
    out[b, h, t] = prod_{u = c0}^{t} a_{u,h}, c0 the first token of t's chunk
    (the factor that carries a chunk's entering state to token t in the
    chunked solve). a_t: [M, H]; returns [Bt, H, T]."""
    H = a_t.shape[1]
    av = np.asarray(a_t, np.float64).reshape(batch, seqlen, H)
    out = np.empty((batch, H, seqlen))
    for c0 in range(0, seqlen, chunk):
        run = np.ones((batch, H))
        for t in range(c0, min(seqlen, c0 + chunk)):
            run = run * av[:, t]
            out[:, :, t] = run
    return out
