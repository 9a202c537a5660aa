"""The Swimba mixer as a literal per-token recurrence in fp64 (oracle).

TEST INFRASTRUCTURE: only tests, the smoke check and the benchmark's CPU
baseline use this module. It imports numpy and nothing from the HIP path.

Readings adopted where the pages leave a step open (all argued in the design
notes of the repository):
  * Per head h the state is an N x P matrix; B and C are N-vectors, X is a
    P-vector, so the injection is the outer product B X^T (rank one per
    expert). B and C come in G groups shared by H/G consecutive heads.
  * The router is linear without bias; pi_t is the softmax over ALL experts;
    the mix uses pi at the selected experts without renormalising.
  * Top-k order: descending logit, equal logits -> lower expert index first.
  * The transition is a scalar a_h per head, constant in time, applied as is
    (no discretisation); h_{-1} is the given initial state or zero.
  * Expert projections are linear without bias; one expert's rows are laid
    out X (H*P) | B (G*N) | C (G*N).

Pins (tests/test_oracle_pins.py): k = E = 1 against the textbook quadratic
(attention-like) form of a scalar-decay SSM; the separated-trajectory
identity; Theorem 3.4 equality under static routing and its bound under
dynamic routing; a chunked fp64 solve; the BIBO bound of Theorem 3.3; dense
brute force with explicit powers on T <= 8; the Theorem 3.5 sigmoid
construction (tests/golden/); linearity, relabelling, causality, split and
resume, decode == prefill; projection against an explicit triple loop; the
output projection against an explicit double loop, the identity and a
column selection.
"""
from __future__ import annotations

import dataclasses

import numpy as np

TIE_MARGIN = 1e-5


@dataclasses.dataclass
class Routing:
    logits: np.ndarray   # [M, E]  g_t = W_r u_t
    pi: np.ndarray       # [M, E]  softmax over all experts
    idx: np.ndarray      # [M, k]  selected experts, descending logit
    w: np.ndarray        # [M, k]  pi at the selected experts
    margin: np.ndarray   # [M]     smallest logit gap that decides idx

    @property
    def flagged(self) -> np.ndarray:
        return self.margin < TIE_MARGIN


@dataclasses.dataclass
class Streams:
    X: np.ndarray        # [M, k, H, P]  X_t^(e) of the selected experts
    B: np.ndarray        # [M, k, G, N]  B_t^(e)
    C: np.ndarray        # [M, k, G, N]  C_t^(e)


def route(u: np.ndarray, w_router: np.ndarray, top_k: int) -> Routing:
    """Token router and top-k active set.

    [notes] Method, key design 1: pi_t = softmax(g_t), K_t a top-k sparse set;
    [gist-en] Technical Summary 2, Architecture Details, "Expert Routing";
    [notes] flowchart: the router R(.) reads the token feature.
    u: [M, D]; w_router: [E, D]. Logits and softmax in fp64.
    """
    u = np.asarray(u, dtype=np.float64)
    wr = np.asarray(w_router, dtype=np.float64)
    E = wr.shape[0]
    if not 1 <= top_k <= E:
        raise ValueError("top_k must lie in [1, E]")
    g = u @ wr.T
    gmax = g.max(axis=1, keepdims=True) if g.shape[0] else np.zeros((0, 1))
    ex = np.exp(g - gmax)
    pi = ex / ex.sum(axis=1, keepdims=True)
    # Stable sort of -g: descending logits, equal logits keep ascending index.
    order = np.argsort(-g, axis=1, kind="stable")
    idx = order[:, :top_k]
    w = np.take_along_axis(pi, idx, axis=1)
    if E == 1:
        margin = np.full(g.shape[0], np.inf)
    else:
        gs = np.take_along_axis(g, order, axis=1)
        last = min(top_k, E - 1)
        margin = (gs[:, :last] - gs[:, 1:last + 1]).min(axis=1)
    return Routing(logits=g, pi=pi, idx=idx.astype(np.int64), w=w, margin=margin)


def tie_alternatives(routing: Routing, m: int) -> list:
    """Every ordered top-k selection of token m that a near-tie leaves open.

    The top-k set of [notes] Method, key design 1 is decided by the logits;
    where two of the leading logits lie within TIE_MARGIN of each other, a
    computation in another precision may order them either way, and both
    orders are correct. The fp64 logits are sorted (descending, exact ties to
    the lower index) and split into runs whose consecutive gaps are below the
    margin; any order that permutes experts inside a run is a valid order,
    and its first k entries a valid selection. Returns the distinct
    selections (tuples of expert ids), the unperturbed one first.
    """
    import itertools

    g = routing.logits[m]
    k = routing.idx.shape[1]
    order = list(np.argsort(-g, kind="stable"))
    runs, cur = [], [order[0]]
    for e in order[1:]:
        if g[cur[-1]] - g[e] < TIE_MARGIN:
            cur.append(e)
        else:
            runs.append(cur)
            cur = [e]
    runs.append(cur)
    # only runs that start among the first k positions can change the selection
    pos, lead = 0, []
    for r in runs:
        if pos >= k:
            break
        lead.append(r)
        pos += len(r)
    out, seen = [], set()
    for perm in itertools.product(*[itertools.permutations(r) for r in lead]):
        sel = tuple(int(e) for e in itertools.chain(*perm))[:k]
        if sel not in seen:
            seen.add(sel)
            out.append(sel)
    return out


def with_selection(routing: Routing, m: int, sel) -> Routing:
    """The routing with token m's ordered selection replaced by ``sel`` (one
    of ``tie_alternatives(routing, m)``); its weights are pi at ``sel``."""
    idx = routing.idx.copy()
    idx[m] = np.asarray(sel, dtype=np.int64)
    w = routing.w.copy()
    w[m] = routing.pi[m, idx[m]]
    return Routing(logits=routing.logits, pi=routing.pi, idx=idx, w=w, margin=routing.margin)


def expert_streams(u: np.ndarray, w_experts: np.ndarray, idx: np.ndarray,
                   nheads: int, headdim: int, ngroups: int, dstate: int,
                   heads=None) -> Streams:
    """Expert-specific linear projections of the same token.

    [notes] Method, key design 1: each expert e maps X_t to its candidate
    streams B_t^(e), C_t^(e), X_t^(e); [gist-en] Technical Summary 2,
    "Parameter Mixing", first bullet. Only selected experts are evaluated.
    w_experts: [E, W, D] with rows X | B | C. ``heads`` keeps only the X rows
    of those heads (X is then [M, k, len(heads), P]); B and C are always whole.
    """
    u = np.asarray(u, dtype=np.float64)
    M, k = idx.shape
    HP, GN = nheads * headdim, ngroups * dstate
    W = w_experts.shape[1]
    if W != HP + 2 * GN:
        raise ValueError("expert width must be H*P + 2*G*N")
    hs = np.arange(nheads) if heads is None else np.asarray(heads)
    rows_x = (hs[:, None] * headdim + np.arange(headdim)[None, :]).ravel()
    keep = np.concatenate([rows_x, np.arange(HP, W)])
    nx = rows_x.size
    z = np.zeros((M, k, keep.size))
    for e in range(w_experts.shape[0]):
        rows, slots = np.nonzero(idx == e)
        if rows.size:
            we = np.asarray(w_experts[e][keep], dtype=np.float64)
            z[rows, slots] = u[rows] @ we.T
    X = z[..., :nx].reshape(M, k, hs.size, headdim)
    B = z[..., nx:nx + GN].reshape(M, k, ngroups, dstate)
    C = z[..., nx + GN:].reshape(M, k, ngroups, dstate)
    return Streams(X=X, B=B, C=C)


def mix_streams(streams: Streams, w: np.ndarray):
    """Parameter-space mix of the selected experts' streams.

    [notes] Method, key design 1, mixing equation: U~_t = sum_{e in K_t}
    pi_{t,e} B_t^(e) X_t^(e), C~_t = sum_{e in K_t} pi_{t,e} C_t^(e).
    Returns the factors the recurrence consumes: B_hat = pi * B per slot (so
    that U~ = sum_j B_hat_j X_j^T), X per slot, and the mixed readout C~.
    """
    B_hat = w[:, :, None, None] * streams.B
    C_mix = np.einsum("mk,mkgn->mgn", w, streams.C)
    return B_hat, streams.X, C_mix


def recurrence(B_hat: np.ndarray, X: np.ndarray, C_mix: np.ndarray, a: np.ndarray,
               h_init: np.ndarray | None, batch: int, seqlen: int, heads=None):
    """Single-trajectory selective SSM, one token at a time.

    [notes] Method, key design 1, state equation: h_t = A h_{t-1} + U~_t,
    Y_t = C~_t^T h_t; key design 2: A is shared by all experts and steps.
    [gist-en] Technical Summary 2, the state update equation.

    B_hat [M,k,G,N] (pi folded in), X [M,k,Hs,P] for the heads in ``heads``
    (all heads when None), C_mix [M,G,N], a [H] and h_init [Bt,H,N,P] over all
    heads. The injection U~ (N x P per head) is formed explicitly every step.
    Returns y [Bt,T,Hs,P] and the final state [Bt,Hs,N,P].
    """
    M, k, G, N = B_hat.shape
    H = a.shape[0]
    heads = np.arange(H) if heads is None else np.asarray(heads)
    P = X.shape[-1]
    grp = heads // (H // G)
    Bh = B_hat.reshape(batch, seqlen, k, G, N)
    Xh = X.reshape(batch, seqlen, k, heads.size, P)
    Ch = C_mix.reshape(batch, seqlen, G, N)
    av = np.asarray(a, dtype=np.float64)[heads][None, :, None, None]
    if h_init is None:
        h = np.zeros((batch, heads.size, N, P))
    else:
        h = np.array(np.asarray(h_init, dtype=np.float64)[:, heads], copy=True)
    y = np.zeros((batch, seqlen, heads.size, P))
    for t in range(seqlen):
        Bt_ = Bh[:, t][:, :, grp, :]                              # [Bt,k,Hs,N]
        # U~_t = sum_j B_hat_j X_j^T: batched (N x k) @ (k x P)
        U = np.matmul(Bt_.transpose(0, 2, 3, 1), Xh[:, t].transpose(0, 2, 1, 3))
        h = av * h + U
        c = Ch[:, t][:, grp, :]                                   # [Bt,Hs,N]
        y[:, t] = np.matmul(c[:, :, None, :], h)[:, :, 0, :]
    return y, h


def forward(u: np.ndarray, w_router: np.ndarray, w_experts: np.ndarray, a: np.ndarray,
            h_init, *, nheads: int, headdim: int, ngroups: int, dstate: int,
            top_k: int, heads=None, routing: Routing | None = None) -> dict:
    """The whole mixer: route, project, mix, recur, read out.

    u: [Bt, T, D]. ``heads`` restricts X, y and the state to those heads (the
    routing, B and C never depend on the head); "X" is then over those heads. ``routing`` lets a caller pass
    a routing the oracle itself produced (for example a different top-k
    choice at a flagged near-tie).
    """
    Bt, T, D = u.shape
    uf = u.reshape(Bt * T, D)
    r = routing if routing is not None else route(uf, w_router, top_k)
    s = expert_streams(uf, w_experts, r.idx, nheads, headdim, ngroups, dstate, heads=heads)
    B_hat, X, C_mix = mix_streams(s, r.w)
    y, hT = recurrence(B_hat, X, C_mix, a, h_init, Bt, T, heads=heads)
    return {"y": y, "h_final": hT, "routing": r, "B_hat": B_hat, "X": X, "C_mix": C_mix}


def output_project(y: np.ndarray, w_out: np.ndarray) -> np.ndarray:
    """The single output projection after the recurrence, in fp64.

    [gist-en] Technical Summary section 2, Architecture Details: the state
    update is followed by one output projection. Read as the map of each
    token's H*P readout back to d_model with no bias: out_t = W_out y_t.
    y: [M, H, P] or [M, H*P]; w_out: [D, H*P]. Returns [M, D].
    """
    yf = np.asarray(y, np.float64)
    yf = yf.reshape(yf.shape[0], -1)
    return yf @ np.asarray(w_out, np.float64).T


def decode_step(u_t: np.ndarray, w_router: np.ndarray, w_experts: np.ndarray, a: np.ndarray,
                h: np.ndarray, *, nheads: int, headdim: int, ngroups: int, dstate: int,
                top_k: int, heads=None, routing: Routing | None = None) -> dict:
    """One recurrent decode step: the same recurrence for a single token.

    [notes] Method, key design 1 (recurrent form); [notes] key findings, vLLM
    decoding. u_t: [Bt, D]; h: [Bt, H, N, P] (or the heads in ``heads``).
    ``routing`` as for ``forward``.
    """
    Bt = u_t.shape[0]
    h_full = h
    if heads is not None:
        h_full = np.zeros((Bt, nheads) + h.shape[2:])
        h_full[:, np.asarray(heads)] = h
    out = forward(u_t[:, None, :], w_router, w_experts, a, h_full, nheads=nheads,
                  headdim=headdim, ngroups=ngroups, dstate=dstate, top_k=top_k, heads=heads,
                  routing=routing)
    return {"y": out["y"][:, 0], "h": out["h_final"], "routing": out["routing"]}
