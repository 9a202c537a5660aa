"""Pins of the separated-SSM MoE oracle (oracle/separated.py) against what
the pages and mathematics fix, and planted mistakes each pin set must catch.

Theorem 3.4 ([notes] Method, key design 2) gives an equality under static
routing with a shared readout and a bound under dynamic routing; k = E = 1
reduces to a textbook SSM; the dense case k = E is checked against the
independent per-expert formulation of tests/pins.py; k < E against brute
force with explicit powers.
"""
from __future__ import annotations

import numpy as np
import pytest

import pins
from oracle import separated as osep
from oracle import swimba as osw
from selective_ssm_parameter_amd import synth


def tiny(seed=11, **kw):
    base = dict(batch=2, seqlen=7, d_model=8, nheads=2, headdim=3, dstate=4, ngroups=1,
                n_experts=3, top_k=2, chunk=4, dtype=synth.F32, a_lo=0.5, a_hi=0.95)
    base.update(kw)
    return synth.small("tiny", seed, **base)


def h_per_expert(wl, seed=5, scale=0.3):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((wl.batch, wl.n_experts, wl.nheads, wl.dstate, wl.headdim)) * scale


def sep(wl, inp, h0, **kw):
    return osep.separated_forward(inp["u"], inp["w_router"], inp["w_experts"], inp["a"], h0,
                                  nheads=wl.nheads, headdim=wl.headdim, ngroups=wl.ngroups,
                                  dstate=wl.dstate, top_k=wl.top_k, **kw)


def mix(wl, inp, h0):
    return osw.forward(inp["u"], inp["w_router"], inp["w_experts"], inp["a"], h0,
                       nheads=wl.nheads, headdim=wl.headdim, ngroups=wl.ngroups,
                       dstate=wl.dstate, top_k=wl.top_k)


def rel(x, y):
    return float(np.max(np.abs(x - y)) / max(np.max(np.abs(y)), 1e-300))


# ---------------------------------------------------------------- checks

def check_theorem34_equality():
    # static routing (W_r = 0: pi = 1/E, k = E) and one shared readout matrix,
    # every trajectory started from the same state: separated == mixed
    wl = tiny(41, n_experts=3, top_k=3, seqlen=8, nheads=2, ngroups=2, dstate=3, headdim=2)
    inp = synth.make_inputs(wl)
    inp["w_router"] = np.zeros_like(inp["w_router"])
    HP, GN = wl.nheads * wl.headdim, wl.ngroups * wl.dstate
    we = inp["w_experts"].copy()
    we[:, HP + GN:] = we[0, HP + GN:][None]
    inp["w_experts"] = we
    h0 = h_per_expert(wl)[:, :1]
    h0e = np.repeat(h0, wl.n_experts, axis=1)
    ys = sep(wl, inp, h0e)["y"]
    ym = mix(wl, inp, h0[:, 0])["y"]
    assert rel(ys, ym) < 1e-12
    # and they differ once the readouts differ
    inp2 = dict(inp, w_experts=synth.make_inputs(wl)["w_experts"])
    assert rel(sep(wl, inp2, h0e)["y"], mix(wl, inp2, h0[:, 0])["y"]) > 1e-3


def check_theorem34_bound():
    # dynamic routing: |y_sep - y_mix| <= max_e |C^(e)| sum_e pi_e |h^(e) - h|
    # per (sequence, token, head), with the states after every token
    wl = tiny(43, n_experts=4, top_k=2, seqlen=6, nheads=2, dstate=3, headdim=2)
    inp = synth.make_inputs(wl)
    h0 = h_per_expert(wl, 7)
    h0m = h0.sum(axis=1) / wl.n_experts
    ys = sep(wl, inp, h0)["y"]
    ym = mix(wl, inp, h0m)["y"]
    _, _, Call = pins.dense_streams(inp["u"].reshape(-1, wl.d_model), inp["w_experts"],
                                    wl.nheads, wl.headdim, wl.ngroups, wl.dstate)
    r = osw.route(inp["u"].reshape(-1, wl.d_model), inp["w_router"], wl.top_k)
    checked = 0
    for t in range(wl.seqlen):
        sub = dict(inp, u=inp["u"][:, :t + 1])
        hs = sep(wl.replace(seqlen=t + 1), sub, h0)["h_final"]        # [Bt,E,H,N,P]
        hm = mix(wl.replace(seqlen=t + 1), sub, h0m)["h_final"]       # [Bt,H,N,P]
        for b in range(wl.batch):
            m = b * wl.seqlen + t
            for h in range(wl.nheads):
                cmax = max(np.linalg.norm(Call[m, e, 0]) for e in r.idx[m])
                rhs = cmax * sum(r.pi[m, e] * np.linalg.norm(hs[b, e, h] - hm[b, h], 2)
                                 for e in r.idx[m])
                lhs = np.linalg.norm(ys[b, t, h] - ym[b, t, h])
                assert lhs <= rhs * (1 + 1e-12) + 1e-14
                checked += lhs > 0
    assert checked > 0


def check_single_expert():
    # k = E = 1: one trajectory with pi = 1, the textbook quadratic form
    wl = tiny(21, n_experts=1, top_k=1, seqlen=11, nheads=3, dstate=5, headdim=4)
    inp = synth.make_inputs(wl)
    h0 = h_per_expert(wl, 9)
    out = sep(wl, inp, h0)
    we = inp["w_experts"][0].astype(np.float64)
    HP, N = wl.nheads * wl.headdim, wl.dstate
    for b in range(wl.batch):
        uu = inp["u"][b].astype(np.float64)
        Xall, Bm, Cm = uu @ we[:HP].T, uu @ we[HP:HP + N].T, uu @ we[HP + N:].T
        for h in range(wl.nheads):
            X = Xall[:, h * wl.headdim:(h + 1) * wl.headdim]
            want = pins.quadratic_form_ssm(Bm, Cm, X, inp["a"][h], h0[b, 0, h])
            assert rel(out["y"][b, :, h], want) < 1e-11


def check_dense_against_pins():
    # k = E: every expert injects every step; states against the per-expert
    # formulation of tests/pins.py (every trajectory from h_init), y = the
    # pi-weighted sum of the readouts
    wl = tiny(47, n_experts=3, top_k=3, seqlen=9, nheads=2, ngroups=2, dstate=3, headdim=2)
    inp = synth.make_inputs(wl)
    h0 = h_per_expert(wl, 11)[:, 0]
    out = sep(wl, inp, np.repeat(h0[:, None], wl.n_experts, axis=1))
    hs, pi, mask, C = pins.separated_trajectories(
        inp["u"], inp["w_router"], inp["w_experts"], inp["a"], h0, wl.nheads, wl.headdim,
        wl.ngroups, wl.dstate, wl.top_k, weighted=False)
    assert rel(out["h_final"], hs[:, -1]) < 1e-12
    grp = np.arange(wl.nheads) // (wl.nheads // wl.ngroups)
    Ce = C.reshape(wl.batch, wl.seqlen, wl.n_experts, wl.ngroups, -1)[:, :, :, grp]
    w = (pi * mask).reshape(wl.batch, wl.seqlen, wl.n_experts)
    y = np.einsum("bte,btehn,btehnp->bthp", w, Ce, hs)
    assert rel(out["y"], y) < 1e-12


def check_brute_force_topk(seed, **kw):
    # k < E: explicit powers and sums, the selection from a full Python sort
    wl = tiny(seed, **kw)
    inp = synth.make_inputs(wl)
    h0 = h_per_expert(wl, seed + 1)
    out = sep(wl, inp, h0)
    Bt, T, E, H, P = wl.batch, wl.seqlen, wl.n_experts, wl.nheads, wl.headdim
    uf = inp["u"].reshape(Bt * T, -1).astype(np.float64)
    g = uf @ np.asarray(inp["w_router"], np.float64).T
    pi = pins.softmax_rows(g)
    mask, _ = pins.topk_mask_bruteforce(g, wl.top_k)
    X, B, C = pins.dense_streams(uf, inp["w_experts"], H, P, wl.ngroups, wl.dstate)
    for b in range(Bt):
        for h in range(H):
            gi = h // (H // wl.ngroups)
            a = float(inp["a"][h])
            for t in range(T):
                y = np.zeros(P)
                for e in range(E):
                    st = a ** (t + 1) * h0[b, e, h]
                    for s in range(t + 1):
                        ms = b * T + s
                        st = st + a ** (t - s) * mask[ms, e] * np.outer(B[ms, e, gi], X[ms, e, h])
                    m = b * T + t
                    y += mask[m, e] * pi[m, e] * (C[m, e, gi] @ st)
                    if t == T - 1:
                        assert rel(out["h_final"][b, e, h], st) < 1e-12
                assert rel(out["y"][b, t, h], y) < 1e-11


def check_unselected_expert_decays():
    # an expert that is never selected injects nothing: its state is a^T h_init
    wl = tiny(53, n_experts=4, top_k=2, seqlen=10)
    inp = synth.make_inputs(wl)
    # feature 0 of u is a constant 1 that only expert 3's router row reads,
    # with weight -1000
    inp["u"] = inp["u"].copy()
    inp["u"][..., 0] = 1.0
    inp["w_router"] = inp["w_router"].copy()
    inp["w_router"][:, 0] = 0.0
    inp["w_router"][3] = 0.0
    inp["w_router"][3, 0] = -1000.0
    h0 = h_per_expert(wl, 13)
    out = sep(wl, inp, h0)
    assert not np.any(out["routing"].idx == 3)
    want = (inp["a"].astype(np.float64)[None, :, None, None] ** wl.seqlen) * h0[:, 3]
    assert rel(out["h_final"][:, 3], want) < 1e-13


def check_head_subset():
    wl = tiny(57, n_experts=4, top_k=2, seqlen=9, nheads=4, ngroups=2)
    inp = synth.make_inputs(wl)
    h0 = h_per_expert(wl, 15)
    full = sep(wl, inp, h0)
    part = sep(wl, inp, h0, heads=[1, 3])
    assert rel(part["y"], full["y"][:, :, [1, 3]]) < 1e-13
    assert rel(part["h_final"], full["h_final"][:, :, [1, 3]]) < 1e-13


CHECKS = [
    check_theorem34_equality,
    check_theorem34_bound,
    check_single_expert,
    check_dense_against_pins,
    lambda: check_brute_force_topk(61),
    lambda: check_brute_force_topk(63, n_experts=4, top_k=1, nheads=4, ngroups=2),
    lambda: check_brute_force_topk(65, n_experts=5, top_k=3, seqlen=5),
    check_unselected_expert_decays,
    check_head_subset,
]


@pytest.mark.parametrize("i", range(len(CHECKS)))
def test_separated_pin(i):
    CHECKS[i]()


# ---------------------------------------------------------------- mutants

_orig_rec = osep.separated_recurrence


def rec_readout_unweighted(B, X, C, mask, pi, a, h_init, batch, seqlen, heads=None):
    return _orig_rec(B, X, C, mask, np.ones_like(pi), a, h_init, batch, seqlen, heads)


def rec_injection_weighted(B, X, C, mask, pi, a, h_init, batch, seqlen, heads=None):
    # pi folded into the injection as in the mixed design
    Bw = B * pi[:, :, None, None]
    return _orig_rec(Bw, X, C, mask, pi, a, h_init, batch, seqlen, heads)


def rec_readout_all_experts(B, X, C, mask, pi, a, h_init, batch, seqlen, heads=None):
    # every expert read out, selected or not (C of unselected experts is 0
    # here, so this differs only through the weights' mask)
    M, E = mask.shape
    Cf = C + (1 - mask)[:, :, None, None]
    return _orig_rec(B, X, Cf, np.ones_like(mask), pi, a, h_init, batch, seqlen, heads)


def rec_unselected_frozen(B, X, C, mask, pi, a, h_init, batch, seqlen, heads=None):
    # an unselected expert's state held instead of decayed: emulated one step
    # at a time by splitting the sequence
    Bt, T = batch, seqlen
    E = mask.shape[1]
    H = a.shape[0]
    hs = np.arange(H) if heads is None else np.asarray(heads)
    h = None if h_init is None else np.array(h_init, np.float64, copy=True)
    ys = []
    for t in range(T):
        rows = np.arange(Bt) * T + t
        y, hn = _orig_rec(B[rows], X[rows], C[rows], mask[rows], pi[rows], a, h, Bt, 1, heads)
        if h is None:
            h = np.zeros((Bt, E, H) + hn.shape[3:])
        keep = mask[rows].astype(bool)
        new = np.array(h, copy=True)
        for b in range(Bt):
            for e in range(E):
                if keep[b, e]:
                    new[b, e][hs] = hn[b, e]
        h = new
        ys.append(y)
    return np.concatenate(ys, axis=1), h[:, :, hs]


def rec_transposed_x(B, X, C, mask, pi, a, h_init, batch, seqlen, heads=None):
    M, E, Hs, P = X.shape
    Xt = X.reshape(M, E, P, Hs).transpose(0, 1, 3, 2).copy()
    return _orig_rec(B, Xt, C, mask, pi, a, h_init, batch, seqlen, heads)


MUTANTS = {
    "readout_unweighted": rec_readout_unweighted,
    "injection_weighted": rec_injection_weighted,
    "readout_all_experts": rec_readout_all_experts,
    "unselected_frozen": rec_unselected_frozen,
    "transposed_x": rec_transposed_x,
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_separated_mutant_is_caught(name, monkeypatch):
    monkeypatch.setattr(osep, "separated_recurrence", MUTANTS[name])
    failures = 0
    for check in CHECKS:
        try:
            check()
        except AssertionError:
            failures += 1
    assert failures > 0, f"no pin caught the planted mistake {name}"
