"""Planted mistakes in the oracle must be caught by at least one pin.

Each mutant replaces one oracle function (on the CPU only) with a plausible
wrong variant: a dropped term, a wrong sign or index, a transposed operand.
The pins of test_oracle_pins.py are then re-run and at least one must fail.
"""
from __future__ import annotations

import numpy as np
import pytest

import test_oracle_pins as tp
from oracle import swimba as osw

_orig_route = osw.route
_orig_mix = osw.mix_streams
_orig_rec = osw.recurrence
_orig_streams = osw.expert_streams
_orig_outproj = osw.output_project


def mix_unweighted(streams, w):
    return _orig_mix(streams, np.ones_like(w))


def mix_renormalised(streams, w):
    return _orig_mix(streams, w / w.sum(axis=1, keepdims=True))


def mix_c_unweighted(streams, w):
    B_hat, X, _ = _orig_mix(streams, w)
    return B_hat, X, streams.C.sum(axis=1)


def route_ties_high(u, w_router, top_k):
    r = _orig_route(u, w_router, top_k)
    g = r.logits
    E = g.shape[1]
    # break equal logits toward the higher index
    order = np.array([sorted(range(E), key=lambda e: (-row[e], -e)) for row in g])
    r.idx = order[:, :top_k]
    r.w = np.take_along_axis(r.pi, r.idx, axis=1)
    return r


def route_pi_over_selected(u, w_router, top_k):
    r = _orig_route(u, w_router, top_k)
    sel = np.take_along_axis(r.logits, r.idx, axis=1)
    ex = np.exp(sel - sel.max(axis=1, keepdims=True))
    r.w = ex / ex.sum(axis=1, keepdims=True)
    return r


def rec_decay_after_injection(B_hat, X, C_mix, a, h_init, batch, seqlen, heads=None):
    # h_t = a (h_{t-1} + U_t): the injection is decayed once too often
    y, h = _orig_rec(B_hat, X, C_mix, a, h_init, batch, seqlen, heads)
    heads_ = np.arange(a.shape[0]) if heads is None else np.asarray(heads)
    ah = a[heads_][None, None, :, None]
    return y * ah, h * a[heads_][None, :, None, None]


def rec_ignores_h_init(B_hat, X, C_mix, a, h_init, batch, seqlen, heads=None):
    return _orig_rec(B_hat, X, C_mix, a, None, batch, seqlen, heads)


def rec_wrong_group(B_hat, X, C_mix, a, h_init, batch, seqlen, heads=None):
    # head h reads group h % G instead of h // (H/G)
    G = B_hat.shape[2]
    H = a.shape[0]
    heads_ = np.arange(H) if heads is None else np.asarray(heads)
    ys, hs = [], []
    for i, h in enumerate(heads_):
        g = int(h) % G
        Bw = np.repeat(B_hat[:, :, g:g + 1], G, axis=2)
        Cw = np.repeat(C_mix[:, g:g + 1], G, axis=1)
        y, hT = _orig_rec(Bw, X[:, :, i:i + 1], Cw, a, h_init, batch, seqlen, heads=[h])
        ys.append(y)
        hs.append(hT)
    return np.concatenate(ys, axis=2), np.concatenate(hs, axis=1)


def streams_b_c_swapped(u, w_experts, idx, nheads, headdim, ngroups, dstate, heads=None):
    s = _orig_streams(u, w_experts, idx, nheads, headdim, ngroups, dstate, heads)
    return osw.Streams(X=s.X, B=s.C, C=s.B)


def streams_transposed_x(u, w_experts, idx, nheads, headdim, ngroups, dstate, heads=None):
    s = _orig_streams(u, w_experts, idx, nheads, headdim, ngroups, dstate, heads)
    M, k, H, P = s.X.shape
    return osw.Streams(X=s.X.reshape(M, k, P, H).transpose(0, 1, 3, 2).copy(), B=s.B, C=s.C)


def outproj_transposed_y(y, w_out):
    # the readout taken as [P, H] instead of [H, P]
    yf = np.asarray(y, np.float64)
    if yf.ndim == 3:
        yf = yf.transpose(0, 2, 1)
    return _orig_outproj(yf, w_out)


def outproj_weight_transposed(y, w_out):
    # W_out indexed [H*P, D]: reshape instead of transpose
    w = np.asarray(w_out, np.float64)
    return _orig_outproj(y, w.reshape(w.shape[1], w.shape[0]).T)


MUTANTS = {
    "mix_unweighted": ("mix_streams", mix_unweighted),
    "mix_renormalised": ("mix_streams", mix_renormalised),
    "mix_c_unweighted": ("mix_streams", mix_c_unweighted),
    "route_ties_high": ("route", route_ties_high),
    "route_pi_over_selected": ("route", route_pi_over_selected),
    "rec_decay_after_injection": ("recurrence", rec_decay_after_injection),
    "rec_ignores_h_init": ("recurrence", rec_ignores_h_init),
    "rec_wrong_group": ("recurrence", rec_wrong_group),
    "streams_b_c_swapped": ("expert_streams", streams_b_c_swapped),
    "streams_transposed_x": ("expert_streams", streams_transposed_x),
    "outproj_transposed_y": ("output_project", outproj_transposed_y),
    "outproj_weight_transposed": ("output_project", outproj_weight_transposed),
}

CHECKS = [
    tp.check_router_sigmoid_and_ties,
    tp.check_plain_ssm_k1_e1,
    tp.check_separated_identity,
    tp.check_theorem34,
    lambda: tp.check_chunked(3),
    tp.check_theorem35,
    tp.check_metamorphic,
    lambda: tp.check_brute_force(91),
    lambda: tp.check_brute_force(93, top_k=3, n_experts=3, nheads=4, ngroups=2),
    lambda: tp.check_brute_force(95, n_experts=4, top_k=2, d_model=1),
    tp.check_output_projection,
]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(osw, attr, fn)
    failures = 0
    for check in CHECKS:
        try:
            check()
        except AssertionError:
            failures += 1
    assert failures > 0, f"no pin caught the planted mistake {name}"
