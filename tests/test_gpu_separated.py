"""GPU parity of the separated-SSM MoE (swimba_separated_forward) against the
fp64 oracle of oracle/separated.py: y and every expert's final state, on
small shapes (ragged, with initial states, dense k = E, two groups, fp32) and
at the c2 sizes on sampled (sequence, head) pairs."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from gpu_util import TOL, check_routing, dev, host, say, slice_err, sub_routing, tdt, upload
from oracle import separated as osep
from oracle import swimba as osw
from selective_ssm_parameter_amd import binding as sb
from selective_ssm_parameter_amd import synth

pytestmark = pytest.mark.gpu


def W(name, seed, **kw):
    base = dict(batch=2, seqlen=300, d_model=256, nheads=4, headdim=64, dstate=128, ngroups=1,
                n_experts=4, top_k=2, chunk=64, dtype=synth.BF16, a_lo=0.9, a_hi=0.999)
    base.update(kw)
    return synth.small(name, seed, **base)


def h_per_expert(wl, scale=0.3):
    rng = np.random.default_rng(2000 + wl.seed)
    return (rng.standard_normal((wl.batch, wl.n_experts, wl.nheads, wl.dstate, wl.headdim))
            * scale).astype(np.float32)


CASES = [
    ("e4_k1", W("q1", 901, top_k=1), False),
    ("e4_k2_h0", W("q2", 902), True),
    ("e8_k2_ragged_L128", W("q3", 903, n_experts=8, seqlen=333, chunk=128), True),
    ("e3_k3_dense", W("q4", 904, n_experts=3, top_k=3, seqlen=200), True),
    ("e6_k2_g2_n64_L32", W("q5", 905, n_experts=6, ngroups=2, dstate=64, chunk=32, seqlen=150), False),
    ("e8_k4_short", W("q6", 906, n_experts=8, top_k=4, seqlen=9, batch=3), True),
    ("f32_e4_k1", W("q7", 907, dtype=synth.F32, seqlen=130, dstate=32), True),
]


def run_sep(wl, d, h0):
    dims = sb.dims_of(wl)
    buf = sb.separated_forward(dims, d["u"], d["w_router"], d["w_experts"], d["a"],
                               None if h0 is None else dev(h0, torch.float32))
    torch.cuda.synchronize()
    return buf


@pytest.mark.parametrize("name,wl,with_h0", CASES, ids=[c[0] for c in CASES])
def test_separated_forward(name, wl, with_h0):
    say(f"[separated] {name} T={wl.seqlen} E={wl.n_experts} k={wl.top_k} {wl.dtype}")
    inp = synth.make_inputs(wl)
    h0 = h_per_expert(wl) if with_h0 else None
    buf = run_sep(wl, upload(wl, inp), h0)
    r = osw.route(inp["u"].reshape(wl.tokens, -1), inp["w_router"], wl.top_k)
    r = check_routing(host(buf.topk_idx).astype(np.int64), None, r, wl)
    ref = osep.separated_forward(inp["u"], inp["w_router"], inp["w_experts"], inp["a"], h0,
                                 nheads=wl.nheads, headdim=wl.headdim, ngroups=wl.ngroups,
                                 dstate=wl.dstate, top_k=wl.top_k, routing=r)
    ey = slice_err(host(buf.y).reshape(wl.batch, wl.seqlen, wl.nheads, 64), ref["y"])
    shape = (wl.batch * wl.n_experts, wl.nheads, wl.dstate, 64)
    eh = slice_err(host(buf.h_final).reshape(shape), ref["h_final"].reshape(shape), (0, 1))
    say(f"  y err {ey:.3e}  h_final err {eh:.3e}")
    assert ey < TOL[wl.dtype] and eh < TOL[wl.dtype]


def test_separated_no_tokens_passes_states():
    wl = W("q8", 908, seqlen=0)
    h0 = h_per_expert(wl)
    dims = sb.dims_of(wl)
    hf = torch.full(h0.shape, 3.0, device="cuda")
    a = dev(synth.make_inputs(wl)["a"], torch.float32)
    sb.swimba_separated_forward(dims, None, None, None, a, dev(h0, torch.float32), None, hf, None,
                                None)
    torch.cuda.synchronize()
    assert np.array_equal(host(hf), h0.astype(np.float64))


def test_separated_reduces_to_swimba_with_one_expert():
    # E = k = 1: one trajectory with pi = 1, the Swimba layer itself
    wl = W("q9", 909, n_experts=1, top_k=1, seqlen=260)
    inp = synth.make_inputs(wl)
    d = upload(wl, inp)
    sep = run_sep(wl, d, None)
    mix = sb.forward(sb.dims_of(wl), d["u"], d["w_router"], d["w_experts"], d["a"])
    torch.cuda.synchronize()
    ys, ym = host(sep.y), host(mix.y)
    e = slice_err(ys.reshape(wl.batch, wl.seqlen, wl.nheads, 64),
                  ym.reshape(wl.batch, wl.seqlen, wl.nheads, 64))
    say(f"  separated vs Swimba at E = k = 1: {e:.3e}")
    assert e < TOL[wl.dtype]


def test_separated_full_size_c2():
    # the c2 sizes (8 x 2048 tokens, d_model 768, 24 heads, E = 8, k = 2):
    # 64 trajectories; sampled (sequence, head) pairs over whole sequences
    wl = synth.WORKLOADS["c2"]
    say(f"[separated] c2 full size: M={wl.tokens} E={wl.n_experts} k={wl.top_k}")
    inp = synth.make_inputs(wl)
    buf = run_sep(wl, upload(wl, inp), None)
    M, T = wl.tokens, wl.seqlen
    r = osw.route(inp["u"].reshape(M, -1), inp["w_router"], wl.top_k)
    r = check_routing(host(buf.topk_idx).astype(np.int64), None, r, wl)
    y = buf.y.view(wl.batch, T, wl.nheads, 64)
    hf = buf.h_final
    for b, heads in [(0, [0, 13]), (7, [23])]:
        ref = osep.separated_forward(inp["u"][b:b + 1], inp["w_router"], inp["w_experts"],
                                     inp["a"], None, nheads=wl.nheads, headdim=wl.headdim,
                                     ngroups=wl.ngroups, dstate=wl.dstate, top_k=wl.top_k,
                                     heads=heads, routing=sub_routing(r, slice(b * T, (b + 1) * T)))
        ey = slice_err(host(y[b:b + 1, :, heads]), ref["y"])
        got_h = host(hf[b][:, heads])                       # [E, Hs, N, P]
        eh = slice_err(got_h, ref["h_final"][0], (0, 1))
        say(f"  b={b} heads={heads}: y err {ey:.3e} h_final err {eh:.3e}")
        assert ey < TOL[wl.dtype] and eh < TOL[wl.dtype]
