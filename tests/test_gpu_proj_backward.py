"""GPU parity of the backward of router, expert projections and mix.

swimba_expert_project_mix_backward (through the C ABI) against the fp64
oracle's mix_backward -> project_backward -> route_backward on the same
seeded inputs and upstream gradients; every expected value comes from the
oracle. Inputs are chosen free of top-k near-ties (checked), since the top-k
set decides which expert's weights a token's gradient reaches.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from gpu_util import TOL, dev, host, say, tdt
from oracle import backward as ob
from oracle import swimba as osw
from selective_ssm_parameter_amd import binding as sb
from selective_ssm_parameter_amd import synth

pytestmark = pytest.mark.gpu


def W(name, seed, **kw):
    base = dict(batch=2, seqlen=300, d_model=128, nheads=3, headdim=64, dstate=128, ngroups=1,
                n_experts=4, top_k=2, chunk=64, dtype=synth.BF16, a_lo=0.9, a_hi=0.999)
    base.update(kw)
    return synth.small(name, seed, **base)


def upstream(wl):
    """Seeded gradients of B_hat, X_hat and C~ (what the scan's backward hands on)."""
    rng = np.random.default_rng(wl.seed + 57)
    M, k, H, G, N, P = wl.tokens, wl.top_k, wl.nheads, wl.ngroups, wl.dstate, wl.headdim
    dB = rng.standard_normal((M, k, G, N)).astype(np.float32)
    dX = rng.standard_normal((M, k, H, P)).astype(np.float32)
    dC = rng.standard_normal((M, G, N)).astype(np.float32)
    return dB, dX, dC


def oracle_grads(wl, inp, dB, dX, dC):
    uf = np.asarray(inp["u"], np.float64).reshape(wl.tokens, wl.d_model)
    wr = np.asarray(inp["w_router"], np.float64)
    we = np.asarray(inp["w_experts"], np.float64)
    r = osw.route(uf, wr, wl.top_k)
    assert not r.flagged.any(), "pick a seed without top-k near-ties"
    s = osw.expert_streams(uf, we, r.idx, wl.nheads, wl.headdim, wl.ngroups, wl.dstate)
    dBs, dCs, dw = ob.mix_backward(s, r.w, dB.astype(np.float64), dC.astype(np.float64))
    du_p, dW = ob.project_backward(uf, we, r.idx, dX.astype(np.float64), dBs, dCs)
    du_r, dWr, _ = ob.route_backward(uf, wr, r, dw)
    return du_p + du_r, dWr, dW


def run_gpu(wl, inp, dB, dX, dC):
    dims = sb.dims_of(wl)
    dt = tdt(wl)
    M, D, E = wl.tokens, wl.d_model, wl.n_experts
    Wd = wl.nheads * wl.headdim + 2 * wl.ngroups * wl.dstate
    f32 = torch.float32
    du = torch.full((M, D), float("nan"), dtype=f32, device="cuda")
    dWr = torch.full((E, D), float("nan"), dtype=f32, device="cuda")
    dW = torch.full((E, Wd, D), float("nan"), dtype=f32, device="cuda")
    ws, _ = sb.workspace(dims, sb.CALL_PROJECT_BACKWARD)
    sb.swimba_expert_project_mix_backward(
        dims, dev(np.reshape(inp["u"], (M, D)), dt), dev(inp["w_router"], dt),
        dev(inp["w_experts"], dt), dev(dB, f32), dev(dX, f32), dev(dC, f32), du, dWr, dW, ws)
    torch.cuda.synchronize()
    return host(du), host(dWr), host(dW)


def row_err(got, ref):
    """max over rows of max_i |d_i| / max(|ref_i|, rms(ref row)); rows = last axis."""
    got = np.asarray(got, np.float64).reshape(-1, ref.shape[-1])
    ref = np.asarray(ref, np.float64).reshape(-1, ref.shape[-1])
    rms = np.sqrt(np.mean(ref * ref, axis=1, keepdims=True))
    den = np.maximum(np.abs(ref), rms)
    den = np.where(den > 0, den, 1.0)
    return float(np.max(np.abs(got - ref) / den)) if ref.size else 0.0


CASES = [
    ("c1_f32", synth.WORKLOADS["c1"]),
    ("bf16_k2_e4", W("q1", 901)),
    ("bf16_k3_e5_g2_ragged", W("q2", 902, n_experts=5, top_k=3, nheads=4, ngroups=2, dstate=32,
                               seqlen=77)),
    ("bf16_e16_d256", W("q3", 903, n_experts=16, d_model=256, seqlen=400, dstate=64)),
    ("bf16_k8_e8", W("q4", 904, n_experts=8, top_k=8, dstate=16, seqlen=50)),
    ("bf16_e256_sparse", W("q5", 905, n_experts=256, top_k=2, seqlen=40, dstate=16)),
    ("f32_d160_ragged", W("q6", 906, dtype=synth.F32, d_model=160, seqlen=130, dstate=32)),
    ("bf16_one_token", W("q7", 907, batch=1, seqlen=1)),
]


@pytest.mark.parametrize("name,wl", CASES, ids=[c[0] for c in CASES])
def test_project_backward(name, wl):
    say(f"[proj_bwd] {name} M={wl.tokens} D={wl.d_model} E={wl.n_experts} k={wl.top_k} "
        f"N={wl.dstate} G={wl.ngroups} {wl.dtype}")
    inp = synth.make_inputs(wl)
    dB, dX, dC = upstream(wl)
    ref = oracle_grads(wl, inp, dB, dX, dC)
    got = run_gpu(wl, inp, dB, dX, dC)
    tol = TOL[wl.dtype]
    e_du = row_err(got[0], ref[0])
    e_dwr = row_err(got[1], ref[1])
    # experts no pair reached have an all-zero gradient, exactly
    used = np.zeros(wl.n_experts, bool)
    used[np.unique(osw.route(np.reshape(inp["u"], (wl.tokens, -1)).astype(np.float64),
                             np.asarray(inp["w_router"], np.float64), wl.top_k).idx)] = True
    e_dw = row_err(got[2][used], ref[2][used])
    say(f"  du {e_du:.2e} dW_router {e_dwr:.2e} dW_experts {e_dw:.2e} "
        f"(experts used {used.sum()}/{wl.n_experts})")
    assert np.all(got[2][~used] == 0)
    assert e_du < tol and e_dwr < tol and e_dw < tol


def test_project_backward_deterministic():
    wl = W("q8", 908, n_experts=8, seqlen=500)
    inp = synth.make_inputs(wl)
    dB, dX, dC = upstream(wl)
    r1 = run_gpu(wl, inp, dB, dX, dC)
    r2 = run_gpu(wl, inp, dB, dX, dC)
    for x, y in zip(r1, r2):
        assert np.array_equal(x, y)


def test_project_backward_no_tokens():
    wl = W("q9", 909, seqlen=0)
    dims = sb.dims_of(wl)
    Wd = wl.nheads * wl.headdim + 2 * wl.ngroups * wl.dstate
    dWr = torch.full((wl.n_experts, wl.d_model), 3.0, device="cuda")
    dW = torch.full((wl.n_experts, Wd, wl.d_model), 3.0, device="cuda")
    sb.swimba_expert_project_mix_backward(dims, None, None, None, None, None, None, None, dWr, dW,
                                          None)
    torch.cuda.synchronize()
    assert np.all(host(dWr) == 0) and np.all(host(dW) == 0)


def test_project_backward_saved_forward_is_bitwise_equal():
    """The variant that takes the forward's routing, B_hat and projection
    workspace returns bitwise what the recomputing call returns."""
    wl = W("q10", 910, n_experts=8, seqlen=333)
    inp = synth.make_inputs(wl)
    dB, dX, dC = upstream(wl)
    dims = sb.dims_of(wl)
    dt = tdt(wl)
    M, D, E = wl.tokens, wl.d_model, wl.n_experts
    Wd = wl.nheads * wl.headdim + 2 * wl.ngroups * wl.dstate
    u = dev(np.reshape(inp["u"], (M, D)), dt)
    wr, we = dev(inp["w_router"], dt), dev(inp["w_experts"], dt)
    buf = sb.alloc_buffers(dims, "cuda", logits=True)
    sb.swimba_route_topk(dims, u, wr, buf.topk_idx, buf.topk_w, buf.logits)
    sb.swimba_expert_project_mix(dims, u, we, buf.topk_idx, buf.topk_w, buf.B_hat, buf.X_hat,
                                 buf.C_mix, buf.ws_project)
    f32 = torch.float32
    outs = []
    for saved in (False, True):
        du = torch.full((M, D), float("nan"), dtype=f32, device="cuda")
        dWr = torch.full((E, D), float("nan"), dtype=f32, device="cuda")
        dW = torch.full((E, Wd, D), float("nan"), dtype=f32, device="cuda")
        args = (dev(dB, f32), dev(dX, f32), dev(dC, f32), du, dWr, dW)
        if saved:
            ws, _ = sb.workspace(dims, sb.CALL_PROJECT_BACKWARD_SAVED)
            sb.swimba_expert_project_mix_backward_saved(dims, u, wr, we, buf.topk_idx, buf.topk_w,
                                                        buf.logits, buf.B_hat, buf.ws_project,
                                                        *args, ws)
        else:
            ws, _ = sb.workspace(dims, sb.CALL_PROJECT_BACKWARD)
            sb.swimba_expert_project_mix_backward(dims, u, wr, we, *args, ws)
        torch.cuda.synchronize()
        outs.append([host(du), host(dWr), host(dW)])
    for a, b in zip(*outs):
        assert np.array_equal(a, b)
