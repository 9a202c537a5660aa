"""Helpers shared by the GPU parity tests: upload, download, comparison.

Inputs come from ``selective_ssm_parameter_amd.synth``; expected values come
from the fp64 oracle only.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

from oracle import swimba as osw
from selective_ssm_parameter_amd import binding as sb
from selective_ssm_parameter_amd import synth

TOL = {synth.F32: 1e-4, synth.BF16: 2e-2}
# Intermediate streams: one rounding (fp16 for bf16 inputs, unit roundoff
# 2^-11) of an fp32-accumulated dot product.
STREAM_TOL = {synth.F32: 1e-5, synth.BF16: 2e-3}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(x, dtype, device="cuda"):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(device=device, dtype=dtype)


def host(t) -> np.ndarray:
    return t.detach().to(torch.float64).cpu().numpy()


def tdt(wl):
    """torch element type of u, the weights and y."""
    return torch.bfloat16 if wl.dtype == synth.BF16 else torch.float32


def sdt(wl):
    """torch element type of the streams B_hat, X_hat, C_mix."""
    return torch.float16 if wl.dtype == synth.BF16 else torch.float32


def upload(wl, inp, device="cuda"):
    dt = tdt(wl)
    return {
        "u": dev(inp["u"].reshape(-1, wl.d_model), dt, device),
        "w_router": dev(inp["w_router"], dt, device),
        "w_experts": dev(inp["w_experts"], dt, device),
        "a": dev(inp["a"], torch.float32, device),
        "h_init": None if inp["h_init"] is None else dev(inp["h_init"], torch.float32, device),
    }


def round_stream(x, wl):
    """The value of a stream element as the library stores it, as fp64."""
    x = np.asarray(x, dtype=np.float32)
    if wl.dtype == synth.BF16:
        return x.astype(np.float16).astype(np.float64)
    return x.astype(np.float64)


def slice_err(got, ref, axes_slice=(0, 2), floor=0.0):
    """max over (batch, head) slices of max_i |d_i| / max(|ref_i|, rms(ref slice), floor).

    got/ref: [Bt, T, H, P] (y) or [Bt, H, N, P] (states, use axes (0, 1)).
    ``floor`` bounds the denominator from below: an fp32 output cannot hold a
    value below the smallest normal fp32 number to relative precision, so
    fp32 outputs whose exact values underflow are compared against it."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    worst = 0.0
    a0, a1 = axes_slice
    for i in range(ref.shape[a0]):
        for j in range(ref.shape[a1]):
            r = np.take(np.take(ref, i, axis=a0), j, axis=a1 - 1)
            g = np.take(np.take(got, i, axis=a0), j, axis=a1 - 1)
            if r.size == 0:
                continue
            rms = np.sqrt(np.mean(r * r))
            den = np.maximum(np.maximum(np.abs(r), rms), floor)
            den = np.where(den > 0, den, 1.0)
            worst = max(worst, float(np.max(np.abs(g - r) / den)))
    return worst


# smallest normal fp32 number: the floor of the relative metric for fp32 outputs
F32_TINY = float(np.finfo(np.float32).tiny)


def rel_err(got, ref):
    """max_i |d_i| / max(|ref_i|, rms(ref)) over the whole tensor."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    if ref.size == 0:
        return 0.0
    rms = np.sqrt(np.mean(ref * ref))
    den = np.maximum(np.abs(ref), rms)
    den = np.where(den > 0, den, 1.0)
    return float(np.max(np.abs(got - ref) / den))


def check_routing(idx_gpu, w_gpu, r: osw.Routing, wl):
    """Index parity, bit-exact except at flagged near-ties. Returns the
    oracle's routing for the selection the GPU made: at every token where the
    GPU's ordered selection differs from the oracle's, that selection must be
    one of the alternatives the oracle itself derives from its fp64 logits
    (``osw.tie_alternatives``), and the returned routing takes the oracle's
    alternative there (its weights are the oracle's pi). No value of the GPU
    enters the returned routing; its indices only pick among the oracle's."""
    idx_gpu = np.asarray(idx_gpu)
    diff = np.any(idx_gpu != r.idx, axis=1)
    bad = diff & ~r.flagged
    assert not bad.any(), f"top-k mismatch at unflagged tokens {np.nonzero(bad)[0][:10]}"
    out = r
    for m in np.nonzero(diff)[0]:
        alts = osw.tie_alternatives(r, int(m))
        sel = tuple(int(e) for e in idx_gpu[m])
        assert sel in alts, f"token {m}: selection {sel} is not a near-tie alternative {alts}"
        out = osw.with_selection(out, int(m), sel)
    ok = ~diff
    if w_gpu is not None and ok.any():
        werr = np.max(np.abs(np.asarray(w_gpu)[ok] - r.w[ok]) / np.maximum(r.w[ok], 1e-30))
        assert werr < 1e-5, f"top-k weight relative error {werr}"
    if diff.any():
        say(f"  near-tie tokens with the other valid order: {np.nonzero(diff)[0].tolist()}")
    return out


def sub_routing(r: osw.Routing, rows) -> osw.Routing:
    """The routing of the token rows ``rows`` (a slice or index array)."""
    return osw.Routing(logits=r.logits[rows], pi=r.pi[rows], idx=r.idx[rows], w=r.w[rows],
                       margin=r.margin[rows])


def oracle_forward(wl, inp, heads=None, routing=None):
    return osw.forward(inp["u"], inp["w_router"], inp["w_experts"], inp["a"], inp["h_init"],
                       nheads=wl.nheads, headdim=wl.headdim, ngroups=wl.ngroups,
                       dstate=wl.dstate, top_k=wl.top_k, heads=heads, routing=routing)


def run_forward(wl, d, logits=False):
    dims = sb.dims_of(wl)
    buf = sb.alloc_buffers(dims, "cuda", logits=logits)
    sb.forward(dims, d["u"], d["w_router"], d["w_experts"], d["a"], d["h_init"], buf)
    torch.cuda.synchronize()
    return buf
