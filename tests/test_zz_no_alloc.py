"""The allocation-free decode step against the decode step with a caller
workspace: the same kernels, so the outputs must agree bit for bit, on two
calls in a row (the second on a smaller batch, so the scratch holds the first
call's larger contents when it starts)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from gpu_util import TOL, dev, host, say, slice_err, tdt, upload
from oracle import swimba as osw
from selective_ssm_parameter_amd import binding as sb
from selective_ssm_parameter_amd import synth

pytestmark = pytest.mark.gpu


def _case(wl, batch):
    w = wl.replace(batch=batch)
    inp = synth.make_inputs(w)
    rng = np.random.default_rng(900 + batch)
    inp["h_init"] = (rng.standard_normal((batch, w.nheads, w.dstate, w.headdim))
                     * np.sqrt(0.1)).astype(np.float32)
    return w, inp


@pytest.mark.parametrize("first,second", [(256, 37), (64, 5)])
def test_decode_noalloc_matches_workspace_call(first, second):
    base = synth.WORKLOADS["c5"].replace(name="noalloc", seed=777, d_model=512, n_experts=16)
    for batch in (first, second):
        wl, inp = _case(base, batch)
        say(f"[noalloc] batch {batch} E={wl.n_experts} k={wl.top_k}")
        d = upload(wl, inp)
        dims = sb.dims_of(wl)
        dt = tdt(wl)
        ut = dev(synth.decode_token(wl, 0), dt)
        h_ws, h_na = d["h_init"].clone(), d["h_init"].clone()
        y_ws = torch.empty(batch, wl.nheads, 64, dtype=dt, device="cuda")
        y_na = torch.full_like(y_ws, float("nan"))
        i_ws = torch.empty(batch, wl.top_k, dtype=torch.int32, device="cuda")
        i_na = torch.full_like(i_ws, -7)
        ws, _ = sb.workspace(dims, sb.CALL_DECODE)
        sb.swimba_decode_step(dims, ut, d["w_router"], d["w_experts"], d["a"], h_ws, y_ws, i_ws,
                              ws)
        sb.swimba_decode_step_noalloc(dims, ut, d["w_router"], d["w_experts"], d["a"], h_na,
                                      y_na, i_na)
        torch.cuda.synchronize()
        assert torch.equal(i_na, i_ws)
        assert torch.equal(y_na, y_ws)
        assert torch.equal(h_na, h_ws)
        # and both against the oracle on a few rows
        rows = [0, batch - 1]
        ref = osw.decode_step(synth.decode_token(wl, 0)[rows], inp["w_router"], inp["w_experts"],
                              inp["a"], inp["h_init"][rows].astype(np.float64),
                              nheads=wl.nheads, headdim=64, ngroups=1, dstate=wl.dstate,
                              top_k=wl.top_k)
        if not ref["routing"].flagged.any():
            assert slice_err(host(y_na)[rows][:, None], ref["y"][:, None]) < TOL[wl.dtype]


def test_decode_noalloc_rejects_oversized_dims():
    wl = synth.WORKLOADS["c5"].replace(batch=1024, top_k=8)
    dims = sb.dims_of(wl)
    need = sb.lib().swimba_workspace_size(dims, sb.CALL_DECODE)
    assert need > 32 << 20
    u = torch.zeros(8, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(sb.SwimbaError, match="SWIMBA_ERR_WORKSPACE"):
        sb.swimba_decode_step_noalloc(dims, u, u, u, u.float(), u.float(), u, None)
