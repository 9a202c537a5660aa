"""Throughput of the Swimba mixer hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input:
route + top-k, expert projection with the mix epilogue, the chunked scan over
the batch (prefill), then one recurrent decode step of every sequence from
the prefill's final state. Inputs are resident in HBM before timing starts.

Prints ONE JSON line. ``value`` is tokens per second (prefill tokens plus the
decoded tokens) over the timed steps. ``roofline`` describes the kernel with
the largest share of the step (found in an untimed pass with events around
every kernel); inside the timed region the library records a HIP event pair
around each launch of that kernel only, on the stream it runs on.
``cpu_baseline`` is the fp64 oracle timed on a bounded sample of the same
workload on this host's cores.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

METRIC = "Swimba mixer tokens/sec on 1 MI355X + % of MFMA/HBM roofline"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16/fp16 matrix-core peak
PEAK_FP32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0


def workload(name):
    from selective_ssm_parameter_amd import synth
    return synth.WORKLOADS[name]


def kernel_models(wl):
    """Algorithmic work per launch of each kernel, for one prefill of ``wl``.

    Returns {kernel: (bound, flops, bytes)}. Bytes count each tensor a kernel
    must read or write once; flops count multiply-adds as 2."""
    M, D, E, k = wl.tokens, wl.d_model, wl.n_experts, wl.top_k
    H, P, N, G, L = wl.nheads, wl.headdim, wl.dstate, wl.ngroups, wl.chunk
    W, HP, GN = wl.width, H * P, G * N
    ei = 2 if wl.dtype == "bf16" else 4       # inputs, weights, y
    es = 2 if wl.dtype == "bf16" else 4       # streams (fp16 for bf16 inputs)
    pairs = M * k
    used_experts = E
    proj_bytes = (M * D * ei + used_experts * W * D * ei + pairs * (HP + GN) * es
                  + pairs * GN * 4 + pairs * 8)
    nc = -(-wl.seqlen // L)
    # causal (token, slot) pairs per chunk, per head: L(L+1)/2 * k
    causal = wl.batch * nc * L * (L + 1) // 2 * k
    scan_flops = (2 * causal * GN                     # Gram, shared by heads of a group
                  + 2 * causal * H * P                # masked y_intra
                  + 2 * M * H * N * P                 # readout of the entering state
                  + 2 * pairs * H * N * P)            # chunk carry
    scan_bytes = pairs * (HP + GN) * es + M * GN * es + M * HP * ei
    return {
        "route_topk": ("hbm", 2 * M * D * E, M * D * ei + E * D * ei + pairs * 8),
        "expert_project": ("mfma", 2 * pairs * D * W, proj_bytes),
        "scan_chunk_output": ("hbm", scan_flops, scan_bytes),
    }


def run_gpu(args):
    import torch

    from selective_ssm_parameter_amd import binding as sb
    from selective_ssm_parameter_amd import synth

    wl = workload(args.config)
    dev = "cuda:0"
    torch.cuda.set_device(0)
    inp = synth.make_inputs(wl)
    dt = torch.bfloat16 if wl.dtype == synth.BF16 else torch.float32

    def up(x, t=dt):
        return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(dev, t)

    u = up(inp["u"].reshape(wl.tokens, -1))
    wr, we, a = up(inp["w_router"]), up(inp["w_experts"]), up(inp["a"], torch.float32)
    dims = sb.dims_of(wl)
    buf = sb.alloc_buffers(dims, dev)
    ddims = sb.dims_of(wl, seqlen=1)
    dws, _ = sb.workspace(ddims, sb.CALL_DECODE, dev)
    u_dec = up(synth.decode_token(wl, 0))
    y_dec = torch.empty(wl.batch, wl.nheads, wl.headdim, dtype=dt, device=dev)
    stream = torch.cuda.current_stream()

    def step():
        # prefill the batch, then decode one more token of every sequence,
        # updating the prefill's final state in place
        sb.forward(dims, u, wr, we, a, None, buf)
        sb.swimba_decode_step(ddims, u_dec, wr, we, a, buf.h_final, y_dec, None, dws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # Per-kernel breakdown (events around every kernel), outside the timed region.
    sb.profile_select(None)
    sb.profile_enable(True)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    report = json.loads(sb.profile_report())
    sb.profile_enable(False)
    models = kernel_models(wl)
    kernels = {n: {"launches": r["launches"], "avg_us": 1e3 * r["ms"] / r["launches"]}
               for n, r in report.items()}
    dom = max((n for n in models if n in report), key=lambda n: report[n]["ms"])

    # Reference timing without any events (reported beside the value).
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed_plain = time.perf_counter() - t0

    # The timed region: the dominant kernel is bracketed by HIP events recorded
    # on the stream it runs on.
    sb.profile_select(dom)
    sb.profile_enable(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    rep_dom = json.loads(sb.profile_report())
    sb.profile_enable(False)
    sb.profile_select(None)

    tokens = wl.tokens + wl.batch
    value = tokens * args.steps / elapsed
    bound, flops, nbytes = models[dom]
    avg_s = rep_dom[dom]["ms"] / rep_dom[dom]["launches"] / 1e3
    if bound == "mfma":
        achieved = flops / avg_s / 1e12
        peak = PEAK_BF16_TFLOPS if wl.dtype == "bf16" else PEAK_FP32_TFLOPS
        roof = {"kernel": dom, "bound": "mfma", "achieved": achieved, "peak": peak,
                "unit": "TFLOP/s", "frac": achieved / peak, "traffic": None,
                "algorithmic_flops": flops, "avg_us": avg_s * 1e6}
    else:
        achieved = nbytes / avg_s / 1e9
        roof = {"kernel": dom, "bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": achieved / PEAK_HBM_GBS, "traffic": None,
                "algorithmic_bytes": nbytes, "avg_us": avg_s * 1e6}
    return {
        "wl": wl, "value": value, "elapsed": elapsed, "kernels": kernels, "roofline": roof,
        "value_without_events": tokens * args.steps / elapsed_plain,
    }


def cpu_baseline(wl, budget_s=20.0):
    """The fp64 oracle on a bounded sample: the first rows of the batch, all
    heads, whole sequences; rows are added until ``budget_s`` is used."""
    from oracle import swimba as osw
    from selective_ssm_parameter_amd import synth
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    inp = synth.make_inputs(wl)
    done_tokens, spent, rows = 0, 0.0, 0
    while rows < wl.batch and spent < budget_s:
        t0 = time.perf_counter()
        osw.forward(inp["u"][rows:rows + 1], inp["w_router"], inp["w_experts"], inp["a"], None,
                    nheads=wl.nheads, headdim=wl.headdim, ngroups=wl.ngroups,
                    dstate=wl.dstate, top_k=wl.top_k)
        spent += time.perf_counter() - t0
        done_tokens += wl.seqlen
        rows += 1
    return {"value": done_tokens / spent, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{rows} of {wl.batch} sequences x {wl.seqlen} tokens, all heads, "
                      f"prefill only, {spent:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="c2", choices=["c1", "c2", "c3", "c4"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1"}))
        sys.exit(2)
    r = run_gpu(args)
    wl = r["wl"]
    out = {
        "metric": METRIC,
        "value": r["value"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": 1e3 * r["elapsed"] / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {
            "workload": (f"Swimba mixer prefill + 1 decode step, {wl.dtype}: batch {wl.batch}, "
                         f"T={wl.seqlen}, d_model={wl.d_model}, heads={wl.nheads}, "
                         f"P={wl.headdim}, N={wl.dstate}, E={wl.n_experts}, "
                         f"top-k={wl.top_k}, chunk {wl.chunk}"),
            "global_batch": wl.batch, "seq_len": wl.seqlen, "parallelism": "none",
        },
        "roofline": r["roofline"],
        "kernels": r["kernels"],
        "value_without_events": r["value_without_events"],
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
