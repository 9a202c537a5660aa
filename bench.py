"""Throughput of the Swimba mixer hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input:
route + top-k, expert projection with the mix epilogue, and the chunked scan
over the batch (prefill). The default workload is the largest prefill
(batch 4 x 8192 tokens, d_model 2048, 64 heads, E = 16, k = 2, chunk 128).
Inputs are resident in HBM before timing starts.
The recurrent decode workload (``--config c5``: batch 256, one token per
sequence per step, the N x P state of every head resident in HBM) times
decode steps alone: one step = one token of every sequence.

Prints ONE JSON line. ``value`` is tokens per second over the timed steps.
``roofline`` describes the kernel with the largest share of the step (found
in an untimed pass with events around every kernel): inside the timed region
the library records a HIP event pair around that kernel's launch, on the
stream it runs on, in one step of every EVENT_EVERY (each pair holds the
stream for ~10 us, so bracketing every step would inflate the step time the
value comes from); its average over those launches gives ``achieved``.
``roofline_scan`` is the scan's chunk-output kernel (the intra-chunk and
readout work), timed in the untimed pass. ``scan_pipeline`` sums the
scan's kernels (from the untimed pass) against the bytes the scan must move
at least: its input streams once and y once.
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


CALIB_BYTES = 256 << 20     # plain device-to-device copy used to scale HBM counters
CALIB_COPIES = 3
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "selective_ssm_parameter_amd", "csrc")
# Kernel symbol pattern -> the name the library's profiler gives the launch.
KERNEL_NAMES = [
    (r"pbwd_dz_kernel", "proj_bwd_dz"),
    (r"pbwd_router_kernel", "proj_bwd_router"),
    # (type, MODE): MODE 0 is du; the demangled name of MODE 1 varies
    (r"pbwd_gemm_kernel.*Li0EEE", "proj_bwd_du"),
    (r"pbwd_gemm_kernel", "proj_bwd_dw"),
    (r"pbwd_du_sum_kernel", "proj_bwd_du_sum"),
    (r"pbwd_dwr_sum_kernel", "proj_bwd_dwr_sum"),
    (r"pbwd_dwr_kernel", "proj_bwd_dwr"),
    (r"bwd_slice_sum_kernel", "scan_bwd_slice_sum"),
    (r"bwd_local_kernel", "scan_bwd_local"),
    (r"bwd_sweep_kernel", "scan_bwd_sweep"),
    (r"bwd_grad_kernel", "scan_bwd_grad"),
    (r"bwd_da_kernel", "scan_bwd_da"),
    (r"route_kernel|route_big_kernel", "route_topk"),
    (r"bucket_count_kernel", "bucket_count"),
    (r"bucket_place_kernel", "bucket_place"),
    # template arguments (type, tile config, PLAIN, ...): PLAIN right after the config
    (r"proj_kernel.*EEELb1E", "output_project"),
    (r"proj_kernel|proj_skinny_kernel", "expert_project"),
    (r"mix_c_kernel", "mix_c"),
    (r"mix_decay_kernel", "mix_decay"),
    (r"scan_gram_kernel", "scan_gram"),
    # (types, NP, KS, BT, WITH_Y, TV): WITH_Y follows the block size
    (r"scan_kernel.*Li\d+ELb0ELb[01]E|scan_carry_kernel", "scan_segment_state"),
    (r"scan_combine_kernel", "scan_state_pass"),
    (r"scan_kernel.*Li\d+ELb1ELb[01]E|scan_block_kernel", "scan_chunk_output"),
    (r"state_copy_kernel", "state_copy"),
    (r"sep_scatter_kernel", "sep_scatter"),
    (r"sep_sum_kernel", "sep_sum"),
    (r"decode_state_kernel", "decode_state"),
    (r"copyBuffer", "copy (runtime blit)"),
]
# Sources a kernel's machine code depends on (a change voids stored counters).
KERNEL_SOURCES = {
    "route_topk": ["route.hip"],
    "expert_project": ["project.hip"],
    "scan_chunk_output": ["scan.hip"],
    "decode_state": ["decode.hip"],
    "mix_decay": ["decay.hip"],
    "scan_bwd_grad": ["scan_bwd.hip"],
    "proj_bwd_du": ["proj_bwd.hip"],
    "proj_bwd_dw": ["proj_bwd.hip"],
}


def kernel_label(symbol):
    import re
    for pat, name in KERNEL_NAMES:
        if re.search(pat, symbol):
            return name
    return symbol[:60]


def source_digest(kernel):
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel] + ["common.hpp", "launch.hpp", "lds_tiles.hpp"]:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def profile_key(wl_name, decay="shared", backward=False):
    """Name of a workload's profile summaries: the expert-mixed decay runs
    other kernels (or the same ones with other work) and has its own, and so
    does the training step (forward + backward)."""
    return wl_name + ("_mixed" if decay == "mixed" else "") + ("_train" if backward else "")


def parse_key(key):
    """(workload name, mixed, backward) of a profile key."""
    backward = key.endswith("_train")
    key = key.removesuffix("_train")
    return key.removesuffix("_mixed"), key.endswith("_mixed"), backward


def traffic_file(key):
    return os.path.join(PROFILES, f"swimba_step_{key}_hbm_traffic.md")


def stored_traffic(kernel, key):
    """HBM bytes per launch of ``kernel`` from the committed counter summary
    of profile ``key``, or None when there is none or the kernel's sources
    changed since."""
    path = traffic_file(key)
    if kernel not in KERNEL_SOURCES or not os.path.exists(path):
        return None
    for line in open(path):
        parts = line.split()
        if len(parts) == 4 and parts[0] == "traffic:" and parts[1] == kernel:
            return int(parts[2]) if parts[3] == source_digest(kernel) else None
    return None


def workload(name):
    from selective_ssm_parameter_amd import synth
    return synth.WORKLOADS[name]


def is_decode(wl):
    return wl.decode_steps > 0


def kernel_models(wl, mixed=False):
    """Algorithmic work per launch of each kernel, for one prefill of ``wl``
    (one decode step for the decode workload). ``mixed``: the expert-mixed
    decay (its mixing kernel, and the scan reading the running log2 decay).

    Returns {kernel: (bound, flops, bytes)}. Bytes count each tensor a kernel
    must read or write once; flops count multiply-adds as 2."""
    if is_decode(wl):
        return decode_models(wl, mixed)
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
    models = {
        "route_topk": ("hbm", 2 * M * D * E, M * D * ei + E * D * ei + pairs * 8),
        "expert_project": ("mfma", 2 * pairs * D * W, proj_bytes),
        "scan_chunk_output": ("hbm", scan_flops, scan_bytes + (M * H * 4 if mixed else 0)),
    }
    if mixed:
        # reads the routing and the expert decays, writes the running log2 decay
        models["mix_decay"] = ("hbm", 2 * pairs * H, pairs * 8 + E * H * 4 + M * H * 4)
    return models


def decode_models(wl, mixed=False):
    """One decode step of every sequence: the state update reads and writes
    each head's fp32 N x P state once; the projection reads the weights of
    every expert some token chose (all E at this batch size)."""
    Bt, D, E, k = wl.batch, wl.d_model, wl.n_experts, wl.top_k
    H, P, N, G = wl.nheads, wl.headdim, wl.dstate, wl.ngroups
    W, HP, GN = wl.width, H * P, G * N
    ei = 2 if wl.dtype == "bf16" else 4
    es = 2 if wl.dtype == "bf16" else 4
    pairs = Bt * k
    state = 2 * Bt * H * N * P * 4
    streams = pairs * (HP + GN) * es + pairs * GN * 4
    return {
        "route_topk": ("hbm", 2 * Bt * D * E, Bt * D * ei + E * D * ei + pairs * 8),
        "expert_project": ("hbm", 2 * pairs * D * W,
                           Bt * D * ei + E * W * D * ei + streams + pairs * 8),
        "decode_state": ("hbm", 4 * pairs * H * N * P,
                         state + streams + Bt * HP * ei + (E * H * 4 + pairs * 8 if mixed else 0)),
    }


def backward_models(wl):
    """Algorithmic work per launch for one training step of prefill ``wl``:
    the forward's kernels (kernel_models) and the backward's. Scan backward
    per (chunk of L tokens, head), R = k L (token, slot) pairs, products
    restricted to causal pairs counted at half the dense cost:
      local:  S = B_hat^T X (2NPR), R = C~^T dy (2NPL)
      grad:   Gm = C~ B_hat^T (LRN, once per group), D = dy X^T (LRP),
              dX (PRL + 2PRN), dB_hat (NRL + 2NRP), dC~ (NLR + 2NLP)
    bytes: the streams and dy read once; the two local chunk-state sets
    [nc, H, N, P] written by local in the operand type (fp16 for bf16
    problems) and read by the sweep, which writes the entering states H_c and
    F_c for grad to read in the same type (fp16 rows with one fp32 factor per
    row of P for bf16 problems); the fp32 gradients written once. Projection
    backward: two grouped GEMMs of 2 (pairs) W D flops each; the dz kernel
    also copies each pair's token row of u into sorted order for the dW GEMM."""
    M, D, E, k = wl.tokens, wl.d_model, wl.n_experts, wl.top_k
    H, P, N, G = wl.nheads, wl.headdim, wl.dstate, wl.ngroups
    W, HP, GN = wl.width, H * P, G * N
    ei = 2 if wl.dtype == "bf16" else 4
    es = 2 if wl.dtype == "bf16" else 4
    pairs = M * k
    L = 64 if wl.dtype == "bf16" else 32
    nch = wl.batch * -(-wl.seqlen // L)          # chunks over the batch
    R = k * L
    states = nch * H * N * (P * es + (4 if es == 2 else 0))  # one entering-state set
    lstates = nch * H * N * P * es                # one local chunk-state set
    streams = pairs * (HP + GN) * es + M * GN * es
    dy = M * HP * ei
    grad_flops = nch * (G * L * R * N + H * (L * R * P + P * R * L + 2 * P * R * N + N * R * L
                                             + 2 * N * R * P + N * L * R + 2 * N * L * P))
    models = dict(kernel_models(wl))
    models.update({
        "scan_bwd_local": ("hbm", nch * H * (2 * N * P * R + 2 * N * P * L),
                           streams + dy + 2 * lstates),
        "scan_bwd_sweep": ("hbm", 0, 2 * lstates + 2 * states),
        "scan_bwd_grad": ("hbm", grad_flops,
                          streams + dy + 2 * states + pairs * (HP + GN) * 4 + M * GN * 4),
        "proj_bwd_dz": ("hbm", 0, pairs * (HP + GN) * 4 + M * GN * 4 + pairs * GN * (es + 4)
                        + pairs * W * ei + pairs * 8 + 2 * pairs * D * ei),
        "proj_bwd_router": ("hbm", 2 * M * E * D, M * E * 4 + pairs * 8 + E * D * ei
                            + M * D * 4 + M * E * 4),
        "proj_bwd_du": ("mfma", 2 * pairs * W * D, pairs * W * ei + E * W * D * ei
                        + pairs * D * 4),
        "proj_bwd_du_sum": ("hbm", 0, pairs * D * 4 + 2 * M * D * 4),
        "proj_bwd_dw": ("mfma", 2 * pairs * W * D, pairs * W * ei + pairs * D * ei
                        + E * W * D * 4),
        "proj_bwd_dwr": ("hbm", 2 * M * E * D, M * E * 4 + M * D * ei + E * D * 4),
    })
    return models


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

    wr, we, a = up(inp["w_router"]), up(inp["w_experts"]), up(inp["a"], torch.float32)
    mixed = getattr(args, "decay", "shared") == "mixed"
    backward = getattr(args, "backward", False)
    a_exp = up(synth.expert_decays(wl), torch.float32) if mixed else None
    if not is_decode(wl):
        u = up(inp["u"].reshape(wl.tokens, -1))
        dims = sb.dims_of(wl)
        buf = sb.alloc_buffers(dims, dev)
    ddims = sb.dims_of(wl, seqlen=1)
    if is_decode(wl):
        dws, _ = sb.workspace(ddims, sb.CALL_DECODE, dev)
        y_dec = torch.empty(wl.batch, wl.nheads, wl.headdim, dtype=dt, device=dev)
    stream = torch.cuda.current_stream()

    if is_decode(wl):
        # decode only: the state starts from the workload's initial state and
        # is updated in place; tokens cycle through a few seeded draws
        h_state = up(inp["h_init"], torch.float32)
        toks = [up(synth.decode_token(wl, i)) for i in range(8)]
        count = [0]

        def step():
            if mixed:
                sb.swimba_decode_step_mixed(ddims, toks[count[0] % len(toks)], wr, we, a_exp,
                                            h_state, y_dec, None, dws)
            else:
                sb.swimba_decode_step(ddims, toks[count[0] % len(toks)], wr, we, a, h_state,
                                      y_dec, None, dws)
            count[0] += 1
    else:
        log_decay = (torch.empty(wl.batch, wl.nheads, wl.seqlen, dtype=torch.float32, device=dev)
                     if mixed else None)
        if backward:
            # the forward keeps its routing (with logits), B_hat and projection
            # workspace for the backward, which reuses them
            dy = up(synth.output_gradient(wl))
            buf = sb.alloc_buffers(dims, dev, logits=True)
            grads = sb.alloc_grads(dims, dev, saved=True)

        def step():
            if backward:
                # training step: the prefill forward, then every gradient of
                # <dy, y> (u, W_r, W_exp, a, the initial state)
                sb.forward(dims, u, wr, we, a, None, buf)
                sb.backward(dims, u, wr, we, a, None, dy, None, buf, grads, saved=True)
                return
            # prefill the batch
            if mixed:
                sb.forward_mixed(dims, u, wr, we, a_exp, None, buf, log_decay)
            else:
                sb.forward(dims, u, wr, we, a, None, buf)

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
    if is_decode(wl):  # the library names decode launches decode_<kernel>
        report = {n[len("decode_"):]: r for n, r in report.items() if n.startswith("decode_")}
    models = backward_models(wl) if backward else kernel_models(wl, mixed)
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
    # on the stream it runs on, in one step of every EVENT_EVERY.
    sb.profile_select(("decode_" if is_decode(wl) else "") + dom)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        sb.profile_enable(i % EVENT_EVERY == 0)
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    rep_dom = json.loads(sb.profile_report())
    if is_decode(wl):
        rep_dom = {n[len("decode_"):]: r for n, r in rep_dom.items() if n.startswith("decode_")}
    sb.profile_enable(False)
    sb.profile_select(None)

    if args.copy_calibration:
        # A plain copy of known size, last in the process, to scale the HBM
        # byte counters of the kernels above.
        src = torch.ones(CALIB_BYTES // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(CALIB_COPIES):
            dst.copy_(src)
        torch.cuda.synchronize()

    tokens = wl.batch if is_decode(wl) else wl.tokens
    value = tokens * args.steps / elapsed
    key = profile_key(wl.name, "mixed" if mixed else "shared", backward)

    def roofline(name, rep):
        bound, flops, nbytes = models[name]
        avg_s = rep[name]["ms"] / rep[name]["launches"] / 1e3
        if bound == "mfma":
            achieved = flops / avg_s / 1e12
            peak = PEAK_BF16_TFLOPS if wl.dtype == "bf16" else PEAK_FP32_TFLOPS
            return {"kernel": name, "bound": "mfma", "achieved": achieved, "peak": peak,
                    "unit": "TFLOP/s", "frac": achieved / peak,
                    "traffic": stored_traffic(name, key),
                    "algorithmic_flops": flops, "avg_us": avg_s * 1e6}
        achieved = nbytes / avg_s / 1e9
        return {"kernel": name, "bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": achieved / PEAK_HBM_GBS,
                "traffic": stored_traffic(name, key),
                "algorithmic_bytes": nbytes, "avg_us": avg_s * 1e6,
                "algorithmic_flops": flops,
                "mfma_frac": flops / avg_s / 1e12 / PEAK_BF16_TFLOPS}

    res = {
        "wl": wl, "value": value, "elapsed": elapsed, "kernels": kernels,
        "roofline": roofline(dom, rep_dom),
        "value_without_events": tokens * args.steps / elapsed_plain,
    }
    if SCAN_KERNEL in report and SCAN_KERNEL != dom:
        res["roofline_scan"] = roofline(SCAN_KERNEL, report)
    if not is_decode(wl) and not backward:
        # the scan's kernels together against the bytes it must move at least
        names = [n for n in SCAN_PIPELINE if n in kernels]
        us = sum(kernels[n]["avg_us"] for n in names)
        nbytes = models[SCAN_KERNEL][2]
        res["scan_pipeline"] = {"kernels": names, "avg_us": us, "bound": "hbm",
                                "algorithmic_bytes": nbytes,
                                "achieved": nbytes / us / 1e3, "unit": "GB/s",
                                "frac": nbytes / us / 1e3 / PEAK_HBM_GBS}
    if is_decode(wl):
        # Every kernel of a decode step is bound by HBM, and a kernel's time
        # also carries the write-back of dirty lines the one before it left
        # (the state update's writes drain while the next step's projection
        # reads): the whole step's algorithmic bytes over the step time.
        step_bytes = sum(m[2] for m in models.values())
        step_s = elapsed / args.steps
        res["step_roofline"] = {"bound": "hbm", "achieved": step_bytes / step_s / 1e9,
                                "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                "frac": step_bytes / step_s / 1e9 / PEAK_HBM_GBS,
                                "algorithmic_bytes": step_bytes}
    return res


SCAN_KERNEL = "scan_chunk_output"
EVENT_EVERY = 4  # timed steps per step with events around the dominant kernel
SCAN_PIPELINE = ("scan_gram", "scan_segment_state", "scan_state_pass", "scan_chunk_output")
E_SWEEP = (4, 8, 16, 32, 64)


def e_sweep(args):
    """Prefill tokens/s at the c3 dimensions with E experts, k = 2, for each E
    in E_SWEEP (seed 30 + E): the recurrence has no E term and projection
    FLOPs depend on k only, so only the weight bytes and the router grow with
    E. Prints one JSON line per E and writes a markdown table."""
    import torch

    from selective_ssm_parameter_amd import binding as sb
    from selective_ssm_parameter_amd import synth

    dev = "cuda:0"
    torch.cuda.set_device(0)
    rows = []
    for E in E_SWEEP:
        wl = synth.WORKLOADS["c3"].replace(name=f"c3_E{E}", seed=30 + E, n_experts=E)
        inp = synth.make_inputs(wl)

        def up(x, t=torch.bfloat16):
            return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(dev, t)

        u = up(inp["u"].reshape(wl.tokens, -1))
        wr, we, a = up(inp["w_router"]), up(inp["w_experts"]), up(inp["a"], torch.float32)
        del inp
        dims = sb.dims_of(wl)
        buf = sb.alloc_buffers(dims, dev)
        for _ in range(args.warmup):
            sb.forward(dims, u, wr, we, a, None, buf)
        torch.cuda.synchronize()
        sb.profile_select(None)
        sb.profile_enable(True)
        for _ in range(args.steps):
            sb.forward(dims, u, wr, we, a, None, buf)
        torch.cuda.synchronize()
        report = json.loads(sb.profile_report())
        sb.profile_enable(False)
        t0 = time.perf_counter()
        for _ in range(args.steps):
            sb.forward(dims, u, wr, we, a, None, buf)
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
        kern = {n: 1e3 * r["ms"] / r["launches"] for n, r in report.items()}
        row = {"E": E, "k": wl.top_k, "tokens_per_s": wl.tokens * args.steps / elapsed,
               "ms_per_step": 1e3 * elapsed / args.steps, "kernels_us": kern,
               "weight_MB": E * wl.width * wl.d_model * 2 / 1e6}
        rows.append(row)
        print(json.dumps(row), flush=True)
        del u, wr, we, a, buf
        torch.cuda.empty_cache()
    if args.out:
        base = rows[0]["tokens_per_s"]
        names = [n for n in rows[0]["kernels_us"]]
        lines = ["# Prefill tokens/s against the number of experts (c3 dimensions, k = 2)", "",
                 "Command (from the repository root, after building the library):", "",
                 "    " + (" ".join(args.command) or "python bench.py --e-sweep"), "",
                 f"Batch 4 x T 8192 tokens, d_model 2048, 64 heads, P 64, N 128, chunk 128, "
                 f"bf16; seed 30 + E; {args.steps} timed steps after {args.warmup} warm-up "
                 "steps; per-kernel times from HIP events around each launch in a separate "
                 "pass.", "",
                 "| E | weights MB | tokens/s (M) | vs E=4 | ms/step | "
                 + " | ".join(n + " us" for n in names) + " |",
                 "|---:|---:|---:|---:|---:|" + "---:|" * len(names)]
        for r in rows:
            lines.append(f"| {r['E']} | {r['weight_MB']:.0f} | {r['tokens_per_s'] / 1e6:.2f} | "
                         f"{r['tokens_per_s'] / base:.3f} | {r['ms_per_step']:.3f} | "
                         + " | ".join(f"{r['kernels_us'].get(n, 0):.1f}" for n in names) + " |")
        open(args.out, "w").write("\n".join(lines) + "\n")


def library_gemm(args):
    """The fused expert projection beside the vendor GEMM library (hipBLASLt,
    through torch.mm) on the same shapes, for c2, c3 and c4: the library's
    dense GEMM of all (token, slot) rows against one expert's weights (the
    same FLOPs with no routing, gather or mix), and one library GEMM per
    expert over an equal share of the rows (the unfused grouped form). Writes
    a markdown table; a context for the projection's roofline fraction."""
    import torch

    from selective_ssm_parameter_amd import binding as sb
    from selective_ssm_parameter_amd import synth

    dev = "cuda:0"
    torch.cuda.set_device(0)

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return 1e3 * e0.elapsed_time(e1) / args.steps

    rows = []
    for name in ("c2", "c3", "c4"):
        wl = synth.WORKLOADS[name]
        inp = synth.make_inputs(wl)

        def up(x, t=torch.bfloat16):
            return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(dev, t)

        u = up(inp["u"].reshape(wl.tokens, -1))
        wr, we, a = up(inp["w_router"]), up(inp["w_experts"]), up(inp["a"], torch.float32)
        del inp
        dims = sb.dims_of(wl)
        buf = sb.alloc_buffers(dims, dev)
        for _ in range(args.warmup):
            sb.forward(dims, u, wr, we, a, None, buf)
        torch.cuda.synchronize()
        sb.profile_select("expert_project")
        sb.profile_enable(True)
        for _ in range(args.steps):
            sb.forward(dims, u, wr, we, a, None, buf)
        torch.cuda.synchronize()
        rep = json.loads(sb.profile_report())["expert_project"]
        sb.profile_enable(False)
        sb.profile_select(None)
        ours = 1e3 * rep["ms"] / rep["launches"]
        del buf
        R, D, W, E = wl.tokens * wl.top_k, wl.d_model, wl.width, wl.n_experts
        A = torch.randn(R, D, device=dev, dtype=torch.bfloat16)
        out = torch.empty(R, W, device=dev, dtype=torch.bfloat16)
        dense = timed(lambda: torch.mm(A, we[0].t(), out=out))
        share = R // E
        parts = [(A[e * share:(e + 1) * share], out[e * share:(e + 1) * share]) for e in range(E)]

        def grouped():
            for e, (ae, oe) in enumerate(parts):
                torch.mm(ae, we[e].t(), out=oe)
        per_expert = timed(grouped)
        flops = 2.0 * R * D * W
        row = {"workload": name, "rows": R, "d_model": D, "width": W, "E": E,
               "fused_us": ours, "library_dense_us": dense, "library_per_expert_us": per_expert,
               "fused_frac": flops / ours / 1e6 / PEAK_BF16_TFLOPS,
               "dense_frac": flops / dense / 1e6 / PEAK_BF16_TFLOPS,
               "per_expert_frac": flops * (share * E / R) / per_expert / 1e6 / PEAK_BF16_TFLOPS}
        rows.append(row)
        print(json.dumps(row), flush=True)
        del u, wr, we, a, A, out, parts
        torch.cuda.empty_cache()
    if args.out:
        lines = ["# Expert projection beside the vendor GEMM library", "",
                 "Command (from the repository root, after building the library):", "",
                 "    " + (" ".join(args.command) or "python bench.py --library-gemm"), "",
                 "fused: `expert_project` of a prefill step (routing gather, the w-weighted "
                 "B and C epilogue and the stream writes included), HIP events around each "
                 "launch. library dense: one `torch.mm` (hipBLASLt) of all k M rows against "
                 "one expert's [W, d_model] weights, bf16 out. library per expert: one "
                 "`torch.mm` per expert over M k / E rows each. Fractions of the 2500 "
                 f"TFLOP/s dense bf16 peak; {args.steps} timed calls after {args.warmup} "
                 "warm-up calls.", "",
                 "| workload | rows k M | d_model | W | E | fused us | frac | library dense us "
                 "| frac | library per expert us | frac |",
                 "|---|---:|---:|---:|---:|---:|---:|---:|---:|---:|---:|"]
        for r in rows:
            lines.append(f"| {r['workload']} | {r['rows']} | {r['d_model']} | {r['width']} | "
                         f"{r['E']} | {r['fused_us']:.1f} | {r['fused_frac']:.3f} | "
                         f"{r['library_dense_us']:.1f} | {r['dense_frac']:.3f} | "
                         f"{r['library_per_expert_us']:.1f} | {r['per_expert_frac']:.3f} |")
        open(args.out, "w").write("\n".join(lines) + "\n")


SEP_POINTS = [(2, 2), (4, 2), (8, 2), (16, 2), (32, 2), (8, 1), (8, 4)]


def separated_sweep(args):
    """Prefill tokens/s of the MoE over separated SSMs (one state trajectory
    per expert) beside Swimba's single trajectory, at the c2 dimensions
    (batch 8 x 2048 tokens, d_model 768, 24 heads, chunk 64) for each
    (E, k) in SEP_POINTS (seed 40 + E + 100 k). One JSON line per point and a
    markdown table: the separated layer's cost grows with E (its E
    trajectories are all scanned), Swimba's does not."""
    import torch

    from selective_ssm_parameter_amd import binding as sb
    from selective_ssm_parameter_amd import synth

    dev = "cuda:0"
    torch.cuda.set_device(0)
    rows = []

    def timed(fn, steps, warmup):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        sb.profile_select(None)
        sb.profile_enable(True)
        fn()
        torch.cuda.synchronize()
        rep = json.loads(sb.profile_report())
        sb.profile_enable(False)
        t0 = time.perf_counter()
        for _ in range(steps):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / steps, {n: 1e3 * r["ms"] / r["launches"]
                                                    for n, r in rep.items()}

    for E, k in SEP_POINTS:
        wl = synth.WORKLOADS["c2"].replace(name=f"c2_E{E}_k{k}", seed=40 + E + 100 * k,
                                           n_experts=E, top_k=k)
        inp = synth.make_inputs(wl)

        def up(x, t=torch.bfloat16):
            return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(dev, t)

        u = up(inp["u"].reshape(wl.tokens, -1))
        wr, we, a = up(inp["w_router"]), up(inp["w_experts"]), up(inp["a"], torch.float32)
        del inp
        dims = sb.dims_of(wl)
        buf = sb.alloc_buffers(dims, dev)
        sbuf = sb.alloc_separated(dims, dev)
        t_mix, k_mix = timed(lambda: sb.forward(dims, u, wr, we, a, None, buf), args.steps,
                             args.warmup)
        t_sep, k_sep = timed(lambda: sb.separated_forward(dims, u, wr, we, a, None, sbuf),
                             args.steps, args.warmup)
        row = {"E": E, "k": k, "swimba_tokens_per_s": wl.tokens / t_mix,
               "separated_tokens_per_s": wl.tokens / t_sep, "swimba_ms": 1e3 * t_mix,
               "separated_ms": 1e3 * t_sep, "swimba_kernels_us": k_mix,
               "separated_kernels_us": k_sep,
               "state_MB": {"swimba": wl.batch * wl.nheads * wl.dstate * wl.headdim * 4 / 1e6,
                            "separated": E * wl.batch * wl.nheads * wl.dstate * wl.headdim
                            * 4 / 1e6}}
        rows.append(row)
        print(json.dumps(row), flush=True)
        del u, wr, we, a, buf, sbuf
        torch.cuda.empty_cache()
    if args.out:
        lines = ["# Separated-SSM MoE against Swimba: prefill tokens/s against E and k "
                 "(c2 dimensions)", "",
                 "Command (from the repository root, after building the library):", "",
                 "    " + (" ".join(args.command) or "python bench.py --separated"), "",
                 "Batch 8 x T 2048 tokens, d_model 768, 24 heads, P 64, N 128, chunk 64, bf16; "
                 "seed 40 + E + 100 k. Swimba: one state trajectory per head (route, project + "
                 "mix, scan). Separated: one trajectory per expert and head (route, the same "
                 "projection of the selected pairs, per-expert streams, Bt x E scans of k = 1, "
                 f"the sum over experts). {args.steps} timed steps after {args.warmup} warm-up "
                 "steps each; per-kernel times from HIP events in one extra pass.", "",
                 "| E | k | Swimba tokens/s (M) | separated tokens/s (M) | separated / Swimba "
                 "time | Swimba scan us | separated scan us | state MB (Swimba / separated) |",
                 "|---:|---:|---:|---:|---:|---:|---:|---:|"]
        scan = ("scan_gram", "scan_segment_state", "scan_state_pass", "scan_chunk_output")
        for r in rows:
            sm = sum(r["swimba_kernels_us"].get(n, 0) for n in scan)
            ss = sum(r["separated_kernels_us"].get(n, 0) for n in scan)
            lines.append(f"| {r['E']} | {r['k']} | {r['swimba_tokens_per_s'] / 1e6:.2f} | "
                         f"{r['separated_tokens_per_s'] / 1e6:.2f} | "
                         f"{r['separated_ms'] / r['swimba_ms']:.2f} | {sm:.1f} | {ss:.1f} | "
                         f"{r['state_MB']['swimba']:.0f} / {r['state_MB']['separated']:.0f} |")
        open(args.out, "w").write("\n".join(lines) + "\n")


def output_projection(args):
    """The output projection after the recurrence on every token of the
    workload (out = W_out y, [M, H*P] -> [M, D]): one JSON line with its
    TFLOP/s and fraction of the matrix-core peak, and the oracle's rate on a
    sample of rows."""
    import torch

    from oracle import swimba as osw
    from selective_ssm_parameter_amd import binding as sb
    from selective_ssm_parameter_amd import synth

    wl = workload(args.config)
    dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    K = wl.nheads * wl.headdim
    inp = synth.output_projection_inputs(wl)
    y = torch.from_numpy(inp["y"].reshape(wl.tokens, K)).to("cuda:0", dt)
    w = torch.from_numpy(inp["w_out"]).to("cuda:0", dt)
    out = torch.empty(wl.tokens, wl.d_model, dtype=dt, device="cuda:0")
    dims = sb.dims_of(wl)
    for _ in range(args.warmup):
        sb.swimba_output_project(dims, y, w, out)
    torch.cuda.synchronize()
    sb.profile_select("output_project")
    sb.profile_enable(True)
    for _ in range(args.steps):
        sb.swimba_output_project(dims, y, w, out)
    torch.cuda.synchronize()
    rep = json.loads(sb.profile_report())["output_project"]
    sb.profile_enable(False)
    sb.profile_select(None)
    avg_s = rep["ms"] / rep["launches"] / 1e3
    flops = 2 * wl.tokens * K * wl.d_model
    peak = PEAK_BF16_TFLOPS if wl.dtype == "bf16" else PEAK_FP32_TFLOPS
    rows = min(wl.tokens, 2048)
    t0 = time.perf_counter()
    osw.output_project(inp["y"][:rows], inp["w_out"])
    cpu_s = time.perf_counter() - t0
    print(json.dumps({
        "metric": "Swimba output projection tokens/sec on 1 MI355X", "value": wl.tokens / avg_s,
        "unit": "tokens/s", "dtype": wl.dtype, "data": "synthetic",
        "config": {"workload": f"output projection of {args.config}: M={wl.tokens}, "
                               f"H*P={K} -> d_model={wl.d_model}"},
        "roofline": {"bound": "mfma", "achieved": flops / avg_s / 1e12, "peak": peak,
                     "unit": "TFLOP/s", "frac": flops / avg_s / 1e12 / peak,
                     "avg_us": avg_s * 1e6, "algorithmic_flops": flops},
        "cpu_baseline": {"value": rows / cpu_s, "unit": "tokens/s", "kind": "oracle",
                         "sample": f"first {rows} tokens, {cpu_s:.2f} s"}}), flush=True)


def cpu_baseline(wl, budget_s=20.0, mixed=False):
    """The fp64 oracle on a bounded sample: the first rows of the batch, all
    heads, whole sequences; rows are added until ``budget_s`` is used."""
    from oracle import mixed_decay as md
    from oracle import swimba as osw
    from selective_ssm_parameter_amd import synth
    if is_decode(wl):
        return cpu_baseline_decode(wl, budget_s, mixed)
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    inp = synth.make_inputs(wl)
    done_tokens, spent, rows = 0, 0.0, 0
    while rows < wl.batch and spent < budget_s:
        t0 = time.perf_counter()
        if mixed:
            md.forward_tv(inp["u"][rows:rows + 1], inp["w_router"], inp["w_experts"],
                          synth.expert_decays(wl), None, nheads=wl.nheads, headdim=wl.headdim,
                          ngroups=wl.ngroups, dstate=wl.dstate, top_k=wl.top_k)
        else:
            osw.forward(inp["u"][rows:rows + 1], inp["w_router"], inp["w_experts"], inp["a"],
                        None, nheads=wl.nheads, headdim=wl.headdim, ngroups=wl.ngroups,
                        dstate=wl.dstate, top_k=wl.top_k)
        spent += time.perf_counter() - t0
        done_tokens += wl.seqlen
        rows += 1
    return {"value": done_tokens / spent, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{rows} of {wl.batch} sequences x {wl.seqlen} tokens, all heads, "
                      f"prefill only, {spent:.1f} s"}


def cpu_baseline_backward(wl, budget_s=20.0):
    """The fp64 oracle's forward + backward (forward_backward) on prefixes of
    sequence 0 (128, 256, ... tokens, all heads), until ``budget_s`` is used."""
    from oracle import backward as ob
    from selective_ssm_parameter_amd import synth
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    inp = synth.make_inputs(wl)
    dy = synth.output_gradient(wl).reshape(wl.batch, wl.seqlen, wl.nheads, wl.headdim)
    done, spent, T, runs = 0, 0.0, 128, []
    while spent < budget_s:
        T = min(T, wl.seqlen)
        t0 = time.perf_counter()
        ob.forward_backward(inp["u"][:1, :T], inp["w_router"], inp["w_experts"], inp["a"], None,
                            dy[:1, :T], None, nheads=wl.nheads, headdim=wl.headdim,
                            ngroups=wl.ngroups, dstate=wl.dstate, top_k=wl.top_k)
        spent += time.perf_counter() - t0
        done += T
        runs.append(T)
        if T == wl.seqlen:
            break
        T *= 2
    return {"value": done / spent, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"forward + backward of the first {', '.join(map(str, runs))} tokens of "
                      f"sequence 0, all heads, {spent:.1f} s"}


def cpu_baseline_decode(wl, budget_s, mixed=False):
    """The fp64 oracle's decode step on growing slices of the batch (all
    heads, the workload's initial state) until ``budget_s`` is used."""
    from oracle import swimba as osw
    from selective_ssm_parameter_amd import synth
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    from oracle import mixed_decay as md
    inp = synth.make_inputs(wl)
    ae = synth.expert_decays(wl)
    done, spent, step, rows = 0, 0.0, 0, 8
    while spent < budget_s and step < wl.decode_steps:
        u_t = synth.decode_token(wl, step)[:rows]
        t0 = time.perf_counter()
        if mixed:
            md.decode_step_tv(u_t, inp["w_router"], inp["w_experts"], ae, inp["h_init"][:rows],
                              nheads=wl.nheads, headdim=wl.headdim, ngroups=wl.ngroups,
                              dstate=wl.dstate, top_k=wl.top_k)
        else:
            osw.decode_step(u_t, inp["w_router"], inp["w_experts"], inp["a"],
                            inp["h_init"][:rows], nheads=wl.nheads, headdim=wl.headdim,
                            ngroups=wl.ngroups, dstate=wl.dstate, top_k=wl.top_k)
        spent += time.perf_counter() - t0
        done += rows
        step += 1
    return {"value": done / spent, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{step} decode steps of {rows} of {wl.batch} sequences, all heads, "
                      f"{spent:.1f} s"}


def find_csv(d, suffix):
    import glob
    hits = sorted(glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True))
    if not hits:
        sys.exit(f"no *{suffix} under {d}")
    return hits[0]


def summarize_trace(trace_dir, wl_name, out, command, bench_json=None):
    """Per-kernel durations from a ``rocprofv3 --kernel-trace --stats`` run,
    grouped by kernel and grid size (prefill and decode launch the same
    kernels on different grids)."""
    import csv
    import collections
    rows = list(csv.DictReader(open(find_csv(trace_dir, "kernel_trace.csv"))))
    groups = collections.OrderedDict()
    for r in rows:
        key = (kernel_label(r["Kernel_Name"]), int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"])
               * int(r["Grid_Size_Z"]) // max(1, int(r["Workgroup_Size_X"])
                                            * int(r["Workgroup_Size_Y"])
                                            * int(r["Workgroup_Size_Z"])))
        groups.setdefault(key, []).append(
            (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    total = sum(sum(v) for v in groups.values())
    stats = find_csv(trace_dir, "kernel_stats.csv")
    base, mixed, backward = parse_key(wl_name)
    kind = ("decode steps" if is_decode(workload(base)) else
            "training step (prefill forward + backward)" if backward else
            "bench step (prefill)")
    what = f"workload {base}" + (", expert-mixed decay" if mixed else "")
    lines = [f"# Kernel durations, {kind} on {what}", "",
             "Command (from the repository root, after building the library):", "",
             "    " + command, "",
             f"Source: `{os.path.basename(stats)}` and the kernel trace of that run; "
             "durations in microseconds, grouped by kernel and workgroup count.", "",
             "| kernel | workgroups | launches | avg us | min us | max us | share |",
             "|---|---:|---:|---:|---:|---:|---:|"]
    for (name, wgs), v in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
        lines.append(f"| {name} | {wgs} | {len(v)} | {sum(v) / len(v):.1f} | {min(v):.1f} | "
                     f"{max(v):.1f} | {100 * sum(v) / total:.1f}% |")
    if bench_json:
        line = [ln for ln in open(bench_json) if ln.startswith("{")][-1]
        roof = json.loads(line)["roofline"]
        lines += ["", f"The JSON line of the same run reports, for its dominant kernel "
                      f"{roof['kernel']}, an average of {roof['avg_us']:.1f} us per launch "
                      f"(HIP events on the launch stream, one timed step in four) and "
                      f"{roof['achieved']:.1f} {roof['unit']} = {100 * roof['frac']:.1f}% "
                      f"of the {roof['peak']:.0f} {roof['unit']} peak."]
    open(out, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize_pmc(fetch_dir, write_dir, wl_name, out, commands):
    """HBM bytes per launch from FETCH_SIZE and WRITE_SIZE runs, each scaled by
    what the same counter reads for the trailing copy of CALIB_BYTES."""
    import csv
    import collections

    def per_dispatch(d, counter):
        vals, names = collections.defaultdict(float), {}
        for r in csv.DictReader(open(find_csv(d, "counter_collection.csv"))):
            if r["Counter_Name"] != counter:
                continue
            i = int(r["Dispatch_Id"])
            vals[i] += float(r["Counter_Value"])
            wgs = (int(r["Grid_Size"]) // max(1, int(r["Workgroup_Size"])))
            names[i] = (kernel_label(r["Kernel_Name"]), wgs)
        return vals, names

    res = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        vals, names = per_dispatch(d, counter)
        last_lib = max(i for i, n in names.items() if not n[0].startswith("copy"))
        calib = [i for i, n in names.items() if n[0].startswith("copy") and i > last_lib]
        if not calib:
            sys.exit(f"no calibration copy after the last library kernel in {d}")
        kib = sum(vals[i] for i in calib) / CALIB_COPIES
        scale = CALIB_BYTES / (kib * 1024.0)
        by = collections.defaultdict(list)
        known = {name for _, name in KERNEL_NAMES}
        for i, n in names.items():
            if i not in calib and n[0] in known and not n[0].startswith("copy"):
                by[n].append(vals[i] * 1024.0 * scale)
        res[counter] = (kib, scale, {k: sum(v) / len(v) for k, v in by.items()})
    fk, fs, fetch = res["FETCH_SIZE"]
    wk, ws_, write = res["WRITE_SIZE"]
    base, mixed, backward = parse_key(wl_name)
    wl = workload(base)
    models = backward_models(wl) if backward else kernel_models(wl, mixed)
    what = f"workload {base}" + (", expert-mixed decay" if mixed else "")
    step = "training step" if backward else "bench step"
    lines = [f"# HBM traffic per launch, {step} on {what}", "",
             "Commands (from the repository root, after building the library):", ""]
    lines += ["    " + c for c in commands]
    lines += ["",
              f"Calibration: the run ends with {CALIB_COPIES} device copies of "
              f"{CALIB_BYTES >> 20} MiB; per copy FETCH_SIZE read {fk:.0f} KiB (scale {fs:.4f}) "
              f"and WRITE_SIZE {wk:.0f} KiB (scale {ws_:.4f}). Counter KiB x 1024 x scale "
              "= bytes.", "",
              ("Every launch is a decode step's." if is_decode(wl) else
               "The forward's kernels launch twice per step (the backward recomputes the "
               "routing and the projection); the algorithmic bytes are per launch."
               if backward else
               "Every launch is the prefill's; the algorithmic bytes are per launch."), "",
              "| kernel | workgroups | read MB | written MB | traffic MB | algorithmic MB |",
              "|---|---:|---:|---:|---:|---:|"]
    keys = sorted(set(fetch) | set(write), key=lambda k: -(fetch.get(k, 0) + write.get(k, 0)))
    best = {}
    for k in keys:
        rd, wr = fetch.get(k, 0.0), write.get(k, 0.0)
        big = k[0] in models and k[1] == max(kk[1] for kk in keys if kk[0] == k[0])
        alg = f"{models[k[0]][2] / 1e6:.1f}" if big else "-"
        lines.append(f"| {k[0]} | {k[1]} | {rd / 1e6:.1f} | {wr / 1e6:.1f} | "
                     f"{(rd + wr) / 1e6:.1f} | {alg} |")
        if k[0] in KERNEL_SOURCES and (k[0] not in best or k[1] > best[k[0]][0]):
            best[k[0]] = (k[1], rd + wr)
    lines += ["", "Machine-readable (kernel, bytes per launch at the largest grid, "
              "digest of the sources the kernel is built from):", ""]
    for k, (_, b) in sorted(best.items()):
        lines.append(f"traffic: {k} {int(round(b))} {source_digest(k)}")
    open(out, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


# Counter passes of the SQ summary (each within one rocprofv3 --pmc run's
# hardware limits: at most 8 SQ, 2 TA and 2 GRBM counters).
SQ_PASSES = [
    "SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_INSTS_VALU_MFMA_MOPS_F16 "
    "SQ_INSTS_MFMA SQ_INSTS_VALU SQ_INSTS_SALU SQ_INSTS_LDS SQ_WAVES GRBM_GUI_ACTIVE",
    "SQ_WAVE_CYCLES SQ_WAIT_INST_ANY SQ_WAIT_INST_LDS SQ_LDS_BANK_CONFLICT "
    "SQ_INSTS_LDS_LOAD_BANDWIDTH SQ_ACTIVE_INST_VALU SQ_ACTIVE_INST_LDS SQ_ACTIVE_INST_SCA "
    "TA_TA_BUSY GRBM_GUI_ACTIVE",
]
N_XCD, N_CU, N_SIMD = 8, 256, 1024


def summarize_sq(dirs, wl_name, out, commands):
    """Matrix-core and issue counters per kernel from rocprofv3 --pmc runs of
    the SQ_PASSES sets: per-dispatch averages, and the derived figures
    (MFMA busy per SIMD, the clock the run held, instruction mix per wave,
    issue stalls, LDS read rate, texture-unit busy)."""
    import csv
    import collections
    vals = collections.defaultdict(lambda: collections.defaultdict(list))
    durs = collections.defaultdict(list)
    for d in dirs:
        seen = set()
        for r in csv.DictReader(open(find_csv(d, "counter_collection.csv"))):
            lab = kernel_label(r["Kernel_Name"])
            wgs = int(r["Grid_Size"]) // max(1, int(r["Workgroup_Size"]))
            key = (lab, wgs)
            vals[key][r["Counter_Name"]].append(float(r["Counter_Value"]))
            did = (d, r["Dispatch_Id"])
            if did not in seen:
                seen.add(did)
                durs[key].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    mean = {k: {c: sum(v) / len(v) for c, v in cs.items()} for k, cs in vals.items()}
    base, mixed, backward = parse_key(wl_name)
    lines = [f"# Matrix-core and issue counters per kernel, bench step (prefill) on workload "
             f"{base}", "", "Commands (from the repository root, after building the library):",
             ""] + ["    " + c for c in commands] + [
        "", "Per-dispatch averages over the profiled steps. Derived: clock = GRBM_GUI_ACTIVE "
        f"per XCD / duration (kernels of 50 us or more); MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (GUI cycles x {N_SIMD} "
        "SIMDs); MFMA TFLOP/s = 512 x (MOPS_BF16 + MOPS_F16) / duration; issue stall = "
        "SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES (wave-cycles waiting to issue); LDS read B/clk/CU "
        f"= 64 x SQ_INSTS_LDS_LOAD_BANDWIDTH / (GUI cycles x {N_CU}); TA busy = TA_TA_BUSY / "
        f"(GUI cycles x {N_CU}). Durations come from the counter runs (kernels serialised).",
        "", "| kernel | WGs | us | clock GHz | MFMA busy | MFMA TFLOP/s | MFMA / wave | "
        "VALU / wave | SALU / wave | LDS / wave | issue stall | LDS-wait share | "
        "LDS read B/clk/CU | LDS bank-conflict cycles | TA busy |",
        "|---|---:|---:|---:|---:|---:|---:|---:|---:|---:|---:|---:|---:|---:|---:|"]
    order = sorted(mean, key=lambda k: -sum(durs[k]) / max(1, len(durs[k])))
    for key in order:
        m = mean[key]
        dur = sum(durs[key]) / len(durs[key])
        gui = m.get("GRBM_GUI_ACTIVE", 0.0) / N_XCD
        if dur < 2.0 or gui <= 0:
            continue
        waves = max(1.0, m.get("SQ_WAVES", 1.0))

        def g(c, f=lambda x: x, fmt="{:.3g}"):
            return fmt.format(f(m[c])) if c in m else "-"
        mops = m.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0) + m.get("SQ_INSTS_VALU_MFMA_MOPS_F16", 0.0)
        wc = m.get("SQ_WAVE_CYCLES", 0.0)
        lines.append(
            f"| {key[0]} | {key[1]} | {dur:.1f} | "
            + (f"{gui / dur / 1e3:.2f}" if dur >= 50 else "-") + " | "
            + g("SQ_VALU_MFMA_BUSY_CYCLES", lambda x: 100 * x / (gui * N_SIMD), "{:.1f}%") + " | "
            + f"{512 * mops / dur / 1e6:.0f} | "
            + g("SQ_INSTS_MFMA", lambda x: x / waves, "{:.0f}") + " | "
            + g("SQ_INSTS_VALU", lambda x: x / waves, "{:.0f}") + " | "
            + g("SQ_INSTS_SALU", lambda x: x / waves, "{:.0f}") + " | "
            + g("SQ_INSTS_LDS", lambda x: x / waves, "{:.0f}") + " | "
            + (g("SQ_WAIT_INST_ANY", lambda x: 100 * x / wc, "{:.0f}%") if wc else "-") + " | "
            + (g("SQ_WAIT_INST_LDS", lambda x: 100 * x / wc, "{:.0f}%") if wc else "-") + " | "
            + g("SQ_INSTS_LDS_LOAD_BANDWIDTH", lambda x: 64 * x / (gui * N_CU), "{:.1f}") + " | "
            + g("SQ_LDS_BANK_CONFLICT", lambda x: x, "{:.3g}") + " | "
            + g("TA_TA_BUSY", lambda x: 100 * x / (gui * N_CU), "{:.0f}%") + " |")
    open(out, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="c3", choices=["c1", "c2", "c3", "c4", "c5"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--decay", default="shared", choices=["shared", "mixed"],
                    help="mixed: the expert-mixed diagonal transition (per-expert decays "
                         "mixed per token) instead of one shared decay per head")
    ap.add_argument("--backward", action="store_true",
                    help="time the training step: the prefill forward and the whole backward")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="end with copies of known size (scales HBM counters)")
    ap.add_argument("--summarize-trace", metavar="DIR",
                    help="write a markdown summary of a rocprofv3 kernel-trace run")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write the HBM traffic summary of two rocprofv3 --pmc runs")
    ap.add_argument("--summarize-sq", nargs="+", metavar="DIR",
                    help="write the matrix-core / issue counter summary of rocprofv3 --pmc "
                         "runs of the SQ_PASSES counter sets")
    ap.add_argument("--out", help="summary file to write")
    ap.add_argument("--output-projection", action="store_true",
                    help="time the output projection alone on the --config workload")
    ap.add_argument("--e-sweep", action="store_true",
                    help="prefill tokens/s at the c3 dimensions for E in 4..64 (k = 2)")
    ap.add_argument("--separated", action="store_true",
                    help="tokens/s of the MoE over separated SSMs beside Swimba's, at the c2 "
                         "dimensions for several E and k")
    ap.add_argument("--library-gemm", action="store_true",
                    help="the expert projection beside hipBLASLt (torch.mm) on the c2, c3 and "
                         "c4 shapes")
    ap.add_argument("--bench-json", help="the JSON output of the profiled bench run")
    ap.add_argument("--command", action="append", default=[],
                    help="the command(s) that produced the profile, for the summary")
    args = ap.parse_args()
    key = profile_key(args.config, args.decay, args.backward)
    if args.summarize_trace:
        summarize_trace(args.summarize_trace, key,
                        args.out or os.path.join(PROFILES, f"swimba_step_{key}_kernel_trace.md"),
                        " ".join(args.command), args.bench_json)
        return
    if args.summarize_sq:
        summarize_sq(args.summarize_sq, key,
                     args.out or os.path.join(PROFILES, f"swimba_step_{key}_sq_counters.md"),
                     args.command)
        return
    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc[0], args.summarize_pmc[1], key,
                      args.out or traffic_file(key), args.command)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1"}))
        sys.exit(2)
    if args.backward and (args.decay != "shared" or is_decode(workload(args.config))):
        print(json.dumps({"error": "--backward times prefill workloads with the shared decay"}))
        sys.exit(2)
    if args.e_sweep:
        e_sweep(args)
        return
    if args.separated:
        separated_sweep(args)
        return
    if args.output_projection:
        output_projection(args)
        return
    if args.library_gemm:
        library_gemm(args)
        return
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
            "workload": ((f"Swimba mixer training step (prefill forward + backward to u, W_r, "
                          f"W_exp, a, h_init), {wl.dtype}: batch {wl.batch}, T={wl.seqlen}, "
                          f"d_model={wl.d_model}, heads={wl.nheads}, P={wl.headdim}, "
                          f"N={wl.dstate}, E={wl.n_experts}, top-k={wl.top_k}, chunk {wl.chunk}")
                         if args.backward else
                         (f"Swimba recurrent decode step, {wl.dtype}: batch {wl.batch}, "
                         f"one token per sequence per step, d_model={wl.d_model}, "
                         f"heads={wl.nheads}, P={wl.headdim}, N={wl.dstate} fp32 state per "
                         f"head in HBM, E={wl.n_experts}, top-k={wl.top_k}")
            if is_decode(wl) else
                        (f"Swimba mixer prefill (forward), {wl.dtype}: batch {wl.batch}, "
                         f"T={wl.seqlen}, d_model={wl.d_model}, heads={wl.nheads}, "
                         f"P={wl.headdim}, N={wl.dstate}, E={wl.n_experts}, "
                         f"top-k={wl.top_k}, chunk {wl.chunk}"))
            + (", expert-mixed decay (per-expert decays mixed per token)"
               if args.decay == "mixed" else ""),
            "global_batch": wl.batch, "seq_len": wl.seqlen, "parallelism": "none",
        },
        "roofline": r["roofline"],
        "kernels": r["kernels"],
        "value_without_events": r["value_without_events"],
    }
    for extra in ("roofline_scan", "scan_pipeline", "step_roofline"):
        if extra in r:
            out[extra] = r[extra]
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = (cpu_baseline_backward(wl) if args.backward else
                               cpu_baseline(wl, mixed=args.decay == "mixed"))
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
