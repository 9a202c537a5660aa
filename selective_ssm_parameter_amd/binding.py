"""Python binding of the Swimba C ABI (``include/swimba.h``).

Argument marshalling only: every step of the mixer runs in the HIP kernels of
``libswimba.so``. PyTorch provides device memory and the current stream. The
library must have been built (``python -m selective_ssm_parameter_amd.build``);
there is no fallback of any kind: a missing library raises.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libswimba.so")

F32, BF16 = 0, 1
(CALL_ROUTE, CALL_PROJECT, CALL_SCAN, CALL_DECODE, CALL_SCAN_BACKWARD, CALL_PROJECT_BACKWARD,
 CALL_PROJECT_BACKWARD_SAVED, CALL_SEPARATED) = (0, 1, 2, 3, 4, 5, 6, 7)

STATUS = {
    0: "SWIMBA_OK", -1: "SWIMBA_ERR_NULL", -2: "SWIMBA_ERR_DIMS", -3: "SWIMBA_ERR_UNSUPPORTED",
    -4: "SWIMBA_ERR_WORKSPACE", -5: "SWIMBA_ERR_ALIGN", -6: "SWIMBA_ERR_HIP",
}

EXPORTS = (
    "swimba_abi_version", "swimba_last_error", "swimba_workspace_size", "swimba_route_topk",
    "swimba_expert_project_mix", "swimba_ssd_chunk_scan", "swimba_decode_step",
    "swimba_output_project", "swimba_profile_enable", "swimba_profile_report",
    "swimba_profile_select", "swimba_mix_decay", "swimba_ssd_chunk_scan_mixed",
    "swimba_decode_step_mixed", "swimba_decode_step_noalloc", "swimba_ssd_chunk_scan_backward",
    "swimba_expert_project_mix_backward", "swimba_expert_project_mix_backward_saved",
    "swimba_separated_forward",
)


class SwimbaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


class Dims(ctypes.Structure):
    _fields_ = [(name, ctypes.c_int32) for name in (
        "batch", "seqlen", "d_model", "nheads", "headdim", "dstate", "ngroups", "n_experts",
        "top_k", "chunk", "dtype", "reserved")]

    def __repr__(self):
        return "Dims(" + ", ".join(f"{n}={getattr(self, n)}" for n, _ in self._fields_) + ")"


_lib = None


def lib() -> ctypes.CDLL:
    """Load libswimba.so (once). Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m selective_ssm_parameter_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    P, S, I32, SZ = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    D = ctypes.POINTER(Dims)
    L.swimba_abi_version.restype = I32
    L.swimba_abi_version.argtypes = []
    L.swimba_last_error.restype = ctypes.c_char_p
    L.swimba_last_error.argtypes = []
    L.swimba_workspace_size.restype = SZ
    L.swimba_workspace_size.argtypes = [D, I32]
    L.swimba_route_topk.restype = I32
    L.swimba_route_topk.argtypes = [D, P, P, P, P, P, S]
    L.swimba_expert_project_mix.restype = I32
    L.swimba_expert_project_mix.argtypes = [D, P, P, P, P, P, P, P, P, SZ, S]
    L.swimba_ssd_chunk_scan.restype = I32
    L.swimba_ssd_chunk_scan.argtypes = [D, P, P, P, P, P, P, P, P, SZ, S]
    L.swimba_decode_step.restype = I32
    L.swimba_decode_step.argtypes = [D, P, P, P, P, P, P, P, P, SZ, S]
    L.swimba_output_project.restype = I32
    L.swimba_output_project.argtypes = [D, P, P, P, S]
    L.swimba_mix_decay.argtypes = [D, P, P, P, P, S]
    L.swimba_mix_decay.restype = I32
    L.swimba_ssd_chunk_scan_mixed.argtypes = [D, P, P, P, P, P, P, P, P, SZ, S]
    L.swimba_ssd_chunk_scan_mixed.restype = I32
    L.swimba_decode_step_noalloc.restype = I32
    L.swimba_decode_step_noalloc.argtypes = [D, P, P, P, P, P, P, P, S]
    L.swimba_decode_step_mixed.argtypes = [D, P, P, P, P, P, P, P, P, SZ, S]
    L.swimba_decode_step_mixed.restype = I32
    L.swimba_ssd_chunk_scan_backward.argtypes = [D, P, P, P, P, P, P, P, P, P, P, P, P, P, SZ, S]
    L.swimba_ssd_chunk_scan_backward.restype = I32
    L.swimba_expert_project_mix_backward.argtypes = [D, P, P, P, P, P, P, P, P, P, P, SZ, S]
    L.swimba_expert_project_mix_backward.restype = I32
    L.swimba_expert_project_mix_backward_saved.argtypes = [D, P, P, P, P, P, P, P, P, SZ, P, P,
                                                           P, P, P, P, P, SZ, S]
    L.swimba_expert_project_mix_backward_saved.restype = I32
    L.swimba_separated_forward.argtypes = [D, P, P, P, P, P, P, P, P, P, SZ, S]
    L.swimba_separated_forward.restype = I32
    L.swimba_profile_enable.restype = I32
    L.swimba_profile_enable.argtypes = [I32]
    L.swimba_profile_report.restype = I32
    L.swimba_profile_report.argtypes = [ctypes.c_char_p, SZ]
    L.swimba_profile_select.restype = I32
    L.swimba_profile_select.argtypes = [ctypes.c_char_p]
    _lib = L
    return L


def _check(status: int):
    if status != 0:
        raise SwimbaError(status, lib().swimba_last_error().decode())


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_contiguous():
        raise ValueError("tensors passed to the Swimba library must be contiguous")
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream if isinstance(stream, int) else stream.cuda_stream


def make_dims(batch, seqlen, d_model, nheads, headdim, dstate, ngroups, n_experts, top_k,
              chunk, dtype) -> Dims:
    dt = {"f32": F32, "bf16": BF16, F32: F32, BF16: BF16}[dtype]
    return Dims(batch, seqlen, d_model, nheads, headdim, dstate, ngroups, n_experts, top_k,
                chunk, dt, 0)


def dims_of(wl, batch=None, seqlen=None) -> Dims:
    """Dims of a ``synth.Workload`` (optionally with another batch or seqlen)."""
    return make_dims(wl.batch if batch is None else batch, wl.seqlen if seqlen is None else seqlen,
                     wl.d_model, wl.nheads, wl.headdim, wl.dstate, wl.ngroups, wl.n_experts,
                     wl.top_k, wl.chunk, wl.dtype)


def torch_dtype(dims: Dims):
    """Element type of u, the weights and y."""
    return torch.bfloat16 if dims.dtype == BF16 else torch.float32


def stream_dtype(dims: Dims):
    """Element type of B_hat, X_hat and C_mix (fp16 when the inputs are bf16)."""
    return torch.float16 if dims.dtype == BF16 else torch.float32


def abi_version() -> int:
    return lib().swimba_abi_version()


def swimba_workspace_size(dims: Dims, call: int) -> int:
    return lib().swimba_workspace_size(ctypes.byref(dims), call)


def workspace(dims: Dims, call: int, device="cuda"):
    n = swimba_workspace_size(dims, call)
    return torch.empty(max(n, 16), dtype=torch.uint8, device=device), n


# ----------------------------------------------------------------- raw calls

def swimba_route_topk(dims, u, w_router, topk_idx, topk_w, logits=None, stream=None):
    _check(lib().swimba_route_topk(ctypes.byref(dims), _ptr(u), _ptr(w_router), _ptr(topk_idx),
                                   _ptr(topk_w), _ptr(logits), _stream(stream)))


def swimba_expert_project_mix(dims, u, w_experts, topk_idx, topk_w, B_hat, X_hat, C_mix, ws,
                              ws_bytes=None, stream=None):
    nb = ws.numel() if ws_bytes is None else ws_bytes
    _check(lib().swimba_expert_project_mix(
        ctypes.byref(dims), _ptr(u), _ptr(w_experts), _ptr(topk_idx), _ptr(topk_w), _ptr(B_hat),
        _ptr(X_hat), _ptr(C_mix), _ptr(ws), nb, _stream(stream)))


def swimba_ssd_chunk_scan(dims, B_hat, X_hat, C_mix, a, h_init, y, h_final, ws, ws_bytes=None,
                          stream=None):
    nb = (ws.numel() if ws is not None else 0) if ws_bytes is None else ws_bytes
    _check(lib().swimba_ssd_chunk_scan(
        ctypes.byref(dims), _ptr(B_hat), _ptr(X_hat), _ptr(C_mix), _ptr(a), _ptr(h_init), _ptr(y),
        _ptr(h_final), _ptr(ws), nb, _stream(stream)))


def swimba_decode_step(dims, u, w_router, w_experts, a, h, y, topk_idx, ws, ws_bytes=None,
                       stream=None):
    nb = ws.numel() if ws_bytes is None else ws_bytes
    _check(lib().swimba_decode_step(
        ctypes.byref(dims), _ptr(u), _ptr(w_router), _ptr(w_experts), _ptr(a), _ptr(h), _ptr(y),
        _ptr(topk_idx), _ptr(ws), nb, _stream(stream)))


def swimba_decode_step_noalloc(dims, u, w_router, w_experts, a, h, y, topk_idx, stream=None):
    _check(lib().swimba_decode_step_noalloc(
        ctypes.byref(dims), _ptr(u), _ptr(w_router), _ptr(w_experts), _ptr(a), _ptr(h), _ptr(y),
        _ptr(topk_idx), _stream(stream)))


def swimba_separated_forward(dims, u, w_router, w_experts, a, h_init, y, h_final, topk_idx, ws,
                             ws_bytes=None, stream=None):
    nb = (ws.numel() if ws is not None else 0) if ws_bytes is None else ws_bytes
    _check(lib().swimba_separated_forward(
        ctypes.byref(dims), _ptr(u), _ptr(w_router), _ptr(w_experts), _ptr(a), _ptr(h_init),
        _ptr(y), _ptr(h_final), _ptr(topk_idx), _ptr(ws), nb, _stream(stream)))


def swimba_mix_decay(dims, topk_idx, topk_w, a_experts, log_decay, stream=None):
    _check(lib().swimba_mix_decay(ctypes.byref(dims), _ptr(topk_idx), _ptr(topk_w),
                                  _ptr(a_experts), _ptr(log_decay), _stream(stream)))


def swimba_ssd_chunk_scan_mixed(dims, B_hat, X_hat, C_mix, log_decay, h_init, y, h_final, ws,
                                ws_bytes=None, stream=None):
    nb = (ws.numel() if ws is not None else 0) if ws_bytes is None else ws_bytes
    _check(lib().swimba_ssd_chunk_scan_mixed(
        ctypes.byref(dims), _ptr(B_hat), _ptr(X_hat), _ptr(C_mix), _ptr(log_decay), _ptr(h_init),
        _ptr(y), _ptr(h_final), _ptr(ws), nb, _stream(stream)))


def swimba_decode_step_mixed(dims, u, w_router, w_experts, a_experts, h, y, topk_idx, ws,
                             ws_bytes=None, stream=None):
    nb = ws.numel() if ws_bytes is None else ws_bytes
    _check(lib().swimba_decode_step_mixed(
        ctypes.byref(dims), _ptr(u), _ptr(w_router), _ptr(w_experts), _ptr(a_experts), _ptr(h),
        _ptr(y), _ptr(topk_idx), _ptr(ws), nb, _stream(stream)))


def swimba_ssd_chunk_scan_backward(dims, B_hat, X_hat, C_mix, a, h_init, dy, dh_final, dB_hat,
                                   dX_hat, dC_mix, da, dh_init, ws, ws_bytes=None, stream=None):
    nb = (ws.numel() if ws is not None else 0) if ws_bytes is None else ws_bytes
    _check(lib().swimba_ssd_chunk_scan_backward(
        ctypes.byref(dims), _ptr(B_hat), _ptr(X_hat), _ptr(C_mix), _ptr(a), _ptr(h_init),
        _ptr(dy), _ptr(dh_final), _ptr(dB_hat), _ptr(dX_hat), _ptr(dC_mix), _ptr(da),
        _ptr(dh_init), _ptr(ws), nb, _stream(stream)))


def swimba_expert_project_mix_backward(dims, u, w_router, w_experts, dB_hat, dX_hat, dC_mix, du,
                                       dW_router, dW_experts, ws, ws_bytes=None, stream=None):
    nb = (ws.numel() if ws is not None else 0) if ws_bytes is None else ws_bytes
    _check(lib().swimba_expert_project_mix_backward(
        ctypes.byref(dims), _ptr(u), _ptr(w_router), _ptr(w_experts), _ptr(dB_hat), _ptr(dX_hat),
        _ptr(dC_mix), _ptr(du), _ptr(dW_router), _ptr(dW_experts), _ptr(ws), nb,
        _stream(stream)))


def swimba_expert_project_mix_backward_saved(dims, u, w_router, w_experts, topk_idx, topk_w,
                                             logits, B_hat, fwd_ws, dB_hat, dX_hat, dC_mix, du,
                                             dW_router, dW_experts, ws, fwd_ws_bytes=None,
                                             ws_bytes=None, stream=None):
    fnb = (fwd_ws.numel() if fwd_ws is not None else 0) if fwd_ws_bytes is None else fwd_ws_bytes
    nb = (ws.numel() if ws is not None else 0) if ws_bytes is None else ws_bytes
    _check(lib().swimba_expert_project_mix_backward_saved(
        ctypes.byref(dims), _ptr(u), _ptr(w_router), _ptr(w_experts), _ptr(topk_idx),
        _ptr(topk_w), _ptr(logits), _ptr(B_hat), _ptr(fwd_ws), fnb, _ptr(dB_hat), _ptr(dX_hat),
        _ptr(dC_mix), _ptr(du), _ptr(dW_router), _ptr(dW_experts), _ptr(ws), nb,
        _stream(stream)))


def swimba_output_project(dims, y, w_out, out, stream=None):
    _check(lib().swimba_output_project(ctypes.byref(dims), _ptr(y), _ptr(w_out), _ptr(out),
                                       _stream(stream)))


def profile_enable(on: bool):
    _check(lib().swimba_profile_enable(1 if on else 0))


def profile_select(kernel: str | None):
    """Time only kernels of this name (None: every kernel)."""
    _check(lib().swimba_profile_select(kernel.encode() if kernel else None))


def profile_report() -> str:
    buf = ctypes.create_string_buffer(1 << 16)
    n = lib().swimba_profile_report(buf, len(buf))
    if n < 0:
        _check(n)
    return buf.value.decode()


# ----------------------------------------------------------------- helpers

@dataclasses.dataclass
class Buffers:
    topk_idx: torch.Tensor
    topk_w: torch.Tensor
    B_hat: torch.Tensor
    X_hat: torch.Tensor
    C_mix: torch.Tensor
    y: torch.Tensor
    h_final: torch.Tensor
    ws_project: torch.Tensor
    ws_scan: torch.Tensor
    logits: torch.Tensor | None = None


def alloc_buffers(dims: Dims, device="cuda", logits=False) -> Buffers:
    """Every output and workspace of one prefill forward, allocated by torch."""
    M = dims.batch * dims.seqlen
    k, H, P, G, N = dims.top_k, dims.nheads, dims.headdim, dims.ngroups, dims.dstate
    dt = torch_dtype(dims)
    st = stream_dtype(dims)
    ws_p, _ = workspace(dims, CALL_PROJECT, device)
    ws_s, _ = workspace(dims, CALL_SCAN, device)
    return Buffers(
        topk_idx=torch.empty(M, k, dtype=torch.int32, device=device),
        topk_w=torch.empty(M, k, dtype=torch.float32, device=device),
        B_hat=torch.empty(M, k, G, N, dtype=st, device=device),
        X_hat=torch.empty(M, k, H, P, dtype=st, device=device),
        C_mix=torch.empty(M, G, N, dtype=st, device=device),
        y=torch.empty(M, H, P, dtype=dt, device=device),
        h_final=torch.empty(dims.batch, H, N, P, dtype=torch.float32, device=device),
        ws_project=ws_p, ws_scan=ws_s,
        logits=torch.empty(M, dims.n_experts, dtype=torch.float32, device=device) if logits else None,
    )


def forward(dims: Dims, u, w_router, w_experts, a, h_init=None, buf: Buffers | None = None,
            stream=None) -> Buffers:
    """Route -> project + mix -> chunked scan, on the current stream."""
    if buf is None:
        buf = alloc_buffers(dims, u.device)
    swimba_route_topk(dims, u, w_router, buf.topk_idx, buf.topk_w, buf.logits, stream=stream)
    swimba_expert_project_mix(dims, u, w_experts, buf.topk_idx, buf.topk_w, buf.B_hat, buf.X_hat,
                              buf.C_mix, buf.ws_project, stream=stream)
    swimba_ssd_chunk_scan(dims, buf.B_hat, buf.X_hat, buf.C_mix, a, h_init, buf.y, buf.h_final,
                          buf.ws_scan, stream=stream)
    return buf


def forward_mixed(dims: Dims, u, w_router, w_experts, a_experts, h_init=None,
                  buf: Buffers | None = None, log_decay=None, stream=None) -> Buffers:
    """Route -> project + mix -> mixed decay -> chunked scan with it."""
    if buf is None:
        buf = alloc_buffers(dims, u.device)
    if log_decay is None:
        log_decay = torch.empty(dims.batch, dims.nheads, dims.seqlen, dtype=torch.float32,
                                device=u.device)
    swimba_route_topk(dims, u, w_router, buf.topk_idx, buf.topk_w, buf.logits, stream=stream)
    swimba_expert_project_mix(dims, u, w_experts, buf.topk_idx, buf.topk_w, buf.B_hat, buf.X_hat,
                              buf.C_mix, buf.ws_project, stream=stream)
    swimba_mix_decay(dims, buf.topk_idx, buf.topk_w, a_experts, log_decay, stream=stream)
    swimba_ssd_chunk_scan_mixed(dims, buf.B_hat, buf.X_hat, buf.C_mix, log_decay, h_init, buf.y,
                                buf.h_final, buf.ws_scan, stream=stream)
    return buf


@dataclasses.dataclass
class Grads:
    dB_hat: torch.Tensor
    dX_hat: torch.Tensor
    dC_mix: torch.Tensor
    da: torch.Tensor
    dh_init: torch.Tensor
    du: torch.Tensor
    dW_router: torch.Tensor
    dW_experts: torch.Tensor
    ws_scan: torch.Tensor | None
    ws_project: torch.Tensor | None


def alloc_grads(dims: Dims, device="cuda", saved=False) -> Grads:
    """Every output and workspace of one backward pass, allocated by torch
    (float32); saved: the workspace of the call that reuses the forward."""
    M = dims.batch * dims.seqlen
    k, H, P, G, N, E, D = (dims.top_k, dims.nheads, dims.headdim, dims.ngroups, dims.dstate,
                           dims.n_experts, dims.d_model)
    Wd = H * P + 2 * G * N
    f32 = torch.float32
    ws_s, _ = workspace(dims, CALL_SCAN_BACKWARD, device)
    ws_p, _ = workspace(dims, CALL_PROJECT_BACKWARD_SAVED if saved else CALL_PROJECT_BACKWARD,
                        device)
    return Grads(
        dB_hat=torch.empty(M, k, G, N, dtype=f32, device=device),
        dX_hat=torch.empty(M, k, H, P, dtype=f32, device=device),
        dC_mix=torch.empty(M, G, N, dtype=f32, device=device),
        da=torch.empty(H, dtype=f32, device=device),
        dh_init=torch.empty(dims.batch, H, N, P, dtype=f32, device=device),
        du=torch.empty(M, D, dtype=f32, device=device),
        dW_router=torch.empty(E, D, dtype=f32, device=device),
        dW_experts=torch.empty(E, Wd, D, dtype=f32, device=device),
        ws_scan=ws_s, ws_project=ws_p)


def backward(dims: Dims, u, w_router, w_experts, a, h_init, dy, dh_final, fwd: Buffers,
             grads: Grads | None = None, stream=None, saved=False) -> Grads:
    """Gradients of l(y, h_final) given dy and dh_final: the chunked scan's
    backward on the forward's streams, then router, projection and mix. With
    saved, the latter reuses the forward's routing, B_hat and projection
    workspace (fwd must hold logits, and grads come from alloc_grads(saved=True))
    instead of recomputing them."""
    g = grads if grads is not None else alloc_grads(dims, u.device, saved)
    swimba_ssd_chunk_scan_backward(dims, fwd.B_hat, fwd.X_hat, fwd.C_mix, a, h_init, dy,
                                   dh_final, g.dB_hat, g.dX_hat, g.dC_mix, g.da, g.dh_init,
                                   g.ws_scan, stream=stream)
    if saved:
        swimba_expert_project_mix_backward_saved(
            dims, u, w_router, w_experts, fwd.topk_idx, fwd.topk_w, fwd.logits, fwd.B_hat,
            fwd.ws_project, g.dB_hat, g.dX_hat, g.dC_mix, g.du, g.dW_router, g.dW_experts,
            g.ws_project, stream=stream)
    else:
        swimba_expert_project_mix_backward(dims, u, w_router, w_experts, g.dB_hat, g.dX_hat,
                                           g.dC_mix, g.du, g.dW_router, g.dW_experts,
                                           g.ws_project, stream=stream)
    return g


@dataclasses.dataclass
class SeparatedBuffers:
    topk_idx: torch.Tensor
    y: torch.Tensor
    h_final: torch.Tensor
    ws: torch.Tensor


def alloc_separated(dims: Dims, device="cuda") -> SeparatedBuffers:
    """Outputs and workspace of one separated-SSM forward, allocated by torch."""
    M = dims.batch * dims.seqlen
    H, P, N, E = dims.nheads, dims.headdim, dims.dstate, dims.n_experts
    ws, _ = workspace(dims, CALL_SEPARATED, device)
    return SeparatedBuffers(
        topk_idx=torch.empty(M, dims.top_k, dtype=torch.int32, device=device),
        y=torch.empty(M, H, P, dtype=torch_dtype(dims), device=device),
        h_final=torch.empty(dims.batch, E, H, N, P, dtype=torch.float32, device=device),
        ws=ws)


def separated_forward(dims: Dims, u, w_router, w_experts, a, h_init=None,
                      buf: SeparatedBuffers | None = None, stream=None) -> SeparatedBuffers:
    """The MoE over separated SSMs (one trajectory per expert), on the current stream."""
    if buf is None:
        buf = alloc_separated(dims, u.device)
    swimba_separated_forward(dims, u, w_router, w_experts, a, h_init, buf.y, buf.h_final,
                             buf.topk_idx, buf.ws, stream=stream)
    return buf
