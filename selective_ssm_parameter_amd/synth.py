"""Seeded synthetic inputs for the Swimba mixer.

This module only draws random numbers and rounds them to the storage dtype;
it holds none of the mixer's arithmetic. Both the HIP path (through its
callers) and the fp64 oracle consume what it returns, so the two sides always
see bit-identical inputs.

Recipe (fixed draw order, numpy PCG64 ``default_rng(seed)``):
  1. a     ~ U[lo, hi]                 shape [H]        fp32 (never rounded)
  2. W_r   ~ N(0, 1) * sqrt(1/D)       shape [E, D]
  3. W_exp ~ N(0, 1) * sqrt(1/D)       shape [E, W, D], one expert at a time,
           rows ordered X (H*P) | B (G*N) | C (G*N)
  4. u     ~ N(0, 1)                   shape [Bt, T, D]
  5. h_init ~ N(0, 1) * sqrt(v)        shape [Bt, H, N, P] fp32 (when asked)
Decode steps draw their token from ``default_rng([seed, step])``.
The output projection draws from ``default_rng([seed, 7919])``: W_out ~
N(0, 1) * sqrt(1/(H*P)) of shape [D, H*P], then y ~ N(0, 1) of shape
[Bt*T, H, P] (standing in for the readout that feeds it).
The expert-mixed transition draws per-expert decays from
``default_rng([seed, 104729])``: a^(e) ~ U[lo, hi] of shape [E, H], fp32.

bf16 workloads round every tensor except ``a`` and ``h_init`` to bf16 with
round-to-nearest-even; the returned numpy arrays hold the rounded values in
fp32, so widening them to fp64 is exact.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

F32 = "f32"
BF16 = "bf16"


@dataclasses.dataclass(frozen=True)
class Workload:
    """Dimensions of one Swimba mixer call plus the input distribution."""

    name: str
    seed: int
    batch: int
    seqlen: int
    d_model: int
    nheads: int
    headdim: int
    dstate: int
    ngroups: int
    n_experts: int
    top_k: int
    chunk: int
    dtype: str
    a_lo: float
    a_hi: float
    h_init_var: float = 0.0  # 0 => no initial state
    decode_steps: int = 0    # >0 => recurrent decode workload (seqlen == 1)

    @property
    def d_inner(self) -> int:
        return self.nheads * self.headdim

    @property
    def width(self) -> int:
        """Rows of one expert's projection: X | B | C."""
        return self.d_inner + 2 * self.ngroups * self.dstate

    @property
    def tokens(self) -> int:
        return self.batch * self.seqlen

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads: a small fp32 case, three bf16 prefill shapes (the last
# with slow decay over 65536 tokens) and a bf16 recurrent decode.
WORKLOADS = {
    "c1": Workload("c1", 1, 1, 256, 128, 2, 64, 16, 1, 4, 1, 32, F32, 0.9, 0.99),
    "c2": Workload("c2", 2, 8, 2048, 768, 24, 64, 128, 1, 8, 2, 64, BF16, 0.9, 0.999),
    "c3": Workload("c3", 3, 4, 8192, 2048, 64, 64, 128, 1, 16, 2, 128, BF16, 0.9, 0.999),
    "c4": Workload("c4", 4, 1, 65536, 1024, 32, 64, 128, 1, 8, 2, 256, BF16, 0.99, 0.9999),
    "c5": Workload("c5", 5, 256, 1, 2048, 64, 64, 128, 1, 32, 4, 64, BF16, 0.9, 0.999,
                   h_init_var=0.1, decode_steps=512),
}


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to the nearest bf16 (ties to even); result kept in fp32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32)
    lsb = (bits >> np.uint32(16)) & np.uint32(1)
    rounded = (bits + np.uint32(0x7FFF) + lsb) & np.uint32(0xFFFF0000)
    return rounded.view(np.float32)


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    return round_bf16(x) if dtype == BF16 else np.ascontiguousarray(x, dtype=np.float32)


def make_inputs(wl: Workload, batch_rows: int | None = None) -> dict:
    """Draw every input of ``wl`` in the fixed order above.

    ``batch_rows`` keeps only the first rows of u and h_init (the draw itself is
    always the full one, so a row is identical whatever slice is asked for).
    """
    rng = np.random.default_rng(wl.seed)
    H, D, E, W = wl.nheads, wl.d_model, wl.n_experts, wl.width
    a = rng.uniform(wl.a_lo, wl.a_hi, size=H).astype(np.float32)
    scale = np.float32(math.sqrt(1.0 / D))
    w_router = _store(rng.standard_normal((E, D), dtype=np.float32) * scale, wl.dtype)
    w_experts = np.empty((E, W, D), dtype=np.float32)
    for e in range(E):
        w_experts[e] = _store(rng.standard_normal((W, D), dtype=np.float32) * scale, wl.dtype)
    u = _store(rng.standard_normal((wl.batch, wl.seqlen, D), dtype=np.float32), wl.dtype)
    h_init = None
    if wl.h_init_var > 0:
        h_init = (rng.standard_normal((wl.batch, H, wl.dstate, wl.headdim), dtype=np.float32)
                  * np.float32(math.sqrt(wl.h_init_var)))
    if batch_rows is not None:
        u = u[:batch_rows].copy()
        if h_init is not None:
            h_init = h_init[:batch_rows].copy()
    return {"a": a, "w_router": w_router, "w_experts": w_experts, "u": u, "h_init": h_init}


def decode_token(wl: Workload, step: int, batch_rows: int | None = None) -> np.ndarray:
    """Token fed to the decode step ``step``: [Bt, D], same dtype rule as u."""
    rng = np.random.default_rng([wl.seed, step])
    u = rng.standard_normal((wl.batch, wl.d_model), dtype=np.float32)
    if batch_rows is not None:
        u = u[:batch_rows]
    return _store(u, wl.dtype)


def output_projection_inputs(wl: Workload, rows: int | None = None) -> dict:
    """W_out [D, H*P] and y [M, H, P] for the output projection (same dtype
    rule as u); ``rows`` keeps only the first rows of y."""
    rng = np.random.default_rng([wl.seed, 7919])
    HP = wl.nheads * wl.headdim
    w_out = _store(rng.standard_normal((wl.d_model, HP), dtype=np.float32)
                   * np.float32(math.sqrt(1.0 / HP)), wl.dtype)
    y = rng.standard_normal((wl.tokens, wl.nheads, wl.headdim), dtype=np.float32)
    if rows is not None:
        y = y[:rows]
    return {"w_out": w_out, "y": _store(y, wl.dtype)}


def output_gradient(wl: Workload) -> np.ndarray:
    """Upstream gradient dl/dy [M, H, P] of the training step (same dtype rule
    as u), from a stream of its own so every other input is unchanged."""
    rng = np.random.default_rng([wl.seed, 130363])
    dy = rng.standard_normal((wl.tokens, wl.nheads, wl.headdim), dtype=np.float32)
    return _store(dy, wl.dtype)


def expert_decays(wl: Workload) -> np.ndarray:
    """Per-expert, per-head decays a^(e)_h ~ U[a_lo, a_hi] (fp32) for the
    expert-mixed transition, [E, H], from a stream of their own so every other
    input of the workload is unchanged."""
    rng = np.random.default_rng([wl.seed, 104729])
    return rng.uniform(wl.a_lo, wl.a_hi, size=(wl.n_experts, wl.nheads)).astype(np.float32)


def small(name: str, seed: int, **dims) -> Workload:
    """A custom workload for tests; unspecified fields take c1's values."""
    base = WORKLOADS["c1"].replace(name=name, seed=seed)
    return base.replace(**dims)
