"""fp64 CPU oracle of the Swimba (Switch Mamba) mixer forward pass.

TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's CPU
baseline may import or run anything in this package. The product path (the
HIP library and its Python binding) never calls it and shares no code with it.

Sources (all are web pages on arXiv 2603.06938, "Swimba: Switch Mamba Model
Scales State Space Models"):
  [notes]   papernotes.org NeurIPS 2026 notes (Chinese): the only page that
            prints the mixing equations, the recurrence and the stability bound.
  [gist-en] gist.science English summary, "Technical Summary".
  [gist-de] gist.science German summary, "Technische Zusammenfassung".
  [gist-ja] gist.science Japanese summary.

Every function is pinned by tests under ``tests/`` against closed forms,
invariants and brute force (see the list in ``oracle/swimba.py``); none is
parity-unpinned.
"""
from .swimba import (  # noqa: F401
    Routing,
    Streams,
    decode_step,
    expert_streams,
    forward,
    mix_streams,
    recurrence,
    route,
)
