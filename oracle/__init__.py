"""fp64 CPU oracle for coalesced varlen attention: TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package. It shares no code with the HIP library and
never imports it. Every function states the passage of the Zellige page it follows.
"""
from .attention import (PackLayout, default_scale, head_backward, head_backward_delta, head_delta, head_forward,
                        head_probs, head_scores, lse_merge, pack_backward, pack_forward, running_merge)

__all__ = ["PackLayout", "default_scale", "head_backward", "head_backward_delta", "head_delta", "head_forward",
           "head_probs", "head_scores", "lse_merge", "pack_backward", "pack_forward", "running_merge"]
