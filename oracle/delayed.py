"""Delayed-scaling state (amax history, "max" algorithm).

The pages fix only the knobs: the Megatron-LM FP8-vs-BF16 MoE bug report
reproduces with ``--fp8-amax-compute-algo max --fp8-amax-history-len
1024`` (reproduction steps), and the Transformer Engine issue names the
"delayed" recipe. The order of operations is a reading, where the pages
are silent:

1. step t quantizes with the (s, inv) held by the state, which come from
   steps before t, and records the amax of the tensor it quantized;
2. after the step, the amax is written into a ring of length L at
   position pos, and pos advances modulo L;
3. a* = max over the whole ring (slots never written hold 0);
4. if a* is finite and > 0: s = fp32(a*/fmax), inv = fp32(fmax/a*);
   otherwise s and inv keep their previous values. Margin is 0.

Initial state: ring all 0, pos 0, s = inv = 1.

Test infrastructure; see the package docstring.
"""
from __future__ import annotations

import numpy as np

from .formats import Fp8Format


class DelayedState:
    def __init__(self, units: int, fmt: Fp8Format, history_len: int = 1024):
        self.fmt = fmt
        self.L = int(history_len)
        self.history = np.zeros((units, self.L), np.float32)
        self.pos = np.zeros(units, np.int64)
        self.s = np.ones(units, np.float32)
        self.inv = np.ones(units, np.float32)

    def scale(self, u: int):
        return np.float32(self.s[u]), np.float32(self.inv[u])

    def update(self, amax) -> None:
        """Push one amax per unit and recompute (s, inv) from the window max."""
        amax = np.asarray(amax, np.float32).reshape(-1)
        fmax = np.float32(self.fmt.fmax)
        for u in range(self.history.shape[0]):
            self.history[u, self.pos[u]] = amax[u]
            self.pos[u] = (self.pos[u] + 1) % self.L
            a = np.float32(np.max(self.history[u]))
            if np.isfinite(a) and a > 0:
                self.s[u] = np.float32(a / fmax)
                self.inv[u] = np.float32(fmax / a)
