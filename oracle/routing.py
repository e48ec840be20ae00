"""Routing permutation of the MoE dispatch (test infrastructure).

What is computed: the grouped matmul of the float8 MoE pages takes the
routed token rows grouped by expert, with cumulative group offsets (the
torchao float8 MoE training PR overrides grouped_mm for the routed experts,
Summary and Limitations; the Megatron-LM FP8-vs-BF16 MoE bug report's
additional context has TEGroupedMLP pad those per-expert inputs for FP8).
The pages do not fix the order inside an expert group; the reading taken:

* the choices (t, j) of a top-k routing ``expert_ids [T, k]`` are ordered
  stably by expert id, i.e. by (expert, token, choice);
* ``row_index[i]`` is the token of routed row i, ``group_ends[e]`` the
  number of choices with an id <= e (ids in [0, E)), and ``slot_row`` the
  inverse map (choice t * k + j -> its routed row);
* a choice with an id outside [0, E) is not routed: its ``slot_row`` is -1
  and the row slots past the last group hold -1.

The definition is a stable sort (a library primitive) and a cumulative
count; nothing is blocked or reordered beyond it.
"""
from __future__ import annotations

import numpy as np


def route(expert_ids, E: int) -> dict:
    ids = np.asarray(expert_ids, np.int64)
    T, k = ids.shape
    flat = ids.reshape(-1)                                   # choice t * k + j
    valid = (flat >= 0) & (flat < E)
    order = np.argsort(np.where(valid, flat, E), kind="stable")
    nvalid = int(valid.sum())
    row_index = np.full(flat.size, -1, np.int64)
    row_index[:nvalid] = order[:nvalid] // k
    slot_row = np.full(flat.size, -1, np.int64)
    slot_row[order[:nvalid]] = np.arange(nvalid)
    group_ends = np.cumsum(np.bincount(flat[valid], minlength=E)).astype(np.int64)
    return {"group_ends": group_ends, "row_index": row_index, "slot_row": slot_row}
