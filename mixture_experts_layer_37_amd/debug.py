"""Host-side consistency checks of the dispatch maps (MOE_DEBUG=1).

With the environment variable MOE_DEBUG set to 1, the binding downloads the
maps that moe_dispatch, moe_dispatch_fp8 and moe_layer_forward(_fp8) return
(after synchronising their stream) and checks here that they describe a valid
placement: every kept assignment owns one row of its expert's block, every
row of the blocks is owned exactly once, the blocks follow the exclusive scan
of the kept counts, and no expert keeps more than its capacity.  These are
invariants of any correct dispatch (section "专家容量与丢 token" of page
"MoE 与专家并行": per-expert buffers of C slots, over-capacity assignments
dropped); the fill order itself is checked by the tests against the oracle.
Nothing here is on the compute path: with MOE_DEBUG unset no map is read.
"""
from __future__ import annotations

import os

import numpy as np


def enabled() -> bool:
    return os.environ.get("MOE_DEBUG", "0") not in ("", "0")


class DispatchMapError(RuntimeError):
    pass


def check_dispatch_maps(topk_idx, slot, row_token, count, kept, offset, C: int) -> None:
    """Raise DispatchMapError unless the maps are a valid placement.

    topk_idx, slot [T, k]; row_token [rows_max]; count, kept [E]; offset [E+1];
    C the capacity (rows an expert may keep).  Arrays are host numpy arrays.
    """
    idx = np.asarray(topk_idx, dtype=np.int64)
    slot = np.asarray(slot, dtype=np.int64)
    row_token = np.asarray(row_token, dtype=np.int64)
    count = np.asarray(count, dtype=np.int64)
    kept = np.asarray(kept, dtype=np.int64)
    offset = np.asarray(offset, dtype=np.int64)
    E = count.shape[0]
    T = slot.shape[0]

    def fail(msg):
        raise DispatchMapError("dispatch maps: " + msg)

    if offset.shape[0] != E + 1 or offset[0] != 0:
        fail("offset must have E + 1 entries starting at 0")
    if (kept < 0).any() or (kept > count).any() or (kept > C).any():
        fail("kept must lie in [0, min(count, C)]")
    if (kept != np.minimum(count, C)).any():
        fail("kept must equal min(count, C)")
    if (np.diff(offset) != kept).any():
        fail("offset must be the exclusive scan of kept")
    rows = int(offset[-1])
    if rows > row_token.shape[0]:
        fail(f"{rows} kept rows exceed the {row_token.shape[0]} rows of row_token")
    valid = (idx >= 0) & (idx < E)
    if (np.bincount(idx[valid], minlength=E) != count).any():
        fail("count must be the histogram of topk_idx")
    if ((slot < -1) | (slot >= rows)).any():
        fail("slot values must lie in [-1, offset[E])")
    t_of, r_of = np.nonzero(slot >= 0)
    s = slot[t_of, r_of]
    if np.unique(s).shape[0] != s.shape[0] or s.shape[0] != rows:
        fail("every row below offset[E] must be owned by exactly one kept assignment")
    e = idx[t_of, r_of]
    if ((s < offset[e]) | (s >= offset[e + 1])).any():
        fail("a kept assignment's row lies outside its expert's block")
    if (row_token[s] != t_of).any():
        fail("row_token must name the token of each kept row")
    if ((row_token[:rows] < 0) | (row_token[:rows] >= T)).any():
        fail("row_token values must be tokens")
    per_expert_kept = np.bincount(e, minlength=E)
    if (per_expert_kept != kept).any():
        fail("each expert must keep exactly kept[e] assignments")
