"""Ragged sort of routed token rows into contiguous per-expert groups.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the pages fix ("Quantize activations before EP all gather", the
description and the two review comments on ``ragged_sort.py``):

* the activation sort moves the already-quantized rows (``qvalue``) and
  gathers the scale along with them only when the scale is per token
  (its leading dimension equals the token count); a per-tensor or
  per-channel scale is passed through unchanged;
* rows are gathered by ``token_indices_sorted`` into the window of sorted
  rows that belongs to this expert-parallel shard; one variant gathers into
  ``[shard_output_start, shard_output_end)`` of the full sorted buffer, the
  other into a compact window ``[0, gather_end)``;
* the grouped matmul then sees ``group_sizes`` (rows per expert) and
  ``group_offset`` (first expert of this shard).

Readings where the pages are silent or offer two options:

* the sort is stable (a counting sort by expert id that keeps the flat
  order ``t * k + j`` among equal ids), so the permutation is unique;
* the compact window layout is used: local sorted row 0 is the first row of
  expert ``group_offset``; ``group_sizes`` stays the global [E] histogram;
* rows ``[n, M_cap)`` of the sorted buffer and their scales are zero.
"""

import numpy as np

from .quantize import SCALE_ROW_DYNAMIC


def sort_by_expert(expert_ids, num_experts, group_offset, num_local_experts,
                   xq=None, xscale=None, xscale_mode=SCALE_ROW_DYNAMIC, m_cap=None):
    """Stable counting sort of the routed rows by expert.

    expert_ids: int [T, k], each entry in [0, num_experts).
    xq: optional uint8 [T, H] quantized token rows; xscale: their scales
    ([T] in row mode, [1] otherwise).

    Returns a dict with
      perm [T*k] int32   flat routed index f = t*k + j of each sorted row
      inv_pos [T*k] int32 local sorted row of f, or -1 when f is not local
      group_sizes [E] int32
      start, n           first global sorted row of the local window, its length
      xs [m_cap, H] uint8, ss [m_cap] float32 (row mode) or the passed-through
                         tensor scale (other modes)
    """
    ids = np.asarray(expert_ids)
    if ids.ndim != 2:
        raise ValueError("sort_by_expert: expert_ids must be [T, k]")
    T, k = ids.shape
    M = T * k
    flat = ids.reshape(-1).astype(np.int64)
    if M and (flat.min() < 0 or flat.max() >= num_experts):
        raise ValueError("sort_by_expert: expert id out of range")
    perm = np.argsort(flat, kind="stable").astype(np.int64)
    group_sizes = np.bincount(flat, minlength=num_experts).astype(np.int64)
    start = int(group_sizes[:group_offset].sum())
    n = int(group_sizes[group_offset:group_offset + num_local_experts].sum())
    rank = np.empty(M, dtype=np.int64)
    rank[perm] = np.arange(M)
    local = (rank >= start) & (rank < start + n)
    inv_pos = np.where(local, rank - start, -1)
    if m_cap is None:
        m_cap = n
    if m_cap < n:
        raise ValueError("sort_by_expert: m_cap smaller than the local row count")
    out = {
        "perm": perm.astype(np.int32),
        "inv_pos": inv_pos.astype(np.int32),
        "group_sizes": group_sizes.astype(np.int32),
        "start": start,
        "n": n,
    }
    src_tokens = perm[start:start + n] // k
    if xq is not None:
        xq = np.asarray(xq, dtype=np.uint8)
        xs = np.zeros((m_cap, xq.shape[1]), dtype=np.uint8)
        xs[:n] = xq[src_tokens]
        out["xs"] = xs
    if xscale is not None:
        xscale = np.asarray(xscale, dtype=np.float32)
        if xscale_mode == SCALE_ROW_DYNAMIC:
            ss = np.zeros(m_cap, dtype=np.float32)
            ss[:n] = xscale[src_tokens]
            out["ss"] = ss
        else:
            out["ss"] = xscale.copy()
    return out
