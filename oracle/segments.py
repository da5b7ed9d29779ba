"""Per-token adapter ids -> segments (oracle; test infrastructure only).

tinker-ticks, "How the SGMV kernel works": every user's tokens are flattened
into one matrix and a per-row segment index records which adapter owns each
row, so one launch can serve all adapters.  Here that index is made explicit:
`offsets[k]..offsets[k+1]` is key k's range in a stable ordering `perm` of the
tokens (token order kept within a key).  Keys outside [0, n_keys) are invalid;
they sort after every valid key and belong to no segment.
"""
from __future__ import annotations

import numpy as np


def segments(ids, n_keys: int):
    """Return (perm int64 [N], offsets int64 [n_keys+1]).

    offsets[k+1] - offsets[k] = number of tokens with id k; perm lists the
    tokens of key 0 in increasing token index, then key 1, ...; invalid tokens
    follow offsets[n_keys] in increasing token index.
    """
    ids = np.asarray(ids, dtype=np.int64)
    valid = (ids >= 0) & (ids < n_keys)
    counts = np.bincount(ids[valid], minlength=n_keys) if n_keys > 0 else np.zeros(0, np.int64)
    offsets = np.zeros(n_keys + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    key = np.where(valid, ids, n_keys)
    perm = np.argsort(key, kind="stable").astype(np.int64)
    return perm, offsets
