"""Host-side precondition check for debugging: the slot-aliasing rules the
library assumes but never checks on the device (two requests of one launch
must not name the same live slot, and no commit destination may be another
request's source or destination).  It copies the index arrays to the host,
so it belongs in tests and debug builds, not on a hot path."""
from __future__ import annotations

from typing import Optional

import numpy as np


def _host(a) -> Optional[np.ndarray]:
    if a is None:
        return None
    if hasattr(a, "detach"):
        a = a.detach().to("cpu").numpy()
    return np.asarray(a).astype(np.int64)


def check_slot_aliasing(state_indices, *, num_slots: int,
                        null_block_id: int = 0, commit_lens=None,
                        final_state_indices=None,
                        boundary_state_indices=None) -> None:
    """Raise ValueError when the slots of one launch alias.

    Sources (`state_indices`) of live requests must be distinct.  A request
    that commits (commit length > 0, or any when `commit_lens` is None)
    writes its final slot and, if given and live, its boundary slot; each
    of those may be its own source (in place) but not another request's
    source or destination.  Slots <= null_block_id or >= num_slots are null
    and never alias."""
    src = _host(state_indices)
    lens = _host(commit_lens)
    fin = _host(final_state_indices)
    bnd = _host(boundary_state_indices)

    def live(s):
        return null_block_id < s < num_slots

    owner = {}
    for b, s in enumerate(src):
        if live(s):
            if s in owner:
                raise ValueError(f"requests {owner[s]} and {b} both read "
                                 f"slot {s}")
            owner[s] = b
    for b, s in enumerate(src):
        if not live(s) or (lens is not None and lens[b] <= 0):
            continue
        dests = {int(fin[b]) if fin is not None else int(s)}
        if bnd is not None:
            dests.add(int(bnd[b]))
        for d in dests:
            if not live(d) or d == s:
                continue
            if d in owner and owner[d] != b:
                raise ValueError(f"request {b} writes slot {d}, which "
                                 f"request {owner[d]} also uses")
            owner[d] = b
