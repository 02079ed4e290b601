"""Grouping of a mixed-adapter batch by adapter (oracle side).

Test infrastructure only (see ``oracle/__init__.py``).

"Punica: Serving multiple LoRA finetuned LLM as one" (README, Overview) splits the
input batch X into the parts x1..xn that map to each LoRA model and computes each
part's add-on x_i@A_i@B_i; its kernel is "Segmented" for that reason.  The
segment description used here:

* ``seg_indptr``  int32 [n_adapters + 1]: CSR offsets over adapter ids, empty
  adapters included; seg_indptr[a+1] - seg_indptr[a] = number of tokens on a.
* ``sorted_tok``  int32 [T]: token indices ordered by (adapter id, token index),
  i.e. a stable sort, so the result is unique.

Every adapter id must lie in [0, n_adapters); there is no "no adapter" value.
"""

from __future__ import annotations

import numpy as np


def build_segments(adapter_id, n_adapters: int):
    """Return ``(seg_indptr, sorted_tok)`` for per-token adapter ids.

    Raises ValueError if an id is outside [0, n_adapters) or n_adapters < 1.
    """
    if n_adapters < 1:
        raise ValueError("n_adapters must be >= 1")
    ids = np.asarray(adapter_id, dtype=np.int64).reshape(-1)
    if ids.size and (ids.min() < 0 or ids.max() >= n_adapters):
        raise ValueError("adapter id out of range")
    counts = np.bincount(ids, minlength=n_adapters)
    seg_indptr = np.zeros(n_adapters + 1, dtype=np.int32)
    seg_indptr[1:] = np.cumsum(counts)
    sorted_tok = np.argsort(ids, kind="stable").astype(np.int32)
    return seg_indptr, sorted_tok
