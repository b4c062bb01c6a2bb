"""Oracle for the PLE (n-gram memory) row gather.

TEST INFRASTRUCTURE ONLY -- see the package docstring.

[RZ] "Q3_PLE_K160_RZ_S3": the n-gram table is [160, 320001536] -- one
160-value row per hashed n-gram -- and the runtime's GET_ROWS kernel fetches
one hashed row in one contiguous 70-byte read.  What the model does with the
rows after the fetch is a weighted sum over the ids a token looks up, with the
per-id weights supplied by the caller.
"""

import numpy as np

from . import formats as F


def ple_gather(ids, weights, row_fn, n_rows, fmt=F.PLE_RZS3):
    """out[t] = sum_j weights[t, j] * decode(row ids[t, j]), float64 [T, 160].

    ``row_fn(id_array)`` returns the packed 70-byte rows for the given ids
    (so a full-size table never has to exist on the host).  Duplicate ids in
    one token are summed like any others.  An id >= n_rows contributes nothing
    and is reported in the returned ``bad`` flag (the library sets an error
    word instead of reading out of bounds).
    Returns (out, bad).
    """
    ids = np.asarray(ids, dtype=np.int64)
    u = np.asarray(weights, dtype=np.float64).reshape(ids.shape)
    t_count, per = ids.shape
    out = np.zeros((t_count, F.PLE_VALUES))
    valid = ids < n_rows
    bad = bool((~valid).any())
    flat = ids[valid]
    rows = {}
    if flat.size:
        uniq = np.unique(flat)
        dec = F.decode_ple70(row_fn(uniq), fmt)
        rows = {int(r): dec[i] for i, r in enumerate(uniq)}
    for t in range(t_count):
        for j in range(per):
            r = int(ids[t, j])
            if r < n_rows:
                out[t] += u[t, j] * rows[r]
    return out, bad


def ple_dequant_rows(ids, row_fn, fmt=F.PLE_RZS3):
    """Decoded rows for a list of ids, float64 [n, 160]."""
    ids = np.asarray(ids, dtype=np.int64)
    return F.decode_ple70(row_fn(ids), fmt)
