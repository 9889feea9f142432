"""Reference outputs of the symmetric operator at t = 1 for a few rows of a
very long input, from the oracle's dense definition over only the inputs
whose terms can be nonzero (test infrastructure)."""
import numpy as np
import torch

import oracle

# exp(-d) is exactly +0 in float64 once d > 746 (below half the smallest
# subnormal, e^-744.4); a sum that starts at +0 is unchanged by such terms.
ZERO_REACH = 746.0


def dense_rows_near(a, x, rows, width=256.0, progress=None):
    """The dense definition y_i = sum_j exp(-|a_i - a_j|) x_j (t = 1) for the
    listed i, summed over only the j whose term can be nonzero.

    Anchors are put in buckets of `width` by value (an integer key, sorted
    stably on the host); for i in bucket b, every j with |a_i - a_j| <= 746
    lies in buckets b - r .. b + r, r = ceil(746 / width), a contiguous range
    of the bucket order.  Terms outside it are exact zeros, so each row is the
    dense row up to the order of its float64 additions."""
    lo = float(a.min())
    key = np.floor((a.astype(np.float64) - lo) / width).astype(np.int32)
    assert key.max() < 32767
    key = key.astype(np.int16)
    order = torch.from_numpy(np.argsort(key, kind="stable"))
    a_b = torch.from_numpy(a)[order].numpy()
    x_b = torch.from_numpy(x)[order].numpy()
    del order
    start = np.concatenate([[0], np.cumsum(np.bincount(key, minlength=int(key.max()) + 1))])
    r = int(np.ceil(ZERO_REACH / width))
    out = np.empty(rows.size)
    for q, i in enumerate(rows):
        b = int(key[i])
        s0 = start[max(b - r, 0)]
        s1 = start[min(b + r + 1, start.size - 1)]
        out[q] = oracle.apply_dense(a[i:i + 1], x_b[s0:s1], b=a_b[s0:s1])[0]
        if progress and (q + 1) % 64 == 0:
            progress(f"  oracle rows {q + 1}/{rows.size}")
    return out
