"""An independent top-k for pinning the oracle: entries are taken one at a time in
ascending index order and kept in a list ordered by the selection rule.

The rule is the one the page "nvfp4-megamoe-kernel -- dsv4/kernels/indexer/
indexer_score_topk.cu" states for its heap and its final sort (heap_insert and the
closing sort of the main kernel): a larger score ranks first, and of two equal
scores the lower index ranks first; a query's k output slots start out as
(-inf, -1), so slots that no entry fills keep index -1.  Nothing here follows that
page's code: the kept list is maintained with ``bisect`` on the key (-score, index),
and the list never grows past k entries.
"""

import bisect
import math


def insertion_topk(scores, k):
    """(indices, scores) of the k best entries in selection order, -1 / -inf padded."""
    kept = []  # sorted ascending by (-score, index): the best entry first
    for s, v in enumerate(scores):
        key = (-float(v), s)
        if len(kept) == k and key >= kept[-1]:
            continue  # ranks below every kept entry
        bisect.insort(kept, key)
        if len(kept) > k:
            kept.pop()
    idx = [s for _, s in kept] + [-1] * (k - len(kept))
    val = [-nv for nv, _ in kept] + [-math.inf] * (k - len(kept))
    return idx, val
