"""Sequential replay of the listing's heap top-k, used as an independent pin.

"nvfp4-megamoe-kernel -- dsv4/kernels/indexer/indexer_score_topk.cu": the heap is
pre-filled with (-inf, -1); ``heap_insert`` rejects a score that does not beat the
root and otherwise replaces the root and sifts down, a child being "smaller" when
its score is lower or, at equal scores, its index is higher; the final pass is a
selection sort by score descending, ties to the lower index.  Replayed one entry
at a time in ascending s there is no race, and the result is the exact top-k.
"""

import math


def heap_topk(scores, k):
    hs = [-math.inf] * k
    hb = [-1] * k

    def smaller(a, b):
        return hs[a] < hs[b] or (hs[a] == hs[b] and hb[a] > hb[b])

    for s, v in enumerate(scores):
        if v <= hs[0]:
            continue
        hs[0], hb[0] = v, s
        root = 0
        while root < (k >> 1):
            left, right = 2 * root + 1, 2 * root + 2
            small = root
            if left < k and smaller(left, small):
                small = left
            if right < k and smaller(right, small):
                small = right
            if small == root:
                break
            hs[root], hs[small] = hs[small], hs[root]
            hb[root], hb[small] = hb[small], hb[root]
            root = small
    order = list(range(k))
    for i in range(k):
        best = i
        for j in range(i + 1, k):
            if hs[order[j]] > hs[order[best]] or (hs[order[j]] == hs[order[best]] and hb[order[j]] < hb[order[best]]):
                best = j
        order[i], order[best] = order[best], order[i]
    return [hb[o] for o in order], [hs[o] for o in order]
