"""The zig-zag context-parallel split, stated plainly for the tests ([PR8539], item 2 and
test plan: each rank scores its query chunks against the key prefix each chunk sees,
with the chunk's absolute causal offset).

A document of n rows is cut into 2*cp equal chunks; rank r holds chunks r and 2*cp-1-r.
For a chunk starting at row a (within its document) with c rows, the rows' absolute
1-based positions are a+1 .. a+c, so the last row sees floor((a+c)/ratio) compressed
keys: the prefix the chunk is scored against, with causal offset a.
"""
from __future__ import annotations


def share(doc_lens, ratio, cp, rank):
    """[(doc, chunk_start, chunk_rows, prefix_keys, batch_row0, batch_key0)] for one rank."""
    out = []
    row0 = key0 = 0
    for d, n in enumerate(doc_lens):
        c = n // (2 * cp)
        for idx in (rank, 2 * cp - 1 - rank):
            a = idx * c
            out.append((d, a, c, (a + c) // ratio, row0 + a, key0))
        row0 += n
        key0 += n // ratio
    return out
