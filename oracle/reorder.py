"""Reverse Cuthill-McKee reordering, written from its definition.  TEST
INFRASTRUCTURE ONLY (see the package docstring).

The AsyncSparse paper preprocesses every evaluation matrix with reverse
Cuthill-McKee before building its formats (Section IV-A), citing Cuthill and
McKee, "Reducing the bandwidth of sparse symmetric matrices" (1969).  The paper
does not fix a start-vertex rule or tie-breaking, so the oracle fixes them, each
a standard choice from the reordering literature (George and Liu's
pseudo-peripheral search for the start, degree-then-index order for ties):

1. graph: the pattern of A plus its transpose, self loops dropped;
2. each component starts from the unnumbered vertex of least degree (ties:
   least index), then moves to a pseudo-peripheral vertex by George and Liu's
   search: root a level structure there, take the least-degree (then
   least-index) vertex of its last level, and move to it while its level
   structure is taller;
3. Cuthill-McKee numbering: breadth first from that vertex; the unnumbered
   neighbours of each dequeued vertex are numbered by increasing degree, then
   index;
4. the numbering of all components, in order, is reversed.

Plain Python containers only; meant for graphs of up to a few ten thousand
vertices.
"""

from __future__ import annotations

from collections import deque

import numpy as np


def symmetric_adjacency(n: int, row_ptr, col_idx) -> list:
    """Neighbour sets of pattern(A) + pattern(A)^T without self loops."""
    adj = [set() for _ in range(n)]
    for i in range(n):
        for e in range(int(row_ptr[i]), int(row_ptr[i + 1])):
            j = int(col_idx[e])
            if j != i:
                adj[i].add(j)
                adj[j].add(i)
    return adj


def _level_structure(adj, root: int):
    """Breadth-first distances from root, for root's component only."""
    dist = {root: 0}
    queue = deque([root])
    while queue:
        v = queue.popleft()
        for w in adj[v]:
            if w not in dist:
                dist[w] = dist[v] + 1
                queue.append(w)
    return dist


def _pseudo_peripheral(adj, start: int) -> int:
    """George and Liu's search, from `start` (step 2 of the module docstring)."""
    r = start
    dist = _level_structure(adj, r)
    height = max(dist.values())
    while True:
        last = [v for v, d in dist.items() if d == height]
        x = min(last, key=lambda v: (len(adj[v]), v))
        dist_x = _level_structure(adj, x)
        height_x = max(dist_x.values())
        if height_x <= height:
            return r
        r, dist, height = x, dist_x, height_x


def rcm_order(n: int, row_ptr, col_idx) -> np.ndarray:
    """perm[i] = old index of the vertex numbered i (reverse Cuthill-McKee)."""
    adj = symmetric_adjacency(n, row_ptr, col_idx)
    numbered = [False] * n
    order = []
    while len(order) < n:
        free = [v for v in range(n) if not numbered[v]]
        start = min(free, key=lambda v: (len(adj[v]), v))
        root = _pseudo_peripheral(adj, start)
        numbered[root] = True
        queue = deque([root])
        order.append(root)
        while queue:
            v = queue.popleft()
            fresh = sorted((w for w in adj[v] if not numbered[w]), key=lambda w: (len(adj[w]), w))
            for w in fresh:
                numbered[w] = True
                order.append(w)
                queue.append(w)
    order.reverse()
    return np.asarray(order, dtype=np.int32)


def permute_symmetric(n: int, row_ptr, col_idx, values, perm):
    """A' = P A P^T: entry (perm[i], perm[j]) of A becomes entry (i, j)."""
    inv = np.empty(n, dtype=np.int64)
    inv[np.asarray(perm, dtype=np.int64)] = np.arange(n)
    entries = []
    for r in range(n):
        for e in range(int(row_ptr[r]), int(row_ptr[r + 1])):
            entries.append((int(inv[r]), int(inv[int(col_idx[e])]), int(values[e])))
    entries.sort()
    out_ptr = np.zeros(n + 1, dtype=np.int32)
    for i, _, _ in entries:
        out_ptr[i + 1] += 1
    out_ptr = np.cumsum(out_ptr).astype(np.int32)
    out_col = np.asarray([c for _, c, _ in entries], dtype=np.int32)
    out_val = np.asarray([v for _, _, v in entries], dtype=np.uint16)
    return out_ptr, out_col, out_val


def bandwidth(n: int, row_ptr, col_idx) -> int:
    """max |i - j| over the entries (i, j) of a CSR pattern (0 if empty)."""
    best = 0
    for i in range(n):
        for e in range(int(row_ptr[i]), int(row_ptr[i + 1])):
            best = max(best, abs(i - int(col_idx[e])))
    return best
