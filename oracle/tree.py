"""Oracle: draft trees (test infrastructure only; see package header).

Follows
  * "EAGLE: Drafting in Feature Space", section "Drafting a Tree, Not a Chain":
    EAGLE-1 uses one fixed branching pattern for every context (the static
    template here); a chain is the template with fan-out 1.
  * "transformer_math / tm_eagle_deep", section "EAGLE-2: expand and rerank":
    every node carries value = product of the draft confidences on its root
    path; only the highest-value nodes are expanded, each to its top-k
    children; after expansion all generated nodes are pooled and the top m by
    value are kept for verification.
  * "Speculative Decoding Deep Dive III", section "EAGLE-2": V_i = prod_j c_j,
    expand top-k, keep top-m by V.
  * "transformer_math / tm_eagle_deep", section "Tree attention in one
    verification pass": the tree is flattened, every node attends only to its
    ancestors, and its position id is set from its depth.

Readings where the pages are silent (listed in the design notes):
  * the dynamic frontier at step s >= 1 is the top_k nodes of the newest depth
    by value (beam width top_k); unexpanded nodes stay in the pool;
  * ordering keys: top-k by (logit desc, id asc); frontier and rerank by
    (value desc, depth asc, creation index asc), a NaN value below all others;
  * value(root) = 1 and value(child) = float32(value(parent) * conf(child));
  * creation order = (step, frontier rank of the parent, child rank); the
    verify tree lists the kept nodes in creation order, root first;
  * position id of a node = root position + depth; the root sits at n_b for
    EAGLE-1 rounds and at n_b - 1 (the last verified position) for EAGLE-3;
  * each expanded node owns one "slot" (its K/V and feature); a row's slot
    mask has bit j set when slot j is an ancestor-or-self holding K/V.  In
    EAGLE-3 rounds the root's K/V lives in the context cache, so its slot
    holds only the feature and never appears in a mask.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Sequence

import numpy as np

CHAIN, STATIC, DYNAMIC = 0, 1, 2
MAX_SLOTS = 64   # masks are 64-bit


def static_children(template: Sequence[int]):
    """children[node] for a template given as parent-of-node (node i+1)."""
    n = len(template) + 1
    ch: List[List[int]] = [[] for _ in range(n)]
    for i, p in enumerate(template):
        if not (0 <= p <= i):
            raise ValueError("template parents must precede their children")
        ch[p].append(i + 1)
    return ch


def template_depths(template: Sequence[int]):
    dep = [0] * (len(template) + 1)
    for i, p in enumerate(template):
        dep[i + 1] = dep[p] + 1
    return dep


@dataclass
class RequestTree:
    """Node pool and frontier of one request."""
    kind: int
    gamma: int
    top_k: int
    top_m: int
    root_pos: int
    eagle3: bool = False
    template: Sequence[int] = ()
    tok: List[int] = field(default_factory=list)
    parent: List[int] = field(default_factory=list)
    depth: List[int] = field(default_factory=list)
    conf: List[np.float32] = field(default_factory=list)
    value: List[np.float32] = field(default_factory=list)
    slot: List[int] = field(default_factory=list)
    slot_mask: List[int] = field(default_factory=list)   # per slot
    frontier: List[int] = field(default_factory=list)
    tnode: List[int] = field(default_factory=list)        # pool -> template node

    @classmethod
    def start(cls, kind, root_tok, root_pos, gamma, top_k, top_m=0,
              template=(), eagle3=False):
        t = cls(kind=kind, gamma=gamma, top_k=top_k, top_m=top_m,
                root_pos=root_pos, eagle3=eagle3, template=tuple(template))
        t.tok, t.parent, t.depth = [int(root_tok)], [-1], [0]
        t.conf, t.value = [np.float32(1.0)], [np.float32(1.0)]
        t.slot = [0]
        t.slot_mask = [0 if eagle3 else 1]
        t.frontier = [0]
        t.tnode = [0]
        if kind == STATIC:
            t._tch = static_children(template)
        return t

    # -- rows the next draft step runs
    def rows(self):
        """(node, parent_slot, token, position, slot, mask) per frontier row.
        parent_slot is -1 for the root (its input feature comes from the
        target, or, in EAGLE-3 rounds, from the ingest)."""
        out = []
        for u in self.frontier:
            p = self.parent[u]
            out.append((u, -1 if p < 0 else self.slot[p], self.tok[u],
                        self.root_pos + self.depth[u], self.slot[u],
                        self.slot_mask[self.slot[u]]))
        return out

    def _new_node(self, tok, parent, conf, tnode=-1):
        self.tok.append(int(tok))
        self.parent.append(parent)
        self.depth.append(self.depth[parent] + 1)
        c = np.float32(conf)
        self.conf.append(c)
        self.value.append(np.float32(self.value[parent] * c))
        self.slot.append(-1)
        self.tnode.append(tnode)
        return len(self.tok) - 1

    def _give_slots(self, nodes):
        for u in nodes:
            s = len(self.slot_mask)
            if s >= MAX_SLOTS:
                raise ValueError("more than 64 expanded nodes per request")
            self.slot[u] = s
            pm = self.slot_mask[self.slot[self.parent[u]]]
            self.slot_mask.append(pm | (1 << s))

    def key(self, u):
        """Frontier / rerank order: value desc, depth asc, creation index asc.
        A NaN value (from a NaN logit row; values otherwise lie in [0, 1])
        ranks below every other value, so the order stays total."""
        v = float(self.value[u])
        return (-(v if v == v else -1.0), self.depth[u], u)

    def expand(self, step, ids, conf):
        """Append the children produced by draft step `step`.

        ids, conf: [rows, top_k] for the frontier rows in order (ids sorted by
        logit desc, id asc).  Then choose the frontier of step+1.
        """
        ids = np.asarray(ids)
        conf = np.asarray(conf, dtype=np.float32)
        assert ids.shape[0] == len(self.frontier)
        new = []
        for r, u in enumerate(self.frontier):
            if self.kind == CHAIN:
                new.append(self._new_node(ids[r, 0], u, conf[r, 0]))
            elif self.kind == STATIC:
                for rank, tc in enumerate(self._tch[self.tnode[u]]):
                    new.append(self._new_node(ids[r, rank], u, conf[r, rank], tc))
            else:
                for rank in range(self.top_k):
                    new.append(self._new_node(ids[r, rank], u, conf[r, rank]))
        if step + 1 >= self.gamma:
            self.frontier = []
            return
        if self.kind == CHAIN:
            nxt = new
        elif self.kind == STATIC:
            nxt = [u for u in new if len(self._tch[self.tnode[u]]) > 0]
        else:
            nxt = sorted(new, key=self.key)[:self.top_k]
        self._give_slots(nxt)
        self.frontier = nxt

    # -- rerank and the verify tree
    def rerank(self):
        """Pool nodes kept for verification (non-root), in key order."""
        cand = list(range(1, len(self.tok)))
        if self.kind != DYNAMIC:
            return cand
        return sorted(cand, key=self.key)[:self.top_m]

    def final_tree(self):
        """Verify tree: root + kept nodes in creation order.

        Returns dict of arrays: node, tok, parent (position, -1 for root),
        depth, pos (position id), mask (uint64 ancestor-or-self over positions).
        """
        kept = sorted(set(self.rerank()) | {0})
        where = {u: i for i, u in enumerate(kept)}
        T = len(kept)
        if T > 64:
            raise ValueError("verify tree larger than 64 positions")
        par = np.full(T, -1, np.int32)
        mask = np.zeros(T, np.uint64)
        for i, u in enumerate(kept):
            p = self.parent[u]
            if p >= 0:
                if p not in where:
                    raise AssertionError("kept set is not ancestor-closed")
                par[i] = where[p]
            m = np.uint64(1) << np.uint64(i)
            if par[i] >= 0:
                m |= mask[par[i]]
            mask[i] = m
        dep = np.array([self.depth[u] for u in kept], np.int32)
        return dict(node=np.array(kept, np.int32),
                    tok=np.array([self.tok[u] for u in kept], np.int32),
                    parent=par, depth=dep,
                    pos=(self.root_pos + dep).astype(np.int32), mask=mask)

