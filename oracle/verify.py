"""Oracle: greedy tree verification (test infrastructure only).

Follows
  * "EAGLE / DFlash / DSpark" explainer (kaushalya.io), steps "3 - target
    verification" and "4 - output of the round": the target accepts the longest
    matching prefix; after the first rejection later draft tokens are
    discarded; the output is the accepted prefix plus the target's corrected
    token at the rejection point.
  * "transformer_math / tm_eagle_deep", section "Tree attention in one
    verification pass": one target pass gives, for every tree node, the
    target's next-token distribution conditioned on that node's path.

Reading (greedy decoding, the pages leave the sampling rule open here): the
target's choice after node u is argmax of its logits at u, lowest id on ties;
child v of u is accepted iff token(v) equals that choice.  Siblings carry
distinct tokens, so the accepted path is unique.
"""
from __future__ import annotations

import numpy as np


def target_choice(row):
    """Greedy target token: argmax, lowest id among equal maxima."""
    return int(np.flatnonzero(row == row.max())[0])


def verify(tok, parent, logits, gamma):
    """Walk the verify tree of one request from the root.

    tok, parent: [T] verify-tree tokens and parent positions (root = 0,
    parent -1); logits: [T, |V|] target logits per position.
    Returns (accept_len, path [gamma+1], out_tokens [gamma+1]); unused
    entries are -1.  path[0] = 0 (the root); out_tokens lists the accepted
    draft tokens followed by the target's token at the deepest accepted node.
    """
    T = len(tok)
    children = [[] for _ in range(T)]
    for v in range(1, T):
        children[int(parent[v])].append(v)
    path = [0]
    out = []
    u = 0
    while True:
        choice = target_choice(logits[u])
        nxt = [v for v in children[u] if int(tok[v]) == choice]
        if not nxt:
            out.append(choice)
            break
        u = nxt[0]
        path.append(u)
        out.append(int(tok[u]))
    acc = len(path) - 1
    p = np.full(gamma + 1, -1, np.int32)
    o = np.full(gamma + 1, -1, np.int32)
    p[:len(path)] = path
    o[:len(out)] = out
    return acc, p, o
