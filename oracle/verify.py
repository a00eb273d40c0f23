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

Stochastic (lossless) verification, `verify_sample`, follows
  * "Speculative Decoding Deep Dive III", section "EAGLE-1", its
    "Inference" list: a tree draft is checked in one target pass by
    multi-round speculative sampling, which keeps the target's output
    distribution (lossless);
  * "transformer_math / tm_eagle_deep", section "Why draft confidence is a
    usable acceptance proxy": the standard test keeps a drafted token with
    probability min(1, p_target / p_draft).
Reading: p_draft is the probability with which the drafting procedure put
the token forward.  Top-k drafting puts every child forward with certainty,
so the test for a child token x is u < p(x), with p the target distribution
at the parent, softmax(s * logits), renormalised after each rejected sibling
(rejected tokens get probability 0: the residual max(p - q, 0) of a point
mass q).  Siblings are tried in verify-tree order.  When every child is
rejected, or the node has none, one token is drawn from the residual by
inverse CDF over token ids.  Random numbers are inputs: draws[u][i] for the
i-th child of position u, draws[u][16] for the residual draw at u.
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


N_DRAWS = 17          # per verify position: 16 child tests + 1 residual draw


def target_probs(row, inv_temp):
    """Target distribution at one position: softmax(s * logits); the scaled
    logit s * z is formed in fp32 (as the logits are stored), the rest in fp64."""
    v = (np.float32(inv_temp) * np.asarray(row, np.float32)).astype(np.float64)
    e = np.exp(v - v.max())
    return e / e.sum()


def residual_draw(p, excluded, u):
    """Inverse CDF over token ids of p with `excluded` tokens zeroed and the
    rest renormalised: the smallest x whose cumulative mass exceeds u.  With
    no mass left outside `excluded` (the rejected tokens held all of it) the
    token is the last one excluded."""
    r = np.array(p, np.float64)
    r[list(excluded)] = 0.0
    c = np.cumsum(r)
    if not c[-1] > 0.0:
        return int(list(excluded)[-1]) if len(excluded) else 0
    target = u * c[-1]
    x = int(np.searchsorted(c, target, side="right"))
    x = min(x, len(r) - 1)
    while r[x] == 0.0:          # never land on a zero-mass token (u -> 1 edge)
        x -= 1
    return x


def verify_sample(tok, parent, logits, inv_temp, draws, gamma):
    """Multi-round speculative sampling over one request's verify tree.

    tok, parent, logits as for `verify`; draws [T, 17] uniforms in [0, 1).
    Returns (accept_len, path [gamma+1], out_tokens [gamma+1]) in the same
    format as `verify`; the last out token is the one drawn at the deepest
    accepted node (from the residual if some child was rejected there).
    """
    T = len(tok)
    children = [[] for _ in range(T)]
    for v in range(1, T):
        children[int(parent[v])].append(v)
    path = [0]
    out = []
    u = 0
    while True:
        p = target_probs(logits[u], inv_temp)
        kids = children[u] if len(path) - 1 < gamma else []
        resid = p.copy()
        tried = []
        nxt = None
        for i, v in enumerate(kids):
            x = int(tok[v])
            if draws[u][i] < resid[x] / resid.sum():
                nxt = v
                break
            resid[x] = 0.0
            tried.append(x)
        if nxt is None:
            out.append(residual_draw(p, tried, draws[u][N_DRAWS - 1]))
            break
        u = nxt
        path.append(u)
        out.append(int(tok[u]))
    acc = len(path) - 1
    pth = np.full(gamma + 1, -1, np.int32)
    o = np.full(gamma + 1, -1, np.int32)
    pth[:len(path)] = path
    o[:len(out)] = out
    return acc, pth, o
