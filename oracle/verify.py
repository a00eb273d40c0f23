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


# ----------------------------------------------- verification of sampled drafts
# Follows "Speculative Decoding Deep Dive III", section "EAGLE-1", its
# "Inference" list (the drafter samples its tokens and one target pass checks
# the tree by multi-round speculative sampling, keeping the target's
# distribution), and "transformer_math / tm_eagle_deep", section "Why draft
# confidence is a usable acceptance proxy" (keep a drafted token with
# probability min(1, p_target / p_draft)).
#
# Reading: when drafting samples, the children of a node are an ordered sample
# without replacement from the draft distribution q = softmax(s_d * z_draft)
# at that node (Gumbel-top-k gives them in draw order).  They are tested in
# that order; the j-th test uses the residual target r_j and the draft's
# proposal distribution q_j for the j-th draw: q restricted to the tokens not
# drawn before it, renormalised.  x_j is kept with probability
# min(1, r_j(x_j) / q_j(x_j)); after a rejection r_{j+1} = max(r_j - q_j, 0)
# renormalised.  r_1 = p, the target distribution.  When all are rejected one
# token is drawn from the last residual.  Every drawn child takes part, also
# one the verify tree dropped: accepting such a child ends the walk with its
# token (the target has no row below it).


def draft_probs_remaining(row, inv_temp, drawn_before):
    """q_j: softmax(s * z) over the tokens not in `drawn_before`; s * z is
    formed in fp32 (as the drafter forms it), the rest in fp64.  All zero if
    no token is left."""
    v = (np.float32(inv_temp) * np.asarray(row, np.float32)).astype(np.float64)
    keep = np.ones(v.size, bool)
    keep[list(drawn_before)] = False
    out = np.zeros(v.size)
    if not keep.any():
        return out
    e = np.exp(v[keep] - v[keep].max())
    out[keep] = e / e.sum()
    return out


def drafted_tests(p, draft_row, draft_inv_temp, drawn):
    """The successive tests at one node whose children `drawn` (token ids, in
    draw order) came from the draft row `draft_row`.

    Returns (thr, resid, mass): thr[j] = r_j(x_j) / q_j(x_j) (x_j is kept iff
    its uniform is below thr[j]; +inf when q_j(x_j) = 0 < r_j(x_j)); resid =
    the residual after every child was rejected, normalised (all zero when no
    mass is left); mass[j] = the unnormalised residual mass before test j
    relative to p (mass[0] = 1, mass[k] = that of resid).  r_j is the residual
    after rejecting x_1 .. x_{j-1}."""
    r = np.array(p, np.float64)
    thr = []
    mass = [1.0]
    for j, x in enumerate(drawn):
        qj = draft_probs_remaining(draft_row, draft_inv_temp, drawn[:j])
        if qj[x] > 0.0:
            thr.append(r[x] / qj[x])
        else:
            thr.append(np.inf if r[x] > 0.0 else 0.0)
        r = np.maximum(r - qj, 0.0)
        tot = r.sum()
        mass.append(mass[-1] * tot)
        r = r / tot if tot > 0.0 else np.zeros_like(r)
    return np.array(thr, np.float64), r, np.array(mass, np.float64)


def verify_sample_drafted(tok, parent, drawn, logits, inv_temp, draft_rows, draft_inv_temp,
                          draws, gamma):
    """Multi-round speculative sampling over one request's verify tree when
    the children were drawn from the draft.

    tok, parent, logits, draws as for `verify_sample` (draws[u][j] tests the
    j-th drawn child of position u, draws[u][16] is the residual draw);
    drawn[u]: list of (token, verify position or -1) of the children drafting
    drew at position u, in draw order (empty for a node never expanded);
    draft_rows[u]: the draft's logits at u (used when drawn[u] is not empty);
    draft_inv_temp: the drafter's s.  Returns (accept_len, path, out_tokens)
    as `verify_sample`.
    """
    path = [0]
    out = []
    u = 0
    while True:
        p = target_probs(logits[u], inv_temp)
        kids = list(drawn[u]) if len(path) - 1 < gamma else []
        if kids:
            thr, resid, _ = drafted_tests(p, draft_rows[u], draft_inv_temp, [x for x, _ in kids])
        else:
            thr, resid = np.zeros(0), p
        take = None
        for j, (x, v) in enumerate(kids):
            if draws[u][j] < thr[j]:
                take = (int(x), int(v))
                break
        if take is None:
            out.append(residual_draw(resid, [int(x) for x, _ in kids], draws[u][N_DRAWS - 1]))
            break
        out.append(take[0])
        if take[1] < 0:          # a child the verify tree dropped: its token ends the walk
            break
        u = take[1]
        path.append(u)
    acc = len(path) - 1
    pth = np.full(gamma + 1, -1, np.int32)
    o = np.full(gamma + 1, -1, np.int32)
    pth[:len(path)] = path
    o[:len(out)] = out
    return acc, pth, o
