"""Oracle: one full draft-and-verify round (test infrastructure only).

Follows
  * "transformer_math / tm_eagle_deep", section "The recurrence, written out":
    the head rolls forward gamma times; the predicted feature f' of a node is
    the f of its children's rows, and every row's token comes from the frozen
    LM head;
  * "Speculative Decoding Deep Dive III", section "EAGLE-1 ... Inference" and
    the EAGLE-1 / EAGLE-3 input-regime examples: after the verified prefix the
    first row uses the target feature f (EAGLE-1) or the fused g of every
    verified position (EAGLE-3); later rows feed back the head's own output;
  * "transformer_math / tm_eagle_deep", sections "EAGLE-2: expand and rerank"
    and "Tree attention in one verification pass" (see oracle.tree);
  * the explainer's verification steps (see oracle.verify).

Readings (listed in the design notes):
  * EAGLE-3 combination: the layer input is the sum g + emb(t) at verified
    positions and a + emb(t) at later steps (no fc);
  * EAGLE-3 ingest: every verified position j gets x_j = g_j + emb(t_{j+1})
    and contributes K/V at position j to the context cache; only the last
    position's layer output drafts (the other positions' outputs are never
    read), so the full layer runs for that row alone, attending to all
    verified positions of its request;
  * a row attends to its request's whole context plus its ancestor-or-self
    slots; the root row of an EAGLE-1 round sits at position n_b;
  * EAGLE-3 steady state (the next round after a verification, "Speculative
    Decoding Deep Dive III", EAGLE-3 example: each round feeds the fused
    features of the verified tokens): only the positions verified since the
    last round are ingested; their K/V join the cache after the old ones.
  * EAGLE-1 steady state (the same page, EAGLE-1 "Inference": the drafter
    reads the target's features of the verified prefix): the newest positions
    are ingested from the target's features f_{j-1} and tokens t_j through fc
    and the layer's key/value projections; the round's root row stays at n_b.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

from .head import DraftHead, attend
from .tree import CHAIN, DYNAMIC, STATIC, RequestTree
from .sampling import gumbel_topk
from .verify import verify

MAX_SLOTS = 64


def row_forward(head: DraftHead, h, pos, ctx_k, ctx_v, anc_k, anc_v):
    """Decoder layer of ONE row given its input h [d], position, the request's
    context K/V [n, Hkv, hd] and its ancestor slots' K/V [a, Hkv, hd] (self
    excluded; the row's own k, v are appended here).

    Returns (out [d], k [Hkv, hd], v [Hkv, hd])."""
    q, k, v = head.qkv(h[None, :], np.array([pos]))
    K = np.concatenate([ctx_k, anc_k, k], axis=0)
    V = np.concatenate([ctx_v, anc_v, v], axis=0)
    att = attend(q[0], K, V, head.group)
    return head.finish(h[None, :], att[None])[0], k[0], v[0]


def ingest(head: DraftHead, lmh, ctx_tokens, pos0=0):
    """EAGLE-3 verified positions pos0 .. pos0 + n - 1 of ONE request.

    lmh [n, 3d] (the target's low/mid/high features), ctx_tokens [n] (token
    t_{j+1} following position j; the last is the anchor token).
    Returns (K [n, Hkv, hd], V [n, Hkv, hd], h_last [d]): every position's
    rotated key/value and the layer input of the last one."""
    n = lmh.shape[0]
    x = head.latent_input(head.fuse(lmh), ctx_tokens)        # g_j + emb(t_{j+1})
    _, K, V = head.qkv(x, np.arange(pos0, pos0 + n))
    return K, V, x[-1]


def ingest_features(head: DraftHead, feats, tokens, pos0):
    """EAGLE-1 verified positions pos0 .. pos0 + n - 1 of ONE request: the row
    of position j is fc([f_{j-1} ; emb(t_j)]) (the target's feature of the
    position before it, the token at it), as for every context position.
    feats [n, d], tokens [n].  Returns (K [n, Hkv, hd], V [n, Hkv, hd])."""
    n = feats.shape[0]
    h = head.fc_input(feats, tokens)
    _, K, V = head.qkv(h, np.arange(pos0, pos0 + n))
    return K, V


@dataclass
class StepTrace:
    rows: list                      # per request: list of row tuples (RequestTree.rows)
    h_in: np.ndarray                # [M, d] layer inputs
    feat: np.ndarray                # [M, d] layer outputs (f-hat / a)
    logits: np.ndarray              # [M, |V|]
    ids: np.ndarray                 # [M, top_k]
    conf: np.ndarray                # [M, top_k]
    lse: np.ndarray                 # [M]


@dataclass
class RoundResult:
    steps: List[StepTrace] = field(default_factory=list)
    trees: List[RequestTree] = field(default_factory=list)
    final: List[dict] = field(default_factory=list)
    accept_len: Optional[np.ndarray] = None
    accept_path: Optional[np.ndarray] = None
    out_tokens: Optional[np.ndarray] = None


def run_round(cfg, head: DraftHead, n, t_root, k_ctx=None, v_ctx=None,
              f_root=None, lmh=None, ctx_tokens=None, target=None,
              teacher=None, n_new=None):
    """One round for all B requests.

    n [B] context lengths; EAGLE-1 rounds take packed k_ctx/v_ctx
    [sum n, Hkv, hd] and f_root [B, d]; EAGLE-3 rounds take packed lmh
    [sum n, 3d] and ctx_tokens [sum n] -- or, in the steady state (n_new
    given), the K/V of each request's first n - n_new positions in k_ctx /
    v_ctx (segments of n rows) and lmh / ctx_tokens for its newest n_new
    positions only, packed (EAGLE-1: lmh [sum n_new, d] holds the target
    features of the positions before them, ctx_tokens the tokens at them;
    f_root as always).  target [B, T, |V|] are the verification logits
    (verify is skipped when None).
    teacher(step) -> (ids, conf) makes the tree follow someone else's
    discrete choices (teacher forcing); the oracle's own logits are still
    computed and recorded.
    """
    c = head.cfg
    dt = head.dt
    B = cfg.B
    e3 = c.mode == 3
    cu = np.concatenate([[0], np.cumsum(n)]).astype(np.int64)
    cun = None if n_new is None else np.concatenate([[0], np.cumsum(n_new)]).astype(np.int64)
    ctxK, ctxV, root_h = [], [], []
    for b in range(B):
        lo, hi = cu[b], cu[b + 1]
        if e3 and cun is not None:
            # steady state: the old positions' K/V are given, the newest
            # n_new[b] positions are ingested at positions n_old .. n - 1
            n_old = int(n[b]) - int(n_new[b])
            K, V, hl = ingest(head, lmh[cun[b]:cun[b + 1]], ctx_tokens[cun[b]:cun[b + 1]], n_old)
            ctxK.append(np.concatenate([k_ctx[lo:lo + n_old], K]))
            ctxV.append(np.concatenate([v_ctx[lo:lo + n_old], V]))
            root_h.append(hl)
        elif e3:
            K, V, hl = ingest(head, lmh[lo:hi], ctx_tokens[lo:hi])
            ctxK.append(K)
            ctxV.append(V)
            root_h.append(hl)
        elif cun is not None:
            # EAGLE-1 steady state: lmh holds the target features f_{j-1} and
            # ctx_tokens the tokens t_j of the newest n_new[b] positions
            n_old = int(n[b]) - int(n_new[b])
            K, V = ingest_features(head, lmh[cun[b]:cun[b + 1]], ctx_tokens[cun[b]:cun[b + 1]], n_old)
            ctxK.append(np.concatenate([k_ctx[lo:lo + n_old], K]))
            ctxV.append(np.concatenate([v_ctx[lo:lo + n_old], V]))
        else:
            ctxK.append(k_ctx[lo:hi])
            ctxV.append(v_ctx[lo:hi])
    top_k = 1 if cfg.tree == CHAIN else cfg.top_k
    trees = [RequestTree.start(cfg.tree, int(t_root[b]),
                               int(n[b]) - 1 if e3 else int(n[b]),
                               cfg.gamma, top_k, cfg.top_m, cfg.template, e3)
             for b in range(B)]
    sk = np.zeros((B, MAX_SLOTS, c.n_kv, c.head_dim), dt)
    sv = np.zeros_like(sk)
    sf = np.zeros((B, MAX_SLOTS, c.d), dt)
    res = RoundResult(trees=trees)
    for s in range(cfg.gamma):
        rows = [t.rows() for t in trees]
        hs, feats = [], []
        for b in range(B):
            for (u, ps, tok, pos, slot, mask) in rows[b]:
                if e3:
                    if ps < 0:
                        h = root_h[b]
                    else:
                        h = head.latent_input(sf[b, ps], tok)
                else:
                    parent_f = f_root[b] if ps < 0 else sf[b, ps]
                    h = head.fc_input(parent_f[None, :], np.array([tok]))[0]
                anc = [j for j in range(MAX_SLOTS) if (mask >> j) & 1 and j != slot]
                if e3 and ps < 0:
                    # the root row is the last verified position: its own K/V
                    # is already the last context entry
                    q, _, _ = head.qkv(h[None, :], np.array([pos]))
                    att = attend(q[0], ctxK[b], ctxV[b], head.group)
                    out = head.finish(h[None, :], att[None])[0]
                else:
                    out, k, v = row_forward(head, h, pos, ctxK[b], ctxV[b],
                                            sk[b, anc], sv[b, anc])
                    sk[b, slot], sv[b, slot] = k, v
                sf[b, slot] = out
                hs.append(h)
                feats.append(out)
        H = np.stack(hs)
        F = np.stack(feats)
        logits = head.lm_head(F)
        ids, conf, lse = DraftHead.draft_choices(logits, top_k, cfg.inv_temp)
        seed = getattr(cfg, "sample_seed", None)
        if seed is not None:
            # sampled drafting: top_k drawn without replacement (Gumbel-top-k),
            # row key b * 1024 + node; confidences of the drawn ids
            r = 0
            for b in range(B):
                for (u, *_rest) in rows[b]:
                    ids[r] = gumbel_topk(logits[r], top_k, cfg.inv_temp, seed, b * 1024 + u)[0]
                    z = logits[r] * logits.dtype.type(cfg.inv_temp)
                    conf[r] = np.exp(z[ids[r]] - lse[r])
                    r += 1
        res.steps.append(StepTrace(rows, H, F, logits, ids, conf, lse))
        use_ids, use_conf = (ids, conf) if teacher is None else teacher(s)
        r0 = 0
        for b in range(B):
            W = len(rows[b])
            trees[b].expand(s, use_ids[r0:r0 + W], use_conf[r0:r0 + W])
            r0 += W
    res.final = [t.final_tree() for t in trees]
    if target is not None:
        acc, path, out = [], [], []
        for b in range(B):
            f = res.final[b]
            a, p, o = verify(f["tok"], f["parent"], target[b, :len(f["tok"])], cfg.gamma)
            acc.append(a)
            path.append(p)
            out.append(o)
        res.accept_len = np.array(acc, np.int32)
        res.accept_path = np.stack(path)
        res.out_tokens = np.stack(out)
    return res
