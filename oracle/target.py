"""Oracle: the target model's verification pass over the draft tree, and the
compaction of the accepted path's keys and values (test infrastructure only:
imported by tests/, the smoke check and the benchmark's CPU baseline, never
by the product path).

Follows
  * "transformer_math / tm_eagle_deep", section "Tree attention in one
    verification pass": the flattened tree goes through the target in one
    forward pass; each node attends to the context and to its own ancestors,
    and its position id is the root's position plus its depth;
  * "EAGLE / DFlash / DSpark" explainer, section "How speculative decoding
    works", steps 3 and 4: the target's distributions at the tree nodes decide
    acceptance; the accepted prefix joins the sequence for the next round.

Readings where the pages are silent (listed in the design notes):
  * the target is a stack of L pre-norm decoder layers of the same form as the
    draft head's layer (oracle/head.py), then a final RMSNorm and the LM head;
    the embedding and the LM head are the ones the draft head shares;
  * a node attends to itself (ancestor-or-self), as in the draft's tree
    attention;
  * after verification the keys and values the target computed for the root
    and the accepted nodes (path positions 0 .. accept_len) are appended to
    the target's cache, in path order; the rest of the tree is dropped.
"""
from __future__ import annotations

import numpy as np

from .head import DraftHead, attend, rms_norm


def mask_bits(mask, T):
    """Positions set in a 64-bit ancestor-or-self mask."""
    m = int(mask) & ((1 << 64) - 1)
    return [j for j in range(T) if (m >> j) & 1]


def tree_layer(layer, x, pos, masks, ctx, store=None):
    """One decoder layer over the T tree positions of one request: rows x
    [T, d] at position ids pos, row u attending to the layer's context cache
    ctx = (K, V) and to the tree positions in its ancestor-or-self mask.
    Returns (out [T, d], k, v [T, Hkv, hd])."""
    T = len(x)
    q, k, v = layer.qkv(x, np.asarray(pos))
    att = np.empty_like(q)
    ck, cv = ctx
    for u in range(T):
        sel = mask_bits(masks[u], T)
        att[u] = attend(q[u], np.concatenate([ck, k[sel]]), np.concatenate([cv, v[sel]]),
                        layer.group)
    return layer.finish(x, att, store), k, v


def final_logits(x, final_g, eps, lm_head):
    """Final RMSNorm, then the shared LM head: logits [T, V]."""
    return rms_norm(x, final_g, eps) @ lm_head.T


def tree_forward(layers, emb, final_g, eps, lm_head, tok, pos, masks, ctx, store=None):
    """Target logits at every verify-tree position of one request.

    layers: list of L DraftHead objects (only their decoder-layer weights are
    used) or a callable l -> DraftHead (so callers can materialise one layer
    at a time); emb [V, d]; final_g [d]; lm_head [V, d]; tok, pos [T];
    masks [T] ancestor-or-self bitmasks over positions; ctx: list of L pairs
    (K [n, Hkv, hd], V [n, Hkv, hd]), the layer's context cache; store:
    optional map applied to the residual stream, after attention and after
    every layer (e.g. rounding to the storage type of a bf16 model).
    Returns (logits [T, V], per-layer tree keys and values [(k, v)] of shape
    [T, Hkv, hd]).
    """
    get = layers if callable(layers) else (lambda l: layers[l])
    x = emb[np.asarray(tok)]
    kv_tree = []
    for l in range(len(ctx)):
        x, k, v = tree_layer(get(l), x, pos, masks, ctx[l], store)
        if store is not None:
            x = store(x)
        kv_tree.append((k, v))
    return final_logits(x, final_g, eps, lm_head), kv_tree


def causal_forward(layers, emb, final_g, eps, lm_head, tokens, pos0, ctx):
    """Plain causal decoding of one token sequence placed at positions
    pos0, pos0 + 1, ... after the context: every token attends to the context,
    to the tokens before it and to itself.  Returns logits [len, V]."""
    S = len(tokens)
    get = layers if callable(layers) else (lambda l: layers[l])
    x = emb[np.asarray(tokens)]
    pos = pos0 + np.arange(S)
    for l in range(len(ctx)):
        layer = get(l)
        q, k, v = layer.qkv(x, pos)
        ck, cv = ctx[l]
        att = np.empty_like(q)
        for i in range(S):
            att[i] = attend(q[i], np.concatenate([ck, k[:i + 1]]), np.concatenate([cv, v[:i + 1]]),
                            layer.group)
        x = layer.finish(x, att)
    return rms_norm(x, final_g, eps) @ lm_head.T


def commit_path(kv_tree, accept_len, path):
    """Keys and values of the root and the accepted nodes, in path order:
    [(k [acc + 1, Hkv, hd], v)] per layer."""
    sel = [int(p) for p in path[:accept_len + 1]]
    return [(k[sel], v[sel]) for k, v in kv_tree]


def layer_heads(cfg, layer_weights, dtype=np.float32):
    """DraftHead objects holding only decoder-layer weights."""
    return [DraftHead(cfg, w, dtype) for w in layer_weights]
