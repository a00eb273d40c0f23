"""Oracle: the EAGLE draft head (test infrastructure only; see package header).

Follows
  * "transformer_math / tm_eagle_deep", section "The recurrence, written out":
    x = concat(f, emb(t)) in R^{2d}; h = fc(x) in R^d; f' = DecoderLayer(h,
    cache); next token from softmax(LM_head(f')).
  * same page, section "What is actually in the head": fc of shape [2d, d],
    one decoder layer (self-attention plus MLP) of width d, shared embedding
    and LM head.
  * "Speculative Decoding Deep Dive III", section "EAGLE-3": g = FC([l; m; h]);
    later draft steps feed back the free latent a plus the token embedding.
  * "EAGLE: Drafting in Feature Space", section "The Mechanism": the LM head is
    one linear layer applied to the feature.

Readings where the pages are silent (each listed in the design notes):
  pre-norm residual layer h1 = h + Attn(N1(h)), out = h1 + MLP(N2(h1)); no
  linear biases; RMSNorm / LayerNorm eps 1e-5; SwiGLU = W_down(silu(W_gate a) *
  W_up a); GELU in its exact erf form; attention scale 1/sqrt(head_dim);
  query head h reads key/value head h // (n_q / n_kv); rotate-half RoPE with
  inv_freq = theta^(-2i/head_dim), angles taken in float64.
"""
from __future__ import annotations

import math

import numpy as np
from scipy.special import erf

ACT_SWIGLU, ACT_GELU = 0, 1
NORM_RMS, NORM_LAYER = 0, 1


# ----------------------------------------------------------------- primitives
def rms_norm(x, g, eps):
    """RMSNorm over the last axis: x / sqrt(mean(x^2) + eps) * g."""
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + x.dtype.type(eps)) * g


def layer_norm(x, g, b, eps):
    """LayerNorm over the last axis with gain and bias (population variance)."""
    mu = np.mean(x, axis=-1, keepdims=True)
    xc = x - mu
    var = np.mean(xc * xc, axis=-1, keepdims=True)
    return xc / np.sqrt(var + x.dtype.type(eps)) * g + b


def silu(x):
    return x / (x.dtype.type(1) + np.exp(-x))


def gelu(x):
    """Exact GELU: x * Phi(x) = 0.5 x (1 + erf(x / sqrt 2))."""
    return (x.dtype.type(0.5) * x * (x.dtype.type(1) + erf(x / x.dtype.type(math.sqrt(2.0))))).astype(x.dtype)


def rope(x, pos, theta):
    """Rotate-half rotary embedding.

    x: [R, H, hd]; pos: [R] integer positions.  Pair (i, i + hd/2) of every
    head is rotated by angle pos * theta^(-2i/hd).  theta == 0 disables it.
    """
    if theta == 0:
        return x
    hd = x.shape[-1]
    half = hd // 2
    inv = np.power(float(theta), -2.0 * np.arange(half, dtype=np.float64) / hd)
    ang = np.asarray(pos, dtype=np.float64)[:, None] * inv[None, :]      # [R, half]
    c = np.cos(ang).astype(x.dtype)[:, None, :]
    s = np.sin(ang).astype(x.dtype)[:, None, :]
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def softmax(z):
    m = np.max(z, axis=-1, keepdims=True)
    e = np.exp(z - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def log_softmax(z):
    m = np.max(z, axis=-1, keepdims=True)
    return z - m - np.log(np.sum(np.exp(z - m), axis=-1, keepdims=True))


def attend(q, K, V, group):
    """Plain softmax attention of one row.

    q: [Hq, hd]; K, V: [L, Hkv, hd] (the keys this row may see, any order);
    query head h uses key/value head h // group.  Returns [Hq, hd].
    """
    Hq, hd = q.shape
    out = np.empty_like(q)
    scale = q.dtype.type(1.0 / math.sqrt(hd))
    for h in range(Hq):
        kv = h // group
        s = (K[:, kv, :] @ q[h]) * scale
        p = softmax(s)
        out[h] = p @ V[:, kv, :]
    return out


def topk(logits, k):
    """Top-k ids of a logit row: larger logit first, lower id first on ties."""
    order = np.lexsort((np.arange(logits.shape[-1]), -logits))
    return order[:k].astype(np.int32)


def argmax_lowest(row):
    """Index of the maximum, lowest index on ties."""
    return int(np.flatnonzero(row == row.max())[0])


# ----------------------------------------------------------------- the head
class DraftHead:
    """Random-init (or any) draft head held as float arrays.

    Matrices are stored [out][in] like a linear layer, so y = x @ W.T.  The
    pages' "fc of shape [2d, d]" is the map R^{2d} -> R^d, i.e. W_fc.T.
    """

    def __init__(self, cfg, weights, dtype=np.float32):
        self.cfg = cfg
        self.dt = dtype
        self.w = {k: np.asarray(v, dtype=dtype) for k, v in weights.items()}
        self.d = cfg.d
        self.group = cfg.n_q // cfg.n_kv

    # -- parameter shapes ("What is actually in the head")
    def fc_map_shape(self):
        """Shape of fc as a map in->out, the pages' [2d, d]."""
        return tuple(self.w["w_fc"].T.shape)

    def matrix_param_count(self):
        names = ["w_fc", "w_fuse", "w_q", "w_k", "w_v", "w_o", "w_gate", "w_up", "w_down"]
        return int(sum(self.w[n].size for n in names if n in self.w))

    # -- input assembly
    def fc_input(self, feat, tok):
        """EAGLE-1: x = [f ; emb(t)] (feature first), h = fc(x).  feat [R, d]."""
        x = np.concatenate([feat, self.w["emb"][tok]], axis=-1)
        return x @ self.w["w_fc"].T

    def fuse(self, lmh):
        """EAGLE-3: g = FC([l; m; h]); lmh [R, 3d] already concatenated."""
        return lmh @ self.w["w_fuse"].T

    def latent_input(self, a, tok):
        """EAGLE-3 later steps (and verified positions): a + emb(t)."""
        return a + self.w["emb"][tok]

    # -- decoder layer pieces
    def norm(self, x, which):
        g = self.w[f"norm{which}_g"]
        if self.cfg.norm == NORM_LAYER:
            return layer_norm(x, g, self.w[f"norm{which}_b"], self.cfg.eps)
        return rms_norm(x, g, self.cfg.eps)

    def qkv(self, h, pos):
        """Pre-norm projections with RoPE at the given positions.

        h: [R, d] -> q [R, Hq, hd], k [R, Hkv, hd], v [R, Hkv, hd].
        """
        c = self.cfg
        a = self.norm(h, 1)
        R = h.shape[0]
        q = (a @ self.w["w_q"].T).reshape(R, c.n_q, c.head_dim)
        k = (a @ self.w["w_k"].T).reshape(R, c.n_kv, c.head_dim)
        v = (a @ self.w["w_v"].T).reshape(R, c.n_kv, c.head_dim)
        return rope(q, pos, c.rope_theta), rope(k, pos, c.rope_theta), v

    def mlp(self, x):
        c = self.cfg
        b = self.norm(x, 2)
        if c.act == ACT_SWIGLU:
            z = silu(b @ self.w["w_gate"].T) * (b @ self.w["w_up"].T)
        else:
            z = gelu(b @ self.w["w_up"].T)
        return z @ self.w["w_down"].T

    def finish(self, h, attn, store=None):
        """Given the layer input h [R, d] and attention output [R, Hq, hd]:
        h1 = h + o W_o^T; out = h1 + MLP(N2(h1)).  store: optional map applied
        to the residual stream h1 (e.g. rounding to the storage type of a bf16
        model); the caller applies it to the output."""
        R = h.shape[0]
        h1 = h + attn.reshape(R, -1) @ self.w["w_o"].T
        if store is not None:
            h1 = store(h1)
        return h1 + self.mlp(h1)

    def layer(self, h, pos, keys):
        """One decoder layer over rows h [R, d].

        keys(r, k_r, v_r) -> (K, V): the key/value set row r attends to, given
        its own freshly projected k_r, v_r (so a row can see itself).
        Returns (out [R, d], k [R, Hkv, hd], v [R, Hkv, hd]).
        """
        q, k, v = self.qkv(h, pos)
        att = np.empty_like(q)
        for r in range(h.shape[0]):
            K, V = keys(r, k[r], v[r])
            att[r] = attend(q[r], K, V, self.group)
        return self.finish(h, att), k, v

    # -- LM head, softmax, top-k
    def lm_head(self, f):
        """Frozen LM head: logits = W_LM f (one linear map, no bias)."""
        return f @ self.w["lm_head"].T

    @staticmethod
    def draft_choices(logits, k, inv_temp=1.0):
        """Top-k ids (logit desc, id asc), their confidences
        c = softmax(s * logits)[id] and the log-partition lse of s * logits."""
        R = logits.shape[0]
        ids = np.stack([topk(logits[r], k) for r in range(R)])
        z = logits * logits.dtype.type(inv_temp)
        m = np.max(z, axis=-1, keepdims=True)
        lse = (m + np.log(np.sum(np.exp(z - m), axis=-1, keepdims=True)))[:, 0]
        conf = np.exp(np.take_along_axis(z, ids, axis=-1) - lse[:, None])
        return ids, conf.astype(logits.dtype), lse
