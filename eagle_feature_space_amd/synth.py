"""Seeded synthetic inputs shared by the oracle tests, the GPU tests and the bench.

This module only draws random numbers and rounds them to the storage type.  It
holds none of the method's arithmetic.

Recipe (the pages train on real conversations and measure on public suites;
none of that is available or needed here, only the shapes):
  * numpy PCG64 streams, one per (seed, tensor, chunk), drawn in float32 and
    rounded to bf16 with round-to-nearest-even (fp32 configs keep float32);
  * matrices, the LM head included, ~ N(0, 0.02); the embedding table ~ N(0, 1)
    so that the token input carries real weight in x = [f; emb(t)];
  * norm gains 1 + 0.1 N(0,1), LayerNorm biases 0.1 N(0,1);
  * features f (or EAGLE-3's l, m, h) ~ N(0, 1); token ids uniform in [0, |V|);
  * synthetic context K/V ~ N(0, 1) (already rotated) for EAGLE-1 rounds;
  * synthetic target logits ~ N(0, 1), one row per verify-tree position;
  * the uniforms of stochastic verification ~ U[0, 1) in float32, 17 per
    verify-tree position;
  * target layers drawn like the head's layer (matrices N(0, 0.02), gains
    1 + 0.1 N(0, 1)), a final RMSNorm gain 1 + 0.1 N(0, 1), and a synthetic
    context cache ~ N(0, 1) per layer; the embedding and LM head are the
    head's.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Dict, Optional

import numpy as np

from .configs import (ACT_GELU, ACT_SWIGLU, DTYPE_BF16, DTYPE_F32, MODE_EAGLE1,
                      MODE_EAGLE3, NORM_LAYER, HeadCfg, RoundCfg)

_CHUNK = 1 << 22
_THREADS = max(1, min(16, len(os.sched_getaffinity(0))))


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit pattern (uint16), round to nearest even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit pattern (uint16) -> float32 (exact)."""
    return (np.ascontiguousarray(bits).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _stream(seed: int, tag: int, chunk: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(
        entropy=seed, spawn_key=(tag, chunk))))


def normal(seed: int, tag: int, shape, std: float = 1.0, mean: float = 0.0,
           bf16: bool = True) -> np.ndarray:
    """N(mean, std^2) tensor; bf16 bit pattern (uint16) or float32."""
    total = int(np.prod(shape))
    out = np.empty(total, dtype=np.uint16 if bf16 else np.float32)
    nchunks = (total + _CHUNK - 1) // _CHUNK

    def work(c):
        lo, hi = c * _CHUNK, min(total, (c + 1) * _CHUNK)
        v = _stream(seed, tag, c).standard_normal(hi - lo, dtype=np.float32)
        if std != 1.0:
            v *= np.float32(std)
        if mean != 0.0:
            v += np.float32(mean)
        out[lo:hi] = bf16_bits(v) if bf16 else v

    if nchunks <= 1:
        for c in range(nchunks):
            work(c)
    else:
        with ThreadPoolExecutor(_THREADS) as ex:
            list(ex.map(work, range(nchunks)))
    return out.reshape(shape)


def integers(seed: int, tag: int, shape, lo: int, hi_incl: int) -> np.ndarray:
    return _stream(seed, tag, 0).integers(lo, hi_incl + 1, size=shape,
                                          dtype=np.int64).astype(np.int32)


def f32(a: np.ndarray) -> np.ndarray:
    """Upcast a stored tensor (bf16 bits or float32) to float32."""
    if a.dtype == np.uint16:
        return bf16_to_f32(a)
    return np.asarray(a, dtype=np.float32)


# tags keep every tensor on its own stream
_T = {name: i for i, name in enumerate([
    "w_fc", "w_fuse", "w_q", "w_k", "w_v", "w_o", "w_gate", "w_up", "w_down",
    "norm1_g", "norm1_b", "norm2_g", "norm2_b", "emb", "lm_head",
    "n", "k_ctx", "v_ctx", "f_root", "t_root", "lmh", "ctx_tokens", "target", "n_new",
    "draws", "final_g"])}
_LAYER_TAGS = 64     # tag stride of one target layer


def head_weights(h: HeadCfg, seed: int) -> Dict[str, np.ndarray]:
    """Random-init draft head.  Matrices are stored [out][in] (K contiguous)."""
    bf = h.dtype == DTYPE_BF16
    d = h.d
    w: Dict[str, np.ndarray] = {}
    if h.mode == MODE_EAGLE1:
        w["w_fc"] = normal(seed, _T["w_fc"], (d, 2 * d), 0.02, bf16=bf)
    else:
        w["w_fuse"] = normal(seed, _T["w_fuse"], (d, 3 * d), 0.02, bf16=bf)
    w["w_q"] = normal(seed, _T["w_q"], (h.q_dim, d), 0.02, bf16=bf)
    w["w_k"] = normal(seed, _T["w_k"], (h.kv_dim, d), 0.02, bf16=bf)
    w["w_v"] = normal(seed, _T["w_v"], (h.kv_dim, d), 0.02, bf16=bf)
    w["w_o"] = normal(seed, _T["w_o"], (d, h.q_dim), 0.02, bf16=bf)
    if h.act == ACT_SWIGLU:
        w["w_gate"] = normal(seed, _T["w_gate"], (h.ffn, d), 0.02, bf16=bf)
    w["w_up"] = normal(seed, _T["w_up"], (h.ffn, d), 0.02, bf16=bf)
    w["w_down"] = normal(seed, _T["w_down"], (d, h.ffn), 0.02, bf16=bf)
    w["norm1_g"] = normal(seed, _T["norm1_g"], (d,), 0.1, 1.0, bf16=bf)
    w["norm2_g"] = normal(seed, _T["norm2_g"], (d,), 0.1, 1.0, bf16=bf)
    if h.norm == NORM_LAYER:
        w["norm1_b"] = normal(seed, _T["norm1_b"], (d,), 0.1, bf16=bf)
        w["norm2_b"] = normal(seed, _T["norm2_b"], (d,), 0.1, bf16=bf)
    w["emb"] = normal(seed, _T["emb"], (h.vocab, d), 1.0, bf16=bf)
    w["lm_head"] = normal(seed, _T["lm_head"], (h.vocab, d), 0.02, bf16=bf)
    return w


@dataclass
class RoundInputs:
    n: np.ndarray                      # int32 [B]
    cu_n: np.ndarray                   # int32 [B+1]
    t_root: np.ndarray                 # int32 [B] anchor token (root of the tree)
    k_ctx: Optional[np.ndarray] = None  # [sum n, Hkv, hd] (EAGLE-1 rounds)
    v_ctx: Optional[np.ndarray] = None
    f_root: Optional[np.ndarray] = None  # [B, d] (EAGLE-1 rounds)
    lmh: Optional[np.ndarray] = None     # [sum n, 3d] (EAGLE-3 rounds; new rows only when steady)
    ctx_tokens: Optional[np.ndarray] = None  # int32 [sum n] shifted tokens (EAGLE-3; likewise)
    # EAGLE-3 steady state: n counts old + new positions; request b's newest
    # n_new[b] positions are ingested (packed by cu_new); k_ctx / v_ctx hold the
    # old positions' K/V in each request's segment (new rows zero)
    n_new: Optional[np.ndarray] = None   # int32 [B]
    cu_new: Optional[np.ndarray] = None  # int32 [B+1]


def context_lengths(r: RoundCfg) -> np.ndarray:
    if r.n_range is not None:
        return integers(r.seed_in, _T["n"], (r.B,), r.n_range[0], r.n_range[1])
    assert len(r.n) == r.B
    return np.asarray(r.n, dtype=np.int32)


def round_inputs(r: RoundCfg) -> RoundInputs:
    h = r.head
    bf = h.dtype == DTYPE_BF16
    n = context_lengths(r)
    cu = np.zeros(r.B + 1, dtype=np.int32)
    cu[1:] = np.cumsum(n)
    total = int(cu[-1])
    s = r.seed_in
    t_root = integers(s, _T["t_root"], (r.B,), 0, h.vocab - 1)
    if h.mode == MODE_EAGLE1 and r.new_range is None:
        return RoundInputs(
            n=n, cu_n=cu, t_root=t_root,
            k_ctx=normal(s, _T["k_ctx"], (total, h.n_kv, h.head_dim), bf16=bf),
            v_ctx=normal(s, _T["v_ctx"], (total, h.n_kv, h.head_dim), bf16=bf),
            f_root=normal(s, _T["f_root"], (r.B, h.d), bf16=bf))
    if r.new_range is not None:
        # steady state: n above is the old context; tau new positions follow
        assert r.new_range[0] >= 1, "every request ingests at least its anchor position"
        tau = integers(s, _T["n_new"], (r.B,), r.new_range[0], r.new_range[1])
        n_old = n
        n = (n_old + tau).astype(np.int32)
        cu[1:] = np.cumsum(n)
        total = int(cu[-1])
        cun = np.zeros(r.B + 1, dtype=np.int32)
        cun[1:] = np.cumsum(tau)
        k = normal(s, _T["k_ctx"], (total, h.n_kv, h.head_dim), bf16=bf)
        v = normal(s, _T["v_ctx"], (total, h.n_kv, h.head_dim), bf16=bf)
        for b in range(r.B):
            k[cu[b] + n_old[b]:cu[b + 1]] = 0
            v[cu[b] + n_old[b]:cu[b + 1]] = 0
        ctx = integers(s, _T["ctx_tokens"], (int(cun[-1]),), 0, h.vocab - 1)
        if h.mode == MODE_EAGLE1:
            # the target's features of the positions before the new ones, the
            # tokens at them; the root row keeps its own (f_root, t_root)
            return RoundInputs(n=n, cu_n=cu, t_root=t_root, k_ctx=k, v_ctx=v,
                               f_root=normal(s, _T["f_root"], (r.B, h.d), bf16=bf),
                               lmh=normal(s, _T["lmh"], (int(cun[-1]), h.d), bf16=bf),
                               ctx_tokens=ctx, n_new=tau.astype(np.int32), cu_new=cun)
        ctx[cun[1:] - 1] = t_root
        return RoundInputs(n=n, cu_n=cu, t_root=t_root, k_ctx=k, v_ctx=v,
                           lmh=normal(s, _T["lmh"], (int(cun[-1]), 3 * h.d), bf16=bf),
                           ctx_tokens=ctx, n_new=tau.astype(np.int32), cu_new=cun)
    assert (n >= 1).all(), "EAGLE-3 rounds need at least the anchor position"
    ctx = integers(s, _T["ctx_tokens"], (total,), 0, h.vocab - 1)
    # the shifted token of each request's last position is the anchor token
    ctx[cu[1:] - 1] = t_root
    return RoundInputs(n=n, cu_n=cu, t_root=t_root,
                       lmh=normal(s, _T["lmh"], (total, 3 * h.d), bf16=bf),
                       ctx_tokens=ctx)


def target_logits(r: RoundCfg, positions: Optional[int] = None) -> np.ndarray:
    """Synthetic verification logits [B, positions, |V|] ~ N(0, 1)."""
    T = r.positions if positions is None else positions
    return normal(r.seed_t, _T["target"], (r.B, T, r.head.vocab),
                  bf16=r.head.dtype == DTYPE_BF16)


N_DRAWS = 17


def verify_draws(r: RoundCfg, positions: Optional[int] = None, k: int = 0) -> np.ndarray:
    """Uniforms in [0, 1) for stochastic verification, float32 [B, positions, 17];
    k selects an independent set."""
    T = r.positions if positions is None else positions
    return _stream(r.seed_t, _T["draws"], k).random((r.B, T, N_DRAWS), dtype=np.float32)


def target_layer_weights(h: HeadCfg, seed: int, layer: int) -> Dict[str, np.ndarray]:
    """Decoder-layer weights of target layer `layer` (the head's layer shape)."""
    bf = h.dtype == DTYPE_BF16
    d = h.d
    t = lambda name: _T[name] + _LAYER_TAGS * (layer + 1)
    w: Dict[str, np.ndarray] = {}
    w["w_q"] = normal(seed, t("w_q"), (h.q_dim, d), 0.02, bf16=bf)
    w["w_k"] = normal(seed, t("w_k"), (h.kv_dim, d), 0.02, bf16=bf)
    w["w_v"] = normal(seed, t("w_v"), (h.kv_dim, d), 0.02, bf16=bf)
    w["w_o"] = normal(seed, t("w_o"), (d, h.q_dim), 0.02, bf16=bf)
    if h.act == ACT_SWIGLU:
        w["w_gate"] = normal(seed, t("w_gate"), (h.ffn, d), 0.02, bf16=bf)
    w["w_up"] = normal(seed, t("w_up"), (h.ffn, d), 0.02, bf16=bf)
    w["w_down"] = normal(seed, t("w_down"), (d, h.ffn), 0.02, bf16=bf)
    w["norm1_g"] = normal(seed, t("norm1_g"), (d,), 0.1, 1.0, bf16=bf)
    w["norm2_g"] = normal(seed, t("norm2_g"), (d,), 0.1, 1.0, bf16=bf)
    if h.norm == NORM_LAYER:
        w["norm1_b"] = normal(seed, t("norm1_b"), (d,), 0.1, bf16=bf)
        w["norm2_b"] = normal(seed, t("norm2_b"), (d,), 0.1, bf16=bf)
    return w


def target_final_gain(h: HeadCfg, seed: int) -> np.ndarray:
    return normal(seed, _T["final_g"], (h.d,), 0.1, 1.0, bf16=h.dtype == DTYPE_BF16)


def target_context(r: RoundCfg, layer: int):
    """Synthetic context cache (K, V) [sum n, Hkv, hd] of target layer `layer`."""
    h = r.head
    total = int(context_lengths(r).sum())
    bf = h.dtype == DTYPE_BF16
    t = _LAYER_TAGS * (layer + 1)
    return (normal(r.seed_tm, _T["k_ctx"] + t, (total, h.n_kv, h.head_dim), bf16=bf),
            normal(r.seed_tm, _T["v_ctx"] + t, (total, h.n_kv, h.head_dim), bf16=bf))
