"""Workload shapes for the EAGLE draft-and-verify round.

Pure data: dimensions, tree shapes, seeds.  Nothing here computes any part of
the method.

Sources (page titles as printed in the reference text):
  * "transformer_math / tm_eagle_deep" -- section "The recurrence, written out"
    (x = [f; emb(t)], fc [2d, d], one decoder layer, frozen LM head) and
    section "EAGLE-2: expand and rerank" (top-k expansion, keep top-m by value).
  * "Speculative Decoding Deep Dive III: EAGLE, DFlash" -- section "EAGLE-3"
    (g = FC([l; m; h]), later steps feed back a + emb(t)).
  * "EAGLE: Drafting in Feature Space" -- section "Drafting a Tree, Not a
    Chain" (EAGLE-1 uses one fixed tree shape for every context).
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Optional, Tuple

# enum values shared with include/eagle.h (kept in sync by a host test)
DTYPE_BF16, DTYPE_F32 = 0, 1
ACT_SWIGLU, ACT_GELU = 0, 1
NORM_RMS, NORM_LAYER = 0, 1
MODE_EAGLE1, MODE_EAGLE3 = 1, 3
TREE_CHAIN, TREE_STATIC, TREE_DYNAMIC = 0, 1, 2


@dataclass(frozen=True)
class HeadCfg:
    d: int                  # draft width (also the EAGLE-3 hidden size k)
    vocab: int              # |V|
    n_q: int                # query heads
    n_kv: int               # key/value heads (GQA when n_kv < n_q)
    head_dim: int
    ffn: int                # MLP hidden width
    act: int = ACT_SWIGLU
    norm: int = NORM_RMS
    dtype: int = DTYPE_BF16
    eps: float = 1e-5
    rope_theta: float = 500000.0   # 0 = no positional encoding
    mode: int = MODE_EAGLE1        # EAGLE-1 fc([f; emb]) or EAGLE-3 FC([l; m; h])

    @property
    def q_dim(self) -> int:
        return self.n_q * self.head_dim

    @property
    def kv_dim(self) -> int:
        return self.n_kv * self.head_dim

    @property
    def group(self) -> int:
        return self.n_q // self.n_kv


@dataclass(frozen=True)
class RoundCfg:
    name: str
    head: HeadCfg
    B: int
    n: Tuple[int, ...] = ()           # fixed per-request context lengths (len B) ...
    n_range: Optional[Tuple[int, int]] = None   # ... or uniform integers in [lo, hi]
    # EAGLE-3 steady-state round: each request already holds n (above) context
    # positions and ingests tau ~ U{lo..hi} newly verified ones (the previous
    # round's accepted path and corrected token) instead of all of them
    new_range: Optional[Tuple[int, int]] = None
    # target verification pass: L decoder layers of the head's shape (sharing
    # its embedding and LM head) produce the target logits (0: synthetic logits)
    target_layers: int = 0
    seed_tm: int = 0
    # sampled drafting: children drawn by Gumbel-top-k with this 64-bit round
    # seed (None: the top_k by logit)
    sample_seed: Optional[int] = None
    tree: int = TREE_CHAIN
    gamma: int = 4                    # draft depth = number of draft steps
    top_k: int = 1
    top_m: int = 0                    # nodes kept by rerank (dynamic trees)
    template: Tuple[int, ...] = ()    # static tree: parent of template node i+1
    inv_temp: float = 1.0             # s in conf = softmax(s * logits)
    tree_attend: bool = False         # the round includes the verify-side tree attention
    seed_w: int = 0
    seed_in: int = 0
    seed_t: int = 0
    note: str = ""

    @property
    def n_final(self) -> int:
        """Non-root nodes of the final (verified) tree per request."""
        if self.tree == TREE_CHAIN:
            return self.gamma
        if self.tree == TREE_STATIC:
            return len(self.template)
        return self.top_m

    @property
    def positions(self) -> int:
        """Positions per request in the verify tree (root + n_final)."""
        return self.n_final + 1


# EAGLE-1 static tree used at the 8B shape: 25 non-root nodes, depth 4, max
# fan-out (4, 3, 2, 1) per depth.  Entry i is the parent of node i+1 (node 0
# is the root); siblings are listed in rank order (rank r = the r-th best
# token of the parent's top-k).
STATIC_TREE_25 = (0, 0, 0, 0,            # nodes 1-4   (depth 1)
                  1, 1, 1, 2, 2, 2, 3, 3, 4,   # nodes 5-13  (depth 2)
                  5, 5, 8, 8, 11, 11, 13, 13,  # nodes 14-21 (depth 3)
                  14, 16, 18, 20)               # nodes 22-25 (depth 4)

HEAD_TINY_F32 = HeadCfg(d=256, vocab=4096, n_q=4, n_kv=4, head_dim=64, ffn=1024,
                        act=ACT_GELU, norm=NORM_LAYER, dtype=DTYPE_F32,
                        rope_theta=0.0)
HEAD_8B = HeadCfg(d=4096, vocab=128256, n_q=32, n_kv=8, head_dim=128, ffn=14336)
HEAD_8B_E3 = replace(HEAD_8B, mode=MODE_EAGLE3)
HEAD_70B = HeadCfg(d=8192, vocab=128256, n_q=64, n_kv=8, head_dim=128, ffn=28672)

# Inverse temperature for the EAGLE-2 dynamic tree at the 8B shape.  The random
# head's draft logits are rescaled so that the mean top-1 confidence of the
# first draft step is close to 0.6 (calibrated by oracle/calibrate_inv_temp.py).
C2_INV_TEMP = 1.39494

CONFIGS = {
    "c0_tiny_chain": RoundCfg(
        name="c0_tiny_chain", head=HEAD_TINY_F32, B=1, n=(64,), tree=TREE_CHAIN,
        gamma=4, top_k=1, seed_w=1000, seed_in=2000, seed_t=3000,
        note="tiny EAGLE-1 chain, fp32, B=1, n=64, gamma=4, greedy top-1"),
    "c1_8b_static": RoundCfg(
        name="c1_8b_static", head=HEAD_8B, B=1, n=(2048,), tree=TREE_STATIC,
        gamma=4, top_k=4, template=STATIC_TREE_25, seed_w=1001, seed_in=2001,
        seed_t=3001,
        note="Llama-3-8B-shaped head, bf16, B=1, n=2048, static 25-node tree"),
    "c2_8b_dynamic": RoundCfg(
        name="c2_8b_dynamic", head=HEAD_8B, B=8, n=(4096,) * 8, tree=TREE_DYNAMIC,
        gamma=6, top_k=10, top_m=60, inv_temp=C2_INV_TEMP, tree_attend=True, seed_w=1002,
        seed_in=2002, seed_t=3002,
        note="EAGLE-2 dynamic tree on the 8B head, B=8, n=4096, top-k 10, depth 6, top-m 60"),
    "c3_8b_eagle3": RoundCfg(
        name="c3_8b_eagle3", head=HEAD_8B_E3, B=32, n_range=(256, 1024),
        tree=TREE_CHAIN, gamma=7, top_k=1, seed_w=1003, seed_in=2003, seed_t=3003,
        note="EAGLE-3 fused-feature chain, B=32, packed n in [256,1024], gamma=7"),
    # the round after c3_8b_eagle3's: the cache holds n in [256, 1024] positions
    # and each request ingests only the tau in [1, 8] it has just verified
    # the benchmark's round with a real verification pass: a 32-layer target
    # of the 8B head's layer shape (sharing its embedding and LM head)
    "c6_8b_target": RoundCfg(
        name="c6_8b_target", head=HEAD_8B, B=1, n=(2048,), tree=TREE_STATIC,
        gamma=4, top_k=4, template=STATIC_TREE_25, seed_w=1001, seed_in=2001,
        seed_t=3001, target_layers=32, seed_tm=4006,
        note="c1 with a 32-layer 8B-shaped target's tree-attention verification pass"),
    # c2's round in the steady state: each request's cache holds 4096
    # positions and 1..7 newly verified ones are ingested from the target's
    # features before the round
    "c7_8b_dynamic_steady": RoundCfg(
        name="c7_8b_dynamic_steady", head=HEAD_8B, B=8, n=(4096,) * 8, new_range=(1, 7),
        tree=TREE_DYNAMIC, gamma=6, top_k=10, top_m=60, inv_temp=C2_INV_TEMP, seed_w=1002,
        seed_in=2007, seed_t=3007,
        note="EAGLE-2 dynamic tree on the 8B head, B=8, cached n=4096 + 1..7 new positions"),
    # c2 with sampled drafting: each node's 10 children drawn without
    # replacement (Gumbel-top-k) instead of its top 10
    "c8_8b_dynamic_sampled": RoundCfg(
        name="c8_8b_dynamic_sampled", head=HEAD_8B, B=8, n=(4096,) * 8, tree=TREE_DYNAMIC,
        gamma=6, top_k=10, top_m=60, inv_temp=C2_INV_TEMP, seed_w=1002, seed_in=2002,
        seed_t=3002, sample_seed=0x5EED0000C0FFEE,
        note="c2 with sampled drafting (Gumbel-top-k children)"),
    "c5_8b_eagle3_steady": RoundCfg(
        name="c5_8b_eagle3_steady", head=HEAD_8B_E3, B=32, n_range=(256, 1024),
        new_range=(1, 8), tree=TREE_CHAIN, gamma=7, top_k=1, seed_w=1003,
        seed_in=2005, seed_t=3005,
        note="EAGLE-3 steady-state chain, B=32, cached n in [256,1024] + tau in [1,8] new, gamma=7"),
    "c4_70b_dynamic": RoundCfg(
        name="c4_70b_dynamic", head=HEAD_70B, B=64, n=(8192,) * 64,
        tree=TREE_DYNAMIC, gamma=6, top_k=8, top_m=60, seed_w=1004,
        seed_in=2004, seed_t=3004,
        note="70B-shaped head, B=64, n=8192, EAGLE-2 top-k 8, depth 6, top-m 60"),
}

# Small shapes for parity at sizes the oracle finishes in seconds.  They cover
# every tree mode, both dtypes, GQA, RoPE, ragged vocab / MLP / context sizes
# and an empty context.
_HEAD_SMALL = HeadCfg(d=256, vocab=3001, n_q=4, n_kv=2, head_dim=128, ffn=704,
                      rope_theta=10000.0)
SMALL_CONFIGS = {
    "c0r_tiny_chain_rope": replace(
        CONFIGS["c0_tiny_chain"], name="c0r_tiny_chain_rope",
        head=replace(HEAD_TINY_F32, rope_theta=10000.0), seed_w=1100,
        seed_in=2100, seed_t=3100),
    "s1_static": RoundCfg(
        name="s1_static", head=_HEAD_SMALL, B=1, n=(77,), tree=TREE_STATIC,
        gamma=4, top_k=4, template=STATIC_TREE_25, seed_w=1101, seed_in=2101,
        seed_t=3101),
    "s2_dynamic": RoundCfg(
        name="s2_dynamic", head=_HEAD_SMALL, B=3, n=(130, 1, 64),
        tree=TREE_DYNAMIC, gamma=4, top_k=4, top_m=12, inv_temp=4.0,
        seed_w=1102, seed_in=2102, seed_t=3102),
    "s3_eagle3": RoundCfg(
        name="s3_eagle3", head=replace(_HEAD_SMALL, mode=MODE_EAGLE3), B=3,
        n=(33, 100, 7), tree=TREE_CHAIN, gamma=5, top_k=1, seed_w=1103,
        seed_in=2103, seed_t=3103),
    "s4_dynamic_wide": RoundCfg(
        name="s4_dynamic_wide", head=replace(_HEAD_SMALL, d=384, n_q=8, n_kv=2,
                                             ffn=1024, vocab=5000),
        B=5, n=(300, 17, 0, 64, 129), tree=TREE_DYNAMIC, gamma=5, top_k=8,
        top_m=40, inv_temp=6.0, seed_w=1104, seed_in=2104, seed_t=3104),
    # 160 rows per step after the root: the large-M tiled GEMM and LM head,
    # with ragged row, column and vocabulary tiles
    "s5_dynamic_many": RoundCfg(
        name="s5_dynamic_many", head=replace(_HEAD_SMALL, vocab=6016),
        B=20, n=tuple(int(x) for x in (5, 90, 33, 1, 64, 128, 7, 200, 0, 49,
                                       12, 77, 150, 3, 65, 31, 100, 9, 256, 18)),
        tree=TREE_DYNAMIC, gamma=4, top_k=8, top_m=24, inv_temp=5.0,
        seed_w=1105, seed_in=2105, seed_t=3105),
    # fp32 head with RMSNorm and GELU: the row-complete fp32 kernels (2 rows),
    # the GELU epilogue, and 18 rows x 2 heads per kv head (workgroup attention)
    "s6_f32_rms_gelu": RoundCfg(
        name="s6_f32_rms_gelu", head=replace(HEAD_TINY_F32, norm=NORM_RMS, n_kv=2,
                                             rope_theta=10000.0),
        B=2, n=(40, 9), tree=TREE_DYNAMIC, gamma=3, top_k=9, top_m=14, inv_temp=3.0,
        seed_w=1106, seed_in=2106, seed_t=3106),
    # the same with head_dim 128 (fp32 instantiations of both attention kernels)
    "s8_f32_hd128": RoundCfg(
        name="s8_f32_hd128", head=replace(HEAD_TINY_F32, norm=NORM_RMS, n_q=2, n_kv=1,
                                          head_dim=128, rope_theta=10000.0),
        B=2, n=(70, 0), tree=TREE_DYNAMIC, gamma=3, top_k=9, top_m=14, inv_temp=3.0,
        seed_w=1108, seed_in=2108, seed_t=3108),
}

# The maxima of the boundary: top-k 16 with a 64-position verify tree, and a
# chain of 63 steps (positions 0..63 use every bit of the 64-bit masks).
SMALL_CONFIGS["s9_dynamic_topk16"] = RoundCfg(
    name="s9_dynamic_topk16", head=_HEAD_SMALL, B=2, n=(50, 300), tree=TREE_DYNAMIC,
    gamma=3, top_k=16, top_m=63, inv_temp=4.0, seed_w=1109, seed_in=2109, seed_t=3109)
SMALL_CONFIGS["s10_chain_63"] = RoundCfg(
    name="s10_chain_63", head=_HEAD_SMALL, B=1, n=(33,), tree=TREE_CHAIN, gamma=63,
    top_k=1, seed_w=1110, seed_in=2110, seed_t=3110)

# EAGLE-3 steady state: cached contexts (one empty) plus 1..8 newly verified
# positions; a dynamic tree at 3 requests (row-complete kernels) and a chain
# at 20 (split-K kernels at step 0)
SMALL_CONFIGS["s11_eagle3_steady_dynamic"] = RoundCfg(
    name="s11_eagle3_steady_dynamic", head=replace(_HEAD_SMALL, mode=MODE_EAGLE3), B=3,
    n=(0, 40, 120), new_range=(1, 8), tree=TREE_DYNAMIC, gamma=4, top_k=4, top_m=12,
    inv_temp=4.0, seed_w=1111, seed_in=2111, seed_t=3111)
SMALL_CONFIGS["s12_eagle3_steady_chain"] = RoundCfg(
    name="s12_eagle3_steady_chain", head=replace(_HEAD_SMALL, mode=MODE_EAGLE3), B=20,
    n_range=(0, 60), new_range=(1, 8), tree=TREE_CHAIN, gamma=3, top_k=1,
    seed_w=1112, seed_in=2112, seed_t=3112)

# EAGLE-1 steady state: cached contexts plus 1..5 newly verified positions
# ingested from the target's features (a dynamic tree, one empty cache; a
# 20-request chain on the split-K kernels)
SMALL_CONFIGS["s17_eagle1_steady_dynamic"] = RoundCfg(
    name="s17_eagle1_steady_dynamic", head=_HEAD_SMALL, B=3, n=(0, 33, 90),
    new_range=(1, 5), tree=TREE_DYNAMIC, gamma=3, top_k=4, top_m=12, inv_temp=4.0,
    seed_w=1117, seed_in=2117, seed_t=3117)
SMALL_CONFIGS["s18_eagle1_steady_chain"] = RoundCfg(
    name="s18_eagle1_steady_chain", head=_HEAD_SMALL, B=20, n_range=(0, 50), new_range=(1, 5),
    tree=TREE_CHAIN, gamma=3, top_k=1, seed_w=1118, seed_in=2118, seed_t=3118)

# Sampled drafting (Gumbel-top-k over Philox noise) on every LM-head path:
# fused epilogue at <= 32 rows, the 33..63-row kernel, and the tiled GEMM with
# logits partials from 64 rows on
SMALL_CONFIGS["s19_sampled_dynamic"] = RoundCfg(
    name="s19_sampled_dynamic", head=_HEAD_SMALL, B=3, n=(60, 1, 130), tree=TREE_DYNAMIC,
    gamma=4, top_k=4, top_m=12, inv_temp=4.0, seed_w=1119, seed_in=2119, seed_t=3119,
    sample_seed=0x0123456789ABCDEF)
for _i, _b in enumerate((40, 70)):
    SMALL_CONFIGS[f"s20_sampled_chain_b{_b}"] = RoundCfg(
        name=f"s20_sampled_chain_b{_b}", head=replace(_HEAD_SMALL, vocab=3008), B=_b,
        n=tuple((5 * j + _b) % 37 for j in range(_b)), tree=TREE_CHAIN, gamma=2, top_k=1,
        seed_w=1120 + _i, seed_in=2120 + _i, seed_t=3120 + _i, sample_seed=0xFEEDFACE + _i)

# the static template with sampled drafting: every node's children are the
# first draw ranks of its Gumbel-top-k sample (a prefix of the draws)
SMALL_CONFIGS["s22_sampled_static"] = RoundCfg(
    name="s22_sampled_static", head=_HEAD_SMALL, B=4, n=(90, 0, 17, 200), tree=TREE_STATIC,
    gamma=4, top_k=4, template=STATIC_TREE_25, inv_temp=2.0, seed_w=1122, seed_in=2122,
    seed_t=3122, sample_seed=0x5A5A5A5A12345678)

# 264 rows per step after the root: the tiled kernels at their 256-row tile
# height with a ragged second tile of 8 rows (every row checked); |V| = 16400
# and ffn = 8320 give the LM head and gate|up at least 128 tiles, so they run
# on the direct-to-LDS kernel (ragged last vocabulary tile of 16 rows; gate|up
# with the fused SwiGLU epilogue)
SMALL_CONFIGS["s21_dynamic_264"] = RoundCfg(
    name="s21_dynamic_264", head=replace(_HEAD_SMALL, vocab=16400, ffn=8320), B=33,
    n=tuple((13 * j + 5) % 97 + (200 if j % 5 == 0 else 0) for j in range(33)),
    tree=TREE_DYNAMIC, gamma=4, top_k=8, top_m=24, inv_temp=5.0,
    seed_w=1122, seed_in=2122, seed_t=3122)

# 80 rows per step after the root (8 requests x top-k 10) on the 64-K-stage
# tiled GEMM: |V| = 69648 gives the LM head 273 tiles of 256 columns, more than
# one per workgroup (ragged last tile of 16 columns), and d = 832 splits the
# fc's K = 1664 into six 320-wide spans whose last is a single 64-K stage
SMALL_CONFIGS["s24_dynamic_80_v69648"] = RoundCfg(
    name="s24_dynamic_80_v69648", head=replace(_HEAD_SMALL, d=832, vocab=69648), B=8,
    n=(40, 0, 77, 5, 130, 64, 1, 19), tree=TREE_DYNAMIC, gamma=3, top_k=10, top_m=20,
    inv_temp=4.0, seed_w=1124, seed_in=2124, seed_t=3124)

# 72 rows per step after the root (9 requests x top-k 8), the fused LM-head
# epilogue with ragged rows: |V| = 16400 is 65 tiles over 72 workgroups, so
# seven workgroups write empty parts
SMALL_CONFIGS["s25_dynamic_72_v16400"] = RoundCfg(
    name="s25_dynamic_72_v16400", head=replace(_HEAD_SMALL, vocab=16400), B=9,
    n=(3, 90, 0, 41, 200, 17, 64, 8, 129), tree=TREE_DYNAMIC, gamma=3, top_k=8, top_m=16,
    inv_temp=3.0, seed_w=1125, seed_in=2125, seed_t=3125)

# The target's verification pass: a static tree (52 rows, tiled kernels), a
# dynamic tree with an empty context, an fp32 LayerNorm / GELU head, and a
# 12-row chain (row-complete kernels)
SMALL_CONFIGS["s13_target_static"] = RoundCfg(
    name="s13_target_static", head=_HEAD_SMALL, B=2, n=(40, 9), tree=TREE_STATIC, gamma=4,
    top_k=4, template=STATIC_TREE_25, seed_w=1113, seed_in=2113, seed_t=3113,
    target_layers=3, seed_tm=4113)
SMALL_CONFIGS["s14_target_dynamic"] = RoundCfg(
    name="s14_target_dynamic", head=_HEAD_SMALL, B=3, n=(0, 30, 70), tree=TREE_DYNAMIC,
    gamma=3, top_k=4, top_m=12, inv_temp=4.0, seed_w=1114, seed_in=2114, seed_t=3114,
    target_layers=2, seed_tm=4114)
SMALL_CONFIGS["s15_target_f32"] = RoundCfg(
    name="s15_target_f32", head=HEAD_TINY_F32, B=2, n=(33, 64), tree=TREE_DYNAMIC, gamma=3,
    top_k=3, top_m=8, seed_w=1115, seed_in=2115, seed_t=3115, target_layers=2, seed_tm=4115)
SMALL_CONFIGS["s16_target_chain_rows"] = RoundCfg(
    name="s16_target_chain_rows", head=_HEAD_SMALL, B=3, n=(17, 5, 60), tree=TREE_CHAIN,
    gamma=3, top_k=1, seed_w=1116, seed_in=2116, seed_t=3116, target_layers=3, seed_tm=4116)

# Chains whose row count sits on either side of every kernel-dispatch boundary:
# 16 / 17 (row-complete vs split-K streaming), 32 / 33 (streaming vs LDS-staged),
# 63 / 64 (LDS-staged vs tiled GEMM, and the tiled LM head: |V| = 3008 is a
# multiple of 16).  Mixed context lengths including empty ones.
for _i, _b in enumerate((16, 17, 32, 33, 63, 64)):
    SMALL_CONFIGS[f"s7_chain_b{_b}"] = RoundCfg(
        name=f"s7_chain_b{_b}", head=replace(_HEAD_SMALL, vocab=3008), B=_b,
        n=tuple((7 * j + 3 * _b) % 41 for j in range(_b)), tree=TREE_CHAIN, gamma=2,
        top_k=1, seed_w=1107 + _i, seed_in=2107 + _i, seed_t=3107 + _i)

ALL_CONFIGS = {**CONFIGS, **SMALL_CONFIGS}
