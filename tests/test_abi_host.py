"""Host-only checks of libeagle's C-ABI: the library loads, exports every
symbol include/eagle.h declares, sizes its buffers consistently with the tree
shapes, and rejects bad arguments before launching anything.  No GPU needed:
every call here returns before the first HIP call."""
import ctypes
from dataclasses import replace
import os
import re

import numpy as np
import pytest

from eagle_feature_space_amd import binding as E
from eagle_feature_space_amd import configs as C

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(E.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    return E.lib()


def _declared_symbols():
    txt = open(os.path.join(ROOT, "include", "eagle.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(eagle_[a-z_]+)\s*\(", txt)))


def test_exports_every_declared_symbol(lib):
    decl = _declared_symbols()
    assert len(decl) >= 11
    for name in decl:
        assert hasattr(lib, name), name
    assert set(decl) == set(E.EXPORTED)
    assert E.eagle_version().startswith("eagle-mi355x")


def test_enums_match_header():
    txt = open(os.path.join(ROOT, "include", "eagle.h")).read()
    vals = dict(re.findall(r"(EAGLE_[A-Z0-9_]+)\s*=\s*(-?\d+)", txt))
    assert int(vals["EAGLE_BF16"]) == C.DTYPE_BF16 and int(vals["EAGLE_F32"]) == C.DTYPE_F32
    assert int(vals["EAGLE_ACT_SWIGLU"]) == C.ACT_SWIGLU and int(vals["EAGLE_ACT_GELU"]) == C.ACT_GELU
    assert int(vals["EAGLE_NORM_RMS"]) == C.NORM_RMS and int(vals["EAGLE_NORM_LAYER"]) == C.NORM_LAYER
    assert int(vals["EAGLE_MODE_1"]) == C.MODE_EAGLE1 and int(vals["EAGLE_MODE_3"]) == C.MODE_EAGLE3
    assert int(vals["EAGLE_TREE_STATIC"]) == C.TREE_STATIC
    assert int(vals["EAGLE_TREE_DYNAMIC"]) == C.TREE_DYNAMIC
    assert int(vals["EAGLE_ECAPACITY"]) == E.EAGLE_ECAPACITY


def _tree(cfg, state=None, nbytes=0):
    t = E.eagle_tree()
    t.kind, t.B, t.gamma, t.top_k, t.top_m = cfg.tree, cfg.B, cfg.gamma, cfg.top_k, cfg.top_m
    arr = (ctypes.c_int32 * max(1, len(cfg.template)))(*cfg.template)
    t.n_template = len(cfg.template) if cfg.tree == C.TREE_STATIC else 0
    t.template_parent = ctypes.cast(arr, ctypes.POINTER(ctypes.c_int32))
    t.inv_temp = cfg.inv_temp
    t.state, t.state_bytes = state, nbytes
    t._keep = arr
    return t


@pytest.mark.parametrize("name", sorted(C.ALL_CONFIGS))
def test_tree_geometry(lib, name):
    cfg = C.ALL_CONFIGS[name]
    t = _tree(cfg)
    L = E.eagle_tree_layout_of(t)
    assert L.positions == cfg.positions
    rows = [E.eagle_step_rows(t, s) for s in range(cfg.gamma)]
    if cfg.tree == C.TREE_CHAIN:
        assert rows == [1] * cfg.gamma and L.pool_cap == cfg.gamma + 1
    elif cfg.tree == C.TREE_STATIC:
        assert rows == [1, 4, 4, 4] and L.pool_cap == 26
    else:
        assert rows == [1] + [cfg.top_k] * (cfg.gamma - 1)
        assert L.pool_cap == 1 + cfg.top_k + (cfg.gamma - 1) * cfg.top_k ** 2
    assert sum(rows) <= 64
    assert E.eagle_tree_state_bytes(t) == L.total
    offs = sorted(getattr(L, f) for f in E._LAYOUT_FIELDS if f != "total")
    assert all(o % 256 == 0 for o in offs) and offs[-1] < L.total


def _head(cfg):
    h = E.eagle_head()
    for f in ("d", "vocab", "ffn", "act", "norm", "dtype", "mode", "eps", "rope_theta"):
        setattr(h, f, getattr(cfg, f))
    h.n_q_heads, h.n_kv_heads, h.head_dim = cfg.n_q, cfg.n_kv, cfg.head_dim
    fake = 1 << 20      # non-null placeholders; never dereferenced on the host
    for f in ("w_fc", "w_fuse", "w_q", "w_k", "w_v", "w_o", "w_gate", "w_up", "w_down",
              "norm1_g", "norm1_b", "norm2_g", "norm2_b", "emb", "lm_head"):
        setattr(h, f, fake)
    return h


def _kv(cfg, n):
    kv = E.eagle_kv()
    kv.B, kv.max_n, kv.total_n = cfg.B, int(max(n)), int(sum(n))
    for f in ("n", "cu_n", "k_ctx", "v_ctx", "k_slot", "v_slot", "feat_slot"):
        setattr(kv, f, 1 << 20)
    return kv


@pytest.mark.parametrize("name", ["c1_8b_static", "c2_8b_dynamic", "c4_70b_dynamic"])
def test_workspace_sizes(lib, name):
    cfg = C.CONFIGS[name]
    n = list(cfg.n)
    ws = E.eagle_workspace_bytes(_head(cfg.head), _kv(cfg, n), _tree(cfg))
    assert ws > 0
    M = cfg.B * max(E.eagle_step_rows(_tree(cfg), s) for s in range(cfg.gamma))
    # at least the LM-head partials and the activations
    assert ws >= M * cfg.head.ffn * 2
    assert ws < 8 << 30


def test_rejects_bad_arguments_before_launch(lib):
    cfg = C.SMALL_CONFIGS["s2_dynamic"]
    h = _head(cfg.head)
    kv = _kv(cfg, cfg.n)
    t = _tree(cfg, state=1 << 20, nbytes=1 << 30)
    ws = 1 << 20
    # step out of range, null workspace, null f_root at step 0
    assert lib.eagle_draft_step(h, kv, t, cfg.gamma, 1, None, None, None, None, ws, 1 << 40, None) == E.EAGLE_EINVAL
    assert lib.eagle_draft_step(h, kv, t, 0, 1, None, None, None, None, None, 1 << 40, None) == E.EAGLE_EINVAL
    assert lib.eagle_draft_step(h, kv, t, 0, None, None, None, None, None, ws, 1 << 40, None) == E.EAGLE_EINVAL
    # workspace too small
    assert lib.eagle_draft_step(h, kv, t, 0, 1, None, None, None, None, ws, 16, None) == E.EAGLE_ECAPACITY
    # tree state too small
    t2 = _tree(cfg, state=1 << 20, nbytes=64)
    assert lib.eagle_tree_expand_rerank(t2, 0, None) == E.EAGLE_ECAPACITY
    # unsupported head shapes
    for field, val, err in [("head_dim", 96, E.EAGLE_EUNSUPPORTED), ("d", 200, E.EAGLE_EUNSUPPORTED),
                            ("n_kv_heads", 3, E.EAGLE_EUNSUPPORTED), ("dtype", 7, E.EAGLE_EINVAL),
                            ("w_lm_head" if False else "lm_head", None, E.EAGLE_EINVAL)]:
        hb = _head(cfg.head)
        setattr(hb, field, val)
        assert lib.eagle_draft_step(hb, kv, t, 0, 1, None, None, None, None, ws, 1 << 40, None) == err, field
    # tree limits: top_k > 16, top_m larger than the pool, verify tree > 64 positions
    for field, val, err in [("top_k", 17, E.EAGLE_EUNSUPPORTED), ("top_m", 10 ** 6, E.EAGLE_EINVAL),
                            ("gamma", 0, E.EAGLE_EINVAL)]:
        tb = _tree(cfg, state=1 << 20, nbytes=1 << 30)
        setattr(tb, field, val)
        assert lib.eagle_tree_expand_rerank(tb, 0, None) == err, field
    big = C.RoundCfg(name="x", head=cfg.head, B=1, n=(4,), tree=C.TREE_DYNAMIC, gamma=3,
                     top_k=8, top_m=70)
    assert lib.eagle_tree_expand_rerank(_tree(big, 1 << 20, 1 << 30), 0, None) == E.EAGLE_ECAPACITY
    deep = C.RoundCfg(name="x", head=cfg.head, B=1, n=(4,), tree=C.TREE_DYNAMIC, gamma=9,
                      top_k=8, top_m=20)          # 1 + 8*8 expanded rows > 64 slots
    assert lib.eagle_tree_expand_rerank(_tree(deep, 1 << 20, 1 << 30), 0, None) == E.EAGLE_ECAPACITY
    # the draft's inverse temperature: positive, finite, at most EAGLE_MAX_INV_TEMP
    for temp in (0.0, -2.0, float("nan"), float("inf"), 1e30, 65536.5):
        tb = _tree(cfg, state=1 << 20, nbytes=1 << 30)
        tb.inv_temp = temp
        assert lib.eagle_tree_expand_rerank(tb, 0, None) == E.EAGLE_EINVAL, temp
        assert E.eagle_tree_state_bytes(tb) == 0, temp
    tb = _tree(cfg)
    tb.inv_temp = 65536.0
    assert E.eagle_tree_state_bytes(tb) > 0
    # static template deeper than gamma
    st = C.SMALL_CONFIGS["s1_static"]
    bad = C.RoundCfg(name="x", head=st.head, B=1, n=(4,), tree=C.TREE_STATIC, gamma=3, top_k=4,
                     template=st.template)
    assert lib.eagle_tree_expand_rerank(_tree(bad, 1 << 20, 1 << 30), 0, None) == E.EAGLE_EINVAL
    # verify: positions smaller than the tree, bad dtype
    assert lib.eagle_tree_verify(t, 1, 2, 100, 0, 1, 1, 1, None) == E.EAGLE_EINVAL
    assert lib.eagle_tree_verify(t, 1, 64, 100, 5, 1, 1, 1, None) == E.EAGLE_EINVAL
    # stochastic verify: null draws, non-positive or non-finite inv_temp, short positions
    for pos, temp, draws in [(64, 1.0, None), (64, 0.0, 1), (64, -1.0, 1), (64, float("nan"), 1),
                             (64, float("inf"), 1), (2, 1.0, 1)]:
        assert lib.eagle_tree_verify_sample(t, 1, pos, 100, 0, temp, draws, 1, 1, 1, None) == E.EAGLE_EINVAL
    # verification of sampled drafts: only for sampled drafting, draft logits
    # required, vocabularies up to 2^19
    sd = _tree(C.CONFIGS["c8_8b_dynamic_sampled"], state=1 << 20, nbytes=1 << 30)
    sd.sample = 1
    f = lib.eagle_tree_verify_sample_drafted
    assert f(t, 1, 64, 100, 0, 1.0, 1, 1, 1, 1, 1, None) == E.EAGLE_EINVAL       # sample = 0
    for pos, temp, dl, draws, voc in [(64, 1.0, None, 1, 100), (64, 1.0, 1, None, 100),
                                      (64, 0.0, 1, 1, 100), (64, float("nan"), 1, 1, 100),
                                      (2, 1.0, 1, 1, 100), (64, 1.0, 1, 1, 0)]:
        assert f(sd, 1, pos, voc, 0, temp, dl, draws, 1, 1, 1, None) == E.EAGLE_EINVAL
    assert f(sd, 1, 64, (1 << 19) + 1, 0, 1.0, 1, 1, 1, 1, 1, None) == E.EAGLE_EUNSUPPORTED
    assert lib.eagle_strerror(E.EAGLE_ECAPACITY).startswith(b"capacity")


def test_noalloc_step_is_validated(lib):
    """eagle_draft_step_noalloc refuses a workspace larger than its array
    (the 8B EAGLE-2 tree at B 8 needs ~400 MB) and bad arguments, before any
    HIP call; the header's array size matches the binding's."""
    txt = open(os.path.join(ROOT, "include", "eagle.h")).read()
    m = re.search(r"#define EAGLE_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", txt)
    assert m and int(m.group(1)) << int(m.group(2)) == E.NOALLOC_SCRATCH_BYTES
    cfg = C.CONFIGS["c2_8b_dynamic"]
    h, kv = _head(cfg.head), _kv(cfg, list(cfg.n))
    t = _tree(cfg, state=1 << 20, nbytes=1 << 30)
    assert E.eagle_workspace_bytes(h, kv, t) > E.NOALLOC_SCRATCH_BYTES
    assert lib.eagle_draft_step_noalloc(h, kv, t, 0, 1 << 20, None, None, None, None, None) == E.EAGLE_ECAPACITY
    small = C.SMALL_CONFIGS["s2_dynamic"]
    hs, kvs = _head(small.head), _kv(small, list(small.n))
    ts = _tree(small, state=1 << 20, nbytes=1 << 30)
    ts.inv_temp = float("nan")
    assert lib.eagle_draft_step_noalloc(hs, kvs, ts, 0, 1 << 20, None, None, None, None, None) == E.EAGLE_EINVAL


def test_steady_state_kv_is_validated(lib):
    """Steady state: n_new needs cu_new and 1 <= total_new / B; step 0 needs
    the ingest inputs (EAGLE-1 too); the workspace is sized by the new rows."""
    cfg = C.CONFIGS["c5_8b_eagle3_steady"]
    n = [600] * cfg.B
    h, t = _head(cfg.head), _tree(cfg)
    full = E.eagle_workspace_bytes(h, _kv(cfg, n), t)
    kv = _kv(cfg, n)
    kv.n_new, kv.cu_new, kv.total_new = 1 << 20, 1 << 20, 4 * cfg.B
    steady = E.eagle_workspace_bytes(h, kv, t)
    assert 0 < steady < full
    for f, v in [("cu_new", None), ("total_new", cfg.B - 1), ("total_new", sum(n) + 1)]:
        kb = _kv(cfg, n)
        kb.n_new, kb.cu_new, kb.total_new = 1 << 20, 1 << 20, 4 * cfg.B
        setattr(kb, f, v)
        assert E.eagle_workspace_bytes(h, kb, t) == 0, (f, v)
    kb = _kv(cfg, n)
    kb.cu_new = 1 << 20           # cu_new without n_new
    assert E.eagle_workspace_bytes(h, kb, t) == 0
    ts = _tree(cfg, state=1 << 20, nbytes=1 << 30)
    h1 = _head(replace(cfg.head, mode=C.MODE_EAGLE1))
    # EAGLE-1 steady state without its ingest inputs (target features, tokens)
    assert lib.eagle_draft_step(h1, kv, ts, 0, 1, None, None, None, None, 1 << 20, 1 << 40, None) == E.EAGLE_EINVAL
    assert lib.eagle_draft_step(h1, kv, ts, 0, 1, 1 << 20, None, None, None, 1 << 20, 1 << 40, None) == E.EAGLE_EINVAL


def test_target_pass_and_commit_are_validated(lib):
    """The target pass needs every layer's weights and a final gain; its
    workspace covers the B * positions verify rows; eagle_kv_commit refuses
    misaligned buffers and bad shapes before any launch."""
    cfg = C.CONFIGS["c1_8b_static"]
    h, t = _head(cfg.head), _tree(cfg)
    kv = _kv(cfg, list(cfg.n))
    L = 3
    layers = (E.eagle_layer * L)()
    for l in range(L):
        for f, _ in E.eagle_layer._fields_:
            setattr(layers[l], f, 1 << 20)
    tg = E.eagle_target()
    tg.n_layers, tg.layers, tg.final_norm_g = L, layers, 1 << 20
    ws = E.eagle_target_workspace_bytes(h, tg, kv, t)
    assert ws >= cfg.B * cfg.positions * cfg.head.ffn * 2
    for field, val in [("n_layers", 0), ("final_norm_g", None)]:
        tb = E.eagle_target()
        tb.n_layers, tb.layers, tb.final_norm_g = L, layers, 1 << 20
        setattr(tb, field, val)
        assert E.eagle_target_workspace_bytes(h, tb, kv, t) == 0, field
    layers[1].w_down = None
    assert E.eagle_target_workspace_bytes(h, tg, kv, t) == 0
    layers[1].w_down = 1 << 20
    layers[2].v_ctx = None           # a layer without its context cache
    assert E.eagle_target_workspace_bytes(h, tg, kv, t) == 0
    layers[2].v_ctx = 1 << 20
    ts = _tree(cfg, state=1 << 20, nbytes=1 << 30)
    # null logits, k_tree without v_tree, workspace too small
    assert lib.eagle_target_verify_logits(h, tg, kv, ts, None, None, None, None, 1 << 20, 1 << 40, None) == E.EAGLE_EINVAL
    assert lib.eagle_target_verify_logits(h, tg, kv, ts, 1 << 20, 1 << 20, None, None, 1 << 20, 1 << 40, None) == E.EAGLE_EINVAL
    assert lib.eagle_target_verify_logits(h, tg, kv, ts, 1 << 20, None, None, None, 1 << 20, 16, None) == E.EAGLE_ECAPACITY
    # commit: misaligned destination, bad dtype, rows not a 16-byte multiple, no rows
    a = 1 << 20
    assert lib.eagle_kv_commit(ts, 8, 128, 0, a, a, a, a, a, 100, a + 2, a, None) == E.EAGLE_EINVAL
    assert lib.eagle_kv_commit(ts, 8, 128, 9, a, a, a, a, a, 100, a, a, None) == E.EAGLE_EINVAL
    assert lib.eagle_kv_commit(ts, 1, 4, 0, a, a, a, a, a, 100, a, a, None) == E.EAGLE_EINVAL
    assert lib.eagle_kv_commit(ts, 8, 128, 0, a, a, a, a, a, 0, a, a, None) == E.EAGLE_EINVAL
