"""Pins for the CPU oracle: closed forms, textbook reductions, the pages' worked
examples and brute force on tiny inputs.  CPU only."""
import itertools
import json
import math
import os
from dataclasses import replace

import numpy as np
import pytest
from scipy.special import logsumexp
from scipy.special import softmax as sp_softmax

from eagle_feature_space_amd import configs as C
from eagle_feature_space_amd import synth
from oracle import head as H
from oracle import tree as T
from oracle import sampling as SM
from oracle import target as TG
from oracle import verify as VF
from oracle.round import ingest_features, run_round

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _head(cfg, dtype=np.float32, **over):
    w = {k: synth.f32(v).astype(dtype) for k, v in synth.head_weights(cfg, 77).items()}
    w.update(over)
    return H.DraftHead(cfg, w, dtype)


TINY = C.HeadCfg(d=64, vocab=97, n_q=4, n_kv=2, head_dim=16, ffn=96, rope_theta=10000.0)
TINY_E3 = replace(TINY, mode=C.MODE_EAGLE3)


# ------------------------------------------------------------ head structure
def test_fc_shape_and_param_count():
    """fc is a [2d, d] map; trainable matrices ~ 2d^2 + 12d^2
    ("What is actually in the head")."""
    cfg = C.HEAD_TINY_F32
    hd = _head(cfg)
    d = cfg.d
    assert hd.fc_map_shape() == (2 * d, d)
    # MHA + 4x GELU MLP: 2d^2 (fc) + 4d^2 (attention) + 8d^2 (MLP) = 14 d^2
    assert hd.matrix_param_count() == 14 * d * d == 917504
    # 8B shape (GQA 32/8, SwiGLU 14336): 15 d^2, within 7% of 14 d^2
    c1 = C.HEAD_8B
    shapes = dict(w_fc=(c1.d, 2 * c1.d), w_q=(c1.q_dim, c1.d), w_k=(c1.kv_dim, c1.d),
                  w_v=(c1.kv_dim, c1.d), w_o=(c1.d, c1.q_dim), w_gate=(c1.ffn, c1.d),
                  w_up=(c1.ffn, c1.d), w_down=(c1.d, c1.ffn))
    big = H.DraftHead(c1, {k: np.broadcast_to(np.float32(0), s) for k, s in shapes.items()})
    cnt = big.matrix_param_count()
    assert cnt == 15 * c1.d * c1.d
    assert abs(cnt / (14 * c1.d * c1.d) - 1) < 0.075
    assert big.fc_map_shape() == (2 * c1.d, c1.d)


def test_fc_input_feature_first():
    """x = concat(f, emb(t)) with the feature first (the recurrence and the
    (f_can, e_I) example)."""
    d = TINY.d
    eye = np.eye(d, dtype=np.float64)
    zero = np.zeros((d, d))
    hd = _head(TINY, np.float64, w_fc=np.concatenate([eye, zero], 1))
    f = np.random.default_rng(0).standard_normal((3, d))
    tok = np.array([5, 7, 11])
    np.testing.assert_array_equal(hd.fc_input(f, tok), f)
    hd2 = _head(TINY, np.float64, w_fc=np.concatenate([zero, eye], 1))
    np.testing.assert_array_equal(hd2.fc_input(f, tok), hd2.w["emb"][tok])


def test_fuse_concat_order():
    """g = FC([l; m; h]): with FC = [0 | 0 | I] the output is the h segment."""
    d = TINY.d
    eye, z = np.eye(d), np.zeros((d, d))
    lmh = np.random.default_rng(1).standard_normal((4, 3 * d))
    for seg in range(3):
        blocks = [z, z, z]
        blocks[seg] = eye
        hd = _head(TINY_E3, np.float64, w_fuse=np.concatenate(blocks, 1))
        np.testing.assert_array_equal(hd.fuse(lmh), lmh[:, seg * d:(seg + 1) * d])


def test_layer_is_pre_norm_residual():
    """With W_o = 0 and W_down = 0 both residual branches vanish: out == h."""
    hd = _head(TINY, np.float64, w_o=np.zeros((TINY.d, TINY.q_dim)),
               w_down=np.zeros((TINY.d, TINY.ffn)))
    rng = np.random.default_rng(2)
    h = rng.standard_normal((2, TINY.d))
    ck = rng.standard_normal((5, TINY.n_kv, TINY.head_dim))
    out, _, _ = hd.layer(h, np.array([5, 6]), lambda r, k, v: (ck, ck))
    np.testing.assert_array_equal(out, h)


def test_lm_head_orientation():
    """logits = W_LM f with W_LM [|V|, d]: one-hot rows pick feature entries."""
    d, V = TINY.d, TINY.vocab
    W = np.zeros((V, d))
    W[np.arange(V), np.arange(V) % d] = 1.0
    hd = _head(TINY, np.float64, lm_head=W)
    f = np.random.default_rng(3).standard_normal((2, d))
    np.testing.assert_array_equal(hd.lm_head(f), f[:, np.arange(V) % d])


# ------------------------------------------------------------ primitives
def test_norms_closed_form():
    x = np.full((1, 8), 3.0)
    np.testing.assert_allclose(H.rms_norm(x, np.ones(8), 1e-5), 3.0 / math.sqrt(9 + 1e-5))
    r = np.random.default_rng(4).standard_normal((5, 64))
    y = H.rms_norm(r, np.ones(64), 0.0)
    np.testing.assert_allclose(np.sqrt((y * y).mean(-1)), 1.0, rtol=1e-12)
    ln = H.layer_norm(r, np.ones(64), np.full(64, 0.5), 0.0)
    np.testing.assert_allclose(ln.mean(-1), 0.5, atol=1e-12)
    np.testing.assert_allclose(((ln - 0.5) ** 2).mean(-1), 1.0, rtol=1e-12)


def test_activations_textbook_values():
    x = np.array([0.0, 1.0, -1.0, 8.0, -8.0])
    phi1 = 0.8413447460685429                      # standard normal CDF at 1
    np.testing.assert_allclose(H.gelu(x), [0, phi1, -(1 - phi1), 8.0, 0.0], atol=1e-12)
    sig1 = 1 / (1 + math.exp(-1))
    np.testing.assert_allclose(H.silu(x)[:3], [0, sig1, -(1 - sig1)], rtol=1e-14)


def test_rope_closed_forms():
    # head_dim 2: one pair rotated by pos radians (inv_freq = 1)
    x = np.array([[[1.0, 0.0]]])
    for pos in (0, 1, 3):
        y = H.rope(x, np.array([pos]), 10000.0)
        np.testing.assert_allclose(y[0, 0], [math.cos(pos), math.sin(pos)], atol=1e-15)
    rng = np.random.default_rng(5)
    q = rng.standard_normal((1, 1, 32))
    k = rng.standard_normal((1, 1, 32))
    # pairs keep their length
    y = H.rope(q, np.array([123]), 10000.0)
    np.testing.assert_allclose(y[..., :16] ** 2 + y[..., 16:] ** 2,
                               q[..., :16] ** 2 + q[..., 16:] ** 2, rtol=1e-12)
    # scores depend only on the position difference
    def score(a, b):
        return float(np.sum(H.rope(q, np.array([a]), 1e4) * H.rope(k, np.array([b]), 1e4)))
    assert abs(score(10, 3) - score(107, 100)) < 1e-10
    assert abs(score(10, 3) - score(10, 4)) > 1e-6
    np.testing.assert_array_equal(H.rope(q, np.array([7]), 0.0), q)   # theta 0: off


def test_rope_frequency_schedule():
    """Pair i of a head turns by pos * theta^(-2i/hd): with theta = 10^4 and
    hd = 8 the four pairs turn by pos, pos/10, pos/100 and pos/1000 radians
    (a schedule of theta^(-i/hd) or over hd/2 would move pairs 1-3)."""
    hd, half, pos = 8, 4, 5
    for i in range(half):
        x = np.zeros((1, 1, hd))
        x[0, 0, i] = 1.0                      # unit vector on pair i's first axis
        y = H.rope(x, np.array([pos]), 10000.0)[0, 0]
        ang = pos * 10.0 ** (-i)
        want = np.zeros(hd)
        want[i], want[i + half] = math.cos(ang), math.sin(ang)
        np.testing.assert_allclose(y, want, atol=1e-15)
        # the second axis of the pair turns the same way: (0, 1) -> (-sin, cos)
        x2 = np.zeros((1, 1, hd))
        x2[0, 0, i + half] = 1.0
        y2 = H.rope(x2, np.array([pos]), 10000.0)[0, 0]
        want2 = np.zeros(hd)
        want2[i], want2[i + half] = -math.sin(ang), math.cos(ang)
        np.testing.assert_allclose(y2, want2, atol=1e-15)


def test_swiglu_roles():
    """SwiGLU = W_down(silu(W_gate a) * W_up a): with d = ffn, W_gate = c I,
    W_up = W_down = I and c != 1 the MLP branch is silu(c N2(x)) * N2(x),
    which silu(W_up a) * W_gate a = silu(N2(x)) * c N2(x) does not equal."""
    cfg = replace(TINY, ffn=TINY.d)
    eye = np.eye(cfg.d)
    c = 2.5
    hd = _head(cfg, np.float64, w_gate=c * eye, w_up=eye, w_down=eye)
    x = np.random.default_rng(11).standard_normal((3, cfg.d))
    n2 = hd.norm(x, 2)
    want = (c * n2) / (1.0 + np.exp(-c * n2)) * n2
    np.testing.assert_allclose(hd.mlp(x), want, rtol=1e-13, atol=1e-14)
    swapped = n2 / (1.0 + np.exp(-n2)) * (c * n2)
    assert np.max(np.abs(hd.mlp(x) - swapped)) > 1e-2


def test_attention_closed_forms():
    hd = 16
    rng = np.random.default_rng(6)
    q = rng.standard_normal((4, hd))
    # one key: output is that value
    K = rng.standard_normal((1, 2, hd))
    V = rng.standard_normal((1, 2, hd))
    out = H.attend(q, K, V, group=2)
    np.testing.assert_allclose(out[:2], np.repeat(V[:, 0], 2, 0), rtol=1e-14)
    # two keys: weight of key 0 = sigmoid(q.k / sqrt(hd))
    a = 3.0
    q1 = np.zeros((1, hd)); q1[0, 0] = a
    K2 = np.zeros((2, 1, hd)); K2[0, 0, 0] = 1.0
    V2 = np.zeros((2, 1, hd)); V2[0, 0, 1] = 1.0; V2[1, 0, 2] = 1.0
    o = H.attend(q1, K2, V2, group=1)
    p0 = 1 / (1 + math.exp(-a / math.sqrt(hd)))
    np.testing.assert_allclose(o[0, [1, 2]], [p0, 1 - p0], rtol=1e-14)
    # GQA: query heads 0,1 read kv head 0; heads 2,3 read kv head 1
    Kg = rng.standard_normal((5, 2, hd))
    Vg = np.zeros((5, 2, hd)); Vg[:, 0] = 1.0; Vg[:, 1] = -2.0
    og = H.attend(q, Kg, Vg, group=2)
    np.testing.assert_allclose(og[:2], 1.0, rtol=1e-14)
    np.testing.assert_allclose(og[2:], -2.0, rtol=1e-14)


def test_topk_softmax_against_library():
    rng = np.random.default_rng(7)
    z = rng.standard_normal((6, 50)).astype(np.float32)
    z[0, [3, 9, 17]] = 5.0                                # tie at the top
    z[1, [4, 8]] = z[1].max() + 1                         # tie at the top
    ids, conf, lse = H.DraftHead.draft_choices(z, 5, inv_temp=2.5)
    for r in range(6):
        ref = np.argsort(-z[r], kind="stable")[:5]
        np.testing.assert_array_equal(ids[r], ref)
        np.testing.assert_allclose(conf[r], sp_softmax(2.5 * z[r].astype(np.float64))[ref], rtol=2e-6)
        np.testing.assert_allclose(lse[r], logsumexp(2.5 * z[r].astype(np.float64)), rtol=1e-6)
    np.testing.assert_array_equal(ids[0, :3], [3, 9, 17])
    assert VF.target_choice(np.array([1.0, 4.0, 2.0, 4.0])) == 1


# ------------------------------------------------------------ trees
def test_static_template_shape():
    tmpl = C.STATIC_TREE_25
    dep = T.template_depths(tmpl)
    assert len(tmpl) == 25 and max(dep) == 4
    widths = [sum(1 for x in dep[1:] if x == l) for l in (1, 2, 3, 4)]
    assert widths == [4, 9, 8, 4]
    ch = T.static_children(tmpl)
    fan = [max(len(ch[u]) for u in range(26) if dep[u] == l) for l in (0, 1, 2, 3)]
    assert fan == [4, 3, 2, 1]
    rows = [sum(1 for u in range(26) if dep[u] == l and ch[u]) for l in (0, 1, 2, 3)]
    assert rows == [1, 4, 4, 4]


def test_static_expansion_follows_template_ranks():
    """Static tree ("Drafting a Tree, Not a Chain"): a node's template children
    take its top-k ids in rank order; the frontier of the next step is the new
    nodes with template children, in creation order.  Hand-built template
    root -> {1, 2}, 1 -> {3, 4}, 2 -> {5} with known ids per row."""
    tmpl = (0, 0, 1, 1, 2)
    t = T.RequestTree.start(T.STATIC, root_tok=7, root_pos=10, gamma=2, top_k=3,
                            template=tmpl)
    # step 0: one row (the root); ranks 0, 1 become nodes 1, 2
    t.expand(0, np.array([[100, 200, 300]]), np.array([[0.5, 0.25, 0.125]], np.float32))
    assert t.tok == [7, 100, 200] and t.parent == [-1, 0, 0]
    assert t.frontier == [1, 2]                      # both have template children
    rows = t.rows()
    assert [(r[0], r[2], r[3]) for r in rows] == [(1, 100, 11), (2, 200, 11)]
    # step 1: row 0 is node 1 (two children), row 1 is node 2 (one child)
    t.expand(1, np.array([[11, 12, 13], [21, 22, 23]]),
             np.array([[0.5, 0.25, 0.125], [0.75, 0.125, 0.0625]], np.float32))
    assert t.tok == [7, 100, 200, 11, 12, 21]
    assert t.parent == [-1, 0, 0, 1, 1, 2]
    assert t.depth == [0, 1, 1, 2, 2, 2]
    assert [float(v) for v in t.value] == [1.0, 0.5, 0.25, 0.25, 0.125, 0.1875]
    f = t.final_tree()
    assert list(f["tok"]) == [7, 100, 200, 11, 12, 21]
    assert list(f["pos"]) == [10, 11, 11, 12, 12, 12]


def _closure(parent):
    """Ancestor-or-self relation by repeated composition (brute force)."""
    n = len(parent)
    A = np.eye(n, dtype=bool)
    for _ in range(n):
        for u in range(n):
            for v in range(n):
                if A[u, v] and parent[v] >= 0:
                    A[u, parent[v]] = True
    return A


def _random_tree(rng, kind, gamma, top_k, top_m, V=50, template=()):
    t = T.RequestTree.start(kind, int(rng.integers(V)), 17, gamma, top_k, top_m, template)
    for s in range(gamma):
        rows = len(t.frontier)
        ids = np.stack([rng.choice(V, top_k, replace=False) for _ in range(rows)])
        conf = np.sort(rng.dirichlet(np.ones(top_k + 3), size=rows)[:, :top_k], 1)[:, ::-1]
        t.expand(s, ids, conf.astype(np.float32))
    return t


@pytest.mark.parametrize("seed", range(6))
def test_values_masks_and_rerank(seed):
    rng = np.random.default_rng(seed)
    top_k, gamma, top_m = 3, 4, 10
    t = _random_tree(rng, T.DYNAMIC, gamma, top_k, top_m)
    P = len(t.tok)
    assert P == 1 + top_k + (gamma - 1) * top_k * top_k
    # V = product of c along the root path (float64), monotone along edges
    for u in range(1, P):
        prod, w = 1.0, u
        while w > 0:
            prod *= float(t.conf[w])
            w = t.parent[w]
        assert abs(float(t.value[u]) - prod) <= 1e-6 * prod
        assert t.value[u] <= t.value[t.parent[u]]
    # rerank = brute-force sort of the pool by (value desc, depth asc, index asc)
    keyed = sorted(range(1, P), key=lambda u: (-float(t.value[u]), t.depth[u], u))
    assert t.rerank() == keyed[:top_m]
    f = t.final_tree()
    Tn = len(f["tok"])
    assert Tn == top_m + 1
    bits = np.array([[(int(f["mask"][u]) >> v) & 1 for v in range(Tn)] for u in range(Tn)], bool)
    np.testing.assert_array_equal(bits, _closure(f["parent"]))
    np.testing.assert_array_equal(bits.sum(1), f["depth"] + 1)
    np.testing.assert_array_equal(f["pos"], 17 + f["depth"])
    for u in range(Tn):
        for v in range(Tn):
            if bits[u, v]:
                assert f["pos"][v] <= f["pos"][u] and v <= u


def test_nan_values_rank_last_and_keep_the_tree_whole():
    """A NaN confidence (a NaN logit row) gives NaN path values below it; they
    rank after every finite value, so the frontier and the kept set keep
    their sizes, the kept set stays ancestor-closed and fits the verify tree."""
    t = T.RequestTree.start(T.DYNAMIC, root_tok=1, root_pos=0, gamma=3, top_k=3, top_m=7)
    nan = np.float32("nan")
    t.expand(0, np.array([[10, 11, 12]]), np.array([[nan, 0.5, 0.25]], np.float32))
    assert t.frontier == [2, 3, 1]                  # the NaN child last
    t.expand(1, np.array([[20, 21, 22], [30, 31, 32], [40, 41, 42]]),
             np.array([[0.5, 0.25, 0.125], [nan, 0.5, 0.5], [0.5, 0.5, 0.5]], np.float32))
    assert len(t.frontier) == 3 and all(not np.isnan(t.value[u]) for u in t.frontier)
    t.expand(2, np.zeros((3, 3), np.int64), np.full((3, 3), 0.5, np.float32))
    kept = t.rerank()
    assert len(kept) == 7
    assert all(not np.isnan(t.value[u]) for u in kept)
    f = t.final_tree()
    assert len(f["tok"]) == 8 and f["parent"][0] == -1
    assert all(0 <= p < i for i, p in enumerate(f["parent"]) if i > 0)


def test_residual_draw_with_no_mass_left_takes_the_last_rejected():
    """A near-one-hot target whose only mass sat on rejected children leaves
    no residual: the token is the last child rejected."""
    p = np.zeros(8)
    p[3] = 1.0
    assert VF.residual_draw(p, [3], 0.7) == 3
    p2 = np.zeros(8)
    p2[[2, 5]] = 0.5
    assert VF.residual_draw(p2, [5, 2], 0.1) == 2


def test_frontier_is_top_k_of_newest_depth():
    rng = np.random.default_rng(11)
    top_k = 4
    t = T.RequestTree.start(T.DYNAMIC, 1, 0, 3, top_k, 8)
    for s in range(3):
        prev = len(t.tok)
        rows = len(t.frontier)
        ids = np.stack([rng.choice(40, top_k, replace=False) for _ in range(rows)])
        conf = rng.uniform(0.01, 1, (rows, top_k)).astype(np.float32)
        conf[0, 1] = conf[0, 0]                                   # value tie
        t.expand(s, ids, conf)
        if s < 2:
            new = list(range(prev, len(t.tok)))
            brute = sorted(new, key=lambda u: (-float(t.value[u]), u))[:top_k]
            assert t.frontier == brute
            assert all(t.depth[u] == s + 1 for u in t.frontier)


# ------------------------------------------------------------ verification
def test_verify_page_example():
    g = json.load(open(os.path.join(GOLD, "verify_paris_example.json")))
    toks = [g["root_token"]] + g["draft_chain"]
    parent = [-1, 0, 1, 2, 3]
    V = 16
    logits = np.zeros((5, V), np.float32)
    for u, c in enumerate(g["target_choice_per_position"]):
        logits[u, c] = 1.0
    acc, path, out = VF.verify(np.array(toks), np.array(parent), logits, 4)
    assert acc == g["expect_accept_len"]
    assert list(out) == g["expect_out_tokens"]
    assert list(path) == g["expect_path"]


def _all_root_paths(parent):
    T_ = len(parent)
    paths = []
    for u in range(T_):
        p, w = [], u
        while w >= 0:
            p.append(w)
            w = parent[w]
        paths.append(p[::-1])
    return paths


@pytest.mark.parametrize("seed", range(20))
def test_verify_bruteforce(seed):
    rng = np.random.default_rng(100 + seed)
    Tn = int(rng.integers(1, 13))
    parent = [-1] + [int(rng.integers(0, u)) for u in range(1, Tn)]
    V = 6
    # distinct tokens among siblings
    tok = [int(rng.integers(V))]
    kids = {}
    for u in range(1, Tn):
        used = kids.setdefault(parent[u], set())
        choices = [x for x in range(V) if x not in used]
        if not choices:
            parent[u] = 0 if len(kids.get(0, ())) < V else parent[u]
            used = kids.setdefault(parent[u], set())
            choices = [x for x in range(V) if x not in used]
        x = int(rng.choice(choices))
        used.add(x)
        tok.append(x)
    choice = rng.integers(V, size=Tn)
    logits = np.zeros((Tn, V), np.float32)
    logits[np.arange(Tn), choice] = 1.0
    depth = [len(p) - 1 for p in _all_root_paths(parent)]
    gamma = max(depth) + 1
    acc, path, out = VF.verify(np.array(tok), np.array(parent), logits, gamma)
    best = [0]
    for p in _all_root_paths(parent):
        if all(tok[p[i + 1]] == choice[p[i]] for i in range(len(p) - 1)) and len(p) > len(best):
            best = p
    assert acc == len(best) - 1
    assert list(path[:len(best)]) == best
    assert list(out[:acc]) == [tok[u] for u in best[1:]]
    assert out[acc] == choice[best[-1]]


def _mc_chain(alpha, gamma, trials, rng):
    tot = 0
    V = 8
    parent = np.arange(-1, gamma)
    tok = np.array([0] + [1] * gamma)
    for _ in range(trials):
        ok = rng.random(gamma + 1) < alpha
        logits = np.zeros((gamma + 1, V), np.float32)
        logits[np.arange(gamma + 1), np.where(ok, 1, 2)] = 1.0
        acc, _, _ = VF.verify(tok, parent, logits, gamma)
        tot += acc + 1
    return tot / trials


@pytest.mark.parametrize("alpha", [0.5, 0.7, 0.9])
def test_chain_acceptance_geometric_sum(alpha):
    """E[tokens per pass] = (1 - alpha^(gamma+1)) / (1 - alpha)."""
    gamma, trials = 4, 30000
    rng = np.random.default_rng(int(alpha * 100))
    est = _mc_chain(alpha, gamma, trials, rng)
    E = (1 - alpha ** (gamma + 1)) / (1 - alpha)
    # std of the emitted length is < gamma/2; 4 sigma
    assert abs(est - E) < 4 * (gamma / 2) / math.sqrt(trials)


def test_tree_widening_page_numbers():
    g = json.load(open(os.path.join(GOLD, "tree_acceptance_examples.json")))
    rng = np.random.default_rng(5)
    trials = 40000
    # chain, alpha 0.7: P(reach depth 2) = 0.49
    reach2 = 0
    tok = np.array([0, 1, 1])
    for _ in range(trials):
        ok = rng.random(2) < 0.7
        logits = np.zeros((3, 4), np.float32)
        logits[[0, 1], np.where(ok, 1, 2)] = 1.0
        reach2 += VF.verify(tok, np.array([-1, 0, 1]), logits, 2)[0] >= 2
    p = reach2 / trials
    assert abs(p - g["reach_depth2_alpha07_chain"]) < 4 * math.sqrt(0.25 / trials)
    # depth 1 with b = 3 candidates each acceptable w.p. 0.7
    hit = 0
    tok3 = np.array([0, 1, 2, 3])
    for _ in range(trials):
        ok = rng.random(3) < 0.7
        logits = np.zeros((4, 6), np.float32)
        logits[0, (1 + int(np.argmax(ok))) if ok.any() else 5] = 1.0
        hit += VF.verify(tok3, np.array([-1, 0, 0, 0]), logits, 1)[0] >= 1
    p3 = hit / trials
    assert abs(p3 - (1 - 0.3 ** 3)) < 4 * math.sqrt(0.25 / trials)
    assert abs((1 - 0.3 ** 3) - g["reach_depth1_alpha07_b3"]) < 5e-4


# ------------------------------------------------------------ whole-round pins
def _round_cfg(kind, head, B=2, n=(9, 4), gamma=3, top_k=3, top_m=7, template=()):
    return C.RoundCfg(name="pin", head=head, B=B, n=n, tree=kind, gamma=gamma,
                      top_k=top_k, top_m=top_m, template=template, seed_w=5, seed_in=6,
                      seed_t=7)


def _inputs64(cfg):
    inp = synth.round_inputs(cfg)
    out = dict(n=inp.n, t_root=inp.t_root)
    if inp.k_ctx is not None:
        out.update(k_ctx=synth.f32(inp.k_ctx).astype(np.float64),
                   v_ctx=synth.f32(inp.v_ctx).astype(np.float64),
                   f_root=synth.f32(inp.f_root).astype(np.float64))
    else:
        out.update(lmh=synth.f32(inp.lmh).astype(np.float64), ctx_tokens=inp.ctx_tokens)
    return out


def _chain_nodes(tr, u):
    p = []
    while u >= 0:
        p.append(u)
        u = tr.parent[u]
    return p[::-1]


@pytest.mark.parametrize("kind", [T.DYNAMIC, T.STATIC])
def test_tree_attention_equals_causal_chain(kind):
    """Tree-masked attention at every node equals plain causal attention over
    [context ; root -> node chain] with positions n + depth."""
    tmpl = (0, 0, 1, 1, 2, 3, 3, 6) if kind == T.STATIC else ()
    cfg = _round_cfg(kind, TINY, gamma=3 if kind == T.DYNAMIC else 4, template=tmpl)
    hd = _head(TINY, np.float64)
    inp = _inputs64(cfg)
    res = run_round(cfg, hd, **inp)
    cu = np.concatenate([[0], np.cumsum(inp["n"])])
    for b in range(cfg.B):
        tr = res.trees[b]
        ck = inp["k_ctx"][cu[b]:cu[b + 1]]
        cv = inp["v_ctx"][cu[b]:cu[b + 1]]
        # every expanded node's feature, recomputed along its chain
        for s, st in enumerate(res.steps):
            r0 = sum(len(st.rows[bb]) for bb in range(b))
            for i, row in enumerate(st.rows[b]):
                u = row[0]
                chain = _chain_nodes(tr, u)
                Ks, Vs, f = [], [], inp["f_root"][b]
                for depth, w in enumerate(chain):
                    h = hd.fc_input(f[None], np.array([tr.tok[w]]))
                    q, k, v = hd.qkv(h, np.array([inp["n"][b] + depth]))
                    Ks.append(k[0]); Vs.append(v[0])
                    K = np.concatenate([ck, np.stack(Ks)]); V = np.concatenate([cv, np.stack(Vs)])
                    att = H.attend(q[0], K, V, hd.group)
                    f = hd.finish(h, att[None])[0]
                np.testing.assert_allclose(st.feat[r0 + i], f, rtol=1e-10, atol=1e-10)


def test_chain_equals_naive_greedy_decoding():
    """A top-1 chain equals greedy AR decoding of the head with a full causal
    recompute of every drafted row at every step (no slot cache)."""
    cfg = _round_cfg(T.CHAIN, TINY, B=1, n=(11,), gamma=4, top_k=1)
    hd = _head(TINY, np.float64)
    inp = _inputs64(cfg)
    res = run_round(cfg, hd, **inp)
    n = int(inp["n"][0])
    toks = [int(inp["t_root"][0])]
    for s in range(cfg.gamma):
        # recompute all rows 0..s from scratch
        f = inp["f_root"][0]
        hs = []
        feats = []
        for j in range(s + 1):
            h = hd.fc_input(f[None], np.array([toks[j]]))
            hs.append(h[0])
            _, k_all, v_all = hd.qkv(np.stack(hs), n + np.arange(j + 1))
            q, _, _ = hd.qkv(h, np.array([n + j]))
            K = np.concatenate([inp["k_ctx"], k_all]); V = np.concatenate([inp["v_ctx"], v_all])
            f = hd.finish(h, H.attend(q[0], K, V, hd.group)[None])[0]
            feats.append(f)
        logits = hd.lm_head(f[None])[0]
        toks.append(int(np.argmax(logits)))
        np.testing.assert_allclose(res.steps[s].feat[0], f, rtol=1e-10, atol=1e-10)
    assert list(res.final[0]["tok"]) == toks


def test_eagle3_chain_equals_full_causal_recompute():
    """EAGLE-3: verified positions take g_j + emb(t_{j+1}), later steps a +
    emb(t); a top-1 chain equals a full causal recompute of the whole
    sequence at every step (every position's layer output computed)."""
    cfg = _round_cfg(T.CHAIN, TINY_E3, B=2, n=(6, 3), gamma=3, top_k=1)
    hd = _head(TINY_E3, np.float64)
    inp = _inputs64(cfg)
    res = run_round(cfg, hd, **inp)
    cu = np.concatenate([[0], np.cumsum(inp["n"])])
    for b in range(cfg.B):
        lmh = inp["lmh"][cu[b]:cu[b + 1]]
        tk = inp["ctx_tokens"][cu[b]:cu[b + 1]]
        n = len(tk)
        xs = list(hd.fuse(lmh) + hd.w["emb"][tk])
        drafted = []
        for s in range(cfg.gamma):
            X = np.stack(xs)
            L = len(xs)
            q, k, v = hd.qkv(X, np.arange(L))
            outs = np.stack([hd.finish(X[j:j + 1], H.attend(q[j], k[:j + 1], v[:j + 1], hd.group)[None])[0]
                             for j in range(L)])
            a = outs[-1]
            t = int(np.argmax(hd.lm_head(a[None])[0]))
            drafted.append(t)
            np.testing.assert_allclose(res.steps[s].feat[b], a, rtol=1e-10, atol=1e-10)
            xs.append(a + hd.w["emb"][t])
        assert list(res.final[b]["tok"][1:]) == drafted
        assert res.final[b]["pos"][0] == n - 1


# ------------------------------------------------- stochastic verification
@pytest.mark.parametrize("seed", range(8))
def test_verify_sample_with_one_hot_target_is_greedy(seed):
    """A target with all its mass on the argmax (inv_temp -> infinity) makes
    multi-round speculative sampling deterministic: it must return exactly
    what greedy verification returns, on random dynamic trees."""
    rng = np.random.default_rng(300 + seed)
    t = _random_tree(rng, T.DYNAMIC, 4, 3, 10, V=12)
    f = t.final_tree()
    Tn = len(f["tok"])
    logits = rng.standard_normal((Tn, 12))
    # plant some accepted children so paths of every length occur
    for u in range(Tn):
        kids = [v for v in range(Tn) if f["parent"][v] == u]
        if kids and rng.random() < 0.7:
            logits[u, f["tok"][kids[int(rng.integers(len(kids)))]]] = 4.0
    draws = rng.random((Tn, VF.N_DRAWS)) * (1 - 1e-9)
    g = VF.verify(f["tok"], f["parent"], logits.astype(np.float32), 4)
    s_ = VF.verify_sample(f["tok"], f["parent"], logits.astype(np.float32), 1e6, draws, 4)
    assert g[0] == s_[0]
    assert list(g[1]) == list(s_[1]) and list(g[2]) == list(s_[2])


def _sampled(tok, parent, logits, inv_temp, gamma, n, seed):
    rng = np.random.default_rng(seed)
    res = []
    for _ in range(n):
        res.append(VF.verify_sample(tok, parent, logits, inv_temp, rng.random((len(tok), VF.N_DRAWS)), gamma))
    return res


def _close(freq, p, n, z=5.0):
    return np.all(np.abs(freq - p) <= z * np.sqrt(p * (1 - p) / n) + 1.0 / n)


def test_verify_sample_is_lossless():
    """The emitted tokens follow the target: the first ~ p(root), and after an
    accepted child the next ~ p(that child's position), whatever the tree
    proposed (Monte Carlo, fixed seed, 5-sigma bounds per token)."""
    V = 6
    tok = np.array([5, 3, 1, 4, 0])          # root; children 3, 1, 4; 3 -> 0
    parent = np.array([-1, 0, 0, 0, 1])
    rng = np.random.default_rng(7)
    logits = rng.standard_normal((5, V)).astype(np.float32)
    s = 1.3
    n = 30000
    res = _sampled(tok, parent, logits, s, 2, n, 8)
    first = np.array([o[2][0] for o in res])
    p0 = VF.target_probs(logits[0], s)
    assert _close(np.bincount(first, minlength=V) / n, p0, n)
    for child in (1, 2):                     # token 3 (has a child), token 1 (leaf)
        sel = [o for o in res if o[0] >= 1 and o[1][1] == child]
        second = np.array([o[2][1] for o in sel])
        pc = VF.target_probs(logits[child], s)
        assert _close(np.bincount(second, minlength=V) / len(sel), pc, len(sel))
    # a token drawn from the residual is never one the node's children offered
    for acc, path, out in res:
        u = path[acc]
        offered = {int(tok[v]) for v in range(5) if parent[v] == u}
        assert out[acc] not in offered


def test_verify_sample_chain_acceptance_matches_page():
    """Chain whose every drafted token has target probability alpha = 0.7:
    P(reach depth 2) = 0.49 and E[tokens per pass] = (1 - a^(g+1)) / (1 - a)
    ("transformer_math / tm_eagle_deep", Acceptance length under a tree)."""
    g = json.load(open(os.path.join(GOLD, "tree_acceptance_examples.json")))
    V, gamma, a = 10, 3, 0.7
    tok = np.array([9, 1, 2, 3])
    parent = np.array([-1, 0, 1, 2])
    logits = np.zeros((4, V), np.float32)
    for u in range(3):
        logits[u, tok[u + 1]] = np.log(a * (V - 1) / (1 - a))
    n = 20000
    acc = np.array([r[0] for r in _sampled(tok, parent, logits, 1.0, gamma, n, 9)])
    reach2 = (acc >= 2).mean()
    assert abs(reach2 - g["reach_depth2_alpha07_chain"]) <= 5 * np.sqrt(0.49 * 0.51 / n)
    expect = (1 - a ** (gamma + 1)) / (1 - a)
    assert abs((acc + 1).mean() - expect) <= 5 * (acc + 1).std() / np.sqrt(n)


def test_verify_sample_residual_is_inverse_cdf():
    """Brute force on a tiny vocabulary: the residual draw is the token whose
    cumulative-mass interval (rejected tokens removed) contains u."""
    p = np.array([0.1, 0.25, 0.05, 0.3, 0.2, 0.1])
    excl = [3, 0]
    r = p.copy()
    r[excl] = 0
    r /= r.sum()
    edges = np.concatenate([[0], np.cumsum(r)])
    for u in np.linspace(0, 1, 101)[:-1]:
        x = VF.residual_draw(p, excl, u)
        assert x not in excl and edges[x] <= u < edges[x + 1] + 1e-12


# ------------------------------------------------- verification of sampled drafts
def _draft_logp(z, s):
    """log q for q = softmax(s * z), s * z in fp32 (the drafter's arithmetic)."""
    l = (np.float32(s) * np.asarray(z, np.float32)).astype(np.float64)
    return l - logsumexp(l)


@pytest.mark.parametrize("k", [1, 2, 3, 5])
@pytest.mark.parametrize("case", ["random", "draft_is_target", "draft_peaked", "target_peaked",
                                  "target_one_hot"])
def test_drafted_verify_law_is_the_target(k, case):
    """Exact law, brute force over every ordered draw: with children drawn one
    after another without replacement from q (the probability of a sequence is
    the product of q(x_j) / (mass of q not yet drawn)), each tested with
    probability min(1, thr_j) and the residual drawn when all fail, the token
    emitted at a node has the target distribution p exactly ("Speculative
    Decoding Deep Dive III", EAGLE-1 "Inference": multi-round speculative
    sampling keeps the target's distribution)."""
    V = 5
    rng = np.random.default_rng(hash(case) % 1000 + 10 * k)
    zt = rng.standard_normal(V).astype(np.float32)
    zd = rng.standard_normal(V).astype(np.float32)
    st, sd = 1.3, 0.9
    if case == "draft_is_target":
        zd, sd = zt.copy(), st
    elif case == "draft_peaked":
        sd = 40.0
    elif case == "target_peaked":
        zt = (3 * rng.standard_normal(V)).astype(np.float32)
    elif case == "target_one_hot":
        st = 1e4
    p = VF.target_probs(zt, st)
    lq = _draft_logp(zd, sd)
    law = np.zeros(V)
    total = 0.0
    for seq in itertools.permutations(range(V), k):
        rem = list(range(V))
        lp = 0.0
        for x in seq:
            lp += lq[x] - logsumexp(lq[rem])
            rem.remove(x)
        pr = math.exp(lp)
        total += pr
        thr, resid, mass = VF.drafted_tests(p, zd, sd, list(seq))
        # the first rejection leaves the total variation distance sum max(p - q, 0)
        assert abs(mass[1] - np.maximum(p - np.exp(lq), 0).sum()) < 1e-12
        stay = 1.0
        for j, x in enumerate(seq):
            a = min(1.0, thr[j])
            law[x] += pr * stay * a
            stay *= 1.0 - a
        law += pr * stay * resid
    assert abs(total - 1.0) < 1e-12
    np.testing.assert_allclose(law, p, rtol=0, atol=1e-13)


def test_drafted_verify_with_a_certain_draft_is_the_point_mass_rule():
    """A draft with all its mass on one token (s_d -> infinity) that proposes
    that token as the only child reduces the test to the one for top-k
    drafting: keep x iff u < p(x), else draw from p with x removed.  Both
    verifications give the same walk on random chains."""
    rng = np.random.default_rng(55)
    V, gamma = 9, 4
    for _ in range(40):
        tok = rng.integers(0, V, gamma + 1)
        parent = np.arange(-1, gamma)
        logits = rng.standard_normal((gamma + 1, V)).astype(np.float32)
        for u in range(gamma):
            if rng.random() < 0.6:
                logits[u, tok[u + 1]] += 2.5
        drafts = rng.standard_normal((gamma + 1, V)).astype(np.float32)
        for u in range(gamma):
            drafts[u, tok[u + 1]] = drafts[u].max() + 1.0
        drawn = [[(int(tok[u + 1]), u + 1)] if u < gamma else [] for u in range(gamma + 1)]
        draws = rng.random((gamma + 1, VF.N_DRAWS))
        a = VF.verify_sample(tok, parent, logits, 1.1, draws, gamma)
        b = VF.verify_sample_drafted(tok, parent, drawn, logits, 1.1, drafts, 1e5, draws, gamma)
        assert a[0] == b[0] and list(a[1]) == list(b[1]) and list(a[2]) == list(b[2])


def test_drafted_verify_keeps_the_first_child_when_draft_is_the_target():
    """q = p makes the first test's ratio exactly 1: the first drawn child is
    always kept, down to the leaf; a first child the tree dropped ends the walk
    with its token."""
    rng = np.random.default_rng(56)
    V = 7
    logits = rng.standard_normal((4, V)).astype(np.float32)
    tok = np.array([0, 3, 5, 2])
    parent = np.array([-1, 0, 0, 1])
    drawn = [[(3, 1), (5, 2)], [(2, 3)], [], []]
    for _ in range(50):
        draws = rng.random((4, VF.N_DRAWS))
        acc, path, out = VF.verify_sample_drafted(tok, parent, drawn, logits, 0.8, logits, 0.8,
                                                  draws, 2)
        assert acc == 2 and list(path) == [0, 1, 3] and out[:2].tolist() == [3, 2]
        dropped = [[(6, -1), (3, 1)], [(2, 3)], [], []]
        acc, path, out = VF.verify_sample_drafted(tok, parent, dropped, logits, 0.8, logits, 0.8,
                                                  draws, 2)
        assert acc == 0 and list(path) == [0, -1, -1] and list(out) == [6, -1, -1]


def test_drafted_verify_walk_is_lossless():
    """Monte Carlo through the whole walk: a bigram target and a different
    bigram draft; the root's 3 children drawn by Gumbel-top-k, the verify tree
    keeping draw ranks 0 and 2 (rank 1 dropped) and the rank-0 child's 2 drawn
    children.  The first two emitted tokens (the second completed from the
    target when the round stops after one) follow p(x0) p(x1 | x0) within 5
    sigma per cell.  Leaving the dropped child out of the root's tests moves a
    cell by ~20 sigma here."""
    V, st, sd = 5, 1.0, 3.0      # a peaked draft: the dropped child carries real mass
    rng = np.random.default_rng(57)
    Pz = rng.standard_normal((V, V)).astype(np.float32)       # target logits after token a
    Qz = rng.standard_normal((V, V)).astype(np.float32)       # draft logits after token a
    root = 0
    p0 = VF.target_probs(Pz[root], st)
    pn = np.array([VF.target_probs(Pz[a], st) for a in range(V)])
    n = 20000
    joint = np.zeros((V, V))
    gum = lambda z, k: np.argsort(-(np.float32(sd) * z + -np.log(-np.log(rng.random(V)))),
                                  kind="stable")[:k]
    for _ in range(n):
        r = gum(Qz[root], 3)
        c = gum(Qz[r[0]], 2)
        tok = np.array([root, r[0], r[2], c[0], c[1]])
        parent = np.array([-1, 0, 0, 1, 1])
        drawn = [[(int(r[0]), 1), (int(r[1]), -1), (int(r[2]), 2)],
                 [(int(c[0]), 3), (int(c[1]), 4)], [], [], []]
        logits = Pz[tok]
        drafts = Qz[tok]
        acc, path, out = VF.verify_sample_drafted(tok, parent, drawn, logits, st, drafts, sd,
                                                  rng.random((5, VF.N_DRAWS)), 2)
        x0 = int(out[0])
        x1 = int(out[1]) if acc >= 1 else int(rng.choice(V, p=pn[x0]))
        joint[x0, x1] += 1
    want = p0[:, None] * pn
    f = joint / n
    assert np.all(np.abs(f - want) <= 5 * np.sqrt(want * (1 - want) / n) + 1.0 / n)


# ------------------------------------------------- sampled drafting (Gumbel-top-k)
def test_philox_known_answers():
    """Philox4x32-10 against the known-answer vectors published with its
    definition (Salmon et al., SC'11; the Random123 test vectors)."""
    kat = [((0, 0, 0, 0), (0, 0), (0x6627e8d5, 0xe169c58d, 0xbc57ac4c, 0x9b00dbd8)),
           ((0xffffffff,) * 4, (0xffffffff,) * 2, (0x408f276d, 0x41c83b0e, 0xa20bc7c6, 0x6d5451fd)),
           ((0x243f6a88, 0x85a308d3, 0x13198a2e, 0x03707344), (0xa4093822, 0x299f31d0),
            (0xd16cfe09, 0x94fdcceb, 0x5001e420, 0x24126ea1))]
    for ctr, key, want in kat:
        got = SM.philox4x32_10([np.array([x], np.uint64) for x in ctr], key)
        assert [int(w[0]) for w in got] == list(want)


def test_uniforms_are_open_interval_and_gumbel_finite():
    u = SM.uniforms(12345, 7, 4096)
    assert u.dtype == np.float32 and u.min() > 0 and u.max() < 1
    # the extreme bit patterns still give finite Gumbel values
    for bits in (0, 0xFFFFFFFF):
        ue = ((np.uint32(bits) >> np.uint32(9)).astype(np.float32) + np.float32(0.5)) * np.float32(2.0 ** -23)
        assert np.isfinite(-np.log(-np.log(ue)))
    # uniform: 16 equal bins within 5 sigma
    h = np.bincount((SM.uniforms(99, 3, 1 << 16) * 16).astype(int), minlength=16) / (1 << 16)
    assert np.all(np.abs(h - 1 / 16) <= 5 * np.sqrt((1 / 16) * (15 / 16) / (1 << 16)))


def test_gumbel_topk_samples_without_replacement():
    """Gumbel-max draws follow softmax(s * logits); the first two of
    Gumbel-top-2 follow sequential sampling without replacement
    (Monte Carlo over row keys, 5-sigma bounds)."""
    l = np.array([1.0, -0.5, 2.0, 0.3, 0.0, -1.2], np.float32)
    s = 1.3
    p = np.exp(s * l.astype(np.float64))
    p /= p.sum()
    n = 40000
    first = np.zeros(6)
    pair = np.zeros((6, 6))
    for r in range(n):
        ids, _ = SM.gumbel_topk(l, 2, s, 2024, r)
        first[ids[0]] += 1
        pair[ids[0], ids[1]] += 1
    f = first / n
    assert np.all(np.abs(f - p) <= 5 * np.sqrt(p * (1 - p) / n) + 1e-4)
    for i in range(6):
        for j in range(6):
            if i == j:
                assert pair[i, j] == 0
                continue
            q = p[i] * p[j] / (1 - p[i])
            assert abs(pair[i, j] / n - q) <= 5 * np.sqrt(q * (1 - q) / n) + 1e-4


# ------------------------------------------------- target verification pass
def _target(L=3, seed=31):
    w = lambda l: {k: synth.f32(v).astype(np.float64)
                   for k, v in synth.target_layer_weights(TINY, seed, l).items()}
    layers = [H.DraftHead(TINY, w(l), np.float64) for l in range(L)]
    hw = {k: synth.f32(v).astype(np.float64) for k, v in synth.head_weights(TINY, 77).items()}
    g = synth.f32(synth.target_final_gain(TINY, seed)).astype(np.float64)
    return layers, hw["emb"], g, hw["lm_head"]


@pytest.mark.parametrize("kind", [T.DYNAMIC, T.STATIC])
def test_target_tree_pass_equals_causal_decoding(kind):
    """Tree attention over L target layers: the logits at every node equal
    plain causal decoding of the node's root path after the context (fp64)."""
    rng = np.random.default_rng(41 if kind == T.DYNAMIC else 42)
    tmpl = C.STATIC_TREE_25 if kind == T.STATIC else ()
    t = _random_tree(rng, kind, 4, 4 if kind == T.STATIC else 3, 9, V=TINY.vocab, template=tmpl)
    f = t.final_tree()
    layers, emb, g, lm = _target()
    n = 6
    ctx = [(rng.standard_normal((n, TINY.n_kv, TINY.head_dim)),
            rng.standard_normal((n, TINY.n_kv, TINY.head_dim))) for _ in layers]
    pos = np.asarray(f["pos"]) - 17 + n          # root at position n
    logits, _ = TG.tree_forward(layers, emb, g, TINY.eps, lm, f["tok"], pos, f["mask"], ctx)
    for u, path in enumerate(_all_root_paths(f["parent"])):
        ref = TG.causal_forward(layers, emb, g, TINY.eps, lm, [f["tok"][w] for w in path], n, ctx)
        np.testing.assert_allclose(logits[u], ref[-1], rtol=1e-10, atol=1e-10)


def test_committed_path_extends_the_cache():
    """After verification, the cache extended by the accepted path's keys and
    values (root first) makes the next token's logits equal causal decoding
    of the whole accepted sequence."""
    rng = np.random.default_rng(43)
    t = _random_tree(rng, T.DYNAMIC, 3, 3, 8, V=TINY.vocab)
    f = t.final_tree()
    layers, emb, g, lm = _target(L=2)
    n = 5
    ctx = [(rng.standard_normal((n, TINY.n_kv, TINY.head_dim)),
            rng.standard_normal((n, TINY.n_kv, TINY.head_dim))) for _ in layers]
    pos = np.asarray(f["pos"]) - 17 + n
    logits, kv_tree = TG.tree_forward(layers, emb, g, TINY.eps, lm, f["tok"], pos, f["mask"], ctx)
    # plant a path of depth 2 in the target's greedy choices
    kid = [v for v in range(len(f["tok"])) if f["parent"][v] == 0][1]
    kid2 = [v for v in range(len(f["tok"])) if f["parent"][v] == kid][0]
    lg = np.array(logits)
    lg[0, f["tok"][kid]] = lg[kid, f["tok"][kid2]] = 1e3
    acc, path, out = VF.verify(f["tok"], f["parent"], lg, 3)
    assert acc >= 2 and list(path[:3]) == [0, kid, kid2]
    com = TG.commit_path(kv_tree, acc, path)
    new_ctx = [(np.concatenate([ck, k]), np.concatenate([cv, v])) for (ck, cv), (k, v) in zip(ctx, com)]
    nxt = int(out[acc])
    one = TG.causal_forward(layers, emb, g, TINY.eps, lm, [nxt], n + acc + 1, new_ctx)
    seq = [f["tok"][w] for w in path[:acc + 1]] + [nxt]
    full = TG.causal_forward(layers, emb, g, TINY.eps, lm, seq, n, ctx)
    np.testing.assert_allclose(one[0], full[-1], rtol=1e-10, atol=1e-10)


def test_eagle3_steady_state_equals_full_causal_recompute():
    """EAGLE-3 steady state: with the first n - tau positions already in the
    cache (their K/V written out here from the definition, position by
    position) and only the newest tau positions ingested, a top-1 chain drafts
    exactly what a full causal recompute of the whole sequence drafts; and it
    equals the round that ingests all n positions."""
    cfg = _round_cfg(T.CHAIN, TINY_E3, B=2, n=(7, 4), gamma=3, top_k=1)
    hd = _head(TINY_E3, np.float64)
    inp = _inputs64(cfg)
    full = run_round(cfg, hd, **inp)
    tau = np.array([3, 1], np.int32)
    cu = np.concatenate([[0], np.cumsum(inp["n"])])
    k_old = np.zeros((cu[-1], TINY_E3.n_kv, TINY_E3.head_dim))
    v_old = np.zeros_like(k_old)
    lmh_new, tok_new = [], []
    for b in range(cfg.B):
        lmh = inp["lmh"][cu[b]:cu[b + 1]]
        tk = inp["ctx_tokens"][cu[b]:cu[b + 1]]
        n_old = len(tk) - tau[b]
        for j in range(n_old):
            x = hd.fuse(lmh[j:j + 1]) + hd.w["emb"][tk[j:j + 1]]
            _, k, v = hd.qkv(x, np.array([j]))
            k_old[cu[b] + j], v_old[cu[b] + j] = k[0], v[0]
        lmh_new.append(lmh[n_old:])
        tok_new.append(tk[n_old:])
    steady = run_round(cfg, hd, n=inp["n"], t_root=inp["t_root"], k_ctx=k_old, v_ctx=v_old,
                       lmh=np.concatenate(lmh_new), ctx_tokens=np.concatenate(tok_new), n_new=tau)
    for s in range(cfg.gamma):
        np.testing.assert_allclose(steady.steps[s].feat, full.steps[s].feat, rtol=1e-10, atol=1e-10)
    for b in range(cfg.B):
        assert list(steady.final[b]["tok"]) == list(full.final[b]["tok"])
        assert list(steady.final[b]["pos"]) == list(full.final[b]["pos"])
        # and the whole chain against a causal recompute from scratch
        lmh = inp["lmh"][cu[b]:cu[b + 1]]
        tk = inp["ctx_tokens"][cu[b]:cu[b + 1]]
        xs = list(hd.fuse(lmh) + hd.w["emb"][tk])
        for s in range(cfg.gamma):
            X = np.stack(xs)
            q, k, v = hd.qkv(X, np.arange(len(xs)))
            a = hd.finish(X[-1:], H.attend(q[-1], k, v, hd.group)[None])[0]
            t = int(np.argmax(hd.lm_head(a[None])[0]))
            assert steady.final[b]["tok"][s + 1] == t
            xs.append(a + hd.w["emb"][t])


def test_eagle1_steady_state_equals_full_ingest():
    """EAGLE-1 steady state: with every context position's K/V produced by
    ingesting (f_{j-1}, t_j), a round that takes the first n - tau positions'
    K/V as given and ingests only the newest tau (at their own positions)
    drafts exactly what the round over the fully ingested context drafts."""
    cfg = _round_cfg(T.DYNAMIC, TINY, B=2, n=(8, 5), gamma=3, top_k=3, top_m=7)
    hd = _head(TINY, np.float64)
    inp = _inputs64(cfg)
    rng = np.random.default_rng(5)
    n = inp["n"]
    cu = np.concatenate([[0], np.cumsum(n)])
    feats = rng.standard_normal((cu[-1], TINY.d))
    toks = rng.integers(0, TINY.vocab, cu[-1])
    k_full = np.zeros((cu[-1], TINY.n_kv, TINY.head_dim))
    v_full = np.zeros_like(k_full)
    for b in range(cfg.B):
        K, V = ingest_features(hd, feats[cu[b]:cu[b + 1]], toks[cu[b]:cu[b + 1]], 0)
        k_full[cu[b]:cu[b + 1]], v_full[cu[b]:cu[b + 1]] = K, V
    full = run_round(cfg, hd, n=n, t_root=inp["t_root"], k_ctx=k_full, v_ctx=v_full,
                     f_root=inp["f_root"])
    tau = np.array([3, 5], np.int32)          # request 1 ingests its whole context
    k_old, v_old = k_full.copy(), v_full.copy()
    sel = np.concatenate([np.arange(cu[b + 1] - tau[b], cu[b + 1]) for b in range(cfg.B)])
    k_old[sel] = 0
    v_old[sel] = 0
    steady = run_round(cfg, hd, n=n, t_root=inp["t_root"], k_ctx=k_old, v_ctx=v_old,
                       f_root=inp["f_root"], lmh=feats[sel], ctx_tokens=toks[sel], n_new=tau)
    for s in range(cfg.gamma):
        np.testing.assert_allclose(steady.steps[s].feat, full.steps[s].feat, rtol=1e-10, atol=1e-10)
        np.testing.assert_array_equal(steady.steps[s].ids, full.steps[s].ids)
    for b in range(cfg.B):
        assert list(steady.final[b]["tok"]) == list(full.final[b]["tok"])


def test_oracle_float32_tracks_float64():
    cfg = C.CONFIGS["c0_tiny_chain"]
    w = synth.head_weights(cfg.head, cfg.seed_w)
    inp = synth.round_inputs(cfg)
    outs = []
    for dt in (np.float32, np.float64):
        hd = H.DraftHead(cfg.head, {k: synth.f32(v) for k, v in w.items()}, dt)
        res = run_round(cfg, hd, n=inp.n, t_root=inp.t_root,
                        k_ctx=synth.f32(inp.k_ctx).astype(dt), v_ctx=synth.f32(inp.v_ctx).astype(dt),
                        f_root=synth.f32(inp.f_root).astype(dt),
                        teacher=(lambda s, r=outs: (r[0].steps[s].ids, r[0].steps[s].conf)) if outs else None)
        outs.append(res)
    for s in range(cfg.gamma):
        a, b = outs[0].steps[s].logits, outs[1].steps[s].logits
        assert np.abs(a - b).max() <= 1e-4 * np.abs(b).max()


def test_norm_precedes_projections():
    """Pre-norm: with eps = 0, RMSNorm makes q, k, v and the MLP branch
    invariant to a positive rescaling of their input."""
    cfg = replace(TINY, eps=0.0)
    hd = _head(cfg, np.float64)
    h = np.random.default_rng(9).standard_normal((3, cfg.d))
    for a, b in zip(hd.qkv(h, np.arange(3)), hd.qkv(7.5 * h, np.arange(3))):
        np.testing.assert_allclose(a, b, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(hd.mlp(h), hd.mlp(7.5 * h), rtol=1e-10, atol=1e-12)
