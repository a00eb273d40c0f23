"""Parity of the HIP path (through the C-ABI) against the CPU oracle.

Protocol
  P1 draft step, teacher-forced: for every checked row the oracle gets the
     GPU's inputs of that step (tokens, positions, masks, parent features and
     ancestor K/V from the GPU's slots) and recomputes the row.  Logits must
     satisfy max|g - o| / max|o| <= 2e-2 per row; top-k ids must match at
     every rank up to which each oracle gap l(i) - l(i+1) exceeds that
     tolerance; confidences agree in the log domain within 2 s (max logit
     error); the fused softmax/top-k must also equal, exactly, the top-k of
     the GPU's own logits.
  P2 tree logic: the oracle's tree code driven by the GPU's (ids, conf) must
     reproduce the GPU's pool, next-step rows and verify tree bit for bit.
  P3 verify: the oracle's verify on the GPU's verify tree and the same target
     logits gives the same accept_len / path / out_tokens, bit for bit, for
     the synthetic logits and for logits with a planted accepted path.
"""
from __future__ import annotations

import numpy as np

from eagle_feature_space_amd import configs as C
from eagle_feature_space_amd import synth
from oracle import sampling as OS
from oracle import target as OTG
from oracle import tree as OT
from oracle import verify as OV
from oracle.head import DraftHead
from oracle.head import attend as o_attend
from oracle.round import ingest, ingest_features, row_forward

TOL = 2e-2          # logits: max relative error (bf16 inputs, fp32 accumulation)
U64 = (1 << 64) - 1


def rel_err(g, o):
    g = np.asarray(g, np.float64)
    o = np.asarray(o, np.float64)
    den = np.max(np.abs(o))
    return float(np.max(np.abs(g - o)) / den) if den > 0 else float(np.max(np.abs(g)))


def _bits(mask):
    m = int(mask) & U64
    return [j for j in range(64) if (m >> j) & 1]


class Case:
    """Seeded weights, inputs and target logits of one configuration."""

    def __init__(self, cfg: C.RoundCfg, with_oracle=True):
        self.cfg = cfg
        self.w = synth.head_weights(cfg.head, cfg.seed_w)
        self.inp = synth.round_inputs(cfg)
        self.target = synth.target_logits(cfg)
        self.head = DraftHead(cfg.head, {k: synth.f32(v) for k, v in self.w.items()}) if with_oracle else None
        self._ctx = None

    def gpu(self, device="cuda:0"):
        from eagle_feature_space_amd.runner import GpuRound
        return GpuRound(self.cfg, self.w, self.inp, device, keep_tree_kv=self.cfg.target_layers > 0)

    def target_dev(self, device="cuda:0", target=None):
        from eagle_feature_space_amd.runner import to_dev
        return to_dev(self.target if target is None else target, device)

    def ctx(self, gr=None):
        """Per-request context K/V (fp32) the attention reads."""
        cu = self.inp.cu_n
        if self.cfg.head.mode == C.MODE_EAGLE3 or self.inp.n_new is not None:
            from eagle_feature_space_amd.runner import to_f32
            K, V = to_f32(gr.k_ctx), to_f32(gr.v_ctx)
        else:
            if self._ctx is None:
                self._ctx = (synth.f32(self.inp.k_ctx), synth.f32(self.inp.v_ctx))
            K, V = self._ctx
        return [(K[cu[b]:cu[b + 1]], V[cu[b]:cu[b + 1]]) for b in range(self.cfg.B)]


# ------------------------------------------------------------------ P1
def check_step(case: Case, gr, snaps, s, rows=None, report=None):
    cfg, hd = case.cfg, case.head
    snap = snaps[s]
    B = cfg.B
    M = len(snap.rows["node"])
    W = M // B
    e3 = cfg.head.mode == C.MODE_EAGLE3
    inp = case.inp
    cu = inp.cu_n
    ctx = case.ctx(gr)
    f_root = synth.f32(inp.f_root) if not e3 else None
    sel = range(M) if rows is None else rows
    worst = dict(logit=0.0, feat=0.0, kv=0.0, ctxkv=0.0, conf=0.0)
    ingested = {}
    if not e3 and s == 0 and inp.n_new is not None:
        # EAGLE-1 steady state: the newest positions' K/V from the target's
        # features, the cached ones untouched
        for b in range(B):
            lo, hi = inp.cu_new[b], inp.cu_new[b + 1]
            n_old = int(inp.n[b]) - int(inp.n_new[b])
            ck, cv = ctx[b]
            old = slice(cu[b], cu[b] + n_old)
            assert np.array_equal(ck[:n_old], synth.f32(inp.k_ctx[old])), f"request {b}: old K changed"
            assert np.array_equal(cv[:n_old], synth.f32(inp.v_ctx[old])), f"request {b}: old V changed"
            K, V = ingest_features(hd, synth.f32(inp.lmh[lo:hi]), inp.ctx_tokens[lo:hi], n_old)
            worst["ctxkv"] = max(worst["ctxkv"], rel_err(ck[n_old:], K), rel_err(cv[n_old:], V))
    for m in sel:
        b = m // W
        pidx = int(snap.rows["pidx"][m])
        tok = int(snap.rows["tok"][m])
        pos = int(snap.rows["pos"][m])
        slot = int(snap.rows["slot"][m])
        mask = int(snap.rows["mask"][m]) & U64
        sl = slot - b * 64
        ck, cv = ctx[b]
        if e3 and s == 0:
            if b not in ingested:
                if inp.n_new is None:
                    lo, hi, n_old = cu[b], cu[b + 1], 0
                else:  # steady state: only the newest n_new[b] positions are ingested
                    lo, hi = inp.cu_new[b], inp.cu_new[b + 1]
                    n_old = int(inp.n[b]) - int(inp.n_new[b])
                    # the cached positions are left exactly as they were
                    old = slice(cu[b], cu[b] + n_old)
                    assert np.array_equal(ck[:n_old], synth.f32(inp.k_ctx[old])), f"request {b}: old K changed"
                    assert np.array_equal(cv[:n_old], synth.f32(inp.v_ctx[old])), f"request {b}: old V changed"
                K, V, hl = ingest(hd, synth.f32(inp.lmh[lo:hi]), inp.ctx_tokens[lo:hi], n_old)
                worst["ctxkv"] = max(worst["ctxkv"], rel_err(ck[n_old:], K), rel_err(cv[n_old:], V))
                ingested[b] = hl
            h = ingested[b]
            q, _, _ = hd.qkv(h[None], np.array([pos]))
            out = hd.finish(h[None], o_attend(q[0], ck, cv, hd.group)[None])[0]
        else:
            if e3:
                h = hd.latent_input(snap.feat_slot[pidx], tok)
            else:
                feat = f_root[b] if s == 0 else snap.feat_slot[pidx]
                h = hd.fc_input(feat[None], np.array([tok]))[0]
            anc = [b * 64 + j for j in _bits(mask) if j != sl]
            out, k, v = row_forward(hd, h, pos, ck, cv, snap.k_slot[anc], snap.v_slot[anc])
            worst["kv"] = max(worst["kv"], rel_err(snap.k_slot[slot], k), rel_err(snap.v_slot[slot], v))
        worst["feat"] = max(worst["feat"], rel_err(snap.feat[m], out))
        lo = hd.lm_head(out[None])[0]
        lg = snap.logits[m]
        e = rel_err(lg, lo)
        worst["logit"] = max(worst["logit"], e)
        assert e <= TOL, f"step {s} row {m}: logit rel err {e:.3g}"
        rk = b * 1024 + int(snap.rows["node"][m])
        _check_topk(cfg, lg, lo, snap.topk_id[m], snap.topk_conf[m], snap.lse[m], s, m, worst, rk)
    assert worst["feat"] <= TOL, worst
    assert worst["kv"] <= TOL, worst
    assert worst["ctxkv"] <= TOL, worst
    if report is not None:
        for k, v in worst.items():
            report[k] = max(report.get(k, 0.0), v)
    return worst


def _check_topk(cfg, lg, lo, ids, conf, lse, s, m, worst, rk=0):
    K = cfg.top_k
    st = cfg.inv_temp
    if cfg.sample_seed is not None:
        _check_sampled(cfg, lg, lo, ids, s, m, rk)
    else:
        # the fused kernel equals the top-k / softmax of the GPU's own logits
        own = np.lexsort((np.arange(lg.size), -lg))[:K]
        assert list(ids) == list(own), f"step {s} row {m}: fused top-k {ids} != top-k of GPU logits {own}"
    z = st * lg.astype(np.float64)
    zmax = z.max()
    ref_lse = zmax + np.log(np.exp(z - zmax).sum())
    assert abs(lse - ref_lse) <= 1e-5 * max(1.0, abs(ref_lse)) + 1e-5, (lse, ref_lse)
    np.testing.assert_allclose(conf, np.exp(z[ids] - ref_lse), rtol=1e-4, atol=1e-12)
    # against the oracle: wherever the gap between the oracle's i-th and
    # (i+1)-th logits exceeds the tolerance, the top-(i+1) id sets are equal
    # (also after a near-tie further up); ids are equal rank by rank up to the
    # first gap that is not clear
    if cfg.sample_seed is None:
        tol = TOL * np.max(np.abs(lo))
        order = np.lexsort((np.arange(lo.size), -lo))
        srt = lo[order]
        clear = True
        for i in range(K):
            gap_clear = bool(srt[i] - srt[i + 1] > tol)
            clear = clear and gap_clear
            if clear:
                assert ids[i] == order[i], f"step {s} row {m} rank {i}: {ids[i]} != {order[i]}"
            if gap_clear:
                assert set(int(x) for x in ids[:i + 1]) == set(int(x) for x in order[:i + 1]), \
                    f"step {s} row {m}: top-{i + 1} id set {sorted(ids[:i + 1])} != {sorted(order[:i + 1])}"
    err = np.max(np.abs(lg.astype(np.float64) - lo))
    zo = st * lo.astype(np.float64)
    lse_o = zo.max() + np.log(np.exp(zo - zo.max()).sum())
    # confidences that underflow fp32 (deep steps of a random-init head can put
    # lower ranks > 100 logits below the top) compare at the floor
    floor = 1e-30
    for i in range(K):
        c_o = np.exp(zo[ids[i]] - lse_o)
        d = abs(np.log(max(float(conf[i]), floor)) - np.log(max(c_o, floor)))
        worst["conf"] = max(worst["conf"], d)
        assert d <= 2 * st * err + 1e-5, f"step {s} row {m}: log-conf diff {d:.3g} > {2 * st * err:.3g}"


def _clear_prefix(keys, ids, tol, what, s, m):
    """ids must follow the key order at every rank up to which each gap
    between consecutive keys exceeds tol (ties by lowest id)."""
    order = np.lexsort((np.arange(keys.size), -keys.astype(np.float64)))
    srt = keys[order].astype(np.float64)
    for i in range(len(ids)):
        if not srt[i] - srt[i + 1] > tol:
            break
        assert ids[i] == order[i], f"step {s} row {m} rank {i} ({what}): {ids[i]} != {order[i]}"


def _check_sampled(cfg, lg, lo, ids, s, m, rk):
    """Gumbel-top-k: the fused ids are the k largest s * logit + G with the
    oracle's Philox noise, on the GPU's own logits (exact but for keys within
    a few fp32 ulps: the two sides' log differ in the last bit) and on the
    oracle's logits wherever the key gaps exceed the logits tolerance."""
    st = cfg.inv_temp
    key_g = OS.gumbel_keys(lg, st, cfg.sample_seed, rk)
    _clear_prefix(key_g, ids, 1e-5 * max(1.0, float(np.max(np.abs(key_g)))), "own logits", s, m)
    key_o = OS.gumbel_keys(lo, st, cfg.sample_seed, rk)
    _clear_prefix(key_o, ids, st * TOL * float(np.max(np.abs(lo))) + 1e-5, "oracle logits", s, m)


# ------------------------------------------------------------------ P2
def check_tree_logic(case: Case, gr, snaps):
    cfg = case.cfg
    B = cfg.B
    e3 = cfg.head.mode == C.MODE_EAGLE3
    n = case.inp.n
    top_k = 1 if cfg.tree == C.TREE_CHAIN else cfg.top_k
    trees = [OT.RequestTree.start(cfg.tree, int(case.inp.t_root[b]),
                                  int(n[b]) - 1 if e3 else int(n[b]), cfg.gamma, top_k,
                                  cfg.top_m, cfg.template, e3) for b in range(B)]
    for s in range(cfg.gamma):
        snap = snaps[s]
        M = len(snap.rows["node"])
        W = M // B
        for b in range(B):
            ort = trees[b].rows()
            assert len(ort) == W
            for i, (u, ps, tok, pos, slot, mask) in enumerate(ort):
                r = b * W + i
                got = (int(snap.rows["node"][r]), int(snap.rows["tok"][r]), int(snap.rows["pos"][r]),
                       int(snap.rows["slot"][r]), int(snap.rows["mask"][r]) & U64)
                assert got == (u, tok, pos, b * 64 + slot, mask), (s, b, i, got, (u, tok, pos, slot, mask))
                if s > 0:
                    assert int(snap.rows["pidx"][r]) == b * 64 + ps
            ids = snap.topk_id[b * W:(b + 1) * W, :cfg.top_k]
            conf = snap.topk_conf[b * W:(b + 1) * W, :cfg.top_k]
            trees[b].expand(s, ids, conf)
    pv = {k: v.cpu().numpy() for k, v in gr.pool_view().items()}
    fv = {k: v.cpu().numpy() for k, v in gr.final_view().items()}
    for b in range(B):
        t = trees[b]
        P = len(t.tok)
        assert int(pv["count"][b]) == P
        assert list(pv["tok"][b, :P]) == t.tok
        assert list(pv["parent"][b, :P]) == t.parent
        assert list(pv["depth"][b, :P]) == t.depth
        assert list(pv["slot"][b, :P]) == t.slot
        np.testing.assert_array_equal(pv["conf"][b, :P], np.array(t.conf, np.float32))
        np.testing.assert_array_equal(pv["value"][b, :P], np.array(t.value, np.float32))
        f = t.final_tree()
        T = len(f["tok"])
        assert int(fv["count"][b]) == T
        for k in ("node", "tok", "parent", "depth", "pos"):
            assert list(fv[k][b, :T]) == list(f[k]), (b, k)
        assert [int(x) & U64 for x in fv["mask"][b, :T]] == [int(x) for x in f["mask"]]
    return trees


# ------------------------------------------------------------------ P3
def check_verify(case: Case, gr, target_np, gamma):
    fv = {k: v.cpu().numpy() for k, v in gr.final_view().items()}
    acc = gr.accept_len.cpu().numpy()
    path = gr.accept_path.cpu().numpy()
    out = gr.out_tokens.cpu().numpy()
    tgt = synth.f32(target_np)
    for b in range(case.cfg.B):
        T = int(fv["count"][b])
        a, p, o = OV.verify(fv["tok"][b, :T], fv["parent"][b, :T], tgt[b, :T], gamma)
        assert int(acc[b]) == a, (b, int(acc[b]), a)
        assert list(path[b]) == list(p), (b, path[b], p)
        assert list(out[b]) == list(o), (b, out[b], o)
    return acc


def planted_target(case: Case, gr, seed=0):
    """Target logits whose greedy choice follows a random root path of the
    GPU's verify tree for a random number of steps (then leaves it)."""
    rng = np.random.default_rng(seed)
    tgt = synth.f32(case.target).copy()
    fv = {k: v.cpu().numpy() for k, v in gr.final_view().items()}
    V = tgt.shape[-1]
    want = []
    for b in range(case.cfg.B):
        T = int(fv["count"][b])
        par, tok = fv["parent"][b, :T], fv["tok"][b, :T]
        u, depth = 0, 0
        goal = int(rng.integers(0, case.cfg.gamma + 1))
        while depth < goal:
            kids = [v for v in range(T) if par[v] == u]
            if not kids:
                break
            v = kids[int(rng.integers(len(kids)))]
            tgt[b, u, tok[v]] = tgt[b, u].max() + 1.0
            u, depth = v, depth + 1
        # at the stopping node pick a token that is not a child
        kid_toks = {int(tok[v]) for v in range(T) if par[v] == u}
        c = int(rng.integers(V))
        while c in kid_toks:
            c = (c + 1) % V
        tgt[b, u, c] = tgt[b, u].max() + 1.0
        want.append(depth)
    if case.cfg.head.dtype == C.DTYPE_BF16:
        return synth.bf16_bits(tgt), want
    return tgt, want


# ------------------------------------------------------------------ P3s: stochastic verify
# Margins: the kernel forms p in fp32 exponentials with fp64 sums, the oracle in
# fp64, so a decision is fixed wherever the uniform sits clear of its threshold:
# relative 1e-5 for an acceptance test (q = p(x) / residual mass), 1.5e-7 of the
# residual mass for the inverse-CDF draw (at most ~1e-7 relative systematic
# error of fp32 exponentials summed over the row).  Inside a margin either
# outcome is valid and the walk follows the GPU.
ACC_MARGIN = 1e-5
CDF_MARGIN = 1.5e-7


def check_verify_sample(case: Case, gr, target_np, draws, inv_temp):
    gamma = case.cfg.gamma
    fv = {k: v.cpu().numpy() for k, v in gr.final_view().items()}
    acc_g = gr.accept_len.cpu().numpy()
    path_g = gr.accept_path.cpu().numpy()
    out_g = gr.out_tokens.cpu().numpy()
    V = target_np.shape[-1]
    stats = dict(tests=0, draws=0, ambiguous=0, accepted=[])
    for b in range(case.cfg.B):
        T = int(fv["count"][b])
        tok, par = fv["tok"][b, :T], fv["parent"][b, :T]
        kids = [[v for v in range(T) if par[v] == u] for u in range(T)]
        a = int(acc_g[b])
        assert 0 <= a <= gamma and path_g[b, 0] == 0, (b, a, path_g[b])
        u = 0
        for depth in range(a + 1):
            p = OV.target_probs(synth.f32(target_np[b, u]), inv_temp)
            resid = p.copy()
            take = int(path_g[b, depth + 1]) if depth < a else -1
            tried = []
            cand = kids[u] if depth < gamma else []
            if take >= 0:
                assert take in cand, (b, depth, take, cand)
            for i, v in enumerate(cand):
                x = int(tok[v])
                q = resid[x] / resid.sum()
                d = float(draws[b, u, i])
                stats["tests"] += 1
                if abs(d - q) > ACC_MARGIN * q + 1e-12:
                    assert (d < q) == (v == take), (b, u, i, d, q, take)
                else:
                    stats["ambiguous"] += 1
                if v == take:
                    break
                resid[x] = 0.0
                tried.append(x)
            if take >= 0:
                assert out_g[b, depth] == tok[take], (b, depth)
                u = take
                continue
            # the walk stopped at u: residual draw by inverse CDF
            x = int(out_g[b, a])
            assert 0 <= x < V and x not in tried and resid[x] > 0, (b, x, tried)
            c = np.cumsum(resid)
            total = c[-1]
            target = float(draws[b, u, OV.N_DRAWS - 1]) * total
            lo_e = c[x - 1] if x > 0 else 0.0
            tol = CDF_MARGIN * total
            assert lo_e - tol <= target < c[x] + tol, (b, x, lo_e, target, c[x])
            stats["draws"] += 1
            if not (target - lo_e > tol and c[x] - target > tol):
                stats["ambiguous"] += 1
        assert all(o == -1 for o in out_g[b, a + 1:]) and all(pp == -1 for pp in path_g[b, a + 1:])
        stats["accepted"].append(a)
    return stats


def planted_sampling_target(case: Case, gr, seed=0):
    """Target logits that give every drafted child a real chance: at each
    node, each child's token gets a logit about log(1.65 |V|) + U(-2, 3), so a
    lone child's target probability lies in ~(0.1, 0.95) against the N(0, 1)
    background."""
    rng = np.random.default_rng(1000 + seed)
    tgt = case.target.copy()          # stored form (bf16 bits or float32)
    bf = tgt.dtype == np.uint16
    fv = {k: v.cpu().numpy() for k, v in gr.final_view().items()}
    V = tgt.shape[-1]
    base = np.log(1.65 * V)
    for b in range(case.cfg.B):
        T = int(fv["count"][b])
        par, tok = fv["parent"][b, :T], fv["tok"][b, :T]
        for v in range(1, T):
            val = np.float32(base + rng.uniform(-2.0, 3.0))
            tgt[b, par[v], tok[v]] = synth.bf16_bits(np.array([val]))[0] if bf else val
    return tgt


def sampling_checks(case: Case, gr, device, seeds=(0, 1, 2), inv_temps=(1.0, 0.7)):
    """P3s on the synthetic target and on planted targets, several draw sets."""
    import torch
    out = dict(tests=0, draws=0, ambiguous=0, accepted=[])
    T = case.target.shape[1]
    for k in seeds:
        draws = synth.verify_draws(case.cfg, T, k)
        dd = torch.from_numpy(draws).to(device)
        tnp = case.target if k == 0 else planted_sampling_target(case, gr, k)
        s_ = inv_temps[k % len(inv_temps)]
        gr.verify_sample(case.target_dev(device, tnp), s_, dd)
        st = check_verify_sample(case, gr, tnp, draws, s_)
        for key in ("tests", "draws", "ambiguous"):
            out[key] += st[key]
        out["accepted"] += st["accepted"]
    return out


# ------------------------------------------------- P3d: verification of sampled drafts
# The kernel's test of the j-th drawn child compares u_j with r_j(x) / q_j(x),
# formed from fp32 exponentials (relative error ~1e-6 for terms far below the
# row maximum) and residual masses C_j summed from fp32 terms: its absolute
# error is within ~4e-6 (p(x) / q_j(x) + thr) (1 + j) / C_j, with C_j the
# residual mass before the test.  The residual draw's cumulative sums carry an
# absolute error of ~2e-6 (1 + k) / C_final in normalised units.  Inside those
# margins either outcome is valid and the walk follows the GPU.
def _draft_rows_of(snaps, B):
    """(request, pool node) -> row of the stacked draft logits, from the row
    descriptors each step recorded before it ran."""
    where = {}
    off = 0
    for sn in snaps:
        nodes = sn.rows["node"]
        W = len(nodes) // B
        for i, nd in enumerate(nodes):
            where[(i // W, int(nd))] = off + i
        off += len(nodes)
    return where


def check_verify_drafted(case: Case, gr, snaps, target_np, draft_np, draws, inv_temp):
    cfg = case.cfg
    gamma, B, s_d = cfg.gamma, cfg.B, cfg.inv_temp
    fv = {k: v.cpu().numpy() for k, v in gr.final_view().items()}
    pv = {k: v.cpu().numpy() for k, v in gr.pool_view().items()}
    where = _draft_rows_of(snaps, B)
    acc_g = gr.accept_len.cpu().numpy()
    path_g = gr.accept_path.cpu().numpy()
    out_g = gr.out_tokens.cpu().numpy()
    V = target_np.shape[-1]
    stats = dict(tests=0, draws=0, ambiguous=0, dropped=0, accepted=[])
    for b in range(B):
        T = int(fv["count"][b])
        fnode = fv["node"][b, :T]
        cnt = int(pv["count"][b])
        ppar, ptok = pv["parent"][b, :cnt], pv["tok"][b, :cnt]
        pos_of = {int(fnode[v]): v for v in range(T)}
        a = int(acc_g[b])
        assert 0 <= a <= gamma and path_g[b, 0] == 0, (b, a, path_g[b])
        u = 0
        for depth in range(a + 1):
            p = OV.target_probs(synth.f32(target_np[b, u]), inv_temp)
            nd = int(fnode[u])
            kids = [(int(ptok[j]), pos_of.get(j, -1)) for j in range(cnt) if ppar[j] == nd] \
                if depth < gamma else []
            if kids:
                row = draft_np[where[(b, nd)]]
                thr, resid, mass = OV.drafted_tests(p, row, s_d, [x for x, _ in kids])
            else:
                row, thr, resid, mass = None, [], p, np.ones(1)
            if depth < a:
                took = [i for i, (_, v) in enumerate(kids) if v == int(path_g[b, depth + 1])]
                assert len(took) == 1, (b, depth, kids, path_g[b])
                i_take = took[0]
            else:
                x_out = int(out_g[b, a])
                took = [i for i, (x, v) in enumerate(kids) if x == x_out and v < 0]
                i_take = took[0] if took else None
            n_test = len(kids) if i_take is None else i_take + 1
            for j in range(n_test):
                x = kids[j][0]
                qj = OV.draft_probs_remaining(row, s_d, [k[0] for k in kids[:j]])[x]
                th = float(thr[j])
                d = float(draws[b, u, j])
                stats["tests"] += 1
                tol = ACC_MARGIN * th + 4e-6 * (p[x] / max(qj, 1e-300) + th) * (1 + j) / max(mass[j], 1e-300)
                if abs(d - th) > tol:
                    assert (d < th) == (j == i_take), (b, u, j, d, th, i_take)
                else:
                    stats["ambiguous"] += 1
            if i_take is not None:
                x, v = kids[i_take]
                assert out_g[b, depth] == x, (b, depth, out_g[b], x)
                if v < 0:
                    assert depth == a, (b, depth, a)
                    stats["dropped"] += 1
                    break
                u = v
                continue
            # the walk stopped at u: residual draw by inverse CDF
            x = int(out_g[b, a])
            tried = [k[0] for k in kids]
            assert 0 <= x < V and x not in tried, (b, x, tried)
            c = np.cumsum(resid)
            total = c[-1]
            stats["draws"] += 1
            if not total > 0:
                assert x == (tried[-1] if tried else 0), (b, x, tried)
                continue
            target = float(draws[b, u, OV.N_DRAWS - 1]) * total
            lo_e = c[x - 1] if x > 0 else 0.0
            tol = CDF_MARGIN * total + 2e-6 * (1 + len(kids)) / max(mass[-1], 1e-300)
            assert lo_e - tol <= target < c[x] + tol, (b, x, lo_e, target, c[x], tol)
            if not (target - lo_e > tol and c[x] - target > tol):
                stats["ambiguous"] += 1
        assert all(o == -1 for o in out_g[b, a + 1:]) and all(pp == -1 for pp in path_g[b, a + 1:])
        stats["accepted"].append(a)
    return stats


def planted_draft(case: Case, gr, snaps, draft_np, seed=0):
    """Draft logits that make the drawn children likely under the draft: at
    each expanded node every drawn child's logit becomes (log |V| + U(0, 2)) / s,
    so each holds a sizeable share of q."""
    rng = np.random.default_rng(2000 + seed)
    out = draft_np.copy()
    pv = {k: v.cpu().numpy() for k, v in gr.pool_view().items()}
    V = out.shape[-1]
    s = case.cfg.inv_temp
    for (b, nd), r in _draft_rows_of(snaps, case.cfg.B).items():
        cnt = int(pv["count"][b])
        for j in range(cnt):
            if pv["parent"][b, j] == nd:
                out[r, pv["tok"][b, j]] = np.float32((np.log(V) + rng.uniform(0.0, 2.0)) / s)
    return out


def drafted_checks(case: Case, gr, snaps, device, inv_temps=(1.0, 0.7, 1.3)):
    """P3d: the drafted verification on the synthetic target with the draft's
    own logits, on a planted target, and on a planted target and draft."""
    import torch
    out = dict(tests=0, draws=0, ambiguous=0, dropped=0, accepted=[])
    T = case.target.shape[1]
    own = gr.draft_logits.cpu().numpy()
    for k in range(3):
        draws = synth.verify_draws(case.cfg, T, 10 + k)
        dd = torch.from_numpy(draws).to(device)
        tnp = case.target if k == 0 else planted_sampling_target(case, gr, k)
        dnp = own if k < 2 else planted_draft(case, gr, snaps, own, k)
        s_ = inv_temps[k]
        gr.verify_sample_drafted(case.target_dev(device, tnp), s_, dd,
                                 draft_logits=None if k < 2 else torch.from_numpy(dnp).to(device))
        st = check_verify_drafted(case, gr, snaps, tnp, dnp, draws, s_)
        for key in ("tests", "draws", "ambiguous", "dropped"):
            out[key] += st[key]
        out["accepted"] += st["accepted"]
    return out


# ------------------------------------------------------------------ P5: target pass
def _target_layers(cfg):
    """Oracle target layers; materialised one at a time at large widths."""
    h = cfg.head
    make = lambda l: DraftHead(h, {k: synth.f32(v) for k, v in
                                   synth.target_layer_weights(h, cfg.seed_tm, l).items()})
    if h.d > 1024:
        return make
    cache = [make(l) for l in range(cfg.target_layers)]
    return lambda l: cache[l]


def check_target_pass(case: Case, gr):
    """The GPU target logits (and every layer's tree K/V) against the oracle's
    tree pass, per request, on the GPU's verify tree (checked bit-exact in P2):
      * teacher-forced, layer by layer (as P1 for the draft step): the oracle's
        layer l on the GPU's rows entering it gives the GPU's rows leaving it,
        and its keys and values, within the plain 2e-2 bar; the oracle's final
        norm and LM head on the GPU's last rows give its logits within 2e-2;
      * free-running from the embeddings: within 2e-2 plus twice the change
        the oracle itself shows when the residual stream is stored in bf16
        (independent roundings add up over the layers)."""
    from eagle_feature_space_amd.runner import to_f32
    cfg, h = case.cfg, case.cfg.head
    fv = {k: v.cpu().numpy() for k, v in gr.final_view().items()}
    logits = gr.t_logits.cpu().numpy()
    kt = to_f32(gr.k_tree) if gr.k_tree is not None else None
    vt = to_f32(gr.v_tree) if gr.v_tree is not None else None
    hid = to_f32(gr.t_hidden) if gr.t_hidden is not None else None
    layers = _target_layers(cfg)
    emb, lm = case.head.w["emb"], case.head.w["lm_head"]
    g = synth.f32(synth.target_final_gain(h, cfg.seed_tm))
    cu = case.inp.cu_n
    ctx_all = [tuple(synth.f32(a) for a in synth.target_context(cfg, l)) for l in range(cfg.target_layers)]
    worst = dict(t_logit=0.0, t_kv=0.0, t_bound=0.0, t_layer_tf=0.0, t_kv_tf=0.0, t_logit_tf=0.0)
    bf = h.dtype == C.DTYPE_BF16
    rnd = (lambda x: synth.bf16_to_f32(synth.bf16_bits(x))) if bf else None
    for b in range(cfg.B):
        T = int(fv["count"][b])
        ctx = [(K[cu[b]:cu[b + 1]], V[cu[b]:cu[b + 1]]) for K, V in ctx_all]
        tok, pos, msk = fv["tok"][b, :T], fv["pos"][b, :T], fv["mask"][b, :T]
        rows = slice(b * gr.layout.positions, b * gr.layout.positions + T)
        if hid is not None:
            assert np.array_equal(hid[0, rows], emb[tok]), f"request {b}: layer-0 rows"
        # every layer materialised once: free-running (fp32, and storing the
        # residual stream in bf16) and teacher-forced on the GPU's rows
        x, xb = emb[tok], emb[tok]
        kv_free = []
        for l in range(cfg.target_layers):
            lay = layers(l)
            x, k, v = OTG.tree_layer(lay, x, pos, msk, ctx[l])
            kv_free.append((k, v))
            if rnd is not None:
                xb, _, _ = OTG.tree_layer(lay, xb, pos, msk, ctx[l], rnd)
                xb = rnd(xb)
            if hid is None:
                continue
            out, k, v = OTG.tree_layer(lay, hid[l, rows], pos, msk, ctx[l])
            for u in range(T):
                e = rel_err(hid[l + 1, rows][u], out[u])
                worst["t_layer_tf"] = max(worst["t_layer_tf"], e)
                assert e <= TOL, f"target layer {l} request {b} position {u}: teacher-forced rel err {e:.3g}"
            if kt is not None:
                e = max(rel_err(kt[l, b, :T], k), rel_err(vt[l, b, :T], v))
                worst["t_kv_tf"] = max(worst["t_kv_tf"], e)
                assert e <= TOL, f"target K/V layer {l} request {b}: teacher-forced rel err {e:.3g}"
        ref = OTG.final_logits(x, g, h.eps, lm)
        # tolerance of the free-running pass: the one-layer bar plus twice
        # what storing the residual stream in the model dtype does to the
        # oracle itself (independent bf16 roundings add up with depth)
        sens = 0.0
        if rnd is not None:
            ref_b = OTG.final_logits(xb, g, h.eps, lm)
            sens = max(rel_err(ref_b[u], ref[u]) for u in range(T))
        tol = TOL + 2.0 * sens
        worst["t_bound"] = max(worst["t_bound"], tol)
        for u in range(T):
            e = rel_err(logits[b, u], ref[u])
            worst["t_logit"] = max(worst["t_logit"], e)
            assert e <= tol, f"target logits request {b} position {u}: rel err {e:.3g} > {tol:.3g}"
        if hid is not None:
            lt = OTG.final_logits(hid[cfg.target_layers, rows], g, h.eps, lm)
            for u in range(T):
                e = rel_err(logits[b, u], lt[u])
                worst["t_logit_tf"] = max(worst["t_logit_tf"], e)
                assert e <= TOL, f"target logits request {b} position {u}: teacher-forced rel err {e:.3g}"
        if kt is not None:
            for l, (k, v) in enumerate(kv_free):
                e = max(rel_err(kt[l, b, :T], k), rel_err(vt[l, b, :T], v))
                worst["t_kv"] = max(worst["t_kv"], e)
                assert e <= tol, f"target K/V layer {l} request {b}: rel err {e:.3g} > {tol:.3g}"
    return worst


def check_commit(case: Case, gr, device):
    """eagle_kv_commit copies exactly the accepted path's rows (root first) of
    the first and last layer, at an offset, and nothing else."""
    import torch
    cfg, h = case.cfg, case.cfg.head
    G = cfg.gamma + 1
    acc = gr.accept_len.cpu().numpy()
    path = gr.accept_path.cpu().numpy()
    dst_row = torch.tensor([b * G + 1 for b in range(cfg.B)], dtype=torch.int32, device=device)
    rows = cfg.B * G + 2
    for l in sorted({0, cfg.target_layers - 1}):
        kd = torch.zeros((rows, h.n_kv, h.head_dim), dtype=gr.dt, device=device)
        vd = torch.zeros_like(kd)
        gr.commit(l, dst_row, kd, vd)
        kd, vd = kd.cpu(), vd.cpu()
        want_k = torch.zeros_like(kd)
        want_v = torch.zeros_like(vd)
        kt, vt = gr.k_tree[l].cpu(), gr.v_tree[l].cpu()
        for b in range(cfg.B):
            for i in range(int(acc[b]) + 1):
                want_k[b * G + 1 + i] = kt[b, int(path[b, i])]
                want_v[b * G + 1 + i] = vt[b, int(path[b, i])]
        assert torch.equal(kd.view(torch.int16) if kd.dtype == torch.bfloat16 else kd,
                           want_k.view(torch.int16) if kd.dtype == torch.bfloat16 else want_k), l
        assert torch.equal(vd.view(torch.int16) if vd.dtype == torch.bfloat16 else vd,
                           want_v.view(torch.int16) if vd.dtype == torch.bfloat16 else want_v), l
    return [int(a) for a in acc]


# ------------------------------------------------------------------ tree attention
def check_tree_attend(case: Case, gr):
    cfg, hd = case.cfg, case.head
    from eagle_feature_space_amd.runner import to_f32
    fv = {k: v.cpu().numpy() for k, v in gr.final_view().items()}
    out = to_f32(gr.attn_out)
    T = gr.layout.positions
    emb = hd.w["emb"]
    ctx = case.ctx(gr)
    worst = 0.0
    for b in range(cfg.B):
        cnt = int(fv["count"][b])
        tok = fv["tok"][b, :cnt]
        pos = fv["pos"][b, :cnt]
        q, k, v = hd.qkv(emb[tok], pos)
        ck, cv = ctx[b]
        for u in range(cnt):
            sel = _bits(fv["mask"][b, u])
            K = np.concatenate([ck, k[sel]])
            V = np.concatenate([cv, v[sel]])
            ref = o_attend(q[u], K, V, hd.group).reshape(-1)
            got = out[b * T + u]
            err = float(np.max(np.abs(got.astype(np.float64) - ref)))
            allowed = TOL * float(np.max(np.abs(ref))) + attn_bf16_bound(q[u], K, V, hd.group)
            assert err <= allowed, (b, u, err, allowed)
            worst = max(worst, err / allowed)
    return worst


def attn_bf16_bound(q, K, V, group):
    """First-order bound on |O_gpu - O| from bf16 storage: rounding q and k
    (relative 2^-9 each) moves a score by at most 2^-8 |q| |k_i| / sqrt(hd);
    softmax turns score shifts d_i into output shifts of at most
    2 max|d_i| max|v|; P and O are rounded to bf16 once more (2^-8 max|v|)."""
    Hq, hd = q.shape
    b = 0.0
    kn = np.linalg.norm(K, axis=-1)              # [L, Hkv]
    for h in range(Hq):
        kv = h // group
        ds = 2.0 ** -8 * np.linalg.norm(q[h]) * kn[:, kv].max() / np.sqrt(hd)
        vmax = float(np.abs(V[:, kv]).max())
        b = max(b, 2 * ds * vmax + 2.0 ** -8 * vmax)
    return b


# ------------------------------------------------------------------ whole round
def full_check(cfg, attend=None, planted=True, rows_per_step=None, device="cuda:0", sampling=True):
    """Run one round on the GPU and check P1 (all or sampled rows), P2, P3."""
    import time

    import torch
    t0 = time.time()

    def say(msg):
        print(f"  [{cfg.name} {time.time() - t0:6.1f}s] {msg}", flush=True)

    case = Case(cfg)
    say("inputs ready")
    gr = case.gpu(device)
    tgt = case.target_dev(device)
    attend = cfg.tree == C.TREE_DYNAMIC if attend is None else attend
    snaps = gr.run(target=tgt, snapshots=True, attend=attend)
    torch.cuda.synchronize()
    say("GPU round done")
    # every row, every step: confidences are probabilities, so path values
    # never grow and the kept set stays ancestor-closed
    for s, sn in enumerate(snaps):
        over = np.argwhere(sn.topk_conf > 1.0)
        assert over.size == 0, f"step {s}: confidence above 1 at (row, rank) {over[:4].tolist()}"
    report = {}
    for s in range(cfg.gamma):
        rows = None
        if rows_per_step is not None:
            M = len(snaps[s].rows["node"])
            rows = sorted(set(np.linspace(0, M - 1, min(M, rows_per_step)).astype(int).tolist()))
        check_step(case, gr, snaps, s, rows=rows, report=report)
        say(f"step {s} checked")
    check_tree_logic(case, gr, snaps)
    if cfg.target_layers > 0:
        report.update(check_target_pass(case, gr))
        say("target pass checked")
        check_verify(case, gr, gr.t_logits.cpu().numpy(), cfg.gamma)
    else:
        check_verify(case, gr, case.target, cfg.gamma)
    if attend:
        report["attend"] = check_tree_attend(case, gr)
    if planted:
        pt, want = planted_target(case, gr)
        gr.verify(case.target_dev(device, pt))
        acc = check_verify(case, gr, pt, cfg.gamma)
        assert list(acc) == want, (list(acc), want)
        report["planted_accept"] = list(map(int, acc))
        if cfg.target_layers > 0:
            report["committed"] = check_commit(case, gr, device)
    if sampling:
        st = sampling_checks(case, gr, device)
        say(f"stochastic verify checked: {st['tests']} tests, {st['draws']} draws, "
            f"{st['ambiguous']} inside a margin")
        report["sample_accept_hist"] = np.bincount(st["accepted"], minlength=cfg.gamma + 1).tolist()
        report["sample_ambiguous"] = st["ambiguous"]
        if cfg.sample_seed is not None:
            st = drafted_checks(case, gr, snaps, device)
            say(f"drafted verify checked: {st['tests']} tests, {st['draws']} draws, "
                f"{st['dropped']} dropped children kept, {st['ambiguous']} inside a margin")
            report["drafted_accept_hist"] = np.bincount(st["accepted"],
                                                        minlength=cfg.gamma + 1).tolist()
            report["drafted_ambiguous"] = st["ambiguous"]
            report["drafted_dropped_kept"] = st["dropped"]
    torch.cuda.synchronize()
    return report


def smoke_round():
    """Tiny fp32 chain on cuda:0, fully checked against the oracle."""
    import torch
    assert torch.cuda.is_available(), "smoke needs a GPU"
    rep = full_check(C.CONFIGS["c0_tiny_chain"])
    print("smoke c0_tiny_chain ok:", {k: (round(v, 6) if isinstance(v, float) else v) for k, v in rep.items()})
