"""Device-side setup of one draft-and-verify round through the C-ABI.

Uploads a head's weights and a round's inputs into torch device tensors, fills
the C structs and calls the library entry points in order:
  eagle_tree_init, then per step eagle_draft_step + eagle_tree_expand_rerank,
  optionally eagle_tree_attend, then eagle_tree_verify.
All arithmetic of the round happens in libeagle's kernels.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass, field
from typing import Dict, List, Optional

import numpy as np
import torch

from . import binding as E
from . import synth
from .configs import DTYPE_BF16, MODE_EAGLE3, TREE_STATIC, RoundCfg


def to_dev(a: np.ndarray, device) -> torch.Tensor:
    """numpy (bf16 bits as uint16, float32 or int32) -> device tensor."""
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def to_f32(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy()


@dataclass
class StepSnapshot:
    rows: Dict[str, np.ndarray]        # this step's row descriptors
    topk_id: np.ndarray
    topk_conf: np.ndarray
    lse: np.ndarray
    logits: Optional[np.ndarray] = None
    feat: Optional[np.ndarray] = None
    feat_slot: Optional[np.ndarray] = None   # after the step (fp32)
    k_slot: Optional[np.ndarray] = None
    v_slot: Optional[np.ndarray] = None


class GpuRound:
    def __init__(self, cfg: RoundCfg, weights: Dict[str, np.ndarray], inputs, device="cuda:0",
                 keep_tree_kv=False):
        self.cfg = cfg
        h = cfg.head
        self.dev = torch.device(device)
        self.dt = torch.bfloat16 if h.dtype == DTYPE_BF16 else torch.float32
        self.w = {k: to_dev(v, self.dev) for k, v in weights.items()}
        hd = E.eagle_head()
        for f in ("d", "vocab", "ffn", "act", "norm", "dtype", "mode", "eps", "rope_theta"):
            setattr(hd, f, getattr(h, f))
        hd.n_q_heads, hd.n_kv_heads, hd.head_dim = h.n_q, h.n_kv, h.head_dim
        for k, t in self.w.items():
            setattr(hd, k, t.data_ptr())
        self.head = hd

        B = cfg.B
        self.n = to_dev(inputs.n.astype(np.int32), self.dev)
        self.cu_n = to_dev(inputs.cu_n.astype(np.int32), self.dev)
        total = int(inputs.cu_n[-1])
        steady = inputs.n_new is not None
        if h.mode == MODE_EAGLE3:
            if steady:  # the old positions' K/V are already cached
                self.k_ctx = to_dev(inputs.k_ctx, self.dev)
                self.v_ctx = to_dev(inputs.v_ctx, self.dev)
            else:
                self.k_ctx = torch.zeros((max(total, 1), h.n_kv, h.head_dim), dtype=self.dt, device=self.dev)
                self.v_ctx = torch.zeros_like(self.k_ctx)
            self.lmh = to_dev(inputs.lmh, self.dev)
            self.ctx_tokens = to_dev(inputs.ctx_tokens.astype(np.int32), self.dev)
            self.f_root = None
        else:
            self.k_ctx = to_dev(inputs.k_ctx, self.dev) if total else None
            self.v_ctx = to_dev(inputs.v_ctx, self.dev) if total else None
            self.f_root = to_dev(inputs.f_root, self.dev)
            self.lmh = self.ctx_tokens = None
            if steady:   # the target's features and tokens of the new positions
                self.lmh = to_dev(inputs.lmh, self.dev)
                self.ctx_tokens = to_dev(inputs.ctx_tokens.astype(np.int32), self.dev)
        self.k_slot = torch.zeros((B * E.MAX_SLOTS, h.n_kv, h.head_dim), dtype=self.dt, device=self.dev)
        self.v_slot = torch.zeros_like(self.k_slot)
        self.feat_slot = torch.zeros((B * E.MAX_SLOTS, h.d), dtype=self.dt, device=self.dev)
        kv = E.eagle_kv()
        kv.B, kv.max_n, kv.total_n = B, int(inputs.n.max()), total
        kv.n, kv.cu_n = self.n.data_ptr(), self.cu_n.data_ptr()
        kv.k_ctx = self.k_ctx.data_ptr() if self.k_ctx is not None else None
        kv.v_ctx = self.v_ctx.data_ptr() if self.v_ctx is not None else None
        kv.k_slot, kv.v_slot = self.k_slot.data_ptr(), self.v_slot.data_ptr()
        kv.feat_slot = self.feat_slot.data_ptr()
        if steady:
            self.n_new = to_dev(inputs.n_new.astype(np.int32), self.dev)
            self.cu_new = to_dev(inputs.cu_new.astype(np.int32), self.dev)
            kv.total_new = int(inputs.cu_new[-1])
            kv.n_new, kv.cu_new = self.n_new.data_ptr(), self.cu_new.data_ptr()
        self.kv = kv

        tr = E.eagle_tree()
        tr.kind, tr.B, tr.gamma, tr.top_k, tr.top_m = cfg.tree, B, cfg.gamma, cfg.top_k, cfg.top_m
        self._tmpl = (ctypes.c_int32 * max(1, len(cfg.template)))(*cfg.template)
        tr.n_template = len(cfg.template) if cfg.tree == TREE_STATIC else 0
        tr.template_parent = ctypes.cast(self._tmpl, ctypes.POINTER(ctypes.c_int32))
        tr.inv_temp = cfg.inv_temp
        if cfg.sample_seed is not None:
            tr.sample, tr.sample_seed = 1, cfg.sample_seed
        nbytes = E.eagle_tree_state_bytes(tr)
        if nbytes == 0:
            raise E.EagleError(E.EAGLE_EINVAL, "eagle_tree_state_bytes")
        self.state = torch.zeros(nbytes, dtype=torch.uint8, device=self.dev)
        tr.state, tr.state_bytes = self.state.data_ptr(), nbytes
        self.tree = tr
        self.layout = E.eagle_tree_layout_of(tr)
        wsb = E.eagle_workspace_bytes(hd, kv, tr)
        if wsb == 0:
            raise E.EagleError(E.EAGLE_EINVAL, "eagle_workspace_bytes")
        self.ws = torch.empty(wsb, dtype=torch.uint8, device=self.dev)
        self.root_tok = to_dev(inputs.t_root.astype(np.int32), self.dev)
        self.rows = [E.eagle_step_rows(tr, s) for s in range(cfg.gamma)]
        P = self.layout.positions
        self.accept_len = torch.zeros(B, dtype=torch.int32, device=self.dev)
        self.accept_path = torch.zeros((B, cfg.gamma + 1), dtype=torch.int32, device=self.dev)
        self.out_tokens = torch.zeros((B, cfg.gamma + 1), dtype=torch.int32, device=self.dev)
        self.attn_out = None
        self.target = None
        self.noalloc = False      # draft steps through eagle_draft_step_noalloc
        self.draft_logits = None  # sampled drafting: every step's logits, for verification
        if cfg.target_layers > 0:
            self._build_target(keep_tree_kv)

    def _build_target(self, keep_tree_kv):
        """Random-init target layers (the head's layer shape, sharing its
        embedding and LM head) and their context caches, one layer at a time."""
        cfg, h = self.cfg, self.cfg.head
        L = cfg.target_layers
        self.t_w, self.t_ctx = [], []
        layers = (E.eagle_layer * L)()
        for l in range(L):
            w = {k: to_dev(v, self.dev) for k, v in synth.target_layer_weights(h, cfg.seed_tm, l).items()}
            kc, vc = (to_dev(a, self.dev) for a in synth.target_context(cfg, l))
            self.t_w.append(w)
            self.t_ctx.append((kc, vc))
            for k, t in w.items():
                setattr(layers[l], k, t.data_ptr())
            layers[l].k_ctx, layers[l].v_ctx = kc.data_ptr(), vc.data_ptr()
        self.t_final = to_dev(synth.target_final_gain(h, cfg.seed_tm), self.dev)
        tg = E.eagle_target()
        tg.n_layers, tg.layers, tg.final_norm_g = L, layers, self.t_final.data_ptr()
        self._t_layers = layers
        self.target = tg
        P = self.layout.positions
        self.t_logits = torch.empty((cfg.B, P, h.vocab), dtype=torch.float32, device=self.dev)
        self.k_tree = self.v_tree = None
        self.t_hidden = None
        if keep_tree_kv:
            self.t_hidden = torch.zeros((L + 1, cfg.B * P, h.d), dtype=self.dt, device=self.dev)
            self.k_tree = torch.zeros((L, cfg.B, E.MAX_SLOTS, h.n_kv, h.head_dim), dtype=self.dt,
                                      device=self.dev)
            self.v_tree = torch.zeros_like(self.k_tree)
        wsb = E.eagle_target_workspace_bytes(self.head, tg, self.kv, self.tree)
        if wsb == 0:
            raise E.EagleError(E.EAGLE_EINVAL, "eagle_target_workspace_bytes")
        if wsb > self.ws.numel():
            self.ws = torch.empty(wsb, dtype=torch.uint8, device=self.dev)

    def target_logits(self, stream=None):
        """The target's pass over the verify tree -> fp32 logits [B, positions, |V|]
        (with keep_hidden, every layer boundary's rows go to self.t_hidden)."""
        E.eagle_target_verify_logits(self.head, self.target, self.kv, self.tree, self.t_logits,
                                     self.k_tree, self.v_tree, self.ws, self.ws.numel(), stream,
                                     hidden_out=self.t_hidden)
        return self.t_logits

    def commit(self, layer, dst_row, k_dst, v_dst, stream=None):
        """Append the accepted path's K/V of target layer `layer` to (k_dst, v_dst)."""
        h = self.cfg.head
        kt, vt = self.k_tree[layer], self.v_tree[layer]
        E.eagle_kv_commit(self.tree, h.n_kv, h.head_dim, 0 if self.dt == torch.bfloat16 else 1,
                          self.accept_len, self.accept_path, kt, vt, dst_row, k_dst.shape[0],
                          k_dst, v_dst, stream)

    # ------------------------------------------------------------ state views
    def view(self, name, dtype, shape):
        off = getattr(self.layout, name)
        nb = int(np.prod(shape)) * torch.tensor([], dtype=dtype).element_size()
        return self.state[off:off + nb].view(dtype).view(*shape)

    def rows_view(self, step):
        """Row descriptors of draft step `step` (double buffer by parity)."""
        B = self.cfg.B
        R = B * self.layout.max_rows
        M = B * self.rows[step]
        h = (step % 2) * R
        out = {}
        for k, dt in (("node", torch.int32), ("tok", torch.int32), ("pos", torch.int32),
                      ("slot", torch.int32), ("pidx", torch.int32), ("mask", torch.int64)):
            out[k] = self.view("row_" + k, dt, (2 * R,))[h:h + M]
        return out

    def final_view(self):
        B = self.cfg.B
        fv = {k: self.view("f_" + k, torch.int32, (B, E.MAX_POSITIONS))
              for k in ("node", "tok", "parent", "depth", "pos")}
        fv["mask"] = self.view("f_mask", torch.int64, (B, E.MAX_POSITIONS))
        fv["count"] = self.view("f_count", torch.int32, (B,))
        return fv

    def pool_view(self):
        B, P = self.cfg.B, self.layout.pool_cap
        pv = {k: self.view("pool_" + k, torch.int32, (B, P)) for k in ("tok", "parent", "depth", "slot")}
        pv["conf"] = self.view("pool_conf", torch.float32, (B, P))
        pv["value"] = self.view("pool_value", torch.float32, (B, P))
        pv["count"] = self.view("pool_count", torch.int32, (B,))
        return pv

    # ------------------------------------------------------------ round
    def init(self, stream=None):
        E.eagle_tree_init(self.head, self.kv, self.tree, self.root_tok, stream)

    def step(self, s, logits_out=None, feat_out=None, stream=None):
        if self.noalloc:
            E.eagle_draft_step_noalloc(self.head, self.kv, self.tree, s, f_root=self.f_root,
                                       lmh=self.lmh, ctx_tokens=self.ctx_tokens,
                                       logits_out=logits_out, feat_out=feat_out, stream=stream)
            return
        E.eagle_draft_step(self.head, self.kv, self.tree, s, f_root=self.f_root, lmh=self.lmh,
                           ctx_tokens=self.ctx_tokens, logits_out=logits_out, feat_out=feat_out,
                           ws=self.ws, stream=stream)

    def expand(self, s, stream=None):
        E.eagle_tree_expand_rerank(self.tree, s, stream)

    def attend(self, stream=None):
        h = self.cfg.head
        if self.attn_out is None:
            self.attn_out = torch.zeros((self.cfg.B * self.layout.positions, h.q_dim),
                                        dtype=self.dt, device=self.dev)
        E.eagle_tree_attend(self.head, self.kv, self.tree, self.attn_out, self.ws, stream=stream)

    def verify(self, target: torch.Tensor, stream=None):
        dtype = 0 if target.dtype == torch.bfloat16 else 1
        E.eagle_tree_verify(self.tree, target, target.shape[1], target.shape[2], dtype,
                            self.accept_len, self.accept_path, self.out_tokens, stream)

    def verify_sample(self, target: torch.Tensor, inv_temp: float, draws: torch.Tensor, stream=None):
        """Stochastic (lossless) verification; draws [B, positions, 17] fp32 on the device."""
        dtype = 0 if target.dtype == torch.bfloat16 else 1
        assert draws.dtype == torch.float32 and draws.is_contiguous()
        assert tuple(draws.shape) == (self.cfg.B, target.shape[1], E.VERIFY_DRAWS)
        E.eagle_tree_verify_sample(self.tree, target, target.shape[1], target.shape[2], dtype,
                                   inv_temp, draws, self.accept_len, self.accept_path,
                                   self.out_tokens, stream)

    def step_logits(self, s):
        """Step s's block of the draft-logits buffer: fp32 [B * rows_s, V], the
        blocks of steps 0 .. gamma-1 one after another (allocated on first use)."""
        B, V = self.cfg.B, self.cfg.head.vocab
        if self.draft_logits is None:
            self.draft_logits = torch.empty((B * sum(self.rows), V), dtype=torch.float32,
                                            device=self.dev)
        off = B * sum(self.rows[:s])
        return self.draft_logits[off:off + B * self.rows[s]]

    def verify_sample_drafted(self, target: torch.Tensor, inv_temp: float, draws: torch.Tensor,
                              stream=None, draft_logits=None):
        """Lossless verification of a sampled draft, with the draft's
        probabilities from the logits every step kept (run() keeps them), or
        from `draft_logits` of the same layout."""
        dtype = 0 if target.dtype == torch.bfloat16 else 1
        dl = self.draft_logits if draft_logits is None else draft_logits
        assert dl is not None, "no draft logits kept"
        assert dl.dtype == torch.float32 and dl.is_contiguous()
        assert tuple(dl.shape) == (self.cfg.B * sum(self.rows), self.cfg.head.vocab)
        assert draws.dtype == torch.float32 and draws.is_contiguous()
        assert tuple(draws.shape) == (self.cfg.B, target.shape[1], E.VERIFY_DRAWS)
        E.eagle_tree_verify_sample_drafted(self.tree, target, target.shape[1], target.shape[2],
                                           dtype, inv_temp, dl, draws,
                                           self.accept_len, self.accept_path, self.out_tokens,
                                           stream)

    def run(self, target=None, snapshots=False, attend=False, sample=None) -> List[StepSnapshot]:
        """One round; with snapshots=True the state after every draft step is
        copied to the host (for parity checks; synchronises).  sample =
        (inv_temp, draws) verifies by speculative sampling instead of greedily
        (with the draft's probabilities when drafting samples)."""
        cfg = self.cfg
        snaps = []
        keep = self.tree.sample == 1
        self.init()
        for s in range(cfg.gamma):
            M = cfg.B * self.rows[s]
            logits = self.step_logits(s) if keep else None
            feat = None
            if snapshots:
                rows = {k: v.cpu().numpy() for k, v in self.rows_view(s).items()}
                if logits is None:
                    logits = torch.empty((M, cfg.head.vocab), dtype=torch.float32, device=self.dev)
                feat = torch.empty((M, cfg.head.d), dtype=self.dt, device=self.dev)
            self.step(s, logits_out=logits, feat_out=feat)
            if snapshots:
                K = cfg.top_k
                snaps.append(StepSnapshot(
                    rows=rows,
                    topk_id=self.view("topk_id", torch.int32, (M, K)).cpu().numpy(),
                    topk_conf=self.view("topk_conf", torch.float32, (M, K)).cpu().numpy(),
                    lse=self.view("lse", torch.float32, (M,)).cpu().numpy(),
                    logits=logits.cpu().numpy(), feat=to_f32(feat),
                    feat_slot=to_f32(self.feat_slot), k_slot=to_f32(self.k_slot),
                    v_slot=to_f32(self.v_slot)))
            self.expand(s)
        if attend:
            self.attend()
        if self.target is not None:
            target = self.target_logits()
        if target is not None:
            if sample is None:
                self.verify(target)
            elif keep:
                self.verify_sample_drafted(target, *sample)
            else:
                self.verify_sample(target, *sample)
        return snaps
