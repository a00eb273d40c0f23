"""ctypes binding of libeagle.so (include/eagle.h).  Argument marshalling only:
every step of the draft-and-verify round runs in the library's HIP kernels.

Functions keep the C names.  Device buffers are torch tensors (their
data_ptr() is passed); `stream` defaults to torch's current HIP stream.
Loading fails loudly when the library has not been built.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libeagle.so")

c_int32, c_int64, c_float, c_size_t, c_void_p = (ctypes.c_int32, ctypes.c_int64,
                                                 ctypes.c_float, ctypes.c_size_t,
                                                 ctypes.c_void_p)

EAGLE_OK, EAGLE_EINVAL, EAGLE_EUNSUPPORTED, EAGLE_ECAPACITY, EAGLE_EHIP = 0, -1, -2, -3, -4
MAX_SLOTS = 64
MAX_POSITIONS = 64
VERIFY_DRAWS = 17
NOALLOC_SCRATCH_BYTES = 32 << 20   # EAGLE_NOALLOC_SCRATCH_BYTES


class eagle_head(ctypes.Structure):
    _fields_ = [(n, c_int32) for n in ("d", "vocab", "n_q_heads", "n_kv_heads", "head_dim", "ffn",
                                       "act", "norm", "dtype", "mode")] + \
               [("eps", c_float), ("rope_theta", c_float)] + \
               [(n, c_void_p) for n in ("w_fc", "w_fuse", "w_q", "w_k", "w_v", "w_o", "w_gate",
                                        "w_up", "w_down", "norm1_g", "norm1_b", "norm2_g",
                                        "norm2_b", "emb", "lm_head")]


class eagle_kv(ctypes.Structure):
    _fields_ = [("B", c_int32), ("max_n", c_int32), ("total_n", c_int64),
                ("n", c_void_p), ("cu_n", c_void_p), ("k_ctx", c_void_p), ("v_ctx", c_void_p),
                ("k_slot", c_void_p), ("v_slot", c_void_p), ("feat_slot", c_void_p),
                ("total_new", c_int64), ("n_new", c_void_p), ("cu_new", c_void_p)]


class eagle_layer(ctypes.Structure):
    _fields_ = [(n, c_void_p) for n in ("w_q", "w_k", "w_v", "w_o", "w_gate", "w_up", "w_down",
                                        "norm1_g", "norm1_b", "norm2_g", "norm2_b", "k_ctx",
                                        "v_ctx")]


class eagle_target(ctypes.Structure):
    _fields_ = [("n_layers", c_int32), ("layers", ctypes.POINTER(eagle_layer)),
                ("final_norm_g", c_void_p)]


class eagle_tree(ctypes.Structure):
    _fields_ = [("kind", c_int32), ("B", c_int32), ("gamma", c_int32), ("top_k", c_int32),
                ("top_m", c_int32), ("n_template", c_int32),
                ("template_parent", ctypes.POINTER(c_int32)), ("inv_temp", c_float),
                ("state", c_void_p), ("state_bytes", c_size_t),
                ("sample_seed", ctypes.c_uint64), ("sample", c_int32)]


_LAYOUT_FIELDS = ("pool_tok", "pool_parent", "pool_depth", "pool_slot", "pool_conf", "pool_value",
                  "pool_count", "slot_count", "root_pos", "slot_mask",
                  "row_node", "row_tok", "row_pos", "row_slot", "row_pidx", "row_mask",
                  "topk_id", "topk_conf", "lse",
                  "f_node", "f_tok", "f_parent", "f_depth", "f_pos", "f_mask", "f_count",
                  "choice", "choice_part", "status", "total")


class eagle_tree_layout(ctypes.Structure):
    _fields_ = [("pool_cap", c_int32), ("max_rows", c_int32), ("positions", c_int32)] + \
               [(n, c_size_t) for n in _LAYOUT_FIELDS]


_lib = None


def lib():
    """The loaded libeagle.so (raises if it was never built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m eagle_feature_space_amd.build` (there is no fallback)")
    L = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER
    sig = {
        "eagle_version": ([], ctypes.c_char_p),
        "eagle_strerror": ([ctypes.c_int], ctypes.c_char_p),
        "eagle_tree_layout_of": ([P(eagle_tree), P(eagle_tree_layout)], ctypes.c_int),
        "eagle_tree_state_bytes": ([P(eagle_tree)], c_size_t),
        "eagle_step_rows": ([P(eagle_tree), ctypes.c_int], ctypes.c_int),
        "eagle_workspace_bytes": ([P(eagle_head), P(eagle_kv), P(eagle_tree)], c_size_t),
        "eagle_tree_init": ([P(eagle_head), P(eagle_kv), P(eagle_tree), c_void_p, c_void_p],
                            ctypes.c_int),
        "eagle_draft_step": ([P(eagle_head), P(eagle_kv), P(eagle_tree), ctypes.c_int, c_void_p,
                              c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_size_t,
                              c_void_p], ctypes.c_int),
        "eagle_draft_step_noalloc": ([P(eagle_head), P(eagle_kv), P(eagle_tree), ctypes.c_int,
                                      c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p],
                                     ctypes.c_int),
        "eagle_tree_expand_rerank": ([P(eagle_tree), ctypes.c_int, c_void_p], ctypes.c_int),
        "eagle_tree_attend": ([P(eagle_head), P(eagle_kv), P(eagle_tree), c_void_p, c_void_p,
                               c_size_t, c_void_p], ctypes.c_int),
        "eagle_tree_verify": ([P(eagle_tree), c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                               c_void_p, c_void_p, c_void_p, c_void_p], ctypes.c_int),
        "eagle_tree_verify_sample": ([P(eagle_tree), c_void_p, ctypes.c_int, ctypes.c_int,
                                      ctypes.c_int, ctypes.c_float, c_void_p, c_void_p, c_void_p,
                                      c_void_p, c_void_p], ctypes.c_int),
        "eagle_tree_verify_sample_drafted": ([P(eagle_tree), c_void_p, ctypes.c_int, ctypes.c_int,
                                              ctypes.c_int, ctypes.c_float, c_void_p, c_void_p,
                                              c_void_p, c_void_p, c_void_p, c_void_p], ctypes.c_int),
        "eagle_target_verify_logits": ([P(eagle_head), P(eagle_target), P(eagle_kv), P(eagle_tree),
                                        c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_size_t,
                                        c_void_p], ctypes.c_int),
        "eagle_target_workspace_bytes": ([P(eagle_head), P(eagle_target), P(eagle_kv),
                                          P(eagle_tree)], c_size_t),
        "eagle_kv_commit": ([P(eagle_tree), ctypes.c_int, ctypes.c_int, ctypes.c_int, c_void_p,
                             c_void_p, c_void_p, c_void_p, c_void_p, c_int64, c_void_p, c_void_p,
                             c_void_p], ctypes.c_int),
        "eagle_profile_enable": ([ctypes.c_int], ctypes.c_int),
        "eagle_profile_reset": ([], ctypes.c_int),
        "eagle_profile_read": ([ctypes.c_int, P(c_int64), P(c_int64), P(ctypes.c_double),
                                P(ctypes.c_double), P(ctypes.c_double), P(ctypes.c_double)],
                               ctypes.c_int),
    }
    for name, (args, res) in sig.items():
        f = getattr(L, name)
        f.argtypes = args
        f.restype = res
    _lib = L
    return L


EXPORTED = ("eagle_version", "eagle_strerror", "eagle_tree_layout_of", "eagle_tree_state_bytes",
            "eagle_step_rows", "eagle_workspace_bytes", "eagle_tree_init", "eagle_draft_step",
            "eagle_draft_step_noalloc",
            "eagle_tree_expand_rerank", "eagle_tree_attend", "eagle_tree_verify",
            "eagle_tree_verify_sample", "eagle_tree_verify_sample_drafted",
            "eagle_target_verify_logits",
            "eagle_target_workspace_bytes", "eagle_kv_commit",
            "eagle_profile_enable", "eagle_profile_reset", "eagle_profile_read")

PROF_FAMILIES = {"lmhead": 0, "gemm": 1, "attn": 2, "verify": 3, "other": 4}


class EagleError(RuntimeError):
    def __init__(self, status, where):
        super().__init__(f"{where}: {lib().eagle_strerror(status).decode()} ({status})")
        self.status = status


def _ptr(t):
    return None if t is None else (t if isinstance(t, int) else t.data_ptr())


def _stream(stream):
    if stream is not None:
        return stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _check(status, where):
    if status != EAGLE_OK:
        raise EagleError(status, where)
    return status


# ------------------------------------------------------------------ calls
def eagle_version():
    return lib().eagle_version().decode()


def eagle_tree_layout_of(tree):
    out = eagle_tree_layout()
    _check(lib().eagle_tree_layout_of(ctypes.byref(tree), ctypes.byref(out)), "eagle_tree_layout_of")
    return out


def eagle_tree_state_bytes(tree):
    return lib().eagle_tree_state_bytes(ctypes.byref(tree))


def eagle_step_rows(tree, step):
    return lib().eagle_step_rows(ctypes.byref(tree), step)


def eagle_workspace_bytes(head, kv, tree):
    return lib().eagle_workspace_bytes(ctypes.byref(head), ctypes.byref(kv), ctypes.byref(tree))


def eagle_tree_init(head, kv, tree, root_tokens, stream=None):
    return _check(lib().eagle_tree_init(ctypes.byref(head), ctypes.byref(kv), ctypes.byref(tree),
                                        _ptr(root_tokens), _stream(stream)), "eagle_tree_init")


def eagle_draft_step(head, kv, tree, step, f_root=None, lmh=None, ctx_tokens=None,
                     logits_out=None, feat_out=None, ws=None, ws_bytes=None, stream=None):
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size()
    return _check(lib().eagle_draft_step(
        ctypes.byref(head), ctypes.byref(kv), ctypes.byref(tree), step, _ptr(f_root), _ptr(lmh),
        _ptr(ctx_tokens), _ptr(logits_out), _ptr(feat_out), _ptr(ws), ws_bytes,
        _stream(stream)), f"eagle_draft_step({step})")


def eagle_draft_step_noalloc(head, kv, tree, step, f_root=None, lmh=None, ctx_tokens=None,
                             logits_out=None, feat_out=None, stream=None):
    return _check(lib().eagle_draft_step_noalloc(
        ctypes.byref(head), ctypes.byref(kv), ctypes.byref(tree), step, _ptr(f_root), _ptr(lmh),
        _ptr(ctx_tokens), _ptr(logits_out), _ptr(feat_out), _stream(stream)),
        f"eagle_draft_step_noalloc({step})")


def eagle_tree_expand_rerank(tree, step, stream=None):
    return _check(lib().eagle_tree_expand_rerank(ctypes.byref(tree), step, _stream(stream)),
                  f"eagle_tree_expand_rerank({step})")


def eagle_tree_attend(head, kv, tree, out, ws, ws_bytes=None, stream=None):
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size()
    return _check(lib().eagle_tree_attend(ctypes.byref(head), ctypes.byref(kv), ctypes.byref(tree),
                                          _ptr(out), _ptr(ws), ws_bytes, _stream(stream)),
                  "eagle_tree_attend")


def eagle_tree_verify(tree, target_logits, positions, vocab, dtype, accept_len, accept_path,
                      out_tokens, stream=None):
    return _check(lib().eagle_tree_verify(ctypes.byref(tree), _ptr(target_logits), positions, vocab,
                                          dtype, _ptr(accept_len), _ptr(accept_path),
                                          _ptr(out_tokens), _stream(stream)), "eagle_tree_verify")


def eagle_tree_verify_sample(tree, target_logits, positions, vocab, dtype, inv_temp, draws,
                             accept_len, accept_path, out_tokens, stream=None):
    return _check(lib().eagle_tree_verify_sample(ctypes.byref(tree), _ptr(target_logits), positions,
                                                 vocab, dtype, inv_temp, _ptr(draws), _ptr(accept_len),
                                                 _ptr(accept_path), _ptr(out_tokens), _stream(stream)),
                  "eagle_tree_verify_sample")


def eagle_tree_verify_sample_drafted(tree, target_logits, positions, vocab, dtype, inv_temp,
                                     draft_logits, draws, accept_len, accept_path, out_tokens,
                                     stream=None):
    return _check(lib().eagle_tree_verify_sample_drafted(
        ctypes.byref(tree), _ptr(target_logits), positions, vocab, dtype, inv_temp,
        _ptr(draft_logits), _ptr(draws), _ptr(accept_len), _ptr(accept_path), _ptr(out_tokens),
        _stream(stream)),
        "eagle_tree_verify_sample_drafted")


def eagle_target_workspace_bytes(head, target, kv, tree):
    return lib().eagle_target_workspace_bytes(ctypes.byref(head), ctypes.byref(target),
                                              ctypes.byref(kv), ctypes.byref(tree))


def eagle_target_verify_logits(head, target, kv, tree, logits_out, k_tree, v_tree, ws, ws_bytes,
                               stream=None, hidden_out=None):
    return _check(lib().eagle_target_verify_logits(
        ctypes.byref(head), ctypes.byref(target), ctypes.byref(kv), ctypes.byref(tree),
        _ptr(logits_out), _ptr(k_tree), _ptr(v_tree), _ptr(hidden_out), _ptr(ws), ws_bytes,
        _stream(stream)),
        "eagle_target_verify_logits")


def eagle_kv_commit(tree, kv_heads, head_dim, dtype, accept_len, accept_path, k_tree, v_tree,
                    dst_row, dst_rows, k_dst, v_dst, stream=None):
    return _check(lib().eagle_kv_commit(
        ctypes.byref(tree), kv_heads, head_dim, dtype, _ptr(accept_len), _ptr(accept_path),
        _ptr(k_tree), _ptr(v_tree), _ptr(dst_row), dst_rows, _ptr(k_dst), _ptr(v_dst),
        _stream(stream)), "eagle_kv_commit")


def eagle_profile_enable(on=True):
    """on: True (every family), False, or a family bitmask."""
    mask = (1 << len(PROF_FAMILIES)) - 1 if on is True else (0 if on is False else int(on))
    return _check(lib().eagle_profile_enable(mask), "eagle_profile_enable")


def eagle_profile_reset():
    return _check(lib().eagle_profile_reset(), "eagle_profile_reset")


def eagle_profile_read(family):
    """-> dict(launches, timed, ms, bytes, flops, roof_ms) for a kernel family."""
    fam = PROF_FAMILIES[family] if isinstance(family, str) else family
    n, t = c_int64(), c_int64()
    ms, by, fl, rf = ctypes.c_double(), ctypes.c_double(), ctypes.c_double(), ctypes.c_double()
    _check(lib().eagle_profile_read(fam, ctypes.byref(n), ctypes.byref(t), ctypes.byref(ms),
                                    ctypes.byref(by), ctypes.byref(fl), ctypes.byref(rf)),
           "eagle_profile_read")
    return dict(launches=n.value, timed=t.value, ms=ms.value, bytes=by.value, flops=fl.value,
                roof_ms=rf.value)
