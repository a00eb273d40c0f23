"""eagle_draft_step_noalloc (workspace in a library-held device array) against
eagle_draft_step with a caller workspace: two rounds in a row through the
C-ABI, the second one smaller, every draft step's logits, layer outputs,
top-k ids, confidences and log-partitions, the tree and the verify result
compared bit for bit (the same kernels on the same inputs)."""
import numpy as np
import pytest

from eagle_feature_space_amd import configs as C

pytestmark = pytest.mark.gpu


def _round(case, noalloc):
    import torch
    gr = case.gpu()
    gr.noalloc = noalloc
    if noalloc:
        gr.ws = None                  # nothing of the caller's workspace is reachable
    snaps = gr.run(target=case.target_dev(), snapshots=True, attend=False)
    torch.cuda.synchronize()
    fv = {k: v.cpu().numpy() for k, v in gr.final_view().items()}
    res = (gr.accept_len.cpu().numpy(), gr.accept_path.cpu().numpy(), gr.out_tokens.cpu().numpy())
    return snaps, fv, res


def _same(a, b, what):
    a, b = np.asarray(a), np.asarray(b)
    assert a.shape == b.shape, what
    assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), what


@pytest.mark.parametrize("name", ["s5_dynamic_many", "s2_dynamic"])
def test_noalloc_step_equals_workspace_step(name):
    from eagle_feature_space_amd import binding as E
    from tests.parity import Case
    cfg = C.SMALL_CONFIGS[name]
    print(f"\n[noalloc] {name}", flush=True)
    case = Case(cfg, with_oracle=False)
    ref, ref_f, ref_v = _round(case, noalloc=False)
    got, got_f, got_v = _round(case, noalloc=True)
    for s, (r, g) in enumerate(zip(ref, got)):
        for k in ("topk_id", "topk_conf", "lse", "logits", "feat"):
            _same(getattr(g, k), getattr(r, k), f"step {s} {k}")
    for k in ref_f:
        _same(got_f[k], ref_f[k], f"verify tree {k}")
    for a, b, what in zip(got_v, ref_v, ("accept_len", "accept_path", "out_tokens")):
        _same(a, b, what)
    print(f"[noalloc] {name}: {len(ref)} steps bit-identical", flush=True)


def test_noalloc_rejects_a_workspace_beyond_the_array():
    """The 8B EAGLE-2 tree at B 8 needs about 400 MB of workspace: refused on
    the host before anything is launched."""
    from eagle_feature_space_amd import binding as E
    from tests.test_abi_host import _head, _kv, _tree
    cfg = C.CONFIGS["c2_8b_dynamic"]
    h, kv = _head(cfg.head), _kv(cfg, list(cfg.n))
    t = _tree(cfg, state=1 << 20, nbytes=1 << 30)
    assert E.eagle_workspace_bytes(h, kv, t) > E.NOALLOC_SCRATCH_BYTES
    st = E.lib().eagle_draft_step_noalloc(h, kv, t, 0, 1 << 20, None, None, None, None, None)
    assert st == E.EAGLE_ECAPACITY
