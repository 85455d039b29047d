"""rola_forward_noalloc (the library's per-GPU scratch instead of a caller
workspace) against rola_forward on the same inputs: two calls in a row, the
second on a smaller problem, each bit-identical to rola_forward's output and
block map (the same kernels run on either workspace)."""
import numpy as np
import pytest
import torch

from sparse_rank_attention_amd import rola, workloads as W

pytestmark = pytest.mark.gpu


def _case(name, dims, grid, topk, rank, kind):
    w = W.Workload(name, 1, dims[0], dims[1], grid, topk, rank, kind, seed=5)
    q, k, v = W.make_qkv(w)
    wq, wk = W.make_proj(w)
    dev = lambda x: torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
    return w, dev(q), dev(k), dev(v), torch.from_numpy(wq).cuda(), torch.from_numpy(wk).cuda()


def _check_one(w, q, k, v, wq, wk, precision):
    cfg = rola.Config(topk=w.topk, rank=w.rank, precision=precision)
    info = rola.plan(rola.problem(q, w.grid), cfg)
    print("[case] no-alloc forward", w.name, "heads", w.heads, "D", w.head_dim, "nb", info.nb, "kb", info.kb,
          "precision", precision, "workspace", info.workspace_bytes, flush=True)
    ref_map = torch.empty((1, w.heads, info.nb, info.kb), dtype=torch.int32, device="cuda")
    ref = rola.rola_forward(q, k, v, wq, wk, w.grid, cfg, block_idx_out=ref_map)
    out = torch.full_like(ref, float("nan"))
    bmap = torch.full_like(ref_map, -1)
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    rola.rola_forward_noalloc(q, k, v, wq, wk, w.grid, cfg, out, block_idx_out=bmap)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == before
    assert torch.equal(bmap, ref_map)
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))


@pytest.mark.parametrize("precision", [rola.ROLA_PREC_BF16, rola.ROLA_PREC_FP8])
def test_noalloc_matches_forward_on_two_calls(precision):
    big = _case("big", (4, 128), (6, 16, 21), 0.1, 32, "field")     # N = 2016: ragged tail, 32 blocks
    small = _case("small", (2, 64), (3, 8, 10), 0.25, 16, "iid")     # N = 240
    _check_one(*big, precision)
    _check_one(*small, precision)  # the second call reuses the scratch the first one filled


def test_noalloc_rejects_problems_above_its_scratch():
    w = W.WORKLOADS["wan14b_720p_fp8"]
    cfg = rola.Config(topk=w.topk, rank=w.rank, precision=rola.ROLA_PREC_FP8)
    q = torch.zeros((1, w.heads, w.n_pad, w.head_dim), dtype=torch.bfloat16, device="cuda")
    wq = torch.zeros((w.head_dim, w.rank), dtype=torch.float32, device="cuda")
    assert rola.plan(rola.problem(q, w.grid), cfg).workspace_bytes > rola.NOALLOC_SCRATCH_BYTES
    with pytest.raises(rola.RolaError, match="scratch"):
        rola.rola_forward_noalloc(q, q, q, wq, wq, w.grid, cfg, torch.empty_like(q))
    # the C entry point itself returns ROLA_ERR_WORKSPACE before any launch
    prob, c = rola.problem(q, w.grid), cfg.c()
    import ctypes
    st = rola.lib().rola_forward_noalloc(ctypes.byref(prob), ctypes.byref(c), rola._ptr(q), rola._ptr(q),
                                         rola._ptr(q), rola._ptr(wq), rola._ptr(wq), None, None, rola._ptr(q),
                                         rola._stream(None))
    assert st == 4
