"""rola_forward captured as a HIP graph (torch.cuda.CUDAGraph) and replayed.

Every call of the library only launches kernels on its stream (no memset, copy,
allocation or synchronisation), so a forward can be captured as it is and
replayed, which is how a serving loop would run it.  Each case captures one
forward, replays it three times with eager work between the replays (another
forward on other inputs, torch kernels, synchronisations) and checks every
replay bit for bit against the eager forward: the kernels are deterministic, so
a replay must reproduce the eager output and block map exactly.
"""
import numpy as np
import pytest
import torch

from sparse_rank_attention_amd import rola, workloads as W
from tests.conftest import gpu_available

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def _dev(x):
    return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()


def _inputs(w):
    q, k, v = W.make_qkv(w)
    wq, wk = W.make_proj(w)
    return _dev(q), _dev(k), _dev(v), torch.from_numpy(wq).cuda(), torch.from_numpy(wk).cuda()


CASES = [
    ("tiny_bf16", W.WORKLOADS["tiny"], dict()),
    ("tiny_fp8", W.WORKLOADS["tiny"], dict(precision=rola.ROLA_PREC_FP8)),
    ("tiny_complement", W.WORKLOADS["tiny"], dict(lowrank_scope=rola.ROLA_LR_COMPLEMENT)),
    ("d128_f32_gate", W.Workload("g", 1, 2, 128, (5, 16, 16), 0.25, 32, "field", seed=4),
     dict(out_dtype=rola.ROLA_OUT_F32)),
]


@pytest.mark.parametrize("name,w,kw", CASES, ids=[c[0] for c in CASES])
def test_forward_graph_replays_match_eager(name, w, kw):
    print("[case] graph replay", name, flush=True)
    q, k, v, wq, wk = _inputs(w)
    gate = torch.from_numpy(W.make_gate(w)).cuda() if name.endswith("gate") else None
    cfg = rola.Config(topk=w.topk, rank=w.rank, **kw)
    info = rola.plan(rola.problem(q, w.grid), cfg)
    bshape = (w.batch, w.heads, info.nb, info.kb)
    ref_map = torch.empty(bshape, dtype=torch.int32, device="cuda")
    ref = rola.rola_forward(q, k, v, wq, wk, w.grid, cfg, block_idx_out=ref_map, gate=gate)
    # other inputs for the eager work between replays
    w2 = W.Workload(w.name, w.batch, w.heads, w.head_dim, w.grid, w.topk, w.rank, w.kind, seed=w.seed + 7)
    q2, k2, v2, _, _ = _inputs(w2)

    out = torch.empty_like(ref)
    bmap = torch.empty_like(ref_map)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        rola.rola_forward(q, k, v, wq, wk, w.grid, cfg, out=out, block_idx_out=bmap, gate=gate, stream=side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        rola.rola_forward(q, k, v, wq, wk, w.grid, cfg, out=out, block_idx_out=bmap, gate=gate, stream=side)
    torch.cuda.synchronize()
    for rep in range(3):
        out.fill_(float("nan"))
        bmap.fill_(-1)
        other = rola.rola_forward(q2, k2, v2, wq, wk, w.grid, cfg)  # eager work between the replays
        _ = (other.float() @ other.float().transpose(-1, -2).contiguous()).sum()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(bmap, ref_map), (name, rep)
        assert torch.equal(out.view(torch.int16) if out.dtype == torch.bfloat16 else out.view(torch.int32),
                           ref.view(torch.int16) if ref.dtype == torch.bfloat16 else ref.view(torch.int32)), (name, rep)
    del g
