"""The training pair: rola_forward_train keeps the sparse branch's output O_s and
each row's log-sum-exp from the forward's own attention launch, and
rola_backward_saved takes them instead of recomputing the sparse branch.

- The training forward's output and block map equal rola_forward's bit for bit
  (keeping O_s and the log-sum-exp changes nothing else).
- With fp32 output both forms compute O_s with fp32 weights, so the saved pair
  equals the backward's own recompute and every gradient is bit-identical to
  rola_backward's.
- With bf16 output the saved pair comes from the fp16-weight form of the
  forward; the gradients then meet the backward's bar against the oracle
  (the same bar and oracle as tests/test_gpu_backward.py).
"""
import numpy as np
import pytest

import oracle
from oracle import backward as OB
from sparse_rank_attention_amd import workloads as W
from tests.conftest import gpu_available
from tests.test_gpu_backward import CASES, _ratio
from tests.test_gpu_parity import dev, host_f64, say

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def _setup(w, gated, out_f32, complement):
    import torch
    from sparse_rank_attention_amd import rola
    q, k, v = W.make_qkv(w)
    wq, wk = W.make_proj(w)
    g = W.make_gate(w) if gated else None
    do = W.make_dout(w, f32=out_f32)
    cfg = rola.Config(topk=w.topk, rank=w.rank, out_dtype=rola.ROLA_OUT_F32 if out_f32 else rola.ROLA_OUT_BF16,
                      lowrank_scope=rola.ROLA_LR_COMPLEMENT if complement else rola.ROLA_LR_GLOBAL)
    t = dict(q=dev(q), k=dev(k), v=dev(v), wq=torch.from_numpy(wq).cuda(), wk=torch.from_numpy(wk).cuda(),
             gate=torch.from_numpy(g).cuda() if gated else None,
             dout=torch.from_numpy(do).cuda() if out_f32 else dev(do))
    return (q, k, v, wq, wk, g, do), cfg, t


def _forward_pair(w, cfg, t):
    """rola_forward and rola_forward_train on the same inputs: outputs and maps
    must agree bit for bit; returns the training forward's (map, os, lse)."""
    import torch
    from sparse_rank_attention_amd import rola
    info = rola.plan(rola.problem(t["q"], w.grid), cfg)
    shape = (w.batch, w.heads, info.nb, info.kb)
    m1 = torch.empty(shape, dtype=torch.int32, device="cuda")
    m2 = torch.empty(shape, dtype=torch.int32, device="cuda")
    o1 = rola.rola_forward(t["q"], t["k"], t["v"], t["wq"], t["wk"], w.grid, cfg, block_idx_out=m1, gate=t["gate"])
    o2, os_, lse = rola.rola_forward_train(t["q"], t["k"], t["v"], t["wq"], t["wk"], w.grid, cfg,
                                           block_idx_out=m2, gate=t["gate"])
    torch.cuda.synchronize()
    assert torch.equal(m1, m2)
    iv = torch.int32 if o1.dtype == torch.float32 else torch.int16
    assert torch.equal(o1.view(iv), o2.view(iv))
    assert torch.count_nonzero(os_[:, :, w.n_tokens:]).item() == 0
    return m2, os_, lse


@pytest.mark.parametrize("name,w", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("complement", [False, True], ids=["global", "complement"])
def test_saved_pair_equals_recompute_with_fp32_output(name, w, complement):
    import torch
    from sparse_rank_attention_amd import rola
    say("training pair fp32", name, "complement" if complement else "global")
    _, cfg, t = _setup(w, gated=True, out_f32=True, complement=complement)
    bmap, os_, lse = _forward_pair(w, cfg, t)
    args = (t["q"], t["k"], t["v"], t["wq"], t["wk"], w.grid, cfg, bmap, t["dout"])
    ref = rola.rola_backward(*args, gate=t["gate"])
    got = rola.rola_backward(*args, gate=t["gate"], saved=(os_, lse))
    torch.cuda.synchronize()
    for key, a, b in zip(("dq", "dk", "dv", "dwq", "dwk", "dgate"), got, ref):
        iv = torch.int32 if a.dtype == torch.float32 else torch.int16
        assert torch.equal(a.view(iv), b.view(iv)), key


@pytest.mark.parametrize("name,w", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("complement", [False, True], ids=["global", "complement"])
def test_saved_pair_matches_oracle_with_bf16_output(name, w, complement):
    import torch
    from sparse_rank_attention_amd import rola
    say("training pair bf16", name, "complement" if complement else "global")
    (q, k, v, wq, wk, g, do), cfg, t = _setup(w, gated=True, out_f32=False, complement=complement)
    bmap, os_, lse = _forward_pair(w, cfg, t)
    dq, dk, dv, dwq, dwk, dgate = rola.rola_backward(t["q"], t["k"], t["v"], t["wq"], t["wk"], w.grid, cfg, bmap,
                                                     t["dout"], gate=t["gate"], saved=(os_, lse))
    torch.cuda.synchronize()
    flat = lambda x: x.reshape(w.batch * w.heads, w.n_pad, -1)
    kb = oracle.keep_blocks(w.topk, w.nb)
    m_ref = oracle.block_map(flat(q), flat(k), w.n_tokens, kb)
    np.testing.assert_array_equal(bmap.cpu().numpy().reshape(-1, w.nb, kb), m_ref)
    f64 = oracle.widen_bf16
    ref = OB.backward(f64(flat(q)), f64(flat(k)), f64(flat(v)), wq, wk, m_ref, f64(flat(do)), w.n_tokens, w.grid,
                      gate=g, complement=complement)
    n = w.n_tokens
    ratios = {}
    for key, got in (("dq", dq), ("dk", dk), ("dv", dv)):
        gh = flat(host_f64(got))
        assert np.all(gh[:, n:] == 0), key
        ratios[key] = _ratio(gh[:, :n], ref[key][:, :n], True)
    ratios["dwq"] = _ratio(host_f64(dwq), ref["dwq"], False)
    ratios["dwk"] = _ratio(host_f64(dwk), ref["dwk"], False)
    ratios["dgate"] = _ratio(host_f64(dgate), ref["dgate"], False)
    say("training pair bf16", name, "err/bound", {k_: round(v_, 3) for k_, v_ in ratios.items()})
    for key, r in ratios.items():
        assert r <= 1.0, (key, r)


def test_saved_pair_for_heads_beyond_fp16():
    """Heads whose V leaves the fp16 range take the bf16 form (fp32 weights) in the
    forward, also in the training forward: for those heads the saved pair is the
    backward's own recompute, so their dq, dk, dv equal rola_backward's bit for bit
    (the projection gradients sum over all heads and are not compared)."""
    import torch
    from sparse_rank_attention_amd import rola
    from tests.test_gpu_parity import small_workload
    say("training pair, V beyond fp16")
    w = small_workload((5, 9, 13), D=128, H=3, rank=32, topk=0.3, kind="field")
    q, k, v = W.make_qkv(w)
    v = v.copy()
    big = np.array([1.0e5, -7.0e4], dtype=np.float32).view(np.uint32) >> 16  # bf16 99840, -70144
    v[0, 1, 100, 3] = big[0]
    v[0, 2, w.n_tokens - 1, 77] = big[1]
    wq, wk = W.make_proj(w)
    cfg = rola.Config(topk=w.topk, rank=w.rank)
    t = dict(q=dev(q), k=dev(k), v=dev(v), wq=torch.from_numpy(wq).cuda(), wk=torch.from_numpy(wk).cuda(),
             gate=None, dout=dev(W.make_dout(w)))
    bmap, os_, lse = _forward_pair(w, cfg, t)
    args = (t["q"], t["k"], t["v"], t["wq"], t["wk"], w.grid, cfg, bmap, t["dout"])
    ref = rola.rola_backward(*args)
    got = rola.rola_backward(*args, saved=(os_, lse))
    torch.cuda.synchronize()
    for key, a, b in zip(("dq", "dk", "dv"), got[:3], ref[:3]):
        for h in (1, 2):
            assert torch.equal(a[0, h].view(torch.int16), b[0, h].view(torch.int16)), (key, h)
