"""GPU parity of the learned output gate on the low-rank term, O = O_sparse + g O_lr
with g = sigmoid(q . w + b) per token and head, against the CPU oracle.

Same bars as the ungated path: outputs within 2e-2 (bf16) or 6e-2 (fp8,
against the fp8 oracle) of the output RMS, plus half a bf16 ulp per element
when O is stored in bf16; padded rows zero.  Saturated gates are checked as
exact identities (b = +800 gives the ungated output, b = -800 the sparse
branch alone).
"""
import numpy as np
import pytest

import oracle
from sparse_rank_attention_amd import workloads as W
from tests.conftest import gpu_available
from tests.test_gpu_fp8 import bound_ratio8
from tests.test_gpu_parity import (SMALL, _full_inputs, bound_ratio, cfg_of, dev, host_f64, rel_err, say,
                                   small_workload)

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

TOL_BF16 = 2e-2


def _torch():
    import torch
    return torch


def _gate_dev(g):
    return _torch().from_numpy(np.ascontiguousarray(g, dtype=np.float32)).cuda()


@pytest.mark.parametrize("name,w", SMALL, ids=[s[0] for s in SMALL])
@pytest.mark.parametrize("prec", ["bf16", "fp8"])
@pytest.mark.parametrize("out_f32", [False, True], ids=["bf16out", "f32out"])
def test_gated_forward_matches_oracle(name, w, prec, out_f32):
    from sparse_rank_attention_amd import rola
    torch = _torch()
    fp8 = prec == "fp8"
    say("gated forward", name, prec, "f32out" if out_f32 else "bf16out")
    q, k, v = W.make_qkv(w)
    wq, wk = W.make_proj(w)
    g = W.make_gate(w)
    bmap = torch.empty((w.batch, w.heads, w.nb, oracle.keep_blocks(w.topk, w.nb)), dtype=torch.int32, device="cuda")
    cfg = cfg_of(w, out_dtype=rola.ROLA_OUT_F32 if out_f32 else rola.ROLA_OUT_BF16,
                 precision=rola.ROLA_PREC_FP8 if fp8 else rola.ROLA_PREC_BF16)
    out = rola.rola_forward(dev(q), dev(k), dev(v), torch.from_numpy(wq).cuda(), torch.from_numpy(wk).cuda(),
                            w.grid, cfg, block_idx_out=bmap, gate=_gate_dev(g))
    torch.cuda.synchronize()
    m_ref, o_ref = oracle.forward(q[0], k[0], v[0], wq, wk, w.n_tokens, oracle.keep_blocks(w.topk, w.nb), w.grid, fp8=fp8, gate_w=g)
    np.testing.assert_array_equal(bmap.cpu().numpy()[0], m_ref)
    got = host_f64(out)[0]
    assert np.all(got[:, w.n_tokens:] == 0)
    got, ref = got[:, :w.n_tokens], o_ref[:, :w.n_tokens]
    ratio = (bound_ratio8 if fp8 else bound_ratio)(got, ref, not out_f32)
    say("gated forward", name, prec, "err/rms", rel_err(got, ref), "err/bound", ratio)
    assert ratio <= 1.0


@pytest.mark.parametrize("name,w", SMALL[:3], ids=[s[0] for s in SMALL[:3]])
def test_gated_lowrank_alone_and_accumulated(name, w):
    from sparse_rank_attention_amd import rola
    torch = _torch()
    say("gated lowrank", name)
    q, k, v = W.make_qkv(w)
    wq, wk = W.make_proj(w)
    g = W.make_gate(w)
    qd, kd, vd = dev(q), dev(k), dev(v)
    wqd, wkd, gd = torch.from_numpy(wq).cuda(), torch.from_numpy(wk).cuda(), _gate_dev(g)
    cfg = cfg_of(w, out_dtype=rola.ROLA_OUT_F32)
    m_ref = oracle.block_map(q[0], k[0], w.n_tokens, oracle.keep_blocks(w.topk, w.nb))
    bmap = torch.from_numpy(m_ref).cuda().reshape(w.batch, w.heads, w.nb, oracle.keep_blocks(w.topk, w.nb))
    o_lr = rola.rola_lowrank_attn(qd, kd, vd, wqd, wkd, w.grid, cfg, gate=gd)
    o_sum = rola.rola_sparse_attn(qd, kd, vd, bmap, w.grid, cfg)
    rola.rola_lowrank_attn(qd, kd, vd, wqd, wkd, w.grid, cfg, out=o_sum, accumulate=True, gate=gd)
    o_fw = rola.rola_forward(qd, kd, vd, wqd, wkd, w.grid, cfg, gate=gd)
    torch.cuda.synchronize()
    qf, kf, vf = (oracle.widen_bf16(x[0]) for x in (q, k, v))
    rows = np.array([bh * w.n_pad + n for bh in range(w.heads) for n in range(w.n_tokens)])
    sp_ref = oracle.sparse_rows(qf, kf, vf, m_ref, w.n_tokens, rows)
    S, z = oracle.lowrank_state(kf, vf, wk, w.n_tokens, w.grid)
    lr_ref = oracle.lowrank_rows(qf, wq, S, z, w.grid, rows, gate_w=g)
    take = lambda t: host_f64(t)[0][:, :w.n_tokens].reshape(-1, w.head_dim)
    e_lr = rel_err(take(o_lr), lr_ref)
    e_sum = rel_err(take(o_sum), sp_ref + lr_ref)
    say("gated lowrank", name, "lowrank", e_lr, "sum", e_sum)
    assert e_lr <= TOL_BF16 and e_sum <= TOL_BF16
    np.testing.assert_allclose(take(o_fw), take(o_sum), rtol=0, atol=1e-5 * np.abs(take(o_sum)).max())


@pytest.mark.parametrize("prec", ["bf16", "fp8"])
def test_saturated_gates_are_exact(prec):
    """b = +800 makes g exactly 1 (the ungated output, bit for bit); b = -800
    makes it exactly 0 (the sparse branch alone)."""
    from sparse_rank_attention_amd import rola
    torch = _torch()
    say("saturated gates", prec)
    w = small_workload((3, 7, 11), D=128, H=2, rank=32, topk=0.3, kind="field")
    q, k, v = (dev(x) for x in W.make_qkv(w))
    wq, wk = (torch.from_numpy(x).cuda() for x in W.make_proj(w))
    cfg = cfg_of(w, out_dtype=rola.ROLA_OUT_F32,
                 precision=rola.ROLA_PREC_FP8 if prec == "fp8" else rola.ROLA_PREC_BF16)
    g = np.zeros(w.head_dim + 1, dtype=np.float32)
    g[w.head_dim] = 800.0
    bmap = torch.empty((w.batch, w.heads, w.nb, oracle.keep_blocks(w.topk, w.nb)), dtype=torch.int32, device="cuda")
    plain = rola.rola_forward(q, k, v, wq, wk, w.grid, cfg, block_idx_out=bmap)
    open_ = rola.rola_forward(q, k, v, wq, wk, w.grid, cfg, gate=_gate_dev(g))
    g[w.head_dim] = -800.0
    shut = rola.rola_forward(q, k, v, wq, wk, w.grid, cfg, gate=_gate_dev(g))
    sparse = rola.rola_sparse_attn(q, k, v, bmap, w.grid, cfg)
    torch.cuda.synchronize()
    assert torch.equal(open_, plain)
    assert torch.equal(shut, sparse)


def test_gated_invalid_rows_of_inputs_are_ignored():
    """NaN in padded query rows reaches neither the gate of a valid row nor the output."""
    from sparse_rank_attention_amd import rola
    torch = _torch()
    w = small_workload((3, 7, 11), D=64, H=2)
    q, k, v = (dev(x) for x in W.make_qkv(w))
    wq, wk = (torch.from_numpy(x).cuda() for x in W.make_proj(w))
    gd = _gate_dev(W.make_gate(w))
    a = rola.rola_forward(q, k, v, wq, wk, w.grid, cfg_of(w), gate=gd)
    for t in (q, k, v):
        t[:, :, w.n_tokens:] = float("nan")
    b = rola.rola_forward(q, k, v, wq, wk, w.grid, cfg_of(w), gate=gd)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_gated_full_size_sampled():
    """Wan 14B 720P launch (40 heads, N = 75600, 35 kept blocks) with a gate, on
    sampled heads and rows."""
    from sparse_rank_attention_amd import rola
    torch = _torch()
    name = "wan14b_720p"
    say("gated full size", name)
    w, (q, k, v), (wq, wk) = _full_inputs(name)
    g = W.make_gate(w)
    out = rola.rola_forward(dev(q), dev(k), dev(v), torch.from_numpy(wq).cuda(), torch.from_numpy(wk).cuda(),
                            w.grid, cfg_of(w), gate=_gate_dev(g))
    torch.cuda.synchronize()
    rng = np.random.default_rng(7)
    worst = 0.0
    for h in (1, w.heads - 2):
        m_ref = oracle.block_map(q[0, h:h + 1], k[0, h:h + 1], w.n_tokens, oracle.keep_blocks(w.topk, w.nb))
        qbs = sorted({0, w.nb - 1, *rng.integers(0, w.nb, 4).tolist()})
        rows = np.array(sorted({n for qb in qbs for n in (qb * 64, qb * 64 + 31, qb * 64 + 63)
                                if n < w.n_tokens} | {w.n_tokens - 1}))
        qf, kf, vf = (oracle.widen_bf16(x[0, h:h + 1]) for x in (q, k, v))
        sp = oracle.sparse_rows(qf, kf, vf, m_ref, w.n_tokens, rows)
        S, z = oracle.lowrank_state(kf, vf, wk, w.n_tokens, w.grid)
        lr = oracle.lowrank_rows(qf, wq, S, z, w.grid, rows, gate_w=g)
        got = out[0, h, torch.from_numpy(rows).cuda()].float().cpu().numpy().astype(np.float64)
        ratio = bound_ratio(got, sp + lr, True)
        worst = max(worst, rel_err(got, sp + lr))
        assert ratio <= 1.0, (h, ratio)
        assert torch.count_nonzero(out[0, h, w.n_tokens:].float()).item() == 0
    say("gated full size", name, "worst err/rms", worst)
