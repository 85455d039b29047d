"""GPU parity of the complement scope of the low-rank branch (each query block's
low-rank state covers only the key blocks it does not keep) against the CPU oracle.

Same bars as the global scope: block maps bit-exact; outputs within 2e-2 (bf16)
or 6e-2 (fp8, against the fp8 oracle) of the output RMS, plus half a bf16 ulp
per element when O is stored in bf16; padded rows zero.  Keeping every block
leaves nothing to the low-rank term, so the forward must then equal the
sparse branch exactly.
"""
import numpy as np
import pytest

import oracle
from sparse_rank_attention_amd import workloads as W
from tests.conftest import gpu_available
from tests.test_gpu_fp8 import bound_ratio8
from tests.test_gpu_parity import SMALL, _full_inputs, bound_ratio, dev, host_f64, rel_err, say, small_workload

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

TOL_BF16 = 2e-2

CASES = SMALL + [("two_batches", W.Workload("b2", 2, 2, 64, (3, 7, 11), 0.25, 16, "iid", seed=3))]


def _torch():
    import torch
    return torch


def ccfg(w, **kw):
    from sparse_rank_attention_amd import rola
    return rola.Config(topk=w.topk, rank=w.rank, lowrank_scope=rola.ROLA_LR_COMPLEMENT, **kw)


def _flat(w, x):
    return x.reshape(w.batch * w.heads, w.n_pad, w.head_dim)


@pytest.mark.parametrize("name,w", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("prec", ["bf16", "fp8"])
@pytest.mark.parametrize("out_f32", [False, True], ids=["bf16out", "f32out"])
def test_complement_forward_matches_oracle(name, w, prec, out_f32):
    from sparse_rank_attention_amd import rola
    torch = _torch()
    fp8 = prec == "fp8"
    say("complement forward", name, prec, "f32out" if out_f32 else "bf16out")
    q, k, v = W.make_qkv(w)
    wq, wk = W.make_proj(w)
    bmap = torch.empty((w.batch, w.heads, w.nb, oracle.keep_blocks(w.topk, w.nb)), dtype=torch.int32, device="cuda")
    cfg = ccfg(w, out_dtype=rola.ROLA_OUT_F32 if out_f32 else rola.ROLA_OUT_BF16,
               precision=rola.ROLA_PREC_FP8 if fp8 else rola.ROLA_PREC_BF16)
    out = rola.rola_forward(dev(q), dev(k), dev(v), torch.from_numpy(wq).cuda(), torch.from_numpy(wk).cuda(),
                            w.grid, cfg, block_idx_out=bmap)
    torch.cuda.synchronize()
    m_ref, o_ref = oracle.forward(_flat(w, q), _flat(w, k), _flat(w, v), wq, wk, w.n_tokens, oracle.keep_blocks(w.topk, w.nb), w.grid,
                                  fp8=fp8, complement=True)
    np.testing.assert_array_equal(bmap.cpu().numpy().reshape(m_ref.shape), m_ref)
    got = host_f64(out).reshape(o_ref.shape)
    assert np.all(got[:, w.n_tokens:] == 0)
    got, ref = got[:, :w.n_tokens], o_ref[:, :w.n_tokens]
    ratio = (bound_ratio8 if fp8 else bound_ratio)(got, ref, not out_f32)
    say("complement forward", name, prec, "err/rms", rel_err(got, ref), "err/bound", ratio)
    assert ratio <= 1.0


@pytest.mark.parametrize("name,w", CASES[:3], ids=[c[0] for c in CASES[:3]])
def test_complement_lowrank_alone_and_accumulated(name, w):
    """rola_lowrank_attn in the complement scope (it selects the blocks itself)
    against the oracle's complement rows, with and without the output gate, and
    sparse + low-rank (accumulated) against the fused forward."""
    from sparse_rank_attention_amd import rola
    torch = _torch()
    say("complement lowrank", name)
    q, k, v = W.make_qkv(w)
    wq, wk = W.make_proj(w)
    g = W.make_gate(w)
    qd, kd, vd = dev(q), dev(k), dev(v)
    wqd, wkd, gd = torch.from_numpy(wq).cuda(), torch.from_numpy(wk).cuda(), torch.from_numpy(g).cuda()
    cfg = ccfg(w, out_dtype=rola.ROLA_OUT_F32)
    m_ref = oracle.block_map(q[0], k[0], w.n_tokens, oracle.keep_blocks(w.topk, w.nb))
    bmap = torch.from_numpy(m_ref).cuda().reshape(w.batch, w.heads, w.nb, oracle.keep_blocks(w.topk, w.nb))
    o_lr = rola.rola_lowrank_attn(qd, kd, vd, wqd, wkd, w.grid, cfg)
    o_lrg = rola.rola_lowrank_attn(qd, kd, vd, wqd, wkd, w.grid, cfg, gate=gd)
    o_sum = rola.rola_sparse_attn(qd, kd, vd, bmap, w.grid, cfg)
    rola.rola_lowrank_attn(qd, kd, vd, wqd, wkd, w.grid, cfg, out=o_sum, accumulate=True, gate=gd)
    o_fw = rola.rola_forward(qd, kd, vd, wqd, wkd, w.grid, cfg, gate=gd)
    torch.cuda.synchronize()
    worst = 0.0
    for h in range(w.heads):
        qf, kf, vf = (oracle.widen_bf16(x[0, h]) for x in (q, k, v))
        Sb, zb = oracle.lowrank_block_states(kf, vf, wk, w.n_tokens, w.grid)
        rows = np.arange(w.n_tokens)
        lr = oracle.lowrank_rows_complement(qf, wq, Sb, zb, m_ref[h], w.grid, rows)
        lrg = oracle.lowrank_rows_complement(qf, wq, Sb, zb, m_ref[h], w.grid, rows, gate_w=g)
        for got, ref in ((o_lr, lr), (o_lrg, lrg)):
            e = rel_err(host_f64(got)[0, h, :w.n_tokens], ref)
            worst = max(worst, e)
            assert e <= TOL_BF16, (h, e)
    say("complement lowrank", name, "worst err/rms", worst)
    take = lambda t: host_f64(t)[0][:, :w.n_tokens]
    np.testing.assert_allclose(take(o_fw), take(o_sum), rtol=0, atol=1e-5 * np.abs(take(o_sum)).max())


@pytest.mark.parametrize("prec", ["bf16", "fp8"])
def test_complement_keep_all_is_the_sparse_branch(prec):
    from sparse_rank_attention_amd import rola
    torch = _torch()
    say("complement keep all", prec)
    w = small_workload((5, 9, 13), D=128, H=2, rank=32, topk=1.0, kind="field")  # N = 585, nb = 10
    q, k, v = (dev(x) for x in W.make_qkv(w))
    wq, wk = (torch.from_numpy(x).cuda() for x in W.make_proj(w))
    cfg = ccfg(w, out_dtype=rola.ROLA_OUT_F32,
               precision=rola.ROLA_PREC_FP8 if prec == "fp8" else rola.ROLA_PREC_BF16)
    bmap = torch.empty((w.batch, w.heads, w.nb, oracle.keep_blocks(w.topk, w.nb)), dtype=torch.int32, device="cuda")
    out = rola.rola_forward(q, k, v, wq, wk, w.grid, cfg, block_idx_out=bmap)
    lr = rola.rola_lowrank_attn(q, k, v, wq, wk, w.grid, cfg)
    sparse = rola.rola_sparse_attn(q, k, v, bmap, w.grid, cfg)
    torch.cuda.synchronize()
    assert torch.equal(out, sparse)
    assert torch.count_nonzero(lr).item() == 0


def test_complement_full_size_sampled():
    """Wan 14B 720P launch (40 heads, N = 75600, 35 kept blocks) in the
    complement scope, on sampled heads and rows."""
    from sparse_rank_attention_amd import rola
    torch = _torch()
    name = "wan14b_720p"
    say("complement full size", name)
    w, (q, k, v), (wq, wk) = _full_inputs(name)
    bmap = torch.empty((w.batch, w.heads, w.nb, oracle.keep_blocks(w.topk, w.nb)), dtype=torch.int32, device="cuda")
    out = rola.rola_forward(dev(q), dev(k), dev(v), torch.from_numpy(wq).cuda(), torch.from_numpy(wk).cuda(),
                            w.grid, ccfg(w), block_idx_out=bmap)
    torch.cuda.synchronize()
    bmap = bmap.cpu().numpy()
    rng = np.random.default_rng(11)
    worst = 0.0
    for h in (2, w.heads - 3):
        m_ref = oracle.block_map(q[0, h:h + 1], k[0, h:h + 1], w.n_tokens, oracle.keep_blocks(w.topk, w.nb))
        np.testing.assert_array_equal(bmap[0, h], m_ref[0])
        qbs = sorted({0, w.nb // 3, w.nb - 1, *rng.integers(0, w.nb, 3).tolist()})
        rows = np.array(sorted({n for qb in qbs for n in (qb * 64, qb * 64 + 33, qb * 64 + 63)
                                if n < w.n_tokens} | {w.n_tokens - 1}))
        qf, kf, vf = (oracle.widen_bf16(x[0, h:h + 1]) for x in (q, k, v))
        sp = oracle.sparse_rows(qf, kf, vf, m_ref, w.n_tokens, rows)
        Sb, zb = oracle.lowrank_block_states(kf[0], vf[0], wk, w.n_tokens, w.grid)
        lr = oracle.lowrank_rows_complement(qf[0], wq, Sb, zb, m_ref[0], w.grid, rows)
        got = out[0, h, torch.from_numpy(rows).cuda()].float().cpu().numpy().astype(np.float64)
        ratio = bound_ratio(got, sp + lr, True)
        worst = max(worst, rel_err(got, sp + lr))
        assert ratio <= 1.0, (h, ratio)
        assert torch.count_nonzero(out[0, h, w.n_tokens:].float()).item() == 0
    say("complement full size", name, "worst err/rms", worst)
