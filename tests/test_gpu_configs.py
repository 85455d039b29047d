"""GPU parity on configurations the workload tests do not reach: several
batches, non-default rotary split / theta / softmax scale / rank / explicit
block count, and keep ratio 1.0 over more key blocks than the attention
kernels stage in LDS (their union list is then read from global memory).
Same bars as the other parity tests: block maps bit-exact, outputs within
2e-2 (bf16) or 6e-2 (fp8, against the fp8 oracle) of the output RMS."""
import numpy as np
import pytest

import oracle
from sparse_rank_attention_amd import workloads as W
from tests.conftest import gpu_available
from tests.test_gpu_fp8 import bound_ratio8
from tests.test_gpu_parity import bound_ratio, dev, host_f64, rel_err, say

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def _torch():
    import torch
    return torch


@pytest.mark.parametrize("fp8", [False, True], ids=["bf16", "fp8"])
def test_two_batches(fp8):
    from sparse_rank_attention_amd import rola
    torch = _torch()
    w = W.Workload("b2", 2, 2, 64, (3, 7, 11), 0.25, 16, "iid", seed=3)
    say("two batches", "fp8" if fp8 else "bf16")
    q, k, v = W.make_qkv(w)
    wq, wk = W.make_proj(w)
    bmap = torch.empty((w.batch, w.heads, w.nb, oracle.keep_blocks(w.topk, w.nb)), dtype=torch.int32, device="cuda")
    cfg = rola.Config(topk=w.topk, rank=w.rank, out_dtype=rola.ROLA_OUT_F32,
                      precision=rola.ROLA_PREC_FP8 if fp8 else rola.ROLA_PREC_BF16)
    out = rola.rola_forward(dev(q), dev(k), dev(v), torch.from_numpy(wq).cuda(), torch.from_numpy(wk).cuda(),
                            w.grid, cfg, block_idx_out=bmap)
    torch.cuda.synchronize()
    flat = lambda x: x.reshape(w.batch * w.heads, w.n_pad, w.head_dim)
    m_ref, o_ref = oracle.forward(flat(q), flat(k), flat(v), wq, wk, w.n_tokens, oracle.keep_blocks(w.topk, w.nb), w.grid, fp8=fp8)
    np.testing.assert_array_equal(bmap.cpu().numpy().reshape(m_ref.shape), m_ref)
    got = host_f64(out).reshape(o_ref.shape)[:, :w.n_tokens]
    ref = o_ref[:, :w.n_tokens]
    ratio = (bound_ratio8 if fp8 else bound_ratio)(got, ref, False)
    say("two batches err/rms", rel_err(got, ref), "err/bound", ratio)
    assert ratio <= 1.0


def test_custom_rope_scale_rank_and_block_count():
    from sparse_rank_attention_amd import rola
    torch = _torch()
    w = W.Workload("cfg", 1, 2, 64, (2, 9, 14), 0.25, 32, "field", seed=5)  # N = 252, tail 60
    split, theta, scale, kb = (16, 16, 32), 500.0, 0.2, 3
    say("custom config", split, theta, scale, kb)
    q, k, v = W.make_qkv(w)
    wq, wk = W.make_proj(w)
    bmap = torch.empty((1, w.heads, w.nb, kb), dtype=torch.int32, device="cuda")
    cfg = rola.Config(topk=w.topk, rank=w.rank, kb_override=kb, rope_split=split, rope_theta=theta,
                      softmax_scale=scale, out_dtype=rola.ROLA_OUT_F32)
    out = rola.rola_forward(dev(q), dev(k), dev(v), torch.from_numpy(wq).cuda(), torch.from_numpy(wk).cuda(),
                            w.grid, cfg, block_idx_out=bmap)
    torch.cuda.synchronize()
    m_ref, o_ref = oracle.forward(q[0], k[0], v[0], wq, wk, w.n_tokens, kb, w.grid, split=split,
                                  theta=theta, scale=scale)
    np.testing.assert_array_equal(bmap.cpu().numpy()[0], m_ref)
    got = host_f64(out[0])[:, :w.n_tokens]
    ratio = bound_ratio(got, o_ref[:, :w.n_tokens], False)
    say("custom config err/rms", rel_err(got, o_ref[:, :w.n_tokens]), "err/bound", ratio)
    assert ratio <= 1.0


@pytest.mark.parametrize("fp8", [False, True], ids=["bf16", "fp8"])
def test_full_keep_with_list_beyond_lds(fp8):
    """topk = 1.0 over 2100 key blocks (N = 134400): every union list has 2100
    entries, more than the 2048 staged in LDS, so the attention kernels read
    it from global memory.  Sampled rows against dense attention (fp8: on the
    dequantised inputs) plus the low-rank branch."""
    from sparse_rank_attention_amd import rola
    torch = _torch()
    w = W.Workload("long", 1, 1, 64, (1, 1, 2100 * 64), 1.0, 16, "iid", seed=11)
    say("full keep, list beyond LDS", "fp8" if fp8 else "bf16", "nb", w.nb)
    q, k, v = W.make_qkv(w)
    wq, wk = W.make_proj(w)
    bmap = torch.empty((1, 1, w.nb, oracle.keep_blocks(w.topk, w.nb)), dtype=torch.int32, device="cuda")
    cfg = rola.Config(topk=1.0, rank=w.rank, out_dtype=rola.ROLA_OUT_F32,
                      precision=rola.ROLA_PREC_FP8 if fp8 else rola.ROLA_PREC_BF16)
    out = rola.rola_forward(dev(q), dev(k), dev(v), torch.from_numpy(wq).cuda(), torch.from_numpy(wk).cuda(),
                            w.grid, cfg, block_idx_out=bmap)
    torch.cuda.synchronize()
    full = np.tile(np.arange(w.nb, dtype=np.int32), (1, w.nb, 1))
    np.testing.assert_array_equal(bmap.cpu().numpy()[0], full)
    rows = np.array([0, 1, 63, 64, 4095, 70000, w.n_tokens - 65, w.n_tokens - 1])
    qf, kf, vf = (oracle.widen_bf16(x[0]) for x in (q, k, v))
    if fp8:
        qs, ks, vs = (oracle.quant_e4m3(x[0], w.n_tokens)[2] for x in (q, k, v))
    else:
        qs, ks, vs = qf, kf, vf
    sp = oracle.sparse_rows(qs, ks, vs, full, w.n_tokens, rows)
    S, z = oracle.lowrank_state(kf, vf, wk, w.n_tokens, w.grid)
    lr = oracle.lowrank_rows(qf, wq, S, z, w.grid, rows)
    ref = sp + lr
    got = out[0, 0, torch.from_numpy(rows).cuda()].cpu().numpy().astype(np.float64)
    ratio = (bound_ratio8 if fp8 else bound_ratio)(got, ref, False)
    say("full keep err/rms", rel_err(got, ref), "err/bound", ratio)
    assert ratio <= 1.0
