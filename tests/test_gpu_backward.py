"""GPU parity of rola_backward (through the C ABI) against the autograd oracle.

The oracle (oracle/backward.py) differentiates a plain torch fp64 forward that
is pinned to the C oracle and to finite differences.  Both sides use the same
block map (the selection is a constant of the backward) and the same seeded
dL/dO.

Bar, per element: |g - g_ref| <= TOL * rms(g_ref) * (1 + 2^-8) + 2^-8 |g_ref|
for dq, dk, dv (stored in bf16: half an ulp of the stored value, at most
2^-8 of it, as for the forward's bf16 output) and <= TOL * rms(g_ref) for the
fp32 dwq, dwk, dgate; padded rows of dq, dk, dv exactly zero.  TOL = 3e-2:
the forward's 2e-2 widened for the bf16 operands of the backward's products
(the weights P and dS in the dk, dv products; R(q), dL/du and dS in the
low-rank sums over tokens); in dq, whose dS terms cancel over the keys, dS
enters as a bf16 pair (hi + lo), and the weights are renormalised in fp32.
"""
import numpy as np
import pytest

import oracle
from oracle import backward as OB
from sparse_rank_attention_amd import workloads as W
from tests.conftest import gpu_available
from tests.test_gpu_parity import SMALL, dev, host_f64, say, small_workload

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

TOL_BWD = 3e-2


def _torch():
    import torch
    return torch


def _ratio(got, ref, bf16_store):
    """max over elements of |got - ref| / bound (<= 1 passes)."""
    rms = np.sqrt(np.mean(ref ** 2))
    bound = TOL_BWD * rms
    if bf16_store:
        bound = bound * (1 + 2.0 ** -8) + 2.0 ** -8 * np.abs(ref)
    return float(np.max(np.abs(got - ref) / bound))


CASES = SMALL + [("d128_1280", small_workload((5, 16, 16), D=128, H=2, rank=32, topk=0.25, kind="field", seed=2))]


@pytest.mark.parametrize("name,w", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("gated", [False, True], ids=["nogate", "gate"])
@pytest.mark.parametrize("dout_f32", [False, True], ids=["dobf16", "dof32"])
def test_backward_matches_oracle(name, w, gated, dout_f32):
    from sparse_rank_attention_amd import rola
    torch = _torch()
    say("backward", name, "gate" if gated else "nogate", "f32" if dout_f32 else "bf16")
    q, k, v = W.make_qkv(w)
    wq, wk = W.make_proj(w)
    g = W.make_gate(w) if gated else None
    do = W.make_dout(w, f32=dout_f32)
    cfg = rola.Config(topk=w.topk, rank=w.rank, out_dtype=rola.ROLA_OUT_F32 if dout_f32 else rola.ROLA_OUT_BF16)
    qd, kd, vd = dev(q), dev(k), dev(v)
    bmap = rola.rola_select_blocks(qd, kd, w.grid, cfg)
    dod = torch.from_numpy(do).cuda() if dout_f32 else dev(do)
    gd = torch.from_numpy(g).cuda() if gated else None
    dq, dk, dv, dwq, dwk, dgate = rola.rola_backward(qd, kd, vd, torch.from_numpy(wq).cuda(),
                                                     torch.from_numpy(wk).cuda(), w.grid, cfg, bmap, dod, gate=gd)
    torch.cuda.synchronize()
    m_ref = oracle.block_map(q[0], k[0], w.n_tokens, w.kb)
    np.testing.assert_array_equal(bmap.cpu().numpy()[0], m_ref)
    f64 = oracle.widen_bf16
    # an fp32 dout is taken at bf16 precision (the header's contract)
    do_ref = f64(W.to_bf16_bits(do[0])) if dout_f32 else f64(do[0])
    ref = OB.backward(f64(q[0]), f64(k[0]), f64(v[0]), wq, wk, m_ref, do_ref, w.n_tokens, w.grid, gate=g)
    n = w.n_tokens
    ratios = {}
    for key, got in (("dq", dq), ("dk", dk), ("dv", dv)):
        gh = host_f64(got)[0]
        assert np.all(gh[:, n:] == 0), key
        ratios[key] = _ratio(gh[:, :n], ref[key][:, :n], True)
    ratios["dwq"] = _ratio(host_f64(dwq), ref["dwq"], False)
    ratios["dwk"] = _ratio(host_f64(dwk), ref["dwk"], False)
    if gated:
        ratios["dgate"] = _ratio(host_f64(dgate), ref["dgate"], False)
    say("backward", name, "err/bound", {k_: round(v_, 3) for k_, v_ in ratios.items()})
    for key, r in ratios.items():
        assert r <= 1.0, (key, r)


def test_backward_full_size_sampled():
    """The benchmarked backward launch (Wan 14B 720P: 40 heads, N = 75600, 35
    kept blocks of 1182, bf16 dL/dO) against the written-out gradient formulas
    (oracle.backward.backward_sampled, pinned to autograd): dq rows of sampled
    query blocks and dk, dv rows of sampled key blocks in two heads, and the
    projection gradients, which sum over all heads and tokens."""
    from sparse_rank_attention_amd import rola
    from tests.test_gpu_parity import _full_inputs
    torch = _torch()
    name = "wan14b_720p"
    say("backward full size", name)
    w, (q, k, v), (wq, wk) = _full_inputs(name)
    do = W.make_dout(w)
    cfg = rola.Config(topk=w.topk, rank=w.rank)
    qd, kd, vd = dev(q), dev(k), dev(v)
    bmap = rola.rola_select_blocks(qd, kd, w.grid, cfg)
    dq, dk, dv, dwq, dwk, _ = rola.rola_backward(qd, kd, vd, torch.from_numpy(wq).cuda(), torch.from_numpy(wk).cuda(),
                                                 w.grid, cfg, bmap, dev(do))
    torch.cuda.synchronize()
    m_ref = oracle.block_map(q[0], k[0], w.n_tokens, w.kb)
    np.testing.assert_array_equal(bmap.cpu().numpy()[0], m_ref)
    rng = np.random.default_rng(17)
    heads = (1, w.heads - 2)
    pick = lambda: sorted({n for b in {0, w.nb // 2, w.nb - 1, *rng.integers(0, w.nb, 3).tolist()}
                           for n in (b * 64, b * 64 + 33, b * 64 + 63) if n < w.n_tokens})
    q_rows = {h: pick() for h in heads}
    k_rows = {h: pick() for h in heads}
    rq, rk, rv, dwq_ref, dwk_ref, _ = OB.backward_sampled(q[0], k[0], v[0], wq, wk, m_ref, do[0], w.n_tokens, w.grid,
                                                          q_rows, k_rows)
    ratios = {}
    for h in heads:
        for key, got, rows, ref in (("dq", dq, q_rows[h], rq[h]), ("dk", dk, k_rows[h], rk[h]),
                                    ("dv", dv, k_rows[h], rv[h])):
            g = got[0, h, torch.tensor(rows, device="cuda")].float().cpu().numpy().astype(np.float64)
            ratios["%s_h%d" % (key, h)] = _ratio(g, ref, True)
    ratios["dwq"] = _ratio(host_f64(dwq), dwq_ref, False)
    ratios["dwk"] = _ratio(host_f64(dwk), dwk_ref, False)
    say("backward full size", name, "err/bound", {k_: round(v_, 3) for k_, v_ in ratios.items()})
    for key, r in ratios.items():
        assert r <= 1.0, (key, r)
