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
from tests.test_gpu_parity import SMALL, bound_ratio, dev, host_f64, say, small_workload

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

TOL_BWD = 3e-2


def _torch():
    import torch
    return torch


def _ratio(got, ref, bf16_store):
    """max over elements of |got - ref| / bound (<= 1 passes); a reference that is
    exactly zero (no low-rank term at all) must be matched exactly."""
    rms = np.sqrt(np.mean(ref ** 2))
    if rms == 0.0:
        return 0.0 if np.all(got == 0) else float("inf")
    bound = TOL_BWD * rms
    if bf16_store:
        bound = bound * (1 + 2.0 ** -8) + 2.0 ** -8 * np.abs(ref)
    return float(np.max(np.abs(got - ref) / bound))


CASES = SMALL + [("d128_1280", small_workload((5, 16, 16), D=128, H=2, rank=32, topk=0.25, kind="field", seed=2)),
                 ("two_batches", W.Workload("b2", 2, 2, 64, (3, 7, 11), 0.25, 16, "iid", seed=3))]


def _backward_case(name, w, gated, dout_f32, complement=False):
    from sparse_rank_attention_amd import rola
    torch = _torch()
    say("backward", name, "complement" if complement else "global", "gate" if gated else "nogate",
        "f32" if dout_f32 else "bf16")
    q, k, v = W.make_qkv(w)
    wq, wk = W.make_proj(w)
    g = W.make_gate(w) if gated else None
    do = W.make_dout(w, f32=dout_f32)
    cfg = rola.Config(topk=w.topk, rank=w.rank, out_dtype=rola.ROLA_OUT_F32 if dout_f32 else rola.ROLA_OUT_BF16,
                      lowrank_scope=rola.ROLA_LR_COMPLEMENT if complement else rola.ROLA_LR_GLOBAL)
    qd, kd, vd = dev(q), dev(k), dev(v)
    bmap = rola.rola_select_blocks(qd, kd, w.grid, cfg)
    dod = torch.from_numpy(do).cuda() if dout_f32 else dev(do)
    gd = torch.from_numpy(g).cuda() if gated else None
    dq, dk, dv, dwq, dwk, dgate = rola.rola_backward(qd, kd, vd, torch.from_numpy(wq).cuda(),
                                                     torch.from_numpy(wk).cuda(), w.grid, cfg, bmap, dod, gate=gd)
    torch.cuda.synchronize()
    # batches and heads flattened: [B*H, n_pad, D]
    flat = lambda x: x.reshape(w.batch * w.heads, w.n_pad, -1)
    kb = oracle.keep_blocks(w.topk, w.nb)
    m_ref = oracle.block_map(flat(q), flat(k), w.n_tokens, kb)
    np.testing.assert_array_equal(bmap.cpu().numpy().reshape(-1, w.nb, kb), m_ref)
    f64 = oracle.widen_bf16
    # an fp32 dout is taken at bf16 precision (the header's contract)
    do_ref = f64(W.to_bf16_bits(flat(do))) if dout_f32 else f64(flat(do))
    ref = OB.backward(f64(flat(q)), f64(flat(k)), f64(flat(v)), wq, wk, m_ref, do_ref, w.n_tokens, w.grid, gate=g,
                      complement=complement)
    n = w.n_tokens
    ratios = {}
    for key, got in (("dq", dq), ("dk", dk), ("dv", dv)):
        gh = flat(host_f64(got))
        assert np.all(gh[:, n:] == 0), key
        ratios[key] = _ratio(gh[:, :n], ref[key][:, :n], True)
    ratios["dwq"] = _ratio(host_f64(dwq), ref["dwq"], False)
    ratios["dwk"] = _ratio(host_f64(dwk), ref["dwk"], False)
    if gated:
        ratios["dgate"] = _ratio(host_f64(dgate), ref["dgate"], False)
    say("backward", name, "err/bound", {k_: round(v_, 3) for k_, v_ in ratios.items()})
    for key, r in ratios.items():
        assert r <= 1.0, (key, r)


@pytest.mark.parametrize("name,w", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("gated", [False, True], ids=["nogate", "gate"])
@pytest.mark.parametrize("dout_f32", [False, True], ids=["dobf16", "dof32"])
def test_backward_matches_oracle(name, w, gated, dout_f32):
    _backward_case(name, w, gated, dout_f32)


# The complement scope: each query block's low-rank sums run over the key
# blocks it does not keep (single_block keeps its only block: no low-rank term).
@pytest.mark.parametrize("name,w", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("gated,dout_f32", [(False, False), (True, True)], ids=["nogate-dobf16", "gate-dof32"])
def test_backward_complement_matches_oracle(name, w, gated, dout_f32):
    _backward_case(name, w, gated, dout_f32, complement=True)


@pytest.mark.parametrize("saved", [False, True], ids=["recompute", "saved"])
def test_backward_full_size_sampled(saved):
    """The benchmarked backward launch (Wan 14B 720P: 40 heads, N = 75600, 35
    kept blocks of 1182, bf16 dL/dO) against the written-out gradient formulas
    (oracle.backward.backward_sampled, pinned to autograd): dq rows of sampled
    query blocks and dk, dv rows of sampled key blocks in two heads, and the
    projection gradients, which sum over all heads and tokens.  ``saved``: the
    backward takes O_s and the log-sum-exp of rola_forward_train (bf16 output)
    instead of recomputing them."""
    from sparse_rank_attention_amd import rola
    from tests.test_gpu_parity import _full_inputs
    torch = _torch()
    name = "wan14b_720p"
    say("backward full size", name, "saved" if saved else "recompute")
    w, (q, k, v), (wq, wk) = _full_inputs(name)
    do = W.make_dout(w)
    cfg = rola.Config(topk=w.topk, rank=w.rank)
    qd, kd, vd = dev(q), dev(k), dev(v)
    wqd, wkd = torch.from_numpy(wq).cuda(), torch.from_numpy(wk).cuda()
    if saved:
        info = rola.plan(rola.problem(qd, w.grid), cfg)
        bmap = torch.empty((w.batch, w.heads, info.nb, info.kb), dtype=torch.int32, device="cuda")
        _, os_, lse = rola.rola_forward_train(qd, kd, vd, wqd, wkd, w.grid, cfg, block_idx_out=bmap)
        pair = (os_, lse)
    else:
        bmap = rola.rola_select_blocks(qd, kd, w.grid, cfg)
        pair = None
    dq, dk, dv, dwq, dwk, _ = rola.rola_backward(qd, kd, vd, wqd, wkd, w.grid, cfg, bmap, dev(do), saved=pair)
    torch.cuda.synchronize()
    m_ref = oracle.block_map(q[0], k[0], w.n_tokens, oracle.keep_blocks(w.topk, w.nb))
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


@pytest.mark.parametrize("saved", [False, True], ids=["recompute", "saved"])
def test_backward_complement_full_size_sampled(saved):
    """The complement-scope backward at the benchmarked size (Wan 14B 720P, bf16
    dL/dO) against the written-out formulas in that scope
    (oracle.backward.backward_sampled, pinned to autograd): dq rows of sampled
    query blocks and dk, dv rows of sampled key blocks in two heads.  The
    projection gradients sum over all 40 heads; the small cases cover them.
    ``saved``: with O_s and the log-sum-exp of rola_forward_train."""
    from sparse_rank_attention_amd import rola
    from tests.test_gpu_parity import _full_inputs
    torch = _torch()
    name = "wan14b_720p"
    say("backward complement full size", name, "saved" if saved else "recompute")
    w, (q, k, v), (wq, wk) = _full_inputs(name)
    do = W.make_dout(w)
    cfg = rola.Config(topk=w.topk, rank=w.rank, lowrank_scope=rola.ROLA_LR_COMPLEMENT)
    qd, kd, vd = dev(q), dev(k), dev(v)
    wqd, wkd = torch.from_numpy(wq).cuda(), torch.from_numpy(wk).cuda()
    if saved:
        info = rola.plan(rola.problem(qd, w.grid), cfg)
        bmap = torch.empty((w.batch, w.heads, info.nb, info.kb), dtype=torch.int32, device="cuda")
        _, os_, lse = rola.rola_forward_train(qd, kd, vd, wqd, wkd, w.grid, cfg, block_idx_out=bmap)
        pair = (os_, lse)
    else:
        bmap = rola.rola_select_blocks(qd, kd, w.grid, cfg)
        pair = None
    dq, dk, dv, _, _, _ = rola.rola_backward(qd, kd, vd, wqd, wkd, w.grid, cfg, bmap, dev(do), saved=pair)
    torch.cuda.synchronize()
    heads = (1, w.heads - 2)
    maps = bmap.cpu().numpy()[0]
    for h in heads:
        np.testing.assert_array_equal(maps[h], oracle.block_map(q[0][h:h + 1], k[0][h:h + 1], w.n_tokens,
                                                                oracle.keep_blocks(w.topk, w.nb))[0])
    rng = np.random.default_rng(19)
    pick = lambda: sorted({n for b in {0, w.nb // 2, w.nb - 1, *rng.integers(0, w.nb, 3).tolist()}
                           for n in (b * 64, b * 64 + 33, b * 64 + 63) if n < w.n_tokens})
    q_rows = {h: pick() for h in heads}
    k_rows = {h: pick() for h in heads}
    rq, rk, rv, _, _, _ = OB.backward_sampled(q[0], k[0], v[0], wq, wk, maps, do[0], w.n_tokens, w.grid,
                                              q_rows, k_rows, complement=True, heads=heads)
    ratios = {}
    for h in heads:
        for key, got, rows, ref in (("dq", dq, q_rows[h], rq[h]), ("dk", dk, k_rows[h], rk[h]),
                                    ("dv", dv, k_rows[h], rv[h])):
            g = got[0, h, torch.tensor(rows, device="cuda")].float().cpu().numpy().astype(np.float64)
            ratios["%s_h%d" % (key, h)] = _ratio(g, ref, True)
    say("backward complement full size", name, "err/bound", {k_: round(v_, 3) for k_, v_ in ratios.items()})
    for key, r in ratios.items():
        assert r <= 1.0, (key, r)


def test_long_union_lists():
    """Union lists longer than the 2048 entries the kernels stage in LDS: 2051 key blocks
    (N = 131241) with 2000 kept per query block, so that group unions pass 2048 entries.
    The forward's attention kernel then reads the list tail from HBM, and the backward's dq
    takes the per-query-block kernel.  Forward rows and dq rows of sampled query blocks, and
    the projection gradients, against the oracle (dk, dv need every query row's softmax
    at this size and are covered by the other cases)."""
    from sparse_rank_attention_amd import rola
    torch = _torch()
    w = small_workload((3, 41, 1067), D=64, H=1, rank=16, topk=1.0, kind="field", seed=5)
    kb = 2000
    say("long union lists", w.nb, "blocks,", kb, "kept")
    q, k, v = W.make_qkv(w)
    wq, wk = W.make_proj(w)
    do = W.make_dout(w)
    cfg = rola.Config(topk=1.0, rank=w.rank, kb_override=kb)
    qd, kd, vd = dev(q), dev(k), dev(v)
    wqd, wkd = torch.from_numpy(wq).cuda(), torch.from_numpy(wk).cuda()
    bmap = rola.rola_select_blocks(qd, kd, w.grid, cfg)
    out = rola.rola_forward(qd, kd, vd, wqd, wkd, w.grid, cfg)
    dq, dk, dv, dwq, dwk, _ = rola.rola_backward(qd, kd, vd, wqd, wkd, w.grid, cfg, bmap, dev(do))
    torch.cuda.synchronize()
    m_ref = oracle.block_map(q[0], k[0], w.n_tokens, kb)
    np.testing.assert_array_equal(bmap.cpu().numpy()[0], m_ref)
    rows = sorted({n for b in (0, 977, w.nb - 1) for n in (b * 64, b * 64 + 40) if n < w.n_tokens})
    rows_a = np.array(rows)
    qf, kf, vf = (oracle.widen_bf16(x[0]) for x in (q, k, v))
    S, z = oracle.lowrank_state(kf, vf, wk, w.n_tokens, w.grid)
    o_ref = oracle.sparse_rows(qf, kf, vf, m_ref, w.n_tokens, rows_a) + oracle.lowrank_rows(qf, wq, S, z, w.grid,
                                                                                            rows_a)
    got = out[0, 0, torch.tensor(rows, device="cuda")].float().cpu().numpy().astype(np.float64)
    r_fwd = bound_ratio(got, o_ref, True)  # the forward's bar, 2e-2
    rq, _, _, dwq_ref, dwk_ref, _ = OB.backward_sampled(q[0], k[0], v[0], wq, wk, m_ref, do[0], w.n_tokens,
                                                       w.grid, {0: rows}, {0: []})
    g = dq[0, 0, torch.tensor(rows, device="cuda")].float().cpu().numpy().astype(np.float64)
    ratios = {"fwd": r_fwd, "dq": _ratio(g, rq[0], True), "dwq": _ratio(host_f64(dwq), dwq_ref, False),
              "dwk": _ratio(host_f64(dwk), dwk_ref, False)}
    say("long union lists err/bound", {k_: round(v_, 3) for k_, v_ in ratios.items()})
    for key, r in ratios.items():
        assert r <= 1.0, (key, r)


@pytest.mark.parametrize("complement", [False, True], ids=["global", "complement"])
def test_backward_layouts_and_padding(complement):
    """The backward on token-major views ([B, N, H, D] storage, the DiT layout)
    and with NaN in every padded input row (q, k, v and dL/dO rows >= N) gives
    the gradients of the head-major call bit for bit."""
    from sparse_rank_attention_amd import rola
    torch = _torch()
    say("backward layouts", "complement" if complement else "global")
    w = small_workload((3, 7, 11), D=128, H=3, rank=32, topk=0.5, kind="field", seed=6)
    q, k, v = W.make_qkv(w)
    wq, wk = W.make_proj(w)
    do = W.make_dout(w)
    wqd, wkd = torch.from_numpy(wq).cuda(), torch.from_numpy(wk).cuda()
    cfg = rola.Config(topk=w.topk, rank=w.rank,
                      lowrank_scope=rola.ROLA_LR_COMPLEMENT if complement else rola.ROLA_LR_GLOBAL)
    qd, kd, vd, dod = dev(q), dev(k), dev(v), dev(do)
    bmap = rola.rola_select_blocks(qd, kd, w.grid, cfg)
    ref = rola.rola_backward(qd, kd, vd, wqd, wkd, w.grid, cfg, bmap, dod)
    # token-major storage, same values
    tm = [x.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3) for x in (qd, kd, vd, dod)]
    got = rola.rola_backward(tm[0], tm[1], tm[2], wqd, wkd, w.grid, cfg, bmap, tm[3])
    # NaN in the padded rows of every input
    nan_in = [x.clone() for x in (qd, kd, vd, dod)]
    for x in nan_in:
        x[:, :, w.n_tokens:] = float("nan")
    got_nan = rola.rola_backward(nan_in[0], nan_in[1], nan_in[2], wqd, wkd, w.grid, cfg, bmap, nan_in[3])
    torch.cuda.synchronize()
    bits = lambda t: t.contiguous().view(torch.int16) if t.dtype == torch.bfloat16 else t.contiguous().view(torch.int32)
    for name, a, b, c in zip(("dq", "dk", "dv", "dwq", "dwk"), ref[:5], got[:5], got_nan[:5]):
        assert torch.equal(bits(a), bits(b)), ("token-major", name)
        assert torch.equal(bits(a), bits(c)), ("padded NaN", name)
