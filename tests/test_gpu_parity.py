"""GPU parity: librola (through its C ABI) against the CPU oracle on the same seeded inputs.

Bar: block maps and pooled scores bit-exact; outputs within max|O - O_ref| <=
2e-2 * rms(O_ref) over valid rows; padded rows exactly zero.  When the output
is stored in bf16, the correctly rounded storage of a result within that bound
adds up to half a bf16 ulp per element, which is at most 2^-8 |O| (8
significant bits: at the bottom of a binade half an ulp is 2^-8 of the
value), so the bound there is 2e-2 * rms * (1 + 2^-8) + 2^-8 |O_ref| (with
max|O|/rms near 10, rounding alone can reach 4e-2 * rms).
"""
import numpy as np
import pytest

import oracle
from sparse_rank_attention_amd import workloads as W
from tests.conftest import gpu_available

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

TOL_BF16 = 2e-2


def _torch():
    import torch
    return torch


def dev(bits):
    torch = _torch()
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def host_f64(t):
    torch = _torch()
    return t.float().cpu().numpy().astype(np.float64) if t.dtype != torch.float32 else t.cpu().numpy().astype(np.float64)


def rel_err(got, ref):
    rms = np.sqrt(np.mean(ref ** 2))
    return float(np.max(np.abs(got - ref)) / rms)


def bound_ratio(got, ref, bf16_out):
    """max over elements of |got - ref| / bound (<= 1 passes)."""
    rms = np.sqrt(np.mean(ref ** 2))
    bound = TOL_BF16 * rms
    if bf16_out:
        bound = bound * (1 + 2.0 ** -8) + 2.0 ** -8 * np.abs(ref)
    return float(np.max(np.abs(got - ref) / bound))


def say(*a):
    print("[case]", *a, flush=True)


def small_workload(grid, D=64, H=2, rank=16, topk=0.25, kind="iid", seed=0):
    return W.Workload("t", 1, H, D, grid, topk, rank, kind, seed=seed)


def cfg_of(w, **kw):
    from sparse_rank_attention_amd import rola
    return rola.Config(topk=w.topk, rank=w.rank, **kw)


SMALL = [
    ("tiny", W.WORKLOADS["tiny"]),
    ("ragged_d64", small_workload((3, 7, 11), D=64, H=3)),                       # N=231, tail 39
    ("ragged_d128", small_workload((5, 9, 13), D=128, H=2, rank=32, topk=0.3, kind="field")),  # N=585
    ("single_block", small_workload((1, 1, 40), D=128, H=2, rank=32, topk=1.0)),
]


@pytest.mark.parametrize("name,w", SMALL, ids=[s[0] for s in SMALL])
def test_select_blocks_bit_exact(name, w):
    from sparse_rank_attention_amd import rola
    torch = _torch()
    say("select", name)
    q, k, _ = W.make_qkv(w)
    qd, kd = dev(q), dev(k)
    scores = torch.empty((w.batch, w.heads, w.nb, w.nb), dtype=torch.float32, device="cuda")
    bmap = rola.rola_select_blocks(qd, kd, w.grid, cfg_of(w), pooled_scores=scores)
    torch.cuda.synchronize()
    qp = oracle.pool(q.reshape(-1, w.n_pad, w.head_dim), w.n_tokens)
    kp = oracle.pool(k.reshape(-1, w.n_pad, w.head_dim), w.n_tokens)
    s_ref = oracle.scores(qp, kp)
    m_ref = oracle.select(s_ref, oracle.keep_blocks(w.topk, w.nb))
    got_s = scores.cpu().numpy().reshape(s_ref.shape)
    assert np.array_equal(got_s.view(np.uint32), s_ref.view(np.uint32)), "pooled scores differ bitwise"
    np.testing.assert_array_equal(bmap.cpu().numpy().reshape(m_ref.shape), m_ref)


@pytest.mark.parametrize("name,w", SMALL, ids=[s[0] for s in SMALL])
@pytest.mark.parametrize("out_f32", [False, True], ids=["bf16out", "f32out"])
def test_forward_matches_oracle(name, w, out_f32):
    from sparse_rank_attention_amd import rola
    torch = _torch()
    say("forward", name, "f32" if out_f32 else "bf16")
    q, k, v = W.make_qkv(w)
    wq, wk = W.make_proj(w)
    bmap = torch.full((w.batch, w.heads, w.nb, oracle.keep_blocks(w.topk, w.nb)), -1, dtype=torch.int32, device="cuda")
    cfg = cfg_of(w, out_dtype=rola.ROLA_OUT_F32 if out_f32 else rola.ROLA_OUT_BF16)
    out = rola.rola_forward(dev(q), dev(k), dev(v), torch.from_numpy(wq).cuda(), torch.from_numpy(wk).cuda(),
                            w.grid, cfg, block_idx_out=bmap)
    torch.cuda.synchronize()
    m_ref, o_ref = oracle.forward(q[0], k[0], v[0], wq, wk, w.n_tokens, oracle.keep_blocks(w.topk, w.nb), w.grid)
    np.testing.assert_array_equal(bmap.cpu().numpy()[0], m_ref)
    got = host_f64(out)[0]
    assert np.all(got[:, w.n_tokens:] == 0)
    err = rel_err(got[:, :w.n_tokens], o_ref[:, :w.n_tokens])
    ratio = bound_ratio(got[:, :w.n_tokens], o_ref[:, :w.n_tokens], not out_f32)
    say("forward", name, "err/rms", err, "err/bound", ratio)
    assert ratio <= 1.0


@pytest.mark.parametrize("name,w", SMALL[:3], ids=[s[0] for s in SMALL[:3]])
def test_branches_alone_and_composed(name, w):
    from sparse_rank_attention_amd import rola
    torch = _torch()
    say("branches", name)
    q, k, v = W.make_qkv(w)
    wq, wk = W.make_proj(w)
    qd, kd, vd = dev(q), dev(k), dev(v)
    wqd, wkd = torch.from_numpy(wq).cuda(), torch.from_numpy(wk).cuda()
    cfg = cfg_of(w, out_dtype=rola.ROLA_OUT_F32)
    m_ref = oracle.block_map(q[0], k[0], w.n_tokens, oracle.keep_blocks(w.topk, w.nb))
    bmap = torch.from_numpy(m_ref).cuda().reshape(w.batch, w.heads, w.nb, oracle.keep_blocks(w.topk, w.nb))
    o_sp = rola.rola_sparse_attn(qd, kd, vd, bmap, w.grid, cfg)
    o_lr = rola.rola_lowrank_attn(qd, kd, vd, wqd, wkd, w.grid, cfg)
    o_sum = rola.rola_sparse_attn(qd, kd, vd, bmap, w.grid, cfg)
    rola.rola_lowrank_attn(qd, kd, vd, wqd, wkd, w.grid, cfg, out=o_sum, accumulate=True)
    o_fw = rola.rola_forward(qd, kd, vd, wqd, wkd, w.grid, cfg)
    torch.cuda.synchronize()
    qf, kf, vf = (oracle.widen_bf16(x[0]) for x in (q, k, v))
    rows = np.array([bh * w.n_pad + n for bh in range(w.heads) for n in range(w.n_tokens)])
    sp_ref = oracle.sparse_rows(qf, kf, vf, m_ref, w.n_tokens, rows)
    S, z = oracle.lowrank_state(kf, vf, wk, w.n_tokens, w.grid)
    lr_ref = oracle.lowrank_rows(qf, wq, S, z, w.grid, rows)
    take = lambda t: host_f64(t)[0][:, :w.n_tokens].reshape(-1, w.head_dim)
    e_sp = rel_err(take(o_sp), sp_ref)
    e_lr = rel_err(take(o_lr), lr_ref)
    e_sum = rel_err(take(o_sum), sp_ref + lr_ref)
    say("branches", name, "sparse", e_sp, "lowrank", e_lr, "sum", e_sum)
    assert e_sp <= TOL_BF16 and e_lr <= TOL_BF16 and e_sum <= TOL_BF16
    # the fused forward equals the two calls up to fp32 summation order
    np.testing.assert_allclose(take(o_fw), take(o_sum), rtol=0, atol=1e-5 * np.abs(take(o_sum)).max())


def test_full_keep_equals_dense_attention():
    from sparse_rank_attention_amd import rola
    torch = _torch()
    say("dense calibration")
    w = small_workload((2, 10, 19), D=128, H=2, rank=32, topk=1.0)  # N=380, nb=6, tail 60
    q, k, v = W.make_qkv(w)
    cfg = cfg_of(w, out_dtype=rola.ROLA_OUT_F32, kb_override=w.nb)
    bmap = torch.arange(w.nb, dtype=torch.int32, device="cuda").repeat(w.batch, w.heads, w.nb, 1).contiguous()
    out = rola.rola_sparse_attn(dev(q), dev(k), dev(v), bmap, w.grid, cfg)
    torch.cuda.synchronize()
    got = host_f64(out)[0]
    for h in range(w.heads):
        qf, kf, vf = (oracle.widen_bf16(x[0, h, :w.n_tokens]) for x in (q, k, v))
        s = qf @ kf.T / np.sqrt(w.head_dim)
        p = np.exp(s - s.max(axis=1, keepdims=True))
        ref = (p @ vf) / p.sum(axis=1, keepdims=True)
        assert rel_err(got[h, :w.n_tokens], ref) <= TOL_BF16


def test_strided_token_major_layout():
    """Q/K/V/O stored token-major [B, N, H, D] (the DiT layout) give the same result."""
    from sparse_rank_attention_amd import rola
    torch = _torch()
    say("strided layout")
    w = small_workload((3, 7, 11), D=128, H=3, rank=32, topk=0.5, kind="field")
    q, k, v = W.make_qkv(w)
    wq, wk = W.make_proj(w)
    wqd, wkd = torch.from_numpy(wq).cuda(), torch.from_numpy(wk).cuda()
    cfg = cfg_of(w)
    ref = rola.rola_forward(dev(q), dev(k), dev(v), wqd, wkd, w.grid, cfg)
    tm = [dev(x).permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3) for x in (q, k, v)]
    out = torch.empty_like(tm[0])  # same token-major strides
    rola.rola_forward(tm[0], tm[1], tm[2], wqd, wkd, w.grid, cfg, out=out)
    torch.cuda.synchronize()
    assert torch.equal(out.contiguous(), ref)


def test_repeatable_bitwise():
    from sparse_rank_attention_amd import rola
    torch = _torch()
    w = small_workload((5, 9, 13), D=128, H=2, rank=32, topk=0.3, kind="field")
    q, k, v = (dev(x) for x in W.make_qkv(w))
    wq, wk = (torch.from_numpy(x).cuda() for x in W.make_proj(w))
    a = rola.rola_forward(q, k, v, wq, wk, w.grid, cfg_of(w))
    b = rola.rola_forward(q, k, v, wq, wk, w.grid, cfg_of(w))
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_invalid_rows_of_inputs_are_ignored():
    """Garbage (NaN) in padded input rows changes nothing."""
    from sparse_rank_attention_amd import rola
    torch = _torch()
    w = small_workload((3, 7, 11), D=64, H=2)
    q, k, v = (dev(x) for x in W.make_qkv(w))
    wq, wk = (torch.from_numpy(x).cuda() for x in W.make_proj(w))
    a = rola.rola_forward(q, k, v, wq, wk, w.grid, cfg_of(w))
    for t in (q, k, v):
        t[:, :, w.n_tokens:] = float("nan")
    b = rola.rola_forward(q, k, v, wq, wk, w.grid, cfg_of(w))
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_standalone_sparse_bf16_output():
    """rola_sparse_attn with bf16 output (its own fp16 copy of V) against the oracle's sparse rows."""
    from sparse_rank_attention_amd import rola
    torch = _torch()
    say("standalone sparse, bf16 out")
    w = small_workload((5, 9, 13), D=128, H=2, rank=32, topk=0.3, kind="field")
    q, k, v = W.make_qkv(w)
    kb = oracle.keep_blocks(w.topk, w.nb)
    m_ref = oracle.block_map(q[0], k[0], w.n_tokens, kb)
    bmap = torch.from_numpy(m_ref).cuda().reshape(w.batch, w.heads, w.nb, kb)
    out = rola.rola_sparse_attn(dev(q), dev(k), dev(v), bmap, w.grid, cfg_of(w))
    torch.cuda.synchronize()
    qf, kf, vf = (oracle.widen_bf16(x[0]) for x in (q, k, v))
    rows = np.arange(w.n_tokens)
    for h in range(w.heads):
        ref = oracle.sparse_rows(qf[h:h + 1], kf[h:h + 1], vf[h:h + 1], m_ref[h:h + 1], w.n_tokens, rows)
        assert bound_ratio(host_f64(out)[0, h, :w.n_tokens], ref, True) <= 1.0, h


def test_v_beyond_fp16_range_takes_bf16_form():
    """A head whose V holds a value at or beyond 2^16 (outside fp16) is computed by the
    bf16 form: its bf16 output is the fp32 output rounded to bf16, bit for bit, and
    every head still meets the bar; the fused and the standalone calls alike."""
    from sparse_rank_attention_amd import rola
    torch = _torch()
    say("V beyond fp16 range")
    w = small_workload((5, 9, 13), D=128, H=3, rank=32, topk=0.3, kind="field")
    q, k, v = W.make_qkv(w)
    v = v.copy()
    big = np.array([1.0e5, -7.0e4], dtype=np.float32).view(np.uint32) >> 16  # bf16 99840, -70144
    v[0, 1, 100, 3] = big[0]
    v[0, 2, w.n_tokens - 1, 77] = big[1]
    wq, wk = W.make_proj(w)
    qd, kd, vd = dev(q), dev(k), dev(v)
    wqd, wkd = torch.from_numpy(wq).cuda(), torch.from_numpy(wk).cuda()
    kb = oracle.keep_blocks(w.topk, w.nb)
    o16 = rola.rola_forward(qd, kd, vd, wqd, wkd, w.grid, cfg_of(w))
    o32 = rola.rola_forward(qd, kd, vd, wqd, wkd, w.grid, cfg_of(w, out_dtype=rola.ROLA_OUT_F32))
    m_ref = oracle.block_map(q[0], k[0], w.n_tokens, kb)
    bmap = torch.from_numpy(m_ref).cuda().reshape(w.batch, w.heads, w.nb, kb)
    s16 = rola.rola_sparse_attn(qd, kd, vd, bmap, w.grid, cfg_of(w))
    s32 = rola.rola_sparse_attn(qd, kd, vd, bmap, w.grid, cfg_of(w, out_dtype=rola.ROLA_OUT_F32))
    torch.cuda.synchronize()
    for a, b in ((o16, o32), (s16, s32)):
        for h in (1, 2):
            assert torch.equal(a[0, h], b[0, h].to(torch.bfloat16)), h
    _, o_ref = oracle.forward(q[0], k[0], v[0], wq, wk, w.n_tokens, kb, w.grid)
    qf, kf, vf = (oracle.widen_bf16(x[0]) for x in (q, k, v))
    rows = np.arange(w.n_tokens)
    for h in range(w.heads):
        assert bound_ratio(host_f64(o16)[0, h, :w.n_tokens], o_ref[h, :w.n_tokens], True) <= 1.0, h
        sp = oracle.sparse_rows(qf[h:h + 1], kf[h:h + 1], vf[h:h + 1], m_ref[h:h + 1], w.n_tokens, rows)
        assert bound_ratio(host_f64(s16)[0, h, :w.n_tokens], sp, True) <= 1.0, h


# --------------------------------------------------------------- full sizes
FULL = ["wan13b_480p", "wan14b_480p", "wan14b_720p"]
_cache = {}


def _full_inputs(name):
    if name not in _cache:
        _cache.clear()
        w = W.WORKLOADS[name]
        _cache[name] = (w, W.make_qkv(w), W.make_proj(w))
    return _cache[name]


@pytest.mark.parametrize("name", FULL)
def test_full_size_sampled(name):
    """The benchmarked launch (all heads, full N) checked on sampled heads and rows:
    the whole block map of each sampled head bit-exact, sampled output rows
    (first, last, tail and random query blocks) within tolerance, padded rows zero."""
    from sparse_rank_attention_amd import rola
    torch = _torch()
    say("full size", name)
    w, (q, k, v), (wq, wk) = _full_inputs(name)
    bmap = torch.empty((w.batch, w.heads, w.nb, oracle.keep_blocks(w.topk, w.nb)), dtype=torch.int32, device="cuda")
    out = rola.rola_forward(dev(q), dev(k), dev(v), torch.from_numpy(wq).cuda(), torch.from_numpy(wk).cuda(),
                            w.grid, cfg_of(w), block_idx_out=bmap)
    torch.cuda.synchronize()
    bmap = bmap.cpu().numpy()
    rng = np.random.default_rng(123)
    heads = sorted({0, w.heads // 2, w.heads - 1})
    worst = 0.0
    for h in heads:
        m_ref = oracle.block_map(q[0, h:h + 1], k[0, h:h + 1], w.n_tokens, oracle.keep_blocks(w.topk, w.nb))
        np.testing.assert_array_equal(bmap[0, h], m_ref[0], err_msg="head %d" % h)
        qbs = sorted({0, 1, w.nb // 2, w.nb - 1, *rng.integers(0, w.nb, 4).tolist()})
        rows = []
        for qb in qbs:
            rows += [n for n in (qb * 64, qb * 64 + 17, qb * 64 + 40, qb * 64 + 63) if n < w.n_tokens]
        rows += [w.n_tokens - 1]
        rows = np.array(sorted(set(rows)))
        qf, kf, vf = (oracle.widen_bf16(x[0, h:h + 1]) for x in (q, k, v))
        sp = oracle.sparse_rows(qf, kf, vf, m_ref, w.n_tokens, rows)
        S, z = oracle.lowrank_state(kf, vf, wk, w.n_tokens, w.grid)
        lr = oracle.lowrank_rows(qf, wq, S, z, w.grid, rows)
        got = out[0, h, torch.from_numpy(rows).cuda()].float().cpu().numpy().astype(np.float64)
        err = rel_err(got, sp + lr)
        ratio = bound_ratio(got, sp + lr, True)
        worst = max(worst, err)
        assert ratio <= 1.0, (h, err, ratio)
        pad = out[0, h, w.n_tokens:].float()
        assert torch.count_nonzero(pad).item() == 0
    say("full size", name, "worst err/rms", worst)


@pytest.mark.parametrize("name", FULL)
def test_full_size_every_block_map(name):
    """The block map of every head of the benchmarked launch, bit for bit."""
    from sparse_rank_attention_amd import rola
    torch = _torch()
    say("full size, every head's map", name)
    w, (q, k, v), (wq, wk) = _full_inputs(name)
    kb = oracle.keep_blocks(w.topk, w.nb)
    bmap = torch.empty((w.batch, w.heads, w.nb, kb), dtype=torch.int32, device="cuda")
    rola.rola_forward(dev(q), dev(k), dev(v), torch.from_numpy(wq).cuda(), torch.from_numpy(wk).cuda(),
                      w.grid, cfg_of(w), block_idx_out=bmap)
    torch.cuda.synchronize()
    m_ref = oracle.block_map(q[0], k[0], w.n_tokens, kb)  # all heads, threads over heads
    got = bmap.cpu().numpy()[0]
    bad = [h for h in range(w.heads) if not np.array_equal(got[h], m_ref[h])]
    assert not bad, "heads with a differing map: %s" % bad


@pytest.mark.parametrize("name", FULL)
def test_full_size_every_row_bf16(name):
    """Every valid row of the first, middle and last head of the benchmarked launch (bf16
    output) against the bf16 bound, 2e-2 * rms * (1 + 2^-8) + 2^-8 |O_ref|."""
    from sparse_rank_attention_amd import rola
    torch = _torch()
    w, (q, k, v), (wq, wk) = _full_inputs(name)
    kb = oracle.keep_blocks(w.topk, w.nb)
    out = rola.rola_forward(dev(q), dev(k), dev(v), torch.from_numpy(wq).cuda(), torch.from_numpy(wk).cuda(),
                            w.grid, cfg_of(w))
    torch.cuda.synchronize()
    rows = np.arange(w.n_tokens)
    res = {}
    for h in sorted({0, w.heads // 2, w.heads - 1}):
        say("full size bf16 rows", name, "head", h)
        m_ref = oracle.block_map(q[0, h:h + 1], k[0, h:h + 1], w.n_tokens, kb)
        qf, kf, vf = (oracle.widen_bf16(x[0, h:h + 1]) for x in (q, k, v))
        S, z = oracle.lowrank_state(kf, vf, wk, w.n_tokens, w.grid)
        ref = oracle.sparse_rows(qf, kf, vf, m_ref, w.n_tokens, rows) + oracle.lowrank_rows(qf, wq, S, z, w.grid, rows)
        got = out[0, h, :w.n_tokens].float().cpu().numpy().astype(np.float64)
        res[h] = (round(rel_err(got, ref), 5), round(bound_ratio(got, ref, True), 4))
        assert res[h][1] <= 1.0, (h, res[h])
    say("full size bf16 rows", name, "(err/rms, err/bound) per head", res)


@pytest.mark.parametrize("name", FULL)
def test_full_size_every_row_fp32(name):
    """Every valid row of the first, middle and last head of the benchmarked launch,
    with fp32 output, against the plain bar max|O - O_ref| <= 2e-2 * rms(O_ref)
    (no storage term: nothing is rounded to bf16 on the way out)."""
    from sparse_rank_attention_amd import rola
    torch = _torch()
    w, (q, k, v), (wq, wk) = _full_inputs(name)
    kb = oracle.keep_blocks(w.topk, w.nb)
    cfg = cfg_of(w, out_dtype=rola.ROLA_OUT_F32)
    out = rola.rola_forward(dev(q), dev(k), dev(v), torch.from_numpy(wq).cuda(), torch.from_numpy(wk).cuda(),
                            w.grid, cfg)
    torch.cuda.synchronize()
    rows = np.arange(w.n_tokens)
    errs = {}
    for h in sorted({0, w.heads // 2, w.heads - 1}):
        say("full size fp32 rows", name, "head", h)
        m_ref = oracle.block_map(q[0, h:h + 1], k[0, h:h + 1], w.n_tokens, kb)
        qf, kf, vf = (oracle.widen_bf16(x[0, h:h + 1]) for x in (q, k, v))
        S, z = oracle.lowrank_state(kf, vf, wk, w.n_tokens, w.grid)
        ref = oracle.sparse_rows(qf, kf, vf, m_ref, w.n_tokens, rows) + oracle.lowrank_rows(qf, wq, S, z, w.grid, rows)
        got = out[0, h, :w.n_tokens].cpu().numpy().astype(np.float64)
        errs[h] = rel_err(got, ref)
        assert errs[h] <= TOL_BF16, (h, errs[h])
        assert torch.count_nonzero(out[0, h, w.n_tokens:]).item() == 0
    say("full size fp32 rows", name, "err/rms per head", {h: round(e, 5) for h, e in errs.items()})
