"""Pins for the oracle's sparse branch, 3-D rotary embedding, low-rank branch and fp8 codes.

References used here are independent of the oracle: dense softmax attention
and torch's scaled_dot_product_attention (fp64, CPU) as special cases, the
textbook complex-number form of 1-D rotary embedding, the quadratic form of
linear attention, torch's elu and float8_e4m3fn conversion, and closed forms.
"""
import json
import os

import numpy as np

import oracle
import pytest
import torch

from sparse_rank_attention_amd.workloads import to_bf16_bits

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _bf16(rng, shape, scale=1.0):
    x = to_bf16_bits((rng.standard_normal(shape) * scale).astype(np.float32))
    return x, (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _dense_attention(q, k, v, n_valid, scale):
    s = (q[:n_valid] @ k[:n_valid].T) * scale
    s -= s.max(axis=1, keepdims=True)
    p = np.exp(s)
    return (p @ v[:n_valid]) / p.sum(axis=1, keepdims=True)


# ------------------------------------------------------------ sparse branch
@pytest.mark.parametrize("n_valid", [64 * 6, 64 * 5 + 23])
def test_sparse_full_keep_equals_dense(oracle_lib, n_valid):
    rng = np.random.default_rng(20)
    n_pad, d = 64 * 6, 32
    _, q = _bf16(rng, (2, n_pad, d))
    _, k = _bf16(rng, (2, n_pad, d))
    _, v = _bf16(rng, (2, n_pad, d))
    k[:, n_valid:] = 1e3  # padded keys must not be attended
    nb = n_pad // 64
    bmap = np.tile(np.arange(nb, dtype=np.int32), (2, nb, 1))
    rows = np.array([bh * n_pad + n for bh in range(2) for n in range(n_valid)])
    out = oracle_lib.sparse_rows(q, k, v, bmap, n_valid, rows).reshape(2, n_valid, d)
    for bh in range(2):
        ref = _dense_attention(q[bh], k[bh], v[bh], n_valid, d ** -0.5)
        np.testing.assert_allclose(out[bh], ref, rtol=1e-12, atol=1e-12)


def test_sparse_equals_sdpa_with_block_mask(oracle_lib):
    rng = np.random.default_rng(21)
    n_pad, d, nb, kb = 64 * 8, 64, 8, 3
    n_valid = n_pad - 40
    _, q = _bf16(rng, (1, n_pad, d))
    _, k = _bf16(rng, (1, n_pad, d))
    _, v = _bf16(rng, (1, n_pad, d))
    bmap = np.sort(np.stack([rng.choice(nb, kb, replace=False) for _ in range(nb)]), axis=1)[None]
    bmap = bmap.astype(np.int32)
    rows = np.arange(n_valid)
    out = oracle_lib.sparse_rows(q, k, v, bmap, n_valid, rows)
    allowed = np.zeros((n_valid, n_valid), dtype=bool)
    for i in range(nb):
        for j in bmap[0, i]:
            allowed[i * 64:(i + 1) * 64, j * 64:(j + 1) * 64] = True
    allowed = allowed[:n_valid, :n_valid]
    qt, kt, vt = (torch.from_numpy(x[0, :n_valid]) for x in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(
        qt[None], kt[None], vt[None], attn_mask=torch.from_numpy(allowed)[None])
    np.testing.assert_allclose(out, ref[0].numpy(), rtol=1e-10, atol=1e-12)


def test_sparse_constant_v_and_identical_keys(oracle_lib):
    rng = np.random.default_rng(22)
    n_pad, d = 64 * 4, 16
    _, q = _bf16(rng, (1, n_pad, d))
    _, k = _bf16(rng, (1, n_pad, d))
    v = np.full((1, n_pad, d), 0.75)
    bmap = np.array([[[0, 2], [1, 3], [0, 1], [2, 3]]], dtype=np.int32)
    rows = np.arange(n_pad - 10)
    out = oracle_lib.sparse_rows(q, k, v, bmap, n_pad - 10, rows)
    np.testing.assert_allclose(out, 0.75, rtol=1e-14)
    # kb = 1 and all keys of the kept block equal -> mean of V over the block's valid tokens
    k2 = np.repeat(k[:, :1], n_pad, axis=1)
    _, v2 = _bf16(rng, (1, n_pad, d))
    bmap1 = np.array([[[3], [3], [3], [3]]], dtype=np.int32)
    n_valid = n_pad - 10
    out = oracle_lib.sparse_rows(q, k2, v2, bmap1, n_valid, np.arange(n_valid))
    np.testing.assert_allclose(out, np.broadcast_to(v2[0, 192:n_valid].mean(axis=0), out.shape),
                               rtol=1e-12, atol=1e-14)


# ------------------------------------------------------------ 3-D rotary
def test_rope_worked_examples(oracle_lib):
    g = json.load(open(os.path.join(GOLDEN, "rope_worked.json")))
    for case in g["cases"]:
        x = np.zeros(64)
        x[case["in_index"]] = 1.0
        y = oracle_lib.rope3d(x, case["pos"], (16, 24, 24))
        expect = np.zeros(64)
        for i, val in case["out"].items():
            expect[int(i)] = val
        np.testing.assert_allclose(y, expect, atol=1e-15, err_msg=case["why"])


@pytest.mark.parametrize("axis", [0, 1, 2])
def test_rope_single_axis_is_textbook_1d(oracle_lib, axis):
    """On one axis, 3-D RoPE is the usual 1-D rotary embedding: pair p as a complex
    number multiplied by exp(i * pos * theta^(-2p/d_axis))."""
    rng = np.random.default_rng(30 + axis)
    split = (32, 48, 48)
    off = (0, 32, 80)[axis]
    da = split[axis]
    x = rng.standard_normal(128)
    for pos in (0, 1, 7, 44):
        pos3 = [0, 0, 0]
        pos3[axis] = pos
        y = oracle_lib.rope3d(x, pos3, split)
        zc = x[off:off + da:2] + 1j * x[off + 1:off + da:2]
        freq = 10000.0 ** (-np.arange(da // 2) * 2.0 / da)
        zr = zc * np.exp(1j * pos * freq)
        np.testing.assert_allclose(y[off:off + da:2], zr.real, atol=1e-12)
        np.testing.assert_allclose(y[off + 1:off + da:2], zr.imag, atol=1e-12)
        rest = np.ones(128, dtype=bool)
        rest[off:off + da] = False
        np.testing.assert_array_equal(y[rest], x[rest])


def test_rope_norm_and_relative_position(oracle_lib):
    rng = np.random.default_rng(33)
    split = (16, 24, 24)
    x, y = rng.standard_normal(64), rng.standard_normal(64)
    np.testing.assert_allclose(np.linalg.norm(oracle_lib.rope3d(x, (5, 9, 13), split)),
                               np.linalg.norm(x), rtol=1e-13)
    np.testing.assert_array_equal(oracle_lib.rope3d(x, (0, 0, 0), split), x)
    a = oracle_lib.rope3d(x, (2, 3, 4), split) @ oracle_lib.rope3d(y, (5, 7, 11), split)
    b = oracle_lib.rope3d(x, (0, 0, 0), split) @ oracle_lib.rope3d(y, (3, 4, 7), split)
    c = oracle_lib.rope3d(x, (10, 20, 30), split) @ oracle_lib.rope3d(y, (13, 24, 37), split)
    np.testing.assert_allclose([a, c], [b, b], rtol=1e-11)


def test_position_raster_order(oracle_lib):
    grid = (4, 5, 6)
    n = 0
    for t in range(4):
        for h in range(5):
            for w in range(6):
                assert oracle_lib.position(n, grid) == (t, h, w)
                n += 1


# ------------------------------------------------------------ low-rank branch
def test_feature_is_elu_plus_one_of_projected_rotation(oracle_lib):
    rng = np.random.default_rng(40)
    grid = (3, 4, 5)
    w = (rng.standard_normal((64, 16)) / 8).astype(np.float32)
    x = rng.standard_normal(64) * 3
    for n in (0, 17, 59):
        f = oracle_lib.lowrank_feature(x, n, grid, w)
        t, h, ww = oracle_lib.position(n, grid)
        u = torch.from_numpy(oracle_lib.rope3d(x, (t, h, ww), (16, 24, 24)) @ w.astype(np.float64))
        np.testing.assert_allclose(f, (torch.nn.functional.elu(u) + 1).numpy(), rtol=1e-12, atol=1e-15)
        assert np.all(f > 0)


def test_linear_branch_matches_quadratic_form(oracle_lib):
    rng = np.random.default_rng(41)
    grid = (2, 8, 12)
    n_valid = 2 * 8 * 12  # 192 = 3 blocks
    n_pad, d, r = 192, 64, 16
    _, q = _bf16(rng, (2, n_pad, d))
    _, k = _bf16(rng, (2, n_pad, d))
    _, v = _bf16(rng, (2, n_pad, d))
    wq = (rng.standard_normal((d, r)) / 8).astype(np.float32)
    wk = (rng.standard_normal((d, r)) / 8).astype(np.float32)
    S, z = oracle_lib.lowrank_state(k, v, wk, n_valid, grid)
    rows = np.arange(2 * n_pad)
    out = oracle_lib.lowrank_rows(q, wq, S, z, grid, rows).reshape(2, n_pad, d)
    for bh in range(2):
        a = np.stack([oracle_lib.lowrank_feature(q[bh, n], n, grid, wq) for n in range(n_valid)])
        b = np.stack([oracle_lib.lowrank_feature(k[bh, n], n, grid, wk) for n in range(n_valid)])
        att = a @ b.T  # [N, N] kernel weights, all > 0
        ref = (att @ v[bh, :n_valid]) / att.sum(axis=1, keepdims=True)
        np.testing.assert_allclose(out[bh, :n_valid], ref, rtol=1e-10, atol=1e-12)


def test_forward_constant_v_gives_twice_constant(oracle_lib):
    from sparse_rank_attention_amd.workloads import WORKLOADS, make_proj, make_qkv
    w = WORKLOADS["tiny"]
    q, k, _ = make_qkv(w)
    wq, wk = make_proj(w)
    n_valid = w.n_tokens - 37  # exercise a ragged tail with padding
    v = np.full(q.shape, to_bf16_bits(np.array([-1.25], dtype=np.float32))[0], dtype=np.uint16)
    bmap, out = oracle_lib.forward(q[0], k[0], v[0], wq, wk, n_valid, oracle.keep_blocks(w.topk, w.nb), w.grid)
    np.testing.assert_allclose(out[:, :n_valid], -2.5, rtol=1e-12)
    assert np.all(out[:, n_valid:] == 0)


def test_forward_is_sum_of_pinned_parts(oracle_lib):
    from sparse_rank_attention_amd.workloads import WORKLOADS, make_proj, make_qkv
    w = WORKLOADS["tiny"]
    q, k, v = (x[0] for x in make_qkv(w))
    wq, wk = make_proj(w)
    bmap, out = oracle_lib.forward(q, k, v, wq, wk, w.n_tokens, oracle.keep_blocks(w.topk, w.nb), w.grid)
    np.testing.assert_array_equal(bmap, oracle_lib.block_map(q, k, w.n_tokens, oracle.keep_blocks(w.topk, w.nb)))
    qd, kd, vd = (oracle_lib.widen_bf16(x) for x in (q, k, v))
    rows = np.arange(q.shape[0] * w.n_pad)
    sp = oracle_lib.sparse_rows(qd, kd, vd, bmap, w.n_tokens, rows)
    S, z = oracle_lib.lowrank_state(kd, vd, wk, w.n_tokens, w.grid)
    lr = oracle_lib.lowrank_rows(qd, wq, S, z, w.grid, rows)
    np.testing.assert_allclose(out.reshape(-1, w.head_dim), sp + lr, rtol=1e-12, atol=1e-14)


# ------------------------------------------------------------ output gate
def test_gate_closed_forms(oracle_lib):
    rng = np.random.default_rng(47)
    d = 64
    _, q = _bf16(rng, (d,))
    zero = np.zeros(d + 1, dtype=np.float32)
    assert oracle_lib.gate(q, zero) == 0.5
    g = zero.copy()
    g[d] = np.float32(np.log(3.0))
    assert abs(oracle_lib.gate(q, g) - 0.75) < 1e-7  # sigmoid(ln 3) = 3/4 (bias rounded to fp32)
    # a unit weight picks one query component: sigmoid(1 + ln 3 - 1)
    q1 = q.copy()
    q1[17] = 1.0
    g = zero.copy()
    g[17], g[d] = 1.0, np.float32(np.log(3.0) - 1.0)
    assert abs(oracle_lib.gate(q1, g) - 0.75) < 1e-7
    # sigmoid(-u) = 1 - sigmoid(u), and a random gate against torch's sigmoid of the dot product
    w = (rng.standard_normal(d + 1) / 4).astype(np.float32)
    u = torch.tensor(q) @ torch.tensor(w[:d], dtype=torch.float64) + float(w[d])
    assert abs(oracle_lib.gate(q, w) - torch.sigmoid(u).item()) < 1e-15
    assert abs(oracle_lib.gate(q, w) + oracle_lib.gate(q, -w) - 1.0) < 1e-15


def test_forward_gate_scales_only_the_lowrank_term(oracle_lib):
    from sparse_rank_attention_amd.workloads import WORKLOADS, make_proj, make_qkv
    w = WORKLOADS["tiny"]
    q, k, v = (x[0] for x in make_qkv(w))
    wq, wk = make_proj(w)
    d = w.head_dim
    n_valid = w.n_tokens - 37
    qd, kd, vd = (oracle_lib.widen_bf16(x) for x in (q, k, v))
    bmap, plain = oracle_lib.forward(q, k, v, wq, wk, n_valid, oracle.keep_blocks(w.topk, w.nb), w.grid)
    rows = np.arange(q.shape[0] * w.n_pad)
    sp = oracle_lib.sparse_rows(qd, kd, vd, bmap, n_valid, rows)
    S, z = oracle_lib.lowrank_state(kd, vd, wk, n_valid, w.grid)
    lr = oracle_lib.lowrank_rows(qd, wq, S, z, w.grid, rows)
    valid = (rows % w.n_pad) < n_valid
    # a saturated gate is exactly the ungated forward; a shut one leaves the sparse branch alone
    g = np.zeros(d + 1, dtype=np.float32)
    g[d] = 800.0
    _, out = oracle_lib.forward(q, k, v, wq, wk, n_valid, oracle.keep_blocks(w.topk, w.nb), w.grid, gate_w=g)
    np.testing.assert_array_equal(out, plain)
    g[d] = -800.0
    _, out = oracle_lib.forward(q, k, v, wq, wk, n_valid, oracle.keep_blocks(w.topk, w.nb), w.grid, gate_w=g)
    np.testing.assert_allclose(out.reshape(-1, d)[valid], sp[valid], rtol=1e-12, atol=1e-14)
    # constant gate 3/4
    g[d] = np.float32(np.log(3.0))
    _, out = oracle_lib.forward(q, k, v, wq, wk, n_valid, oracle.keep_blocks(w.topk, w.nb), w.grid, gate_w=g)
    gv = 1.0 / (1.0 + np.exp(-np.float64(g[d])))
    np.testing.assert_allclose(out.reshape(-1, d)[valid], (sp + gv * lr)[valid], rtol=1e-12, atol=1e-14)
    # a per-token gate reads the token's own unrotated query: one weight on component 5
    g = np.zeros(d + 1, dtype=np.float32)
    g[5], g[d] = 1.5, -0.25
    _, out = oracle_lib.forward(q, k, v, wq, wk, n_valid, oracle.keep_blocks(w.topk, w.nb), w.grid, gate_w=g)
    qf = qd.reshape(-1, d)
    gt = torch.sigmoid(torch.tensor(1.5 * qf[:, 5] - 0.25)).numpy()[:, None]
    np.testing.assert_allclose(out.reshape(-1, d)[valid], (sp + gt * lr)[valid], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(oracle_lib.lowrank_rows(qd, wq, S, z, w.grid, rows, gate_w=g),
                               gt * lr, rtol=1e-12, atol=1e-14)
    assert np.all(out.reshape(-1, d)[~valid] == 0)


# ------------------------------------------------------------------- fp8
def test_e4m3_values_match_torch():
    pytest.importorskip("torch")
    import oracle
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = np.array([oracle.e4m3_value(c) for c in range(256)])
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(ours))
    np.testing.assert_array_equal(ours[~nan], ref[~nan])


def test_e4m3_encode_matches_torch_rne():
    import oracle
    rng = np.random.default_rng(50)
    y = np.concatenate([rng.uniform(-448, 448, 3000), rng.uniform(-1, 1, 2000) * 2.0 ** -6,
                        np.array([0.0, -0.0, 448.0, -448.0, 2.0 ** -9, 1.5 * 2.0 ** -9])]).astype(np.float32)
    # exact midpoints between neighbouring codes: ties go to the even code
    mids = [(oracle.e4m3_value(c) + oracle.e4m3_value(c + 1)) / 2 for c in range(0, 0x7e)]
    y = np.concatenate([y, np.array(mids, dtype=np.float32)])
    ours = np.array([oracle.e4m3_encode(float(t)) for t in y], dtype=np.uint8)
    ref = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(ours, ref)
    assert oracle.e4m3_encode(1000.0) == 0x7E and oracle.e4m3_encode(-1000.0) == 0xFE


def test_quant_round_trip_bound(oracle_lib):
    rng = np.random.default_rng(51)
    xb, xf = _bf16(rng, (2, 192, 32), scale=3.0)
    n_valid = 170
    codes, scale, deq = oracle_lib.quant_e4m3(xb, n_valid)
    for bh in range(2):
        for c in range(3):
            lo, hi = 64 * c, min(64 * c + 64, n_valid)
            blk = xf[bh, lo:hi]
            amax = np.abs(blk).max()
            assert scale[bh, c] == np.float32(np.float32(amax) / np.float32(448.0))
            err = np.abs(deq[bh, lo:hi] - blk)
            # half an e4m3 step: 2^-4 relative for normals, 2^-10 * scale absolute below 2^-6 * scale
            bound = np.maximum(np.abs(blk) * 2.0 ** -4, 2.0 ** -10 * scale[bh, c]) * (1 + 1e-6)
            assert np.all(err <= bound)
            assert np.isclose(np.abs(deq[bh, lo:hi]).max(), 448.0 * scale[bh, c], rtol=1e-6)
    assert np.all(codes[:, n_valid:] == 0)


# ------------------------------------------------------- complement scope
def _tiny_complement_case(rng, n_valid, n_pad, d, r):
    _, q = _bf16(rng, (n_pad, d))
    _, k = _bf16(rng, (n_pad, d))
    _, v = _bf16(rng, (n_pad, d))
    wq = (rng.standard_normal((d, r)) / 8).astype(np.float32)
    wk = (rng.standard_normal((d, r)) / 8).astype(np.float32)
    return q, k, v, wq, wk


def test_block_states_partition_the_global_state(oracle_lib):
    rng = np.random.default_rng(51)
    grid = (3, 7, 11)  # N = 231: four blocks, the last with 39 tokens
    n_valid, n_pad, d, r = 231, 256, 64, 16
    _, k, v, _, wk = _tiny_complement_case(rng, n_valid, n_pad, d, r)
    Sb, zb = oracle_lib.lowrank_block_states(k, v, wk, n_valid, grid)
    S, z = oracle_lib.lowrank_state(k[None], v[None], wk, n_valid, grid)
    np.testing.assert_allclose(Sb.sum(axis=0), S[0], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(zb.sum(axis=0), z[0], rtol=1e-12)
    # block 3 holds exactly tokens 192..230
    b = np.stack([oracle_lib.lowrank_feature(k[n], n, grid, wk) for n in range(192, 231)])
    np.testing.assert_allclose(zb[3], b.sum(axis=0), rtol=1e-12)
    np.testing.assert_allclose(Sb[3], b.T @ v[192:231], rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("kb", [1, 2, 4])
def test_complement_matches_token_quadratic_form(oracle_lib, kb):
    """Row n of query block i: sum over valid tokens m outside i's kept blocks of
    (a_n . b_m) v_m, over the sum of a_n . b_m (kb = nb leaves nothing: 0)."""
    rng = np.random.default_rng(53 + kb)
    grid = (3, 7, 11)
    n_valid, n_pad, d, r = 231, 256, 64, 16
    q, k, v, wq, wk = _tiny_complement_case(rng, n_valid, n_pad, d, r)
    nb = n_pad // 64
    bmap = np.stack([np.sort(rng.choice(nb, size=kb, replace=False)) for _ in range(nb)]).astype(np.int32)
    Sb, zb = oracle_lib.lowrank_block_states(k, v, wk, n_valid, grid)
    rows = np.arange(n_valid)
    got = oracle_lib.lowrank_rows_complement(q, wq, Sb, zb, bmap, grid, rows)
    a = np.stack([oracle_lib.lowrank_feature(q[n], n, grid, wq) for n in range(n_valid)])
    b = np.stack([oracle_lib.lowrank_feature(k[m], m, grid, wk) for m in range(n_valid)])
    for n in rows:
        keep = np.isin(np.arange(n_valid) // 64, bmap[n // 64], invert=True)
        if not keep.any():
            assert np.all(got[n] == 0)
            continue
        wts = b[keep] @ a[n]
        ref = wts @ v[:n_valid][keep] / wts.sum()
        np.testing.assert_allclose(got[n], ref, rtol=1e-10, atol=1e-12)


def test_forward_complement_scope(oracle_lib):
    """Whole forward: constant V still gives twice the constant, keeping every
    block leaves the sparse branch alone, and the output is the sum of the parts."""
    from sparse_rank_attention_amd.workloads import WORKLOADS, make_proj, make_qkv
    w = WORKLOADS["tiny"]
    q, k, v = (x[0] for x in make_qkv(w))
    wq, wk = make_proj(w)
    n_valid = w.n_tokens - 37
    cval = to_bf16_bits(np.array([0.75], dtype=np.float32))[0]
    _, out = oracle_lib.forward(q, k, np.full_like(v, cval), wq, wk, n_valid, oracle.keep_blocks(w.topk, w.nb), w.grid, complement=True)
    np.testing.assert_allclose(out[:, :n_valid], 1.5, rtol=1e-12)
    qd, kd, vd = (oracle_lib.widen_bf16(x) for x in (q, k, v))
    bmap, out = oracle_lib.forward(q, k, v, wq, wk, n_valid, w.nb, w.grid, complement=True)
    rows = np.arange(q.shape[0] * w.n_pad)
    valid = (rows % w.n_pad) < n_valid
    sp = oracle_lib.sparse_rows(qd, kd, vd, bmap, n_valid, rows)
    np.testing.assert_allclose(out.reshape(-1, w.head_dim)[valid], sp[valid], rtol=1e-12, atol=1e-14)
    g = (np.arange(w.head_dim + 1) % 5 - 2).astype(np.float32) / 8
    bmap, out = oracle_lib.forward(q, k, v, wq, wk, n_valid, oracle.keep_blocks(w.topk, w.nb), w.grid, complement=True, gate_w=g)
    sp = oracle_lib.sparse_rows(qd, kd, vd, bmap, n_valid, rows)
    for bh in range(q.shape[0]):
        Sb, zb = oracle_lib.lowrank_block_states(kd[bh], vd[bh], wk, n_valid, w.grid)
        lr = oracle_lib.lowrank_rows_complement(qd[bh], wq, Sb, zb, bmap[bh], w.grid, np.arange(n_valid),
                                                gate_w=g)
        np.testing.assert_allclose(out[bh, :n_valid], sp[bh * w.n_pad:bh * w.n_pad + n_valid] + lr,
                                   rtol=1e-12, atol=1e-14)
    assert np.all(out[:, n_valid:] == 0)
