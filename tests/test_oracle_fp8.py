"""Pins for the oracle's keep count and its fp8 mode, against things other than
the oracle itself: exact rational arithmetic for the keep count, torch's
float8_e4m3fn rounding for the per-block codes, and, for the fp8 forward, the
composition the definition states (selection and the low-rank branch on the
bf16 values, the sparse branch on the dequantised ones), with the wrong
compositions shown to differ on the same inputs.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from sparse_rank_attention_amd import workloads as W
from sparse_rank_attention_amd.workloads import to_bf16_bits


# ------------------------------------------------------------ keep count
@pytest.mark.parametrize("topk,nb,kb", [(0.25, 16, 4), (0.10, 512, 51), (0.05, 512, 25), (0.03, 1182, 35),
                                        (0.10, 1182, 118), (0.05, 1182, 59), (1.0, 1182, 1182), (0.5, 1, 1),
                                        (0.001, 100, 1)])
def test_keep_blocks_of_the_configurations(topk, nb, kb):
    """configs: 4 of 16 blocks at topk 0.25; floor(topk * nb) at the Wan sizes;
    at least one block, at most all of them."""
    assert oracle.keep_blocks(topk, nb) == kb


def test_keep_blocks_is_the_decimal_floor():
    """floor(topk * nb) computed exactly from the decimal ratio (two decimals,
    0.01 .. 1.00) for block counts up to the library's limit of 4096."""
    rng = np.random.default_rng(7)
    nbs = np.unique(np.concatenate([np.arange(1, 200), rng.integers(200, 4097, 300), [4000, 4096]]))
    for c in range(1, 101):
        t = Fraction(c, 100)
        for nb in nbs:
            want = max(1, min(int(nb), int(t * int(nb))))
            assert oracle.keep_blocks(float(t), int(nb)) == want, (c, nb)


# ------------------------------------------------ per-block e4m3 quantiser
def _blocks_with_mixed_magnitudes(rng, bh, n_pad, d):
    x = rng.standard_normal((bh, n_pad, d)).astype(np.float32)
    # a power-of-two magnitude per (bh, block), so that a scale taken per
    # block, per row or globally would give different codes
    e = rng.integers(-12, 9, size=(bh, n_pad // 64, 1, 1)).astype(np.float32)
    x = (x.reshape(bh, n_pad // 64, 64, d) * np.float32(2.0) ** e).reshape(bh, n_pad, d)
    x[0, 64:128] = 0.0  # an all-zero block
    return to_bf16_bits(x)


def test_block_codes_are_torch_rne_of_the_scaled_block():
    """Codes are torch's RNE e4m3 conversion of x * fl32(448/absmax) per
    (bh, 64-token block), absmax over the block's valid tokens only; the
    scale is fl32(absmax/448) (1 for a zero block); padded rows give code 0."""
    rng = np.random.default_rng(11)
    bh, n_pad, d, n_valid = 2, 256, 32, 211
    xb = _blocks_with_mixed_magnitudes(rng, bh, n_pad, d)
    xb[:, n_valid:] = to_bf16_bits(np.full((bh, n_pad - n_valid, d), 1e4, np.float32))  # ignored padding
    codes, scale, deq = oracle.quant_e4m3(xb, n_valid)
    x = oracle.widen_bf16(xb).astype(np.float32)
    for b in range(bh):
        for c in range(n_pad // 64):
            lo, hi = 64 * c, min(64 * c + 64, n_valid)
            blk = x[b, lo:hi]
            amax = np.float32(np.abs(blk).max())
            if amax == 0:
                assert scale[b, c] == 1.0 and not codes[b, lo:hi].any()
                continue
            y = torch.from_numpy(blk * (np.float32(448.0) / amax))  # fp32 product
            ref = y.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
            np.testing.assert_array_equal(codes[b, lo:hi], ref)
            assert scale[b, c] == np.float32(amax / np.float32(448.0))
            assert (codes[b, lo:hi] & 0x7F).max() == 0x7E
    assert not codes[:, n_valid:].any() and not deq[:, n_valid:].any()
    vals = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    sc = np.repeat(scale.astype(np.float64), 64, axis=1)[:, :, None]
    np.testing.assert_array_equal(deq, vals * sc)


# ----------------------------------------------------- fp8 forward
def _case():
    w = W.Workload("f", 1, 2, 64, (3, 9, 14), 0.25, 16, "field", seed=0)  # 378 tokens: ragged tail
    q, k, v = W.make_qkv(w)
    wq, wk = W.make_proj(w)
    return w, q[0], k[0], v[0], wq, wk


def test_fp8_forward_is_selection_and_lowrank_on_bf16_plus_sparse_on_codes():
    w, q, k, v, wq, wk = _case()
    kb = oracle.keep_blocks(w.topk, w.nb)
    bmap, out = oracle.forward(q, k, v, wq, wk, w.n_tokens, kb, w.grid, fp8=True)

    sel = oracle.block_map(q, k, w.n_tokens, kb)                 # bf16 selection
    qd, kd, vd = (oracle.quant_e4m3(x, w.n_tokens)[2] for x in (q, k, v))
    qf, kf, vf = (oracle.widen_bf16(x) for x in (q, k, v))
    rows = np.array([h * w.n_pad + n for h in range(w.heads) for n in range(w.n_tokens)])
    sp = oracle.sparse_rows(qd, kd, vd, sel, w.n_tokens, rows)   # sparse branch on the codes
    S, z = oracle.lowrank_state(kf, vf, wk, w.n_tokens, w.grid)  # low-rank branch on bf16
    lr = oracle.lowrank_rows(qf, wq, S, z, w.grid, rows)
    want = (sp + lr).reshape(w.heads, w.n_tokens, -1)
    np.testing.assert_array_equal(bmap, sel)
    np.testing.assert_allclose(out[:, :w.n_tokens], want, rtol=1e-12, atol=1e-12)
    assert not out[:, w.n_tokens:].any()

    # the wrong compositions differ on these inputs, so the checks above would see them
    gap = lambda a: np.abs(a.reshape(want.shape) - want).max() / np.sqrt((want ** 2).mean())
    assert gap(oracle.sparse_rows(qf, kf, vf, sel, w.n_tokens, rows) + lr) > 1e-2  # sparse on bf16
    S8, z8 = oracle.lowrank_state(kd, vd, wk, w.n_tokens, w.grid)
    assert gap(sp + oracle.lowrank_rows(qf, wq, S8, z8, w.grid, rows)) > 1e-3      # state on codes
    assert gap(sp + oracle.lowrank_rows(qd, wq, S, z, w.grid, rows)) > 1e-3        # apply on codes
    # selection from the dequantised values gives another map on these inputs
    q8b, k8b = (to_bf16_bits(x.astype(np.float32)) for x in (qd, kd))
    assert not np.array_equal(oracle.block_map(q8b, k8b, w.n_tokens, kb), sel)
